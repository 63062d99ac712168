// Dequantization and the layer objective of page "量化", section GPTQ:
// ||W X - W^ X||_F^2 = 1/2 * sum_r D_r H D_r^T with D = W - W^ and the undamped H = 2 X X^T.
// W^ = s * (code - z) per row and group.  H is symmetric, so the loss comes from half the
// product: 1/2 D H D^T = sum T .* D - 1/2 sum D^2 diag(H) per row, with T = D U and U the
// upper triangle of H (the fp32 MFMA GEMM with a triangular operand mask); the row sums and
// the total are accumulated in double in a fixed order.

#include "gptq_internal.h"

namespace gptq {

namespace {

__global__ void __launch_bounds__(256)
dequant(const uint32_t* __restrict__ qweight, const float* __restrict__ scales,
        const uint8_t* __restrict__ zeros, const void* __restrict__ W, int w_dtype, int64_t d_row,
        int64_t d_col, int bits, int64_t g, float* __restrict__ D, float* __restrict__ W_hat) {
  const int64_t n = d_row * d_col;
  const int64_t words_per_row = d_col * bits / 32;
  const int64_t n_groups = d_col / g;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / d_col, c = i % d_col;
    const int64_t bit = c * bits;
    const uint32_t* wr = qweight + r * words_per_row;
    uint64_t two = wr[bit / 32];
    if ((bit % 32) + bits > 32) two |= (uint64_t)wr[bit / 32 + 1] << 32;
    const uint32_t code = (uint32_t)(two >> (bit % 32)) & mask;
    const float s = scales[r * n_groups + c / g];
    const float z = (float)zeros[r * n_groups + c / g];
    const float wh = s * ((float)code - z);
    const float w = w_dtype == 0 ? (float)static_cast<const _Float16*>(W)[i]
                                 : static_cast<const float*>(W)[i];
    D[i] = w - wh;
    if (W_hat) W_hat[i] = wh;
  }
}

__global__ void __launch_bounds__(256)
grid_check(const float* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t n, int bits,
           unsigned long long* __restrict__ off_grid) {
  const int maxq = (1 << bits) - 1;
  unsigned long long bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float s = scales[i];
    if (!(s > 0.0f) || !(s < 3.0e38f) || (int)zeros[i] > maxq) ++bad;
  }
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
  if ((threadIdx.x & 63) == 0 && bad) atomicAdd(off_grid, bad);
}

__global__ void zero_i64(unsigned long long* p) { *p = 0ull; }

// One wave per row, for T = D U with U the upper triangle of H (diagonal included):
// 1/2 D_r H D_r^T = sum_c T[r][c] D[r][c] - 1/2 sum_c D[r][c]^2 H[c][c], in double.
__global__ void __launch_bounds__(256)
row_loss_upper_k(const float* __restrict__ T, const float* __restrict__ D,
                 const float* __restrict__ H, int64_t d_row, int64_t d_col,
                 double* __restrict__ rows) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= d_row) return;
  double acc = 0.0;
  for (int64_t c = lane; c < d_col; c += 64) {
    const double dv = (double)D[r * d_col + c];
    acc += (double)T[r * d_col + c] * dv - 0.5 * dv * dv * (double)H[c * d_col + c];
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) rows[r] = acc;
}

__global__ void __launch_bounds__(256)
sum_rows(const double* __restrict__ rows, int64_t d_row, double* __restrict__ loss,
         double* __restrict__ row_out) {
  __shared__ double s[256];
  double acc = 0.0;
  for (int64_t r = threadIdx.x; r < d_row; r += 256) {
    acc += rows[r];
    if (row_out) row_out[r] = rows[r];
  }
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = s[0];
}

}  // namespace

size_t check_ws_bytes(int64_t d_row, int64_t d_col) {
  return 2 * align_up((size_t)d_row * d_col * sizeof(float), 256) +
         align_up((size_t)d_row * sizeof(double), 256);
}

hipError_t check_launch(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                        const void* W, int w_dtype, const float* H, int64_t d_row, int64_t d_col,
                        int bits, int group, double* loss, double* row_loss, float* W_hat,
                        int64_t* off_grid, void* ws, hipStream_t s) {
  const size_t mat = align_up((size_t)d_row * d_col * sizeof(float), 256);
  float* D = static_cast<float*>(ws);
  float* T = reinterpret_cast<float*>(static_cast<char*>(ws) + mat);
  double* rows = reinterpret_cast<double*>(static_cast<char*>(ws) + 2 * mat);
  const int64_t g = group == 0 ? d_col : group;
  const int64_t n = d_row * d_col;
  ProfScope ps("check", s);
  hipLaunchKernelGGL(dequant, dim3((unsigned)(ceil_div(n, 256) < 8192 ? ceil_div(n, 256) : 8192)),
                     dim3(256), 0, s, qweight, scales, zeros, W, w_dtype, d_row, d_col, bits, g, D,
                     W_hat);
  const int64_t ng = d_row * (d_col / g);
  unsigned long long* og = reinterpret_cast<unsigned long long*>(off_grid);
  hipLaunchKernelGGL(zero_i64, dim3(1), dim3(1), 0, s, og);
  hipLaunchKernelGGL(grid_check, dim3((unsigned)(ceil_div(ng, 256) < 1024 ? ceil_div(ng, 256) : 1024)),
                     dim3(256), 0, s, scales, zeros, ng, bits, og);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return loss_of_diff_upper(D, H, d_row, d_col, loss, row_loss, T, rows, s, "check_gemm");
}

hipError_t loss_of_diff_upper(const float* D, const float* H, int64_t d_row, int64_t d_col,
                              double* loss, double* row_loss, float* T, double* rows, hipStream_t s,
                              const char* prof_name) {
  // op(B) = H masked to its upper triangle (entries with k > n read as zero)
  GemmArgs ga{d_row, d_col, d_col, D, d_col, 0, 0, H, d_col, 0, 1, T, d_col, 0, 1.0f, 0.0f};
  hipError_t e = gemm_f32(ga, s, prof_name);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_loss_upper_k, dim3((unsigned)ceil_div(d_row, 4)), dim3(256), 0, s, T, D,
                     H, d_row, d_col, rows);
  hipLaunchKernelGGL(sum_rows, dim3(1), dim3(256), 0, s, rows, d_row, loss, row_loss);
  return hipGetLastError();
}


}  // namespace gptq
