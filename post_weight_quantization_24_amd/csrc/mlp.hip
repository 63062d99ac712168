// The MLP of a decoder layer on quantized gate_proj and up_proj (page "大模型常见的量化方式",
// section on the layers of a large model: the LLaMA MLP with gate_proj, up_proj, down_proj;
// read as the LLaMA definition down(silu(gate x) * up x)):
//     Y = silu(X G^T) * (X U^T),  silu(a) = a / (1 + exp(-a)),
// written in float16 as down_proj's calibration input when a block is quantized layer by
// layer.  G and U are dequantized once into one float32 [2 d_ff x d] matrix (gate rows, then
// up rows); the tokens go through in chunks: X chunk to float32, one fp32 MFMA product
// against both weight matrices (N = 2 d_ff), then silu and the product into float16.

#include <cmath>

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int64_t MLP_CHUNK = 8192;   // tokens per product

// W^ rows [row0, row0 + rows) of the packed layer into dst (float32, row stride d).
__global__ void __launch_bounds__(256)
mlp_dequant(const uint32_t* __restrict__ qweight, const float* __restrict__ scales,
            const uint8_t* __restrict__ zeros, int64_t rows, int64_t d, int bits, int64_t g,
            float* __restrict__ dst) {
  const int64_t n = rows * d;
  const int64_t words_per_row = d * bits / 32;
  const int64_t n_groups = d / g;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / d, c = i % d;
    const int64_t bit = c * bits;
    const uint32_t* wr = qweight + r * words_per_row;
    uint64_t two = wr[bit / 32];
    if ((bit % 32) + bits > 32) two |= (uint64_t)wr[bit / 32 + 1] << 32;
    const uint32_t code = (uint32_t)(two >> (bit % 32)) & mask;
    const float s = scales[r * n_groups + c / g];
    const float z = (float)zeros[r * n_groups + c / g];
    dst[i] = (float)((double)s * ((double)code - (double)z));
  }
}

__global__ void __launch_bounds__(256)
mlp_x_to_f32(const _Float16* __restrict__ X, int64_t ldx, int64_t rows, int64_t d,
             float* __restrict__ dst) {
  const int64_t n = rows * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / d, c = i % d;
    dst[i] = (float)X[r * ldx + c];
  }
}

// Y[t][j] = float16(silu(A[t][j]) * A[t][d_ff + j]) for the chunk's rows.
__global__ void __launch_bounds__(256)
mlp_act(const float* __restrict__ A, int64_t rows, int64_t d_ff, _Float16* __restrict__ Y,
        int64_t ldy) {
  const int64_t n = rows * d_ff;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / d_ff, j = i % d_ff;
    const float a = A[t * 2 * d_ff + j];
    const float b = A[t * 2 * d_ff + d_ff + j];
    Y[t * ldy + j] = (_Float16)(a / (1.0f + expf(-a)) * b);
  }
}

unsigned grid_of(int64_t n) {
  const int64_t g = ceil_div(n, 256);
  return (unsigned)(g < 16384 ? g : 16384);
}

}  // namespace

void dequant_rows_f32(const uint32_t* q, const float* sc, const uint8_t* z, int64_t rows,
                      int64_t d, int bits, int64_t g, float* dst, hipStream_t s) {
  hipLaunchKernelGGL(mlp_dequant, dim3(grid_of(rows * d)), dim3(256), 0, s, q, sc, z, rows, d,
                     bits, g, dst);
}

void f16_rows_to_f32(const _Float16* X, int64_t ldx, int64_t rows, int64_t d, float* dst,
                     hipStream_t s) {
  hipLaunchKernelGGL(mlp_x_to_f32, dim3(grid_of(rows * d)), dim3(256), 0, s, X, ldx, rows, d, dst);
}

size_t mlp_ws_bytes(int64_t n_tok, int64_t d, int64_t d_ff) {
  const int64_t t = n_tok < MLP_CHUNK ? n_tok : MLP_CHUNK;
  return align_up((size_t)2 * d_ff * d * sizeof(float), 256) +
         align_up((size_t)t * d * sizeof(float), 256) +
         align_up((size_t)t * 2 * d_ff * sizeof(float), 256);
}

hipError_t mlp_launch(const void* X, int64_t n_tok, int64_t d, int64_t ldx,
                      const uint32_t* qg, const float* sg, const uint8_t* zg,
                      const uint32_t* qu, const float* su, const uint8_t* zu, int64_t d_ff,
                      int bits, int group, void* Y, int64_t ldy, void* ws, hipStream_t s) {
  const int64_t g = group == 0 ? d : group;
  char* p = static_cast<char*>(ws);
  float* Wcat = reinterpret_cast<float*>(p);
  p += align_up((size_t)2 * d_ff * d * sizeof(float), 256);
  const int64_t tmax = n_tok < MLP_CHUNK ? n_tok : MLP_CHUNK;
  float* X32 = reinterpret_cast<float*>(p);
  p += align_up((size_t)tmax * d * sizeof(float), 256);
  float* A = reinterpret_cast<float*>(p);
  hipError_t e;
  {
    ProfScope ps("mlp_elementwise", s);
    dequant_rows_f32(qg, sg, zg, d_ff, d, bits, g, Wcat, s);
    dequant_rows_f32(qu, su, zu, d_ff, d, bits, g, Wcat + d_ff * d, s);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const _Float16* Xh = static_cast<const _Float16*>(X);
  _Float16* Yh = static_cast<_Float16*>(Y);
  for (int64_t t0 = 0; t0 < n_tok; t0 += MLP_CHUNK) {
    const int64_t rows = n_tok - t0 < MLP_CHUNK ? n_tok - t0 : MLP_CHUNK;
    {
      ProfScope ps("mlp_elementwise", s);
      f16_rows_to_f32(Xh + t0 * ldx, ldx, rows, d, X32, s);
    }
    // A = X32 [rows x d] times Wcat^T (op(B)[k][n] = Wcat[n][k])
    if ((e = gemm_f32({rows, 2 * d_ff, d, X32, d, 0, 0, Wcat, d, 1, 0, A, 2 * d_ff, 0, 1.0f, 0.0f},
                      s, "mlp_gemm")) != hipSuccess)
      return e;
    {
      ProfScope ps("mlp_elementwise", s);
      hipLaunchKernelGGL(mlp_act, dim3(grid_of(rows * d_ff)), dim3(256), 0, s, A, rows, d_ff,
                         Yh + t0 * ldy, ldy);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gptq
