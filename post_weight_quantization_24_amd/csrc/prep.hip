// Inverse factor G = Cholesky((H + lambda I)^-1)^T (page "量化", section GPTQ: the
// Cholesky reformulation; damping lambda = frac * mean(diag H) is not on the pages).
//
// G is computed without forming an inverse.  With A = H + lambda I = U U^T, U upper,
// G = U^-1 is upper with G^T G = A^-1 and positive diagonal, hence the same unique
// factor.  A recursion on the 2x2 block split A = [[A11, A12], [A12^T, A22]]:
//     G22 = factor(A22)                     (recursion)
//     P   = A12 G22^T                       (= U12)
//     A12 <- P G22
//     A11 <- A11 - P P^T                    (Schur complement, upper triangle only)
//     G11 = factor(A11)                     (recursion)
//     G12 = -G11 (P G22) = -G11 A12
// All products run on the fp32 MFMA GEMM; blocks of at most 128 are factored and
// inverted by one workgroup in LDS.  Everything happens in the upper triangle of G;
// the strictly lower triangle is zeroed at the end.

#include <climits>

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int NB = 128;           // leaf size
constexpr int LEAF_LD = NB + 1;   // LDS row stride

struct PrepWs {
  double* lambda;
  int* flag;
  float* tmp;
};

PrepWs carve(void* ws, int64_t d) {
  char* p = static_cast<char*>(ws);
  PrepWs w;
  w.lambda = reinterpret_cast<double*>(p);
  w.flag = reinterpret_cast<int*>(p + 8);
  w.tmp = reinterpret_cast<float*>(p + 256);
  return w;
}

// lambda = frac * mean(diag H) in double with a fixed reduction order; flag reset.
__global__ void __launch_bounds__(256)
damp_lambda(const float* __restrict__ H, int64_t d, float frac, double* lambda, int* flag) {
  __shared__ double s[256];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 256) acc += (double)H[i * d + i];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = s[0] / (double)d;
    *lambda = (double)frac * mean;
    *flag = (mean > 0.0 && mean < 1e300) ? INT_MAX : 1;
  }
}

// Upper triangle of G <- upper triangle of H, diagonal + lambda (safe when G == H).
// Row-wise helpers: rows stride over gridDim.y, columns over gridDim.x * 256.
__global__ void __launch_bounds__(256)
copy_damp(const float* H, float* G, int64_t d, const double* lambda) {
  const float lam = (float)*lambda;
  for (int64_t i = blockIdx.y; i < d; i += gridDim.y)
    for (int64_t j = i + blockIdx.x * 256 + threadIdx.x; j < d; j += (int64_t)gridDim.x * 256) {
      float v = H[i * d + j];
      if (j == i) v += lam;
      G[i * d + j] = v;
    }
}

__global__ void __launch_bounds__(256) zero_lower(float* __restrict__ G, int64_t d) {
  for (int64_t i = blockIdx.y; i < d; i += gridDim.y)
    for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < i; j += (int64_t)gridDim.x * 256)
      G[i * d + j] = 0.0f;
}

__global__ void __launch_bounds__(256)
copy_block(const float* __restrict__ src, int64_t lds, float* __restrict__ dst, int64_t ldd,
           int64_t rows, int64_t cols) {
  for (int64_t i = blockIdx.y; i < rows; i += gridDim.y)
    for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < cols; j += (int64_t)gridDim.x * 256)
      dst[i * ldd + j] = src[i * lds + j];
}

dim3 rows_grid(int64_t rows, int64_t cols) {
  const int64_t gx = (cols + 255) / 256;
  return dim3((unsigned)(gx < 1 ? 1 : gx > 64 ? 64 : gx), (unsigned)(rows > 32768 ? 32768 : rows));
}

// Factor the n x n diagonal block at (off, off) as U U^T (U upper) and overwrite its
// upper triangle with G = U^-1.  One workgroup; 16 x 16 threads stride over the block.
__global__ void __launch_bounds__(256)
leaf_factor_invert(float* __restrict__ A, int64_t ld, int64_t off, int n, int* flag) {
  extern __shared__ float smem[];
  float* S = smem;                    // factor, upper triangle
  float* R = smem + NB * LEAF_LD;     // inverse being built, upper triangle
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float* blk = A + off * ld + off;

  for (int i = ty; i < n; i += 16)
    for (int j = tx; j < n; j += 16) {
      S[i * LEAF_LD + j] = (j >= i) ? blk[i * ld + j] : 0.0f;
      R[i * LEAF_LD + j] = (i == j) ? 1.0f : 0.0f;
    }
  __syncthreads();

  // A = U U^T from the bottom-right corner: outer-product updates with unscaled columns.
  for (int k = n - 1; k > 0; --k) {
    const float rp = 1.0f / S[k * LEAF_LD + k];
    for (int j = tx; j < k; j += 16) {
      const float sjk = S[j * LEAF_LD + k] * rp;
      for (int i = ty; i <= j; i += 16) S[i * LEAF_LD + j] -= S[i * LEAF_LD + k] * sjk;
    }
    __syncthreads();
  }
  // pivots are now final on the diagonal
  if (threadIdx.x == 0) {
    for (int k = 0; k < n; ++k) {
      const float p = S[k * LEAF_LD + k];
      if (!(p > 0.0f) || !(p < 3.0e38f)) {
        atomicMin(flag, (int)(off + k) + 1);
        break;
      }
    }
  }
  // scale columns: U[k][k] = sqrt(p_k), U[i][k] = S[i][k] / sqrt(p_k)
  for (int j = tx; j < n; j += 16) {
    const float u = sqrtf(S[j * LEAF_LD + j]);
    for (int i = ty; i < j; i += 16) S[i * LEAF_LD + j] /= u;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256) S[j * LEAF_LD + j] = sqrtf(S[j * LEAF_LD + j]);
  __syncthreads();

  // U G = I, rows from the bottom: row k of R is final at step k.
  for (int k = n - 1; k > 0; --k) {
    const float ru = 1.0f / S[k * LEAF_LD + k];
    for (int j = k + tx; j < n; j += 16) {
      const float gkj = R[k * LEAF_LD + j] * ru;
      for (int i = ty; i < k; i += 16) R[i * LEAF_LD + j] -= S[i * LEAF_LD + k] * gkj;
    }
    __syncthreads();
  }
  for (int i = ty; i < n; i += 16) {
    const float ru = 1.0f / S[i * LEAF_LD + i];
    for (int j = tx; j < n; j += 16)
      if (j >= i) blk[i * ld + j] = R[i * LEAF_LD + j] * ru;
  }
}

hipError_t copy2d(const float* src, int64_t lds, float* dst, int64_t ldd, int64_t rows,
                  int64_t cols, hipStream_t s) {
  hipLaunchKernelGGL(copy_block, rows_grid(rows, cols), dim3(256), 0, s, src, lds, dst, ldd, rows,
                     cols);
  return hipGetLastError();
}

hipError_t factor_rec(float* A, int64_t ld, int64_t off, int64_t n, float* tmp, int* flag,
                      hipStream_t s) {
  hipError_t e;
  if (n <= NB) {
    ProfScope ps("prep_leaf", s);
    hipLaunchKernelGGL(leaf_factor_invert, dim3(1), dim3(256), 2 * NB * LEAF_LD * sizeof(float),
                       s, A, ld, off, (int)n, flag);
    return hipGetLastError();
  }
  int64_t m = (n / 2) / NB * NB;
  if (m == 0) m = n - NB;
  const int64_t r = n - m;
  float* A11 = A + off * ld + off;
  float* A12 = A11 + m;
  float* A22 = A + (off + m) * ld + off + m;

  if ((e = factor_rec(A, ld, off + m, r, tmp, flag, s)) != hipSuccess) return e;
  // P = A12 G22^T   (op(B)[k][j] = G22[j][k], zero for k < j)
  if ((e = gemm_f32({m, r, r, A12, ld, 0, 0, A22, ld, 1, 2, tmp, r, 0, 1.0f, 0.0f}, s,
                    "prep_gemm")) != hipSuccess)
    return e;
  // A12 <- P G22    (G22 upper: zero for k > j)
  if ((e = gemm_f32({m, r, r, tmp, r, 0, 0, A22, ld, 0, 1, A12, ld, 0, 1.0f, 0.0f}, s,
                    "prep_gemm")) != hipSuccess)
    return e;
  // A11 <- A11 - P P^T, upper triangle
  if ((e = gemm_f32({m, m, r, tmp, r, 0, 0, tmp, r, 1, 0, A11, ld, 1, -1.0f, 1.0f}, s,
                    "prep_gemm")) != hipSuccess)
    return e;
  if ((e = factor_rec(A, ld, off, m, tmp, flag, s)) != hipSuccess) return e;
  // G12 = -G11 A12   (G11 upper: zero for k < i)
  if ((e = gemm_f32({m, r, m, A11, ld, 0, 1, A12, ld, 0, 0, tmp, r, 0, -1.0f, 0.0f}, s,
                    "prep_gemm")) != hipSuccess)
    return e;
  return copy2d(tmp, r, A12, ld, m, r, s);
}

bool leaf_attr_done = false;

}  // namespace

size_t prepare_ws_bytes(int64_t d) {
  const int64_t h = d / 2;
  return 256 + (size_t)(h * (d - h) + 64) * sizeof(float);
}

int* prepare_flag_ptr(void* ws, int64_t d) { return carve(ws, d).flag; }

hipError_t prepare_launch(const float* H, float* G, int64_t d, float damp_frac, void* ws,
                          hipStream_t stream) {
  hipError_t e;
  if (!leaf_attr_done) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(leaf_factor_invert),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            2 * NB * LEAF_LD * (int)sizeof(float));
    if (e != hipSuccess) return e;
    leaf_attr_done = true;
  }
  PrepWs w = carve(ws, d);
  {
    ProfScope ps("prep_damp", stream);
    hipLaunchKernelGGL(damp_lambda, dim3(1), dim3(256), 0, stream, H, d, damp_frac, w.lambda,
                       w.flag);
    hipLaunchKernelGGL(copy_damp, rows_grid(d, d), dim3(256), 0, stream, H, G, d, w.lambda);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = factor_rec(G, d, 0, d, w.tmp, w.flag, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(zero_lower, rows_grid(d, d), dim3(256), 0, stream, G, d);
  return hipGetLastError();
}

}  // namespace gptq
