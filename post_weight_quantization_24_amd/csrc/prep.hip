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
// inverted by one workgroup in registers.  Everything happens in the upper triangle of G;
// the strictly lower triangle is zeroed at the end.

#include <climits>

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int NB = 128;           // leaf size

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
// upper triangle with G = U^-1.  One workgroup of 16 x 16 threads; thread (tx, ty) keeps
// the 8 x 8 tile at rows 8ty.., cols 8tx.. of the symmetric block in registers.  Each
// column step publishes one column (and, for the inverse, one row) through
// double-buffered LDS, so a step costs one barrier plus at most 64 register FMAs.
template <int KK>
__device__ __forceinline__ void chol_step(float (&S)[8][8], int k, int tx, int ty, int i0, int j0,
                                          float (*colbuf)[NB], float* diag, int* bad) {
  const int b = k & 1;
  if (tx == (k >> 3)) {
#pragma unroll
    for (int r = 0; r < 8; ++r) colbuf[b][i0 + r] = S[r][KK];
  }
  __syncthreads();
  const float piv = colbuf[b][k];
  if (threadIdx.x == 0) {
    diag[k] = piv;
    if (!(piv > 0.0f) || !(piv < 3.0e38f)) *bad = k;
  }
  if (i0 < k && j0 < k) {
    const float rp = 1.0f / piv;
    // unconditional 16-byte loads (always in bounds), then masks: no branch per element
    const floatx4* cv = reinterpret_cast<const floatx4*>(colbuf[b]);
    const floatx4 i_lo = cv[i0 / 4], i_hi = cv[i0 / 4 + 1], j_lo = cv[j0 / 4], j_hi = cv[j0 / 4 + 1];
    float ci[8], cj[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ci[r] = (i0 + r < k) ? i_lo[r] : 0.0f;
      ci[r + 4] = (i0 + r + 4 < k) ? i_hi[r] : 0.0f;
      cj[r] = (j0 + r < k) ? j_lo[r] * rp : 0.0f;
      cj[r + 4] = (j0 + r + 4 < k) ? j_hi[r] * rp : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int q = 0; q < 8; ++q) S[r][q] = fmaf(-ci[r], cj[q], S[r][q]);
  }
}

template <int KK>
__device__ __forceinline__ void inv_step(const float (&U)[8][8], float (&R)[8][8], int k, int tx,
                                         int ty, int i0, int j0, float (*ucol)[NB],
                                         float (*rrow)[NB], const float* diag) {
  const int b = k & 1;
  if (tx == (k >> 3)) {
#pragma unroll
    for (int r = 0; r < 8; ++r) ucol[b][i0 + r] = U[r][KK];
  }
  if (ty == (k >> 3)) {
#pragma unroll
    for (int q = 0; q < 8; ++q) rrow[b][j0 + q] = R[KK][q];
  }
  __syncthreads();
  if (i0 < k) {
    const float ru = 1.0f / diag[k];
    const floatx4* uv = reinterpret_cast<const floatx4*>(ucol[b]);
    const floatx4* rv = reinterpret_cast<const floatx4*>(rrow[b]);
    const floatx4 u_lo = uv[i0 / 4], u_hi = uv[i0 / 4 + 1], g_lo = rv[j0 / 4], g_hi = rv[j0 / 4 + 1];
    float uc[8], gk[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uc[r] = (i0 + r < k) ? u_lo[r] : 0.0f;
      uc[r + 4] = (i0 + r + 4 < k) ? u_hi[r] : 0.0f;
      gk[r] = g_lo[r] * ru;
      gk[r + 4] = g_hi[r] * ru;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int q = 0; q < 8; ++q) R[r][q] = fmaf(-uc[r], gk[q], R[r][q]);
  }
}

__global__ void __launch_bounds__(256)
leaf_factor_invert(float* __restrict__ A, int64_t ld, int64_t off, int n, int* flag) {
  __shared__ __attribute__((aligned(16))) float colbuf[2][NB];
  __shared__ __attribute__((aligned(16))) float rowbuf[2][NB];
  __shared__ float diag[NB];
  __shared__ int bad;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int i0 = 8 * ty, j0 = 8 * tx;
  float* blk = A + off * ld + off;
  if (threadIdx.x == 0) bad = -1;

  float S[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = i0 + r, j = j0 + q;
      S[r][q] = (i < n && j < n) ? (j >= i ? blk[(int64_t)i * ld + j] : blk[(int64_t)j * ld + i])
                                 : (i == j ? 1.0f : 0.0f);
    }

  // A = U U^T from the bottom-right corner (outer-product form, columns unscaled).
  for (int kb = NB / 8 - 1; kb >= 0; --kb) {
#define GPTQ_CHOL(KK) \
    if (8 * kb + KK < n) chol_step<KK>(S, 8 * kb + KK, tx, ty, i0, j0, colbuf, diag, &bad);
    GPTQ_CHOL(7) GPTQ_CHOL(6) GPTQ_CHOL(5) GPTQ_CHOL(4)
    GPTQ_CHOL(3) GPTQ_CHOL(2) GPTQ_CHOL(1) GPTQ_CHOL(0)
#undef GPTQ_CHOL
  }
  __syncthreads();
  if (threadIdx.x == 0 && bad >= 0) atomicMin(flag, (int)(off + bad) + 1);
  for (int k = threadIdx.x; k < n; k += 256) diag[k] = sqrtf(diag[k]);
  __syncthreads();
  // scale to U: U[i][j] = S[i][j] / sqrt(p_j) above the diagonal, sqrt(p_j) on it
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = i0 + r, j = j0 + q;
      const float dj = j < n ? diag[j] : 1.0f;
      S[r][q] = i < j ? S[r][q] / dj : (i == j ? dj : 0.0f);
    }

  // U G = I from the bottom row up; R holds the rows of G not yet divided by U[i][i].
  float R[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int q = 0; q < 8; ++q) R[r][q] = (i0 + r == j0 + q) ? 1.0f : 0.0f;
  for (int kb = NB / 8 - 1; kb >= 0; --kb) {
#define GPTQ_INV(KK) \
    if (8 * kb + KK < n) inv_step<KK>(S, R, 8 * kb + KK, tx, ty, i0, j0, colbuf, rowbuf, diag);
    GPTQ_INV(7) GPTQ_INV(6) GPTQ_INV(5) GPTQ_INV(4)
    GPTQ_INV(3) GPTQ_INV(2) GPTQ_INV(1) GPTQ_INV(0)
#undef GPTQ_INV
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int i = i0 + r;
    if (i >= n) continue;
    const float ru = 1.0f / diag[i];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int j = j0 + q;
      if (j >= i && j < n) blk[(int64_t)i * ld + j] = R[r][q] * ru;
    }
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
    hipLaunchKernelGGL(leaf_factor_invert, dim3(1), dim3(256), 0, s, A, ld, off, (int)n, flag);
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

}  // namespace

size_t prepare_ws_bytes(int64_t d) {
  const int64_t h = d / 2;
  return 256 + (size_t)(h * (d - h) + 64) * sizeof(float);
}

int* prepare_flag_ptr(void* ws, int64_t d) { return carve(ws, d).flag; }

hipError_t prepare_launch(const float* H, float* G, int64_t d, float damp_frac, void* ws,
                          hipStream_t stream) {
  hipError_t e;
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
