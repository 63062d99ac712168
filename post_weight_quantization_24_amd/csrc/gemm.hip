// float32 GEMM on the matrix cores (v_mfma_f32_32x32x2_f32), with optional triangular
// operand masks and an upper-triangle-only output.  It carries the lazy batch update of
// GPTQ (page "量化", section GPTQ, third improvement: the columns right of a block are
// updated in one matrix product), the products of the blocked inverse-factor
// computation, and the Delta*H product of the loss check.
//
// Workgroup: 256 threads = 2x2 waves, tile 128 x 128, each wave 64 x 64 = 2x2 MFMA
// tiles.  K advances 16 at a time through a single LDS stage (k-major, so every MFMA
// operand read is one conflict-free dword per lane), with the next stage prefetched
// into registers while the current one is multiplied.

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int LDA_S = BM + 4, LDB_S = BN + 4;

struct Dev {
  int64_t M, N, K;
  const float* A; int64_t lda; int transA; int triA;
  const float* B; int64_t ldb; int transB; int triB;
  float* C; int64_t ldc; int triC;
  float alpha, beta;
};

__device__ __forceinline__ bool a_ok(const Dev& g, int64_t m, int64_t k) {
  if (m >= g.M || k >= g.K) return false;
  if (g.triA == 1 && k < m) return false;
  if (g.triA == 2 && k > m) return false;
  return true;
}
__device__ __forceinline__ bool b_ok(const Dev& g, int64_t k, int64_t n) {
  if (n >= g.N || k >= g.K) return false;
  if (g.triB == 1 && k > n) return false;
  if (g.triB == 2 && k < n) return false;
  return true;
}
__device__ __forceinline__ float a_at(const Dev& g, int64_t m, int64_t k) {
  return a_ok(g, m, k) ? (g.transA ? g.A[k * g.lda + m] : g.A[m * g.lda + k]) : 0.0f;
}
__device__ __forceinline__ float b_at(const Dev& g, int64_t k, int64_t n) {
  return b_ok(g, k, n) ? (g.transB ? g.B[n * g.ldb + k] : g.B[k * g.ldb + n]) : 0.0f;
}

// Each thread stages 8 elements of op(A) (128 x 16) and 8 of op(B) (16 x 128): two runs
// of 4 elements along the operand's contiguous direction.
template <bool VEC>
__device__ __forceinline__ void load4(const Dev& g, bool isA, int64_t r, int64_t c,
                                      bool along_c, floatx4& v) {
  // isA: (r, c) = (m, k); else (k, n).  along_c: the 4 elements are (r, c..c+3),
  // otherwise (r..r+3, c).
  bool all = true;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t rr = along_c ? r : r + j, cc = along_c ? c + j : c;
    all = all && (isA ? a_ok(g, rr, cc) : b_ok(g, rr, cc));
  }
  if (VEC && all) {
    // contiguous in memory: A row-major with along k (!transA) or along m (transA)
    const float* p;
    if (isA) p = g.transA ? g.A + c * g.lda + r : g.A + r * g.lda + c;
    else p = g.transB ? g.B + c * g.ldb + r : g.B + r * g.ldb + c;
    v = *reinterpret_cast<const floatx4*>(p);
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t rr = along_c ? r : r + j, cc = along_c ? c + j : c;
    v[j] = isA ? a_at(g, rr, cc) : b_at(g, rr, cc);
  }
}

template <bool VEC>
__global__ void __launch_bounds__(256) gemm_f32_mfma(Dev g) {
  __shared__ __attribute__((aligned(16))) float As[BK * LDA_S];
  __shared__ __attribute__((aligned(16))) float Bs[BK * LDB_S];

  const int64_t tiles_n = (g.N + BN - 1) / BN;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
  const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
  if (g.triC == 1 && m0 >= n0 + BN) return;  // tile entirely below the diagonal

  int64_t k_lo = 0, k_hi = g.K;
  if (g.triA == 1) k_lo = m0;
  if (g.triA == 2) k_hi = k_hi < m0 + BM ? k_hi : m0 + BM;
  if (g.triB == 1) k_hi = k_hi < n0 + BN ? k_hi : n0 + BN;
  if (g.triB == 2) k_lo = k_lo > n0 ? k_lo : n0;
  k_lo = k_lo / BK * BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  floatx16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // A element runs: transA -> along m (4 m's at one k): idx -> k = idx/32, m = (idx%32)*4
  //                 !transA -> along k: idx -> m = idx/4, k = (idx%4)*4
  floatx4 ra[2], rb[2];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + i * 256;
      if (g.transA) load4<VEC>(g, true, m0 + (idx % 32) * 4, k0 + idx / 32, false, ra[i]);
      else load4<VEC>(g, true, m0 + idx / 4, k0 + (idx % 4) * 4, true, ra[i]);
      if (g.transB) load4<VEC>(g, false, k0 + (idx % 4) * 4, n0 + idx / 4, false, rb[i]);
      else load4<VEC>(g, false, k0 + idx / 32, n0 + (idx % 32) * 4, true, rb[i]);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + i * 256;
      if (g.transA) {
        const int k = idx / 32, m = (idx % 32) * 4;
        *reinterpret_cast<floatx4*>(&As[k * LDA_S + m]) = ra[i];
      } else {
        const int m = idx / 4, k = (idx % 4) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) As[(k + j) * LDA_S + m] = ra[i][j];
      }
      if (g.transB) {
        const int n = idx / 4, k = (idx % 4) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) Bs[(k + j) * LDB_S + n] = rb[i][j];
      } else {
        const int k = idx / 32, n = (idx % 32) * 4;
        *reinterpret_cast<floatx4*>(&Bs[k * LDB_S + n]) = rb[i];
      }
    }
  };

  if (k_lo < k_hi) load(k_lo);
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + BK < k_hi) load(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
      const int kr = 2 * kk + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = As[kr * LDA_S + wm * 64 + t * 32 + (lane & 31)];
        b[t] = Bs[kr * LDB_S + wn * 64 + t * 32 + (lane & 31)];
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x], b[y], acc[x][y], 0, 0, 0);
    }
  }

#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + x * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 64 + y * 32 + (lane & 31);
        if (m < g.M && n < g.N && (g.triC == 0 || m <= n)) {
          float* p = g.C + m * g.ldc + n;
          const float v = g.alpha * acc[x][y][r];
          *p = g.beta != 0.0f ? v + g.beta * *p : v;
        }
      }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t gemm_f32(const GemmArgs& a, hipStream_t stream, const char* prof_name) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  Dev g{a.M, a.N, a.K, a.A, a.lda, a.transA, a.triA, a.B, a.ldb, a.transB, a.triB,
        a.C, a.ldc, a.triC, a.alpha, a.beta};
  const bool vec = aligned16(a.A) && aligned16(a.B) && (a.lda % 4 == 0) && (a.ldb % 4 == 0);
  const int64_t grid = ceil_div(a.M, BM) * ceil_div(a.N, BN);
  ProfScope ps(prof_name, stream);
  if (vec) hipLaunchKernelGGL(gemm_f32_mfma<true>, dim3(grid), dim3(256), 0, stream, g);
  else hipLaunchKernelGGL(gemm_f32_mfma<false>, dim3(grid), dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace gptq
