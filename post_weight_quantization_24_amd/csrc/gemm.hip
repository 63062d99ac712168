// float32 GEMM on the matrix cores (v_mfma_f32_32x32x2_f32), with optional triangular
// operand masks and an upper-triangle-only output.  It carries the lazy batch update of
// GPTQ (page "量化", section GPTQ, third improvement: the columns right of a block are
// updated in one matrix product), the products of the blocked inverse-factor
// computation, and the Delta*H product of the loss check.
//
// Workgroup: 256 threads = 2x2 waves; tile BM x BN (128 x 128, or 64 x 64 for problems
// too small to fill the chip); each wave computes (BM/2) x (BN/2) with 32x32 MFMA tiles.
// K advances 16 (128-tiles) or 32 (64-tiles) at a time through two LDS stages stored k-major, so every MFMA operand
// read is one conflict-free dword per lane; the next stage is fetched into registers while
// the current one is multiplied (one barrier per K step).  Interior K steps use unmasked
// 16-byte loads from per-step base pointers with 32-bit offsets; only steps that touch a
// matrix edge or a triangular mask take the per-element masked path.
// With beta = 1 the C tile is loaded into the accumulators before the K loop and alpha
// (+1 or -1) is folded into op(A) as it is staged, so the epilogue is a plain store.

#include "gptq_internal.h"

namespace gptq {

namespace {

struct Dev {
  int64_t M, N, K;
  const float* A; int64_t lda; int triA;
  const float* B; int64_t ldb; int triB;
  float* C; int64_t ldc; int triC;
  float alpha, beta;
  int vec;   // operands and leading dimensions allow 16-byte loads
};

template <int BM, int BN, bool TA, bool TB>
struct Cfg {
  // K per LDS stage: 128 x 128 tiles keep 16 so that staging fits two waves per SIMD.
  static constexpr int BK = BM >= 128 ? 16 : 32;
  static constexpr int LDA_S = BM + 4, LDB_S = BN + 4;
  static constexpr int A_V4 = BM * BK / 4 / 256;   // float4 per thread for the A stage
  static constexpr int B_V4 = BN * BK / 4 / 256;
  static constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 MFMA tiles per wave
  static_assert(A_V4 >= 1 && B_V4 >= 1, "tile too small");
};

// Coordinates of the idx-th 4-element run of a stage.  A runs go along k (!TA) or m (TA);
// B runs go along n (!TB) or k (TB): always the operand's contiguous direction in memory.
template <int BM, int BK, bool TA>
__device__ __forceinline__ void a_coords(int idx, int& ml, int& kl) {
  if (!TA) { ml = idx / (BK / 4); kl = (idx % (BK / 4)) * 4; }
  else { kl = idx / (BM / 4); ml = (idx % (BM / 4)) * 4; }
}
template <int BN, int BK, bool TB>
__device__ __forceinline__ void b_coords(int idx, int& kl, int& nl) {
  if (!TB) { kl = idx / (BN / 4); nl = (idx % (BN / 4)) * 4; }
  else { nl = idx / (BK / 4); kl = (idx % (BK / 4)) * 4; }
}

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

template <int BM, int BN, bool TA, bool TB>
__global__ void __launch_bounds__(256, 2) gemm_f32_mfma(Dev g) {
  using C = Cfg<BM, BN, TA, TB>;
  constexpr int BK = C::BK;
  __shared__ __attribute__((aligned(16))) float As[2][BK * C::LDA_S];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * C::LDB_S];

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
  const bool acc_c = g.beta != 0.0f;
  const float a_scale = acc_c ? g.alpha : 1.0f;   // +-1 when C is accumulated
  const bool edge_mn = (m0 + BM > g.M) || (n0 + BN > g.N);
  const int lda = (int)g.lda, ldb = (int)g.ldb;

  // C tile addressed with 32-bit offsets from its corner
  float* ct = g.C + m0 * g.ldc + n0;
  const int ldc = (int)g.ldc;
  const int m_left = (int)(g.M - m0 < BM ? g.M - m0 : BM);
  const int n_left = (int)(g.N - n0 < BN ? g.N - n0 : BN);
  const int col0 = wn * (BN / 2) + (lane & 31);
  const int row0 = wm * (BM / 2) + 4 * (lane >> 5);

  floatx16 acc[C::TM][C::TN];
#pragma unroll
  for (int x = 0; x < C::TM; ++x)
#pragma unroll
    for (int y = 0; y < C::TN; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = 0.0f;
        const int mr = row0 + x * 32 + 8 * (r >> 2) + (r & 3), nc = col0 + y * 32;
        if (acc_c && mr < m_left && nc < n_left) v = ct[mr * ldc + nc] * g.beta;
        acc[x][y][r] = v;
      }

  floatx4 ra[C::A_V4], rb[C::B_V4];
  // masks are needed when the step touches an edge or a triangle's diagonal
  auto step_masked = [&](int64_t k0) {
    if (!g.vec || edge_mn || k0 + BK > g.K) return true;
    if (g.triA == 1 && k0 < m0 + BM) return true;        // some k < m inside the step
    if (g.triA == 2 && k0 + BK > m0) return true;
    if (g.triB == 1 && k0 + BK > n0) return true;
    if (g.triB == 2 && k0 < n0 + BN) return true;
    return false;
  };
  auto load = [&](int64_t k0) {
    // per-step corners; in-step offsets fit in 32 bits
    const float* pa = TA ? g.A + k0 * g.lda + m0 : g.A + m0 * g.lda + k0;
    const float* pb = TB ? g.B + n0 * g.ldb + k0 : g.B + k0 * g.ldb + n0;
    if (!step_masked(k0)) {
#pragma unroll
      for (int i = 0; i < C::A_V4; ++i) {
        int ml, kl;
        a_coords<BM, BK, TA>(tid + i * 256, ml, kl);
        ra[i] = *reinterpret_cast<const floatx4*>(TA ? pa + kl * lda + ml : pa + ml * lda + kl);
      }
#pragma unroll
      for (int i = 0; i < C::B_V4; ++i) {
        int kl, nl;
        b_coords<BN, BK, TB>(tid + i * 256, kl, nl);
        rb[i] = *reinterpret_cast<const floatx4*>(TB ? pb + nl * ldb + kl : pb + kl * ldb + nl);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < C::A_V4; ++i) {
      int ml, kl;
      a_coords<BM, BK, TA>(tid + i * 256, ml, kl);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int mj = TA ? ml + j : ml, kj = TA ? kl : kl + j;
        ra[i][j] = a_ok(g, m0 + mj, k0 + kj) ? (TA ? pa[kj * lda + mj] : pa[mj * lda + kj]) : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_V4; ++i) {
      int kl, nl;
      b_coords<BN, BK, TB>(tid + i * 256, kl, nl);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kj = TB ? kl + j : kl, nj = TB ? nl : nl + j;
        rb[i][j] = b_ok(g, k0 + kj, n0 + nj) ? (TB ? pb[nj * ldb + kj] : pb[kj * ldb + nj]) : 0.0f;
      }
    }
  };
  auto store = [&](int buf) {
    float* as = As[buf];
    float* bs = Bs[buf];
#pragma unroll
    for (int i = 0; i < C::A_V4; ++i) {
      int ml, kl;
      a_coords<BM, BK, TA>(tid + i * 256, ml, kl);
      const floatx4 va = ra[i] * a_scale;
      if (TA) {
        *reinterpret_cast<floatx4*>(&as[kl * C::LDA_S + ml]) = va;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) as[(kl + j) * C::LDA_S + ml] = va[j];
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_V4; ++i) {
      int kl, nl;
      b_coords<BN, BK, TB>(tid + i * 256, kl, nl);
      if (TB) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bs[(kl + j) * C::LDB_S + nl] = rb[i][j];
      } else {
        *reinterpret_cast<floatx4*>(&bs[kl * C::LDB_S + nl]) = rb[i];
      }
    }
  };

  int buf = 0;
  if (k_lo < k_hi) {
    load(k_lo);
    store(0);
    __syncthreads();
  }
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += BK) {
    const bool more = k0 + BK < k_hi;
    if (more) load(k0 + BK);
    const float* as = As[buf];
    const float* bs = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
      const int kr = 2 * kk + (lane >> 5);
      float a[C::TM], b[C::TN];
#pragma unroll
      for (int t = 0; t < C::TM; ++t) a[t] = as[kr * C::LDA_S + wm * (BM / 2) + t * 32 + (lane & 31)];
#pragma unroll
      for (int t = 0; t < C::TN; ++t) b[t] = bs[kr * C::LDB_S + wn * (BN / 2) + t * 32 + (lane & 31)];
#pragma unroll
      for (int x = 0; x < C::TM; ++x)
#pragma unroll
        for (int y = 0; y < C::TN; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x], b[y], acc[x][y], 0, 0, 0);
    }
    if (more) {
      store(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  const float out_scale = acc_c ? 1.0f : g.alpha;
  const int diag_off = (int)(n0 - m0);   // m <= n  <=>  mr <= nc + diag_off
#pragma unroll
  for (int x = 0; x < C::TM; ++x)
#pragma unroll
    for (int y = 0; y < C::TN; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mr = row0 + x * 32 + 8 * (r >> 2) + (r & 3), nc = col0 + y * 32;
        if (mr < m_left && nc < n_left && (g.triC == 0 || mr <= nc + diag_off))
          ct[mr * ldc + nc] = out_scale * acc[x][y][r];
      }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int BM, int BN>
hipError_t launch(const Dev& g, bool ta, bool tb, hipStream_t s) {
  const int64_t grid = ceil_div(g.M, BM) * ceil_div(g.N, BN);
  if (!ta && !tb) hipLaunchKernelGGL((gemm_f32_mfma<BM, BN, false, false>), dim3(grid), dim3(256), 0, s, g);
  else if (!ta && tb) hipLaunchKernelGGL((gemm_f32_mfma<BM, BN, false, true>), dim3(grid), dim3(256), 0, s, g);
  else if (ta && !tb) hipLaunchKernelGGL((gemm_f32_mfma<BM, BN, true, false>), dim3(grid), dim3(256), 0, s, g);
  else hipLaunchKernelGGL((gemm_f32_mfma<BM, BN, true, true>), dim3(grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_f32(const GemmArgs& a, hipStream_t stream, const char* prof_name) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  // With beta != 0 the accumulators start from beta*C and op(A) is scaled by alpha,
  // which is exact only for alpha = +-1 and beta = 1 (the only uses).
  if (a.beta != 0.0f && !(a.beta == 1.0f && (a.alpha == 1.0f || a.alpha == -1.0f)))
    return hipErrorInvalidValue;
  // 32-bit in-tile offsets; 16-byte loads need aligned operands and leading dimensions
  // (otherwise every step takes the element-wise path).
  if (a.ldc >= (int64_t)1 << 24 || a.lda >= (int64_t)1 << 24 || a.ldb >= (int64_t)1 << 24)
    return hipErrorInvalidValue;
  const int vec = aligned16(a.A) && aligned16(a.B) && !(a.lda % 4) && !(a.ldb % 4);
  Dev g{a.M, a.N, a.K, a.A, a.lda, a.triA, a.B, a.ldb, a.triB, a.C, a.ldc, a.triC, a.alpha, a.beta,
        vec};
  ProfScope ps(prof_name, stream);
  const int64_t big_tiles = ceil_div(a.M, 128) * ceil_div(a.N, 128);
  if (big_tiles >= 192) return launch<128, 128>(g, a.transA, a.transB, stream);
  return launch<64, 64>(g, a.transA, a.transB, stream);
}

}  // namespace gptq
