// Device code of the fp32 MFMA GEMM's register-staged tiles and short-K tiles
// (v_mfma_f32_32x32x2_f32), shared by gemm.hip (the GEMM launches) and prep.hip (launches
// that run GEMM tiles beside the inverse factor's leaf).  See gemm.hip for the design.
#pragma once

#include "gptq_internal.h"

namespace gptq {

namespace {

struct Dev {
  int64_t M, N, K;
  const float* A; int64_t lda; int triA;
  const float* B; int64_t ldb; int triB;
  float* C; int64_t ldc; int triC;
  float alpha, beta;
  int vec;     // operands and leading dimensions allow 16-byte loads
  int order;   // tile order: 0 by rows, 1 by columns, 2 by columns from the last, 3 by rows
               // from the last (a triangular mask makes K per tile vary; long tiles first)
};

// Output tile `tile` of the launch -> tile coordinates, in the order `order`.
__device__ __forceinline__ void tile_origin(const Dev& g, int64_t tile, int BM, int BN, int64_t& m0,
                                            int64_t& n0) {
  const int64_t tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  int64_t i, j;
  if (g.order == 1 || g.order == 2) {
    i = tile % tm;
    j = tile / tm;
    if (g.order == 2) j = tn - 1 - j;
  } else {
    i = tile / tn;
    j = tile % tn;
    if (g.order == 3) i = tm - 1 - i;
  }
  m0 = i * BM;
  n0 = j * BN;
}

template <int BM, int BN, bool TA, bool TB>
struct Cfg {
  // K per LDS stage: 128 x 128 tiles keep 16 so that staging fits two waves per SIMD.
  static constexpr int BK = BM >= 128 ? 16 : 32;
  // Row strides of the k-major stages.  An operand stored with 16-byte writes (op(A) with
  // TA, op(B) without TB) needs a stride that keeps them aligned: +4.  An operand stored one
  // dword at a time has half a wave writing BK/4 k-rows, 4 apart, of 128/BK consecutive
  // columns each; +1 (BK = 32) or +2 (BK = 16) puts those rows on disjoint runs of banks.
  static constexpr int SPAD = BK == 32 ? 1 : 2;
  static constexpr int LDA_S = TA ? BM + 4 : BM + SPAD, LDB_S = TB ? BN + SPAD : BN + 4;
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

// LDS of one workgroup: two stages of op(A) and op(B), k-major.
template <int BM, int BN>
struct Smem {
  static constexpr int BK = BM >= 128 ? 16 : 32;
  float a[2][BK * (BM + 4)];
  float b[2][BK * (BN + 4)];
};

// Output tile `tile` (row-major over the tile grid) of one problem.
template <int BM, int BN, bool TA, bool TB>
__device__ __forceinline__ void gemm_tile(const Dev& g, int64_t tile, Smem<BM, BN>& sm) {
  using C = Cfg<BM, BN, TA, TB>;
  constexpr int BK = C::BK;
  static_assert(BK == Smem<BM, BN>::BK, "stage depth");
  auto& As = sm.a;
  auto& Bs = sm.b;

  int64_t m0, n0;
  tile_origin(g, tile, BM, BN, m0, n0);
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
      // k of this step for lane half h: (kk % 8) + 8 h + 16 (kk / 8).  Any one-to-one choice
      // sums the same products; this one lets consecutive steps' reads pair into one
      // two-address LDS read.
      const int kr = (kk & 7) + 8 * (lane >> 5) + 16 * (kk >> 3);
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

// ---------------------------------------------------------------------------------
// Short-K products (K up to a few hundred): one workgroup per 32 x 32 output tile, the four
// waves split K (wave w takes the 32-wide chunks w, w + 4, ...), operands go straight from
// global memory into the MFMA registers and the four partial tiles are summed in LDS in wave
// order.  A product of this shape is bound by the length of one wave's MFMA chain, not by
// memory, so spreading K over more waves is what shortens it.
// MFMA k slots: within a chunk at k0, lane half h and step i use k = k0 + 16 h + i, so a
// lane reads 16 consecutive k of its row of A (and of B's row when B is stored N x K).
// Loads use addresses clamped into the operands; masked or out-of-range values are zeroed.
constexpr int SK_T = 32;   // output tile edge
constexpr int SK_C = 32;   // k per chunk

// Each wave's share of the 32 x 32 tile at (m0, n0) over the 32-wide k chunks from k_lo
// (a multiple of SK_C) up to k_hi, written to red[wave] (row stride 33); no barrier.
template <bool TB>
__device__ __forceinline__ void small_tile_part(const Dev& g, int64_t m0, int64_t n0, int64_t k_lo,
                                                int64_t k_hi, float* red) {
  const int nch = k_hi > k_lo ? (int)((k_hi - k_lo + SK_C - 1) / SK_C) : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const bool acc_c = g.beta != 0.0f;
  const float a_scale = acc_c ? g.alpha : 1.0f;
  const int64_t m = m0 + l32, n = n0 + l32;                    // this lane's row of A, column of B
  const int64_t mc = m < g.M ? m : g.M - 1, nc = n < g.N ? n : g.N - 1;

  // 16-byte loads need K % 4 == 0: then a clamped run only ever holds k >= K (zeroed)
  const bool vec = g.vec && (g.K & 3) == 0;
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  for (int c = wave; c < nch; c += 4) {
    const int64_t kb = k_lo + (int64_t)c * SK_C + 16 * h;     // first k of this lane
    float a[16], b[16];
    if (vec) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k4 = kb + 4 * j < g.K - 4 ? kb + 4 * j : g.K - 4;
        const floatx4 v = *reinterpret_cast<const floatx4*>(g.A + mc * g.lda + k4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * j + e] = v[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t k = kb + i < g.K ? kb + i : g.K - 1;
        a[i] = g.A[mc * g.lda + k];
      }
    }
    if (TB && vec) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k4 = kb + 4 * j < g.K - 4 ? kb + 4 * j : g.K - 4;
        const floatx4 v = *reinterpret_cast<const floatx4*>(g.B + nc * g.ldb + k4);
#pragma unroll
        for (int e = 0; e < 4; ++e) b[4 * j + e] = v[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t k = kb + i < g.K ? kb + i : g.K - 1;
        b[i] = TB ? g.B[nc * g.ldb + k] : g.B[k * g.ldb + nc];
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t k = kb + i;
      a[i] = a_ok(g, m, k) ? a[i] * a_scale : 0.0f;
      b[i] = b_ok(g, k, n) ? b[i] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], acc, 0, 0, 0);
  }

  // partial tiles -> LDS (row stride 33), summed in wave order by all 256 threads
#pragma unroll
  for (int r = 0; r < 16; ++r)
    red[wave * SK_T * 33 + (8 * (r >> 2) + 4 * h + (r & 3)) * 33 + l32] = acc[r];
}

template <bool TB>
__device__ __forceinline__ void small_tile(const Dev& g, int64_t tile, float* red) {
  int64_t m0, n0;
  tile_origin(g, tile, SK_T, SK_T, m0, n0);
  if (g.triC == 1 && m0 >= n0 + SK_T) return;   // the whole workgroup leaves together

  int64_t k_lo = 0, k_hi = g.K;
  if (g.triA == 1) k_lo = m0;
  if (g.triA == 2) k_hi = k_hi < m0 + SK_T ? k_hi : m0 + SK_T;
  if (g.triB == 1) k_hi = k_hi < n0 + SK_T ? k_hi : n0 + SK_T;
  if (g.triB == 2) k_lo = k_lo > n0 ? k_lo : n0;
  k_lo = k_lo / SK_C * SK_C;

  small_tile_part<TB>(g, m0, n0, k_lo, k_hi, red);
  const int tid = threadIdx.x;
  const bool acc_c = g.beta != 0.0f;
  __syncthreads();
  const float out_scale = acc_c ? 1.0f : g.alpha;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q, mr = e / SK_T, ncl = e % SK_T;
    const int o = mr * 33 + ncl;
    float v = red[o];
    v += red[SK_T * 33 + o];
    v += red[2 * SK_T * 33 + o];
    v += red[3 * SK_T * 33 + o];
    const int64_t gm = m0 + mr, gn = n0 + ncl;
    if (gm < g.M && gn < g.N && (g.triC == 0 || gm <= gn)) {
      float* cp = g.C + gm * g.ldc + gn;
      *cp = acc_c ? *cp + v : out_scale * v;
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Longest tiles first: K per tile shrinks with the column for a lower op(B) (k >= n),
// grows with it for an upper op(B) (k <= n), shrinks with the row for an upper op(A).
int tile_order(const GemmArgs& a) {
  if (a.triB == 2) return 1;
  if (a.triB == 1) return 2;
  if (a.triA == 2) return 3;
  return 0;
}

Dev make_dev(const GemmArgs& a) {
  const int vec = aligned16(a.A) && aligned16(a.B) && !(a.lda % 4) && !(a.ldb % 4);
  return Dev{a.M, a.N, a.K, a.A, a.lda, a.triA, a.B, a.ldb, a.triB, a.C, a.ldc, a.triC, a.alpha,
             a.beta, vec, tile_order(a)};
}

}  // namespace

}  // namespace gptq
