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
// Products with at most one 64 x 64 tile per CU go to a short-K kernel instead (32 x 32
// tiles, K split over the four waves of a workgroup); long-K products with many 128 x 128
// tiles to a direct-to-LDS variant.

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

template <int BM, int BN, bool TA, bool TB>
__global__ void __launch_bounds__(256, 2) gemm_f32_mfma(Dev g) {
  __shared__ __attribute__((aligned(16))) Smem<BM, BN> sm;
  gemm_tile<BM, BN, TA, TB>(g, blockIdx.x, sm);
}

// Two independent problems in one launch (tiles of the first, then of the second); both
// have op(A) = A and share the tile shape and the LDS.
template <int BM, int BN, bool TB1, bool TB2>
__global__ void __launch_bounds__(256, 2) gemm_f32_pair(Dev g1, int64_t tiles1, Dev g2) {
  __shared__ __attribute__((aligned(16))) Smem<BM, BN> sm;
  if ((int64_t)blockIdx.x < tiles1) gemm_tile<BM, BN, false, TB1>(g1, blockIdx.x, sm);
  else gemm_tile<BM, BN, false, TB2>(g2, (int64_t)blockIdx.x - tiles1, sm);
}

// ---------------------------------------------------------------------------------
// Direct-to-LDS variant (op(A) = A row-major M x K; B row-major K x N, or N x K with TB).
// Operand tiles of 16 k per stage are copied from global memory straight into LDS by
// buffer loads (`buffer_load_dwordx4 ... lds`, 1 KB per wave instruction), four stages in
// the ring and three in flight, one barrier per stage.  A k-contiguous tile (A, or B with
// TB) keeps 64-byte rows of 4 16-byte chunks whose slot is XOR-swizzled by (row / 4) % 4,
// so a ds_read_b128 of one chunk per lane is conflict-free; an n-contiguous tile (B) keeps
// its k rows with 64 or 128 bytes of padding per 1 KB copy, so that the two lane halves
// (k and k + 4) read disjoint banks.  MFMA k index: lane half h, step 4u + e of a stage
// uses k = 4 (2u + h) + e, which lets the k-contiguous operand deliver four steps per
// 16-byte read.  Global addresses are clamped into the operands and the stages that touch
// an edge or a triangular mask zero the affected values after the LDS read.
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return rsrc_t{lo, hi & 0xffffu, 0xffffffffu, 0x00020000u};
}

// One wave-wide 1 KB copy: lane l's 16 bytes at byte offset voff land at lds_base + 16 l.
// Inline asm keeps the compiler from treating later LDS reads as dependent on the copy
// (it would wait for the whole ring); explicit vmcnt waits before each stage barrier
// order the copies.  No register output.
__device__ __forceinline__ void dma16(rsrc_t rsrc, uint32_t lds_base, int voff) {
  __asm__ volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "s"(lds_base)
                   : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
}

constexpr int DBK = 16;   // k per stage
constexpr int DNS = 4;    // stages in the ring

// n-contiguous tile of width W floats: rows per 1 KB copy, padding per copy, bytes
__host__ __device__ constexpr int nc_rows(int W) { return 256 / W; }
__host__ __device__ constexpr int nc_pad(int W) { return W == 128 ? 64 : 128; }
__host__ __device__ constexpr int nc_bytes(int W) { return (DBK / nc_rows(W)) * (1024 + nc_pad(W)); }

template <int BM, int BN, bool TB>
struct DCfg {
  static constexpr int A_BYTES = BM * 64;                        // k-contiguous
  static constexpr int B_BYTES = TB ? BN * 64 : nc_bytes(BN);
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_COPIES = BM / 16, B_COPIES = BN / 16;   // 1 KB copies per stage
  static constexpr int CPW = (A_COPIES + B_COPIES) / 4;          // per wave
  static constexpr int TM = BM / 64, TN = BN / 64;
  static_assert((A_COPIES + B_COPIES) % 4 == 0, "copies must split over 4 waves");
};

// k-contiguous tile of `rows` rows starting at element `base` (row stride ld): copy q.
// Rows >= row_lim and k >= k_lim are clamped (their values are masked later).
__device__ __forceinline__ void copy_kc(rsrc_t rsrc, uint32_t lds, int q, int lane, int ld,
                                        int row_lim, int k_lim) {
  const int row = 16 * q + (lane >> 2);
  const int c = (lane & 3) ^ ((row >> 2) & 3);
  const int r = row < row_lim ? row : row_lim - 1;
  const int k = 4 * c < k_lim ? 4 * c : k_lim - 4;
  dma16(rsrc, lds + q * 1024, (r * ld + k) * 4);
}
// n-contiguous tile (DBK rows of W floats): copy q.
template <int W>
__device__ __forceinline__ void copy_nc(rsrc_t rsrc, uint32_t lds, int q, int lane, int ld,
                                        int k_lim, int n_lim) {
  constexpr int CH = W / 4;
  const int kr = q * nc_rows(W) + lane / CH;
  const int ch = lane % CH;
  const int k = kr < k_lim ? kr : k_lim - 1;
  const int n = 4 * ch < n_lim ? 4 * ch : n_lim - 4;
  dma16(rsrc, lds + q * (1024 + nc_pad(W)), (k * ld + n) * 4);
}

// vmcnt wait that leaves `later` stages of CPW copies each in flight (later <= I)
template <int CPW, int I>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (I == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= I) wait_vmcnt<I * CPW>();
    else wait_later<CPW, I - 1>(later);
  }
}

// Output tile `tile` of one problem through a ring of NS stages (NS - 1 in flight).
template <int BM, int BN, bool TB, int NS>
__device__ __forceinline__ void dma_tile(const Dev& g, int64_t tile, char* ring) {
  using C = DCfg<BM, BN, TB>;
  static_assert((NS - 2) * C::CPW <= 63, "vmcnt range");

  int64_t m0, n0;
  tile_origin(g, tile, BM, BN, m0, n0);
  if (g.triC == 1 && m0 >= n0 + BN) return;  // tile entirely below the diagonal

  int64_t k_lo = 0, k_hi = g.K;
  if (g.triA == 1) k_lo = m0;
  if (g.triA == 2) k_hi = k_hi < m0 + BM ? k_hi : m0 + BM;
  if (g.triB == 1) k_hi = k_hi < n0 + BN ? k_hi : n0 + BN;
  if (g.triB == 2) k_lo = k_lo > n0 ? k_lo : n0;
  k_lo = k_lo / DBK * DBK;
  const int nsteps = k_hi > k_lo ? (int)((k_hi - k_lo + DBK - 1) / DBK) : 0;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m_left = (int)(g.M - m0 < BM ? g.M - m0 : BM);
  const int n_left = (int)(g.N - n0 < BN ? g.N - n0 : BN);
  const bool edge_mn = m_left < BM || n_left < BN;
  const uint32_t ring0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)ring);
  const int lda = (int)g.lda, ldb = (int)g.ldb;

  auto issue = [&](int st) {
    const int64_t k0 = k_lo + (int64_t)st * DBK;
    const int k_lim = (int)(g.K - k0 < DBK ? g.K - k0 : DBK);
    const uint32_t sa = ring0 + (st % NS) * C::STAGE, sb = sa + C::A_BYTES;
    const rsrc_t ra = make_rsrc(g.A + m0 * g.lda + k0);
    const rsrc_t rb = make_rsrc(TB ? g.B + n0 * g.ldb + k0 : g.B + k0 * g.ldb + n0);
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) {
      const int q = wave * C::CPW + i;             // copy index over A then B
      if (q < C::A_COPIES) {
        copy_kc(ra, sa, q, lane, lda, m_left, k_lim);
      } else if (TB) {
        copy_kc(rb, sb, q - C::A_COPIES, lane, ldb, n_left, k_lim);
      } else {
        copy_nc<BN>(rb, sb, q - C::A_COPIES, lane, ldb, k_lim, n_left);
      }
    }
  };
  // does stage st need masking (an edge, the end of K, or a triangle's diagonal)?
  auto masked = [&](int st) {
    const int64_t k0 = k_lo + (int64_t)st * DBK;
    if (edge_mn || k0 + DBK > g.K || k0 < k_lo) return true;
    if (g.triA == 1 && k0 < m0 + BM) return true;
    if (g.triA == 2 && k0 + DBK > m0) return true;
    if (g.triB == 1 && k0 + DBK > n0) return true;
    if (g.triB == 2 && k0 < n0 + BN) return true;
    return false;
  };

  floatx16 acc[C::TM][C::TN];
#pragma unroll
  for (int x = 0; x < C::TM; ++x)
#pragma unroll
    for (int y = 0; y < C::TN; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;

#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < nsteps) issue(i);
  for (int s = 0; s < nsteps; ++s) {
    const int later = nsteps - 1 - s < NS - 2 ? nsteps - 1 - s : NS - 2;
    wait_later<C::CPW, NS - 2>(later);
    stage_barrier();
    if (s + NS - 1 < nsteps) issue(s + NS - 1);   // into the buffer read in iteration s - 1
    const char* sa = ring + (s % NS) * C::STAGE;
    const char* sb = sa + C::A_BYTES;
    const int64_t k0 = k_lo + (int64_t)s * DBK;
    const bool msk = masked(s);
#pragma unroll
    for (int u = 0; u < DBK / 8; ++u) {
      const int c = 2 * u + h;                     // chunk: k = 4c .. 4c + 3
      floatx4 a[C::TM];
#pragma unroll
      for (int x = 0; x < C::TM; ++x) {
        const int row = wm * (BM / 2) + 32 * x + l32;
        a[x] = *reinterpret_cast<const floatx4*>(sa + row * 64 + 16 * (c ^ ((row >> 2) & 3)));
        if (msk) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t mg = m0 + row, kg = k0 + 4 * c + e;
            if (!a_ok(g, mg, kg) || kg < k_lo) a[x][e] = 0.0f;
          }
        }
        a[x] = a[x] * g.alpha;
      }
      floatx4 b[C::TN];
#pragma unroll
      for (int y = 0; y < C::TN; ++y) {
        const int col = wn * (BN / 2) + 32 * y + l32;
        if (TB) {
          b[y] = *reinterpret_cast<const floatx4*>(sb + col * 64 + 16 * (c ^ ((col >> 2) & 3)));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kr = 4 * c + e;
            b[y][e] = *reinterpret_cast<const float*>(
                sb + (kr / nc_rows(BN)) * (1024 + nc_pad(BN)) + (kr % nc_rows(BN)) * BN * 4 + col * 4);
          }
        }
        if (msk) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t kg = k0 + 4 * c + e, ng = n0 + col;
            if (!b_ok(g, kg, ng) || kg < k_lo) b[y][e] = 0.0f;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int x = 0; x < C::TM; ++x)
#pragma unroll
          for (int y = 0; y < C::TN; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[x][e], b[y][e], acc[x][y], 0, 0, 0);
    }
  }

  // epilogue: C = alpha op(A) op(B) (+ C when beta = 1); alpha was applied to op(A)
  float* ct = g.C + m0 * g.ldc + n0;
  const int ldc = (int)g.ldc;
  const int diag_off = (int)(n0 - m0);   // m <= n  <=>  mr <= nc + diag_off
  const bool acc_c = g.beta != 0.0f;
#pragma unroll
  for (int x = 0; x < C::TM; ++x)
#pragma unroll
    for (int y = 0; y < C::TN; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mr = wm * (BM / 2) + 32 * x + 8 * (r >> 2) + 4 * h + (r & 3);
        const int nc = wn * (BN / 2) + 32 * y + l32;
        if (mr < m_left && nc < n_left && (g.triC == 0 || mr <= nc + diag_off)) {
          float v = acc[x][y][r];
          if (acc_c) v += ct[mr * ldc + nc];
          ct[mr * ldc + nc] = v;
        }
      }
}

template <int BM, int BN, bool TB, int NS>
__global__ void __launch_bounds__(256, 2) gemm_f32_dma(Dev g) {
  __shared__ __attribute__((aligned(1024))) char ring[NS * DCfg<BM, BN, TB>::STAGE];
  dma_tile<BM, BN, TB, NS>(g, blockIdx.x, ring);
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

template <bool TB>
__global__ void __launch_bounds__(256) gemm_f32_small(Dev g) {
  __shared__ float red[4 * SK_T * 33];
  small_tile<TB>(g, blockIdx.x, red);
}

template <bool TB1, bool TB2>
__global__ void __launch_bounds__(256) gemm_f32_small_pair(Dev g1, int64_t tiles1, Dev g2) {
  __shared__ float red[4 * SK_T * 33];
  if ((int64_t)blockIdx.x < tiles1) small_tile<TB1>(g1, blockIdx.x, red);
  else small_tile<TB2>(g2, (int64_t)blockIdx.x - tiles1, red);
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

template <int BM, int BN, int NS>
hipError_t launch_dma(const Dev& g, bool tb, hipStream_t s) {
  const int64_t grid = ceil_div(g.M, BM) * ceil_div(g.N, BN);
  if (tb) hipLaunchKernelGGL((gemm_f32_dma<BM, BN, true, NS>), dim3(grid), dim3(256), 0, s, g);
  else hipLaunchKernelGGL((gemm_f32_dma<BM, BN, false, NS>), dim3(grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_small(const Dev& g, bool tb, hipStream_t s) {
  const int64_t grid = ceil_div(g.M, SK_T) * ceil_div(g.N, SK_T);
  if (tb) hipLaunchKernelGGL((gemm_f32_small<true>), dim3(grid), dim3(256), 0, s, g);
  else hipLaunchKernelGGL((gemm_f32_small<false>), dim3(grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_small_pair(const Dev& g1, bool tb1, const Dev& g2, bool tb2, hipStream_t s) {
  const int64_t t1 = ceil_div(g1.M, SK_T) * ceil_div(g1.N, SK_T);
  const int64_t grid = t1 + ceil_div(g2.M, SK_T) * ceil_div(g2.N, SK_T);
  if (!tb1 && !tb2) hipLaunchKernelGGL((gemm_f32_small_pair<false, false>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else if (!tb1 && tb2) hipLaunchKernelGGL((gemm_f32_small_pair<false, true>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else if (tb1 && !tb2) hipLaunchKernelGGL((gemm_f32_small_pair<true, false>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else hipLaunchKernelGGL((gemm_f32_small_pair<true, true>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_pair(const Dev& g1, bool tb1, const Dev& g2, bool tb2, hipStream_t s) {
  const int64_t t1 = ceil_div(g1.M, BM) * ceil_div(g1.N, BN);
  const int64_t grid = t1 + ceil_div(g2.M, BM) * ceil_div(g2.N, BN);
  if (!tb1 && !tb2) hipLaunchKernelGGL((gemm_f32_pair<BM, BN, false, false>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else if (!tb1 && tb2) hipLaunchKernelGGL((gemm_f32_pair<BM, BN, false, true>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else if (tb1 && !tb2) hipLaunchKernelGGL((gemm_f32_pair<BM, BN, true, false>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else hipLaunchKernelGGL((gemm_f32_pair<BM, BN, true, true>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  return hipGetLastError();
}

bool valid_args(const GemmArgs& a) {
  // With beta != 0 the accumulators start from beta*C and op(A) is scaled by alpha,
  // which is exact only for alpha = +-1 and beta = 1 (the only uses); 32-bit in-tile offsets.
  if (a.beta != 0.0f && !(a.beta == 1.0f && (a.alpha == 1.0f || a.alpha == -1.0f))) return false;
  return a.ldc < (int64_t)1 << 24 && a.lda < (int64_t)1 << 24 && a.ldb < (int64_t)1 << 24;
}

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

hipError_t gemm_f32_pair(const GemmArgs& a1, const GemmArgs& a2, hipStream_t stream,
                         const char* prof_name) {
  if (a1.M <= 0 || a1.N <= 0) return gemm_f32(a2, stream, prof_name);
  if (a2.M <= 0 || a2.N <= 0) return gemm_f32(a1, stream, prof_name);
  if (a1.transA || a2.transA || !valid_args(a1) || !valid_args(a2)) return hipErrorInvalidValue;
  const Dev g1 = make_dev(a1), g2 = make_dev(a2);
  ProfScope ps(prof_name, stream);
  // few 64 x 64 tiles (at most one per CU): the short-K kernel puts four waves on each 32 x 32
  // tile instead (measured on MI355X: 128^3 pair 9.9 -> 5.6 us, 512^3 22 -> 15 us; at 1024^3,
  // 512 tiles, the 64 x 64 kernel is faster)
  if (ceil_div(a1.M, 64) * ceil_div(a1.N, 64) + ceil_div(a2.M, 64) * ceil_div(a2.N, 64) <= 256)
    return launch_small_pair(g1, a1.transB, g2, a2.transB, stream);
  const int64_t big = ceil_div(a1.M, 128) * ceil_div(a1.N, 128) + ceil_div(a2.M, 128) * ceil_div(a2.N, 128);
  const bool masked = (a1.triA || a1.triB || a1.triC || a2.triA || a2.triB || a2.triC) &&
                      big < 1024;
  if (!masked && big >= 512) return launch_pair<128, 128>(g1, a1.transB, g2, a2.transB, stream);
  return launch_pair<64, 64>(g1, a1.transB, g2, a2.transB, stream);
}

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
  const Dev g = make_dev(a);
  const int vec = g.vec;
  ProfScope ps(prof_name, stream);
  // At most one 64 x 64 tile per CU: the short-K kernel (measured on MI355X: 128^3 9.3 -> 4.9
  // us, 1024^3 with a triangular operand 40 -> 28 us, 4096 x 128 x 128 11 -> 7.7 us)
  if (!a.transA && ceil_div(a.M, 64) * ceil_div(a.N, 64) <= 256)
    return launch_small(g, a.transB, stream);
  const int64_t big_tiles = ceil_div(a.M, 128) * ceil_div(a.N, 128);
  // With a triangular mask K differs per tile: while there are few 128 x 128 tiles per CU
  // (one would wait for the longest), 64 x 64 tiles, longest first, let the dispatcher
  // balance the CUs; with many tiles per CU the larger tiles are more efficient.
  const bool masked = (a.triA || a.triB || a.triC) && big_tiles < 1024;
  // direct-to-LDS path: A row-major, 16-byte rows and chunks that do not straddle an edge
  // (byte offsets inside a 128-row tile stay below 2^31 for leading dimensions < 2^21)
  const bool dma = vec && !a.transA && a.K % 4 == 0 && a.K >= 4 && (a.transB || a.N % 4 == 0) &&
                   a.M >= 64 && a.N >= 64 && a.lda < ((int64_t)1 << 21) &&
                   a.ldb < ((int64_t)1 << 21);
  // Measured on MI355X: 128 x 128 tiles pay off from about two per CU (4096 x 1024 x 1024:
  // 64 x 64 tiles 98 us, 128 x 128 120 us; 4096 x 2048 x 2048: all variants 330-345 us); the
  // direct-to-LDS kernel only for long K on large outputs.
  if (!masked && dma && big_tiles >= 512 && a.K >= 2048)
    return launch_dma<128, 128, DNS>(g, a.transB, stream);
  if (!masked && big_tiles >= 512) return launch<128, 128>(g, a.transA, a.transB, stream);
  return launch<64, 64>(g, a.transA, a.transB, stream);
}

}  // namespace gptq
