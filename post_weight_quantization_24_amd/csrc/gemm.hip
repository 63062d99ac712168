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
// tiles, K split over the four waves of a workgroup); long-K products and product pairs
// with many 128 x 128 tiles to a direct-to-LDS variant.

#include "gptq_internal.h"
#include "gemm_tile.h"

namespace gptq {

namespace {

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
// Operand tiles of 32 k per stage are copied from global memory straight into LDS by
// buffer loads (`buffer_load_dwordx4 ... lds`, 1 KB per wave instruction), two stages in
// the ring and one in flight, one barrier per stage (a ring of four 16-k stages, three in
// flight, took 3-4 % longer with twice the barriers per k; three 32-k stages, 6-24 %
// longer).  A k-contiguous tile (A, or B with TB) keeps 128-byte rows of 8 16-byte chunks
// whose slot is XOR-swizzled by (row / 2) % 8, so a ds_read_b128 of one chunk per lane is
// conflict-free; an n-contiguous tile (B) keeps its k rows with 64 or 128 bytes of padding
// per 1 KB copy, so that the two lane halves (k and k + 4) read disjoint banks.  MFMA k index: lane half h, step 4u + e of a stage
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

constexpr int DBK = 32;   // k per stage
constexpr int DNS = 2;    // stages in the ring

// n-contiguous tile of width W floats: rows per 1 KB copy, padding per copy, bytes
__host__ __device__ constexpr int nc_rows(int W) { return 256 / W; }
__host__ __device__ constexpr int nc_pad(int W) { return W == 128 ? 64 : 128; }
__host__ __device__ constexpr int nc_bytes(int W) { return (DBK / nc_rows(W)) * (1024 + nc_pad(W)); }

// k-contiguous rows: DBK floats, rows per 1 KB copy, 16-byte chunks per row, and the chunk
// swizzle that keeps a ds_read_b128 of one chunk per lane conflict-free
constexpr int KC_ROW = DBK * 4;
constexpr int KC_RPC = 1024 / KC_ROW;
constexpr int KC_CH = DBK / 4;
static_assert(DBK == 16 || DBK == 32, "chunk swizzle defined for 16- and 32-deep stages");
__device__ __forceinline__ int kc_swz(int row) {
  // 16 consecutive rows (one 16-lane read group) land on 16 distinct 16-byte bank positions
  // of the 256-byte bank row: the row's place in the bank row, and the swizzled chunk
  return DBK == 16 ? (row >> 2) & 3 : (row >> 1) & (KC_CH - 1);
}

template <int BM, int BN, bool TB>
struct DCfg {
  static constexpr int A_BYTES = BM * KC_ROW;                    // k-contiguous
  static constexpr int B_BYTES = TB ? BN * KC_ROW : nc_bytes(BN);
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_COPIES = BM / KC_RPC;                   // 1 KB copies per stage
  static constexpr int B_COPIES = TB ? BN / KC_RPC : DBK / nc_rows(BN);
  static constexpr int CPW = (A_COPIES + B_COPIES) / 4;          // per wave
  static constexpr int TM = BM / 64, TN = BN / 64;
  static_assert((A_COPIES + B_COPIES) % 4 == 0, "copies must split over 4 waves");
};

// k-contiguous tile of `rows` rows starting at element `base` (row stride ld): copy q.
// Rows >= row_lim and k >= k_lim are clamped (their values are masked later).
__device__ __forceinline__ void copy_kc(rsrc_t rsrc, uint32_t lds, int q, int lane, int ld,
                                        int row_lim, int k_lim) {
  const int row = KC_RPC * q + lane / KC_CH;
  const int c = (lane % KC_CH) ^ kc_swz(row);
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
    // the stage's operands first (one LDS wait), then its DBK / 2 k-steps of MFMAs
    floatx4 a[DBK / 8][C::TM], b[DBK / 8][C::TN];
#pragma unroll
    for (int u = 0; u < DBK / 8; ++u) {
      const int c = 2 * u + h;                     // chunk: k = 4c .. 4c + 3
#pragma unroll
      for (int x = 0; x < C::TM; ++x) {
        const int row = wm * (BM / 2) + 32 * x + l32;
        a[u][x] = *reinterpret_cast<const floatx4*>(sa + row * KC_ROW + 16 * (c ^ kc_swz(row)));
      }
#pragma unroll
      for (int y = 0; y < C::TN; ++y) {
        const int col = wn * (BN / 2) + 32 * y + l32;
        if (TB) {
          b[u][y] = *reinterpret_cast<const floatx4*>(sb + col * KC_ROW + 16 * (c ^ kc_swz(col)));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kr = 4 * c + e;
            b[u][y][e] = *reinterpret_cast<const float*>(
                sb + (kr / nc_rows(BN)) * (1024 + nc_pad(BN)) + (kr % nc_rows(BN)) * BN * 4 + col * 4);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < DBK / 8; ++u) {
      const int c = 2 * u + h;
      if (msk) {
#pragma unroll
        for (int x = 0; x < C::TM; ++x) {
          const int row = wm * (BM / 2) + 32 * x + l32;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t mg = m0 + row, kg = k0 + 4 * c + e;
            if (!a_ok(g, mg, kg) || kg < k_lo) a[u][x][e] = 0.0f;
          }
        }
#pragma unroll
        for (int y = 0; y < C::TN; ++y) {
          const int col = wn * (BN / 2) + 32 * y + l32;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t kg = k0 + 4 * c + e, ng = n0 + col;
            if (!b_ok(g, kg, ng) || kg < k_lo) b[u][y][e] = 0.0f;
          }
        }
      }
#pragma unroll
      for (int x = 0; x < C::TM; ++x) a[u][x] = a[u][x] * g.alpha;
    }
#pragma unroll
    for (int u = 0; u < DBK / 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int x = 0; x < C::TM; ++x)
#pragma unroll
          for (int y = 0; y < C::TN; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u][x][e], b[u][y][e], acc[x][y], 0, 0, 0);
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

// Two independent problems in one launch, as gemm_f32_pair, through the direct-to-LDS ring.
template <int BM, int BN, bool TB1, bool TB2, int NS>
__global__ void __launch_bounds__(256, 2) gemm_f32_dma_pair(Dev g1, int64_t tiles1, Dev g2) {
  constexpr int S1 = DCfg<BM, BN, TB1>::STAGE, S2 = DCfg<BM, BN, TB2>::STAGE;
  __shared__ __attribute__((aligned(1024))) char ring[NS * (S1 > S2 ? S1 : S2)];
  if ((int64_t)blockIdx.x < tiles1) dma_tile<BM, BN, TB1, NS>(g1, blockIdx.x, ring);
  else dma_tile<BM, BN, TB2, NS>(g2, (int64_t)blockIdx.x - tiles1, ring);
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

template <int BM, int BN, int NS>
hipError_t launch_dma_pair(const Dev& g1, bool tb1, const Dev& g2, bool tb2, hipStream_t s) {
  const int64_t t1 = ceil_div(g1.M, BM) * ceil_div(g1.N, BN);
  const int64_t grid = t1 + ceil_div(g2.M, BM) * ceil_div(g2.N, BN);
  if (!tb1 && !tb2) hipLaunchKernelGGL((gemm_f32_dma_pair<BM, BN, false, false, NS>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else if (!tb1 && tb2) hipLaunchKernelGGL((gemm_f32_dma_pair<BM, BN, false, true, NS>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else if (tb1 && !tb2) hipLaunchKernelGGL((gemm_f32_dma_pair<BM, BN, true, false, NS>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
  else hipLaunchKernelGGL((gemm_f32_dma_pair<BM, BN, true, true, NS>), dim3(grid), dim3(256), 0, s, g1, t1, g2);
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


// The direct-to-LDS kernels' preconditions: A row-major, 16-byte rows and chunks that do not
// straddle an edge (K and, for a row-major B, N multiples of 4), and byte offsets inside a
// 128-row tile below 2^31 (leading dimensions < 2^21).
bool dma_ok(const GemmArgs& a, int vec) {
  return vec && !a.transA && a.K % 4 == 0 && a.K >= 4 && (a.transB || a.N % 4 == 0) &&
         a.M >= 64 && a.N >= 64 && a.lda < ((int64_t)1 << 21) && a.ldb < ((int64_t)1 << 21);
}

// Shortest K at which the direct-to-LDS kernel replaces the register-staged 128 x 128 one.
// Measured on MI355X: from K = 1024 instead, no change; 64 x 64 direct-to-LDS tiles (four
// workgroups per CU) from K = 256, 512 or 1024 in place of the register-staged 64 x 64
// kernel, no change in prepare or quantize at d = 4096 ... 28672 (within 0.5 %).
constexpr int64_t DMA128_MIN_K = 2048;


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
  const bool dma = dma_ok(a1, g1.vec) && dma_ok(a2, g2.vec);
  const int64_t k_min = a1.K < a2.K ? a1.K : a2.K;
  if (!masked && big >= 512 && dma && k_min >= DMA128_MIN_K)
    return launch_dma_pair<128, 128, DNS>(g1, a1.transB, g2, a2.transB, stream);
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
  const bool dma = dma_ok(a, vec);
  // Measured on MI355X: 128 x 128 tiles pay off from about two per CU (4096 x 1024 x 1024:
  // 64 x 64 tiles 98 us, 128 x 128 120 us; 4096 x 2048 x 2048: all variants 330-345 us); the
  // direct-to-LDS kernel only for long K on large outputs.
  if (!masked && dma && big_tiles >= 512 && a.K >= DMA128_MIN_K)
    return launch_dma<128, 128, DNS>(g, a.transB, stream);
  if (!masked && big_tiles >= 512) return launch<128, 128>(g, a.transA, a.transB, stream);
  return launch<64, 64>(g, a.transA, a.transB, stream);
}

}  // namespace gptq
