// Hessian H += 2 X^T X for token-major calibration inputs (page "量化", section GPTQ:
// H = 2 X X^T with X stored d x n_tok there; here X is n_tok x d, one token per row).
//
// Layout of the work:
//   * H is covered by 256 x 256 tiles; only tiles on or below the diagonal are computed
//     (H is symmetric) and the reduce kernel mirrors them.
//   * The token range is cut into `splits` equal ranges; workgroup (split, tile) writes a
//     float32 partial tile into the workspace.  The reduce kernel sums the partials in a
//     fixed order (deterministic, no float atomics), scales by 2, adds into H and writes
//     both triangles.
//   * f16 inputs: v_mfma_f32_32x32x16_f16 (products of f16 values are exact in the f32
//     accumulator).  X rows are channel-contiguous, but MFMA operands need 8 consecutive
//     tokens of one channel per lane, so each thread loads an 8-token x 8-channel block
//     (eight 16-byte row loads), transposes it in registers and writes eight 16-byte
//     channel runs to LDS, stored [channel][token] with a 16-byte pad per channel row so
//     that both the stores and the MFMA operand reads are free of bank conflicts.
//   * f32 inputs (small layers): a VALU kernel with the same partial-tile output.

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int TILE = 256;         // H tile edge
constexpr int BK = 64;            // tokens per LDS stage
constexpr int LDS_ROW = BK + 8;   // halfs per channel row in LDS (16-byte pad)

__device__ __forceinline__ void tile_coords(int tile, int& ti, int& tj) {
  // tile = ti*(ti+1)/2 + tj with 0 <= tj <= ti
  int t = (int)((sqrtf(8.0f * (float)tile + 1.0f) - 1.0f) * 0.5f);
  while ((t + 1) * (t + 2) / 2 <= tile) ++t;
  while (t * (t + 1) / 2 > tile) --t;
  ti = t;
  tj = tile - t * (t + 1) / 2;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One 8x8 f16 block: rows r = tokens, 4 dwords each holding channels (2p, 2p+1).
// Output o[c][p] holds tokens (2p, 2p+1) of channel c.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t x = in[2 * p][m], y = in[2 * p + 1][m];
      out[2 * m][p] = (x & 0xffffu) | (y << 16);
      out[2 * m + 1][p] = (x >> 16) | (y & 0xffff0000u);
    }
  }
}

template <int WAVES_M, int WAVES_N, int TM, int TN>
struct HessCfg {
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NTHREADS = NWAVES * 64;
  static_assert(WAVES_M * TM * 32 == TILE && WAVES_N * TN * 32 == TILE, "tile shape");
  // micro-blocks (8 tokens x 8 channels) per operand per stage: (TILE/8) * (BK/8)
  static constexpr int MB_PER_OPERAND = (TILE / 8) * (BK / 8);
  static constexpr int MB_PER_THREAD = 2 * MB_PER_OPERAND / NTHREADS;
  static_assert(MB_PER_THREAD * NTHREADS == 2 * MB_PER_OPERAND, "loader shape");
};

template <int WAVES_M, int WAVES_N, int TM, int TN>
__global__ void __launch_bounds__(WAVES_M* WAVES_N * 64, 1)
hess_f16_mfma(const _Float16* __restrict__ X, int64_t ldx, int64_t d, int64_t n_tok,
              int64_t tok_per_split, int tiles, float* __restrict__ part) {
  using C = HessCfg<WAVES_M, WAVES_N, TM, TN>;
  __shared__ __attribute__((aligned(16))) _Float16 lds[2 * TILE * LDS_ROW];
  _Float16* lds_a = lds;
  _Float16* lds_b = lds + TILE * LDS_ROW;

  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  int ti, tj;
  tile_coords(tile, ti, tj);
  const int64_t ca0 = (int64_t)ti * TILE;  // channel block of H rows
  const int64_t cb0 = (int64_t)tj * TILE;  // channel block of H cols
  const int64_t t_begin = (int64_t)split * tok_per_split;
  int64_t t_end = t_begin + tok_per_split;
  if (t_end > n_tok) t_end = n_tok;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  floatx16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // loader: micro-block index mb = tid + i*NTHREADS over [A blocks | B blocks];
  // within an operand: tb = mb % 8 (token block), cbk = mb / 8 (channel block).
  u32x4 stage[C::MB_PER_THREAD][8];

  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < C::MB_PER_THREAD; ++i) {
      const int mb = tid + i * C::NTHREADS;
      const int op = mb / C::MB_PER_OPERAND;
      const int r = mb % C::MB_PER_OPERAND;
      const int tb = r % 8;
      const int cbk = r / 8;
      const int64_t ch = (op ? cb0 : ca0) + cbk * 8;
      const bool ch_ok = ch < d;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int64_t t = k0 + tb * 8 + rr;
        if (ch_ok && t < t_end) {
          stage[i][rr] = *reinterpret_cast<const u32x4*>(X + t * ldx + ch);
        } else {
          stage[i][rr] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < C::MB_PER_THREAD; ++i) {
      const int mb = tid + i * C::NTHREADS;
      const int op = mb / C::MB_PER_OPERAND;
      const int r = mb % C::MB_PER_OPERAND;
      const int tb = r % 8;
      const int cbk = r / 8;
      u32x4 tr[8];
      transpose8x8(stage[i], tr);
      _Float16* base = (op ? lds_b : lds_a) + (cbk * 8) * LDS_ROW + tb * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4*>(base + c * LDS_ROW) = tr[c];
    }
  };

  int64_t k0 = t_begin;
  if (k0 < t_end) load_stage(k0);
  for (; k0 < t_end; k0 += BK) {
    __syncthreads();  // previous stage's LDS reads are done
    store_stage();
    __syncthreads();
    if (k0 + BK < t_end) load_stage(k0 + BK);  // prefetch overlaps the MFMAs below
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      half8 af[TM], bf[TN];
      const int koff = kk * 16 + 8 * (lane >> 5);
#pragma unroll
      for (int a = 0; a < TM; ++a)
        af[a] = *reinterpret_cast<const half8*>(
            lds_a + (wm * TM * 32 + a * 32 + (lane & 31)) * LDS_ROW + koff);
#pragma unroll
      for (int b = 0; b < TN; ++b)
        bf[b] = *reinterpret_cast<const half8*>(
            lds_b + (wn * TN * 32 + b * 32 + (lane & 31)) * LDS_ROW + koff);
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  }

  // partial tile [TILE][TILE] for (split, tile)
  float* out = part + ((int64_t)split * tiles + tile) * (int64_t)TILE * TILE;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * TM * 32 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * TN * 32 + b * 32 + (lane & 31);
        out[row * TILE + col] = acc[a][b][r];
      }
}

// f32 inputs: each workgroup computes a 64x64 piece of one partial tile on the VALU.
__global__ void __launch_bounds__(256)
hess_f32_valu(const float* __restrict__ X, int64_t ldx, int64_t d, int64_t n_tok,
              int64_t tok_per_split, int tiles, float* __restrict__ part) {
  __shared__ float sa[16][64 + 4];
  __shared__ float sb[16][64 + 4];
  const int sub = blockIdx.x % 16;
  const int tile = (blockIdx.x / 16) % tiles;
  const int split = blockIdx.x / (16 * tiles);
  int ti, tj;
  tile_coords(tile, ti, tj);
  const int64_t ra = (int64_t)ti * TILE + (sub / 4) * 64;
  const int64_t rb = (int64_t)tj * TILE + (sub % 4) * 64;
  const int64_t t_begin = (int64_t)split * tok_per_split;
  int64_t t_end = t_begin + tok_per_split;
  if (t_end > n_tok) t_end = n_tok;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int64_t k0 = t_begin; k0 < t_end; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int kk = e / 64, c = e % 64;
      const int64_t t = k0 + kk;
      sa[kk][c] = (t < t_end && ra + c < d) ? X[t * ldx + ra + c] : 0.0f;
      sb[kk][c] = (t < t_end && rb + c < d) ? X[t * ldx + rb + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sa[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sb[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* out = part + ((int64_t)split * tiles + tile) * (int64_t)TILE * TILE;
  const int r0 = (sub / 4) * 64 + ty * 4, c0 = (sub % 4) * 64 + tx * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) out[(r0 + i) * TILE + c0 + j] = acc[i][j];
}

// Sum the partial tiles in split order, scale by 2, add into both triangles of H.
// One workgroup per 64x64 sub-block of a lower tile; the mirror goes through LDS so
// that both writes are row-contiguous.
__global__ void __launch_bounds__(256)
hess_reduce(const float* __restrict__ part, int splits, int tiles, int64_t d,
            float* __restrict__ H) {
  __shared__ float s[64][65];
  const int sub = blockIdx.x % 16;
  const int tile = blockIdx.x / 16;
  int ti, tj;
  tile_coords(tile, ti, tj);
  const int sa = sub / 4, sbk = sub % 4;
  if (ti == tj && sbk > sa) return;  // above the diagonal inside a diagonal tile
  const int64_t r0 = (int64_t)ti * TILE + sa * 64;
  const int64_t c0 = (int64_t)tj * TILE + sbk * 64;
  const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
  const bool diag = (r0 == c0);
  for (int rr = ty; rr < 64; rr += 4) {
    float v = 0.0f;
    const int64_t off = (int64_t)(sa * 64 + rr) * TILE + sbk * 64 + tx;
    for (int sp = 0; sp < splits; ++sp)
      v += part[((int64_t)sp * tiles + tile) * (int64_t)TILE * TILE + off];
    v *= 2.0f;
    s[rr][tx] = v;
    const int64_t i = r0 + rr, j = c0 + tx;
    if (i < d && j < d && (!diag || j <= i)) H[i * d + j] += v;
  }
  __syncthreads();
  // mirror: H[c0 + rr][r0 + tx] += s[tx][rr] for entries strictly below the diagonal
  for (int rr = ty; rr < 64; rr += 4) {
    const int64_t i = c0 + rr, j = r0 + tx;  // upper-triangle position (i < j)
    if (i < d && j < d && (!diag || tx > rr)) H[i * d + j] += s[tx][rr];
  }
}

}  // namespace

HessPlan hessian_plan(int64_t d, int64_t n_tok, int x_dtype) {
  HessPlan p{};
  p.d = d;
  p.n_tok = n_tok;
  const int64_t nb = ceil_div(d, TILE);
  p.tiles = (int)(nb * (nb + 1) / 2);
  // Enough workgroups to fill 256 CUs with a short tail, each split >= 2048 tokens.
  const int64_t cus = 256;
  const int64_t min_tok = 2048;
  int best = 1;
  double best_cost = 1e30;
  const int64_t max_split = n_tok / min_tok > 1 ? n_tok / min_tok : 1;
  for (int64_t s = 1; s <= max_split && s <= 64; ++s) {
    const int64_t wgs = p.tiles * s * (x_dtype == 0 ? 1 : 16);
    const double rounds = (double)ceil_div(wgs, cus);
    // time ~ rounds * work per workgroup (1/s), plus partial-tile traffic per split
    const double cost = rounds / (double)s * (x_dtype == 0 ? 1.0 : 1.0 / 16.0) + 0.004 * (double)s;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = (int)s;
    }
  }
  p.splits = best;
  int64_t tps = ceil_div(n_tok, best);
  tps = ceil_div(tps, BK) * BK;
  p.tok_per_split = tps > 0 ? tps : BK;
  p.ws_bytes = (size_t)p.splits * p.tiles * TILE * TILE * sizeof(float);
  return p;
}

hipError_t hessian_launch(const HessPlan& p, float* H, const void* X, int x_dtype, int64_t ldx,
                          void* ws, hipStream_t stream) {
  float* part = static_cast<float*>(ws);
  {
    ProfScope ps("hessian_mfma", stream);
    if (x_dtype == 0) {
      hipLaunchKernelGGL((hess_f16_mfma<2, 2, 4, 4>), dim3(p.tiles * p.splits), dim3(256), 0,
                         stream, static_cast<const _Float16*>(X), ldx, p.d, p.n_tok,
                         p.tok_per_split, p.tiles, part);
    } else {
      hipLaunchKernelGGL(hess_f32_valu, dim3(p.tiles * p.splits * 16), dim3(256), 0, stream,
                         static_cast<const float*>(X), ldx, p.d, p.n_tok, p.tok_per_split,
                         p.tiles, part);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps("hessian_reduce", stream);
    hipLaunchKernelGGL(hess_reduce, dim3(p.tiles * 16), dim3(256), 0, stream, part, p.splits,
                       p.tiles, p.d, H);
  }
  return hipGetLastError();
}

}  // namespace gptq
