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
//     accumulator), fed by direct global-to-LDS copies and transposed LDS reads (below).
//   * f32 inputs (small layers): a VALU kernel with the same partial-tile output.

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int TILE = 256;         // H tile edge

__device__ __forceinline__ void tile_coords(int tile, int& ti, int& tj) {
  // tile = ti*(ti+1)/2 + tj with 0 <= tj <= ti
  int t = (int)((sqrtf(8.0f * (float)tile + 1.0f) - 1.0f) * 0.5f);
  while ((t + 1) * (t + 2) / 2 <= tile) ++t;
  while (t * (t + 1) / 2 > tile) --t;
  ti = t;
  tj = tile - t * (t + 1) / 2;
}

// ---------------------------------------------------------------------------------
// f16 inputs, direct-to-LDS pipeline (the launch path).
//
// Each stage holds 64 tokens x 256 channels of the two channel blocks, copied from X by
// buffer loads that write LDS directly (the buffer covers exactly the workgroup's token
// range, so reads past its end return zeros: no masking for ragged token counts).  LDS
// keeps X's token-major layout; the MFMA operands (8 consecutive tokens of one channel per
// lane) come from transposed LDS reads: within each 16-lane group of ds_read_b64_tr_b16,
// lane i receives element i%4 of the 8-byte pieces addressed by lanes 4m + i/4 (m = 0..3),
// so lane j pointing at (token k0 + j/4, channels c0 + 4(j%4)..) hands lane i channel c0+i
// at tokens k0..k0+3.  The 16-byte slots of a token row are XOR-swizzled by 4*(row % 4)
// so that the four rows such a group touches fall on distinct banks.
// Eight waves in a 2 x 4 grid, each owning a 128 x 64 quarter-column of the tile (128
// accumulator registers), so two waves share each SIMD and one wave's MFMAs cover the
// other's LDS waits.  Against four waves of 128 x 128 (one per SIMD) this reads 1.5x the
// operand bytes from LDS but ran 6-8 % faster on MI355X (q_proj, 11 splits, identical H).
// Two stages: the copies of stage s + 1 are issued, between the first MFMAs, while stage s
// is multiplied.  Measured on MI355X: 64-token stages in a ring of 2 beat 32-token stages in
// rings of 2, 3 or 4; issuing the copies all at once after the barrier, or spread over all
// the MFMAs of a stage, was 4-6 % slower.
constexpr int V2_BK = 64;                                 // tokens per stage
constexpr int V2_NST = 2;                                 // stages in the ring
constexpr int V2_WAVES = 8;                               // 2 x 4 wave grid
constexpr int V2_BFR = 2;                                 // 32-column B fragments per wave
constexpr int V2_CPO = V2_BK / 2 / V2_WAVES;              // 1 KB copies per operand, wave, stage
constexpr int V2_STAGE_HALFS = V2_BK * TILE;              // 16384 halfs = 32 KB per operand
static_assert(V2_BK % 16 == 0 && V2_BK / 4 >= 2 * V2_CPO, "a copy slot per MFMA group");
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_s4;

__device__ __forceinline__ int v2_slot(int row, int chunk) { return chunk ^ (4 * (row & 3)); }

typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));

// Work item of a workgroup for the f16 kernel: splits one after the other (split-major).
// Within a split, lower-triangle tiles are visited by 4 x 4-block super-tiles (row-major
// over the super-tiles, then over the tiles inside one), so that the tiles in flight share
// few channel blocks.  The grid covers the triangle padded to a multiple of 4 blocks; padded
// tiles exit.  Giving each of the 8 XCDs (workgroups go round robin, id % 8) its own token
// ranges when the split count is a multiple of 8 was measured 3-5 % slower than this order
// with the eight-wave kernel (q_proj and 8192-wide layers).
constexpr int SUPER = 4;
__device__ __forceinline__ void super_tile_coords(int t, int& i, int& j) {
  // tiles before super-row S: 16 * S(S-1)/2 (off-diagonal) + 10 * S (diagonal)
  int S = 0;
  while (8 * (S + 1) * S + 10 * (S + 1) <= t) ++S;
  int r = t - (8 * S * (S - 1) + 10 * S);
  if (r < SUPER * SUPER * S) {
    i = SUPER * S + (r % (SUPER * SUPER)) / SUPER;
    j = SUPER * (r / (SUPER * SUPER)) + r % SUPER;
  } else {
    r -= SUPER * SUPER * S;                       // 0..9 inside the diagonal super-tile
    int a = 0;
    while ((a + 1) * (a + 2) / 2 <= r) ++a;
    i = SUPER * S + a;
    j = SUPER * S + (r - a * (a + 1) / 2);
  }
}
__device__ __forceinline__ void hess_work(int id, int padded_tiles, int splits, int& split,
                                          int& ti, int& tj) {
  (void)splits;
  split = id / padded_tiles;
  super_tile_coords(id % padded_tiles, ti, tj);
}

// One wave-wide 1 KB copy global -> LDS: lane l's 16 bytes at buffer offset voff land at
// lds_base + 16 l.  Written as asm so that the compiler's wait insertion does not treat
// every later LDS read as dependent on it (it would drain the whole pipeline); the
// explicit vmcnt waits before each stage barrier order the copies.  No register output.
__device__ __forceinline__ void dma16(rsrc_t rsrc, uint32_t lds_base, int voff) {
  __asm__ volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "s"(lds_base)
                   : "memory", "m0");
}

// Copy q (0..V2_BK/2 - 1) of one operand's stage: a wave-wide 1 KB copy of token rows 2q,
// 2q+1 (V2_CPO per wave).
__device__ __forceinline__ void v2_load_copy(rsrc_t rsrc, short* dst, int tok_in_range, int64_t ldx,
                                             int64_t ch0, int q, int lane) {
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)dst);
  const int row = 2 * q + (lane >> 5);
  const int slot = lane & 31;
  const int chunk = v2_slot(row, slot);            // XOR is an involution
  const int voff = (int)(((int64_t)(tok_in_range + row) * ldx + ch0 + 8 * chunk) * 2);
  dma16(rsrc, __builtin_amdgcn_readfirstlane(lds0 + q * 1024), voff);
}

// Operand fragment for one 32x32x16 MFMA: channels c_base..+31, tokens k_sub..+15 of a stage.
__device__ __forceinline__ half8 v2_frag(const short* stage, int c_base, int k_sub, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int ch = c_base + 16 * (g & 1) + 4 * (j & 3);
  const int chunk = ch >> 3, half_off = (ch & 7);   // 0 or 4 halfs into the chunk
  const int r0 = k_sub + 8 * (g >> 1) + (j >> 2);
  const int r1 = r0 + 4;
  const short* p0 = stage + r0 * TILE + v2_slot(r0, chunk) * 8 + half_off;
  const short* p1 = stage + r1 * TILE + v2_slot(r1, chunk) * 8 + half_off;
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p0);
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p1);
  const short4v c8[2] = {a, b};
  half8 out;
  __builtin_memcpy(&out, c8, sizeof(out));
  return out;
}

// vmcnt wait with compile-time count (gfx9 encoding; expcnt and lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// vmcnt wait that leaves `later` stages of CPW copies each in flight (later <= I)
template <int CPW, int I>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (I <= 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= I) wait_vmcnt<I * CPW>();
    else wait_later<CPW, I - 1>(later);
  }
}
// Workgroup barrier without the memory fence of __syncthreads (whose release half would
// drain every outstanding load, including the stages meant to stay in flight).  The caller
// has waited for the loads it needs; lgkmcnt(0) retires this wave's LDS reads first.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
}

__global__ void __launch_bounds__(64 * V2_WAVES, 1)
hess_f16_lds(const _Float16* __restrict__ X, int64_t ldx, int64_t d, int64_t n_tok,
             int64_t tok_per_split, int tiles, int padded_tiles, int splits,
             float* __restrict__ part) {
  // V2_NST stages x {A, B} x V2_BK tokens x 256 channels
  __shared__ __attribute__((aligned(16))) short lds[V2_NST * 2 * V2_STAGE_HALFS];

  int split, ti, tj;
  hess_work(blockIdx.x, padded_tiles, splits, split, ti, tj);
  if ((int64_t)ti * TILE >= d) return;   // padding of the super-tile grid
  const int tile = ti * (ti + 1) / 2 + tj;
  const bool diag = ti == tj;
  const int64_t ca0 = (int64_t)ti * TILE, cb0 = (int64_t)tj * TILE;
  const int64_t t_begin = (int64_t)split * tok_per_split;
  int64_t t_end = t_begin + tok_per_split;
  if (t_end > n_tok) t_end = n_tok;
  const int64_t n_here = t_end > t_begin ? t_end - t_begin : 0;
  const int nsteps = (int)((n_here + V2_BK - 1) / V2_BK);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (LDS base in M0)
  const int wm = wave >> 2, wn = wave & 3;   // rows wm * 128 .., columns wn * 64 ..
  // buffer over exactly this workgroup's tokens; bytes beyond it read as zero
  // (built from readfirstlane'd values so that it lives in scalar registers)
  const uint64_t base = reinterpret_cast<uint64_t>(X + (n_here ? t_begin : 0) * ldx);
  const uint32_t base_lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t base_hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const int nbytes = __builtin_amdgcn_readfirstlane((int)(n_here * ldx * 2));
  // buffer descriptor: base, stride 0, size in bytes, raw 32-bit data format
  const rsrc_t rsrc = {base_lo, base_hi & 0xffffu, (uint32_t)nbytes, 0x00020000u};

  floatx16 acc[4][V2_BFR];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < V2_BFR; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  auto stage_a = [&](int st) { return lds + (st % V2_NST) * 2 * V2_STAGE_HALFS; };
  // copy i (0 .. 2 V2_CPO - 1) of this wave's share of stage st: operand A, then operand B
  auto issue_part = [&](int st, int i) {
    short* dst = stage_a(st) + (i >= V2_CPO ? V2_STAGE_HALFS : 0);
    v2_load_copy(rsrc, dst, st * V2_BK, ldx, i >= V2_CPO ? cb0 : ca0,
                 wave * V2_CPO + (i % V2_CPO), lane);
  };
  auto issue = [&](int st) {
#pragma unroll
    for (int i = 0; i < V2_CPO; ++i) issue_part(st, i);
    if (!diag) {
#pragma unroll
      for (int i = V2_CPO; i < 2 * V2_CPO; ++i) issue_part(st, i);
    }
  };

#pragma unroll
  for (int i = 0; i < V2_NST - 1; ++i)
    if (i < nsteps) issue(i);

  if (diag) {
    // A diagonal tile needs only its 36 fragments (32 x 32) on or below the diagonal:
    // (R, C) with C <= R in the 8 x 8 grid (the reduction reads nothing above it).  Each wave
    // keeps a 128 x 64 rectangle of the usual layout (role (dm, dn)) and skips the MFMAs of
    // fragments above the diagonal; the roles need 7, 3, 0, 0 (dm = 0) and 8, 8, 7, 3
    // (dm = 1) fragments.  Waves are placed on the SIMDs round robin (wave w on SIMD w % 4),
    // so roles are permuted to pair 8 with 0 and 7 with 3 on each SIMD: at most 10 MFMAs per
    // SIMD and 16 tokens instead of 16.  Only operand A is staged.
    const int role = (0x17326054u >> (4 * wave)) & 0xf;
    const int dm = role >> 2, dn = role & 3;
    uint32_t need = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < V2_BFR; ++b)
        if (2 * dn + b <= 4 * dm + a) need |= 1u << (a * V2_BFR + b);
    need = __builtin_amdgcn_readfirstlane(need);
    for (int s = 0; s < nsteps; ++s) {
      const int later = nsteps - 1 - s < V2_NST - 2 ? nsteps - 1 - s : V2_NST - 2;
      wait_later<V2_CPO, V2_NST - 2>(later);
      stage_barrier();
      const bool more = s + V2_NST - 1 < nsteps;
      const short* sa = stage_a(s);
#pragma unroll
      for (int kk = 0; kk < V2_BK / 16; ++kk) {
        if (need) {
          half8 af[4], bf[V2_BFR];
#pragma unroll
          for (int a = 0; a < 4; ++a) af[a] = v2_frag(sa, dm * 128 + a * 32, kk * 16, lane);
#pragma unroll
          for (int b = 0; b < V2_BFR; ++b) bf[b] = v2_frag(sa, dn * 64 + b * 32, kk * 16, lane);
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < V2_BFR; ++b)
              if (need & (1u << (a * V2_BFR + b)))
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int part = kk * 4 + a;
          if (more && part < V2_CPO) issue_part(s + V2_NST - 1, part);
        }
      }
    }
    float* out = part + ((int64_t)split * tiles + tile) * (int64_t)TILE * TILE;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < V2_BFR; ++b) {
        if (!(need & (1u << (a * V2_BFR + b)))) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = dm * 128 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = dn * 64 + b * 32 + (lane & 31);
          out[row * TILE + col] = acc[a][b][r];
        }
      }
    return;
  }

  for (int s = 0; s < nsteps; ++s) {
    // stage s has landed once at most `later` stages issued after it are pending
    // (copies retire in order; V2_CPO per operand per wave and stage)
    const int later = nsteps - 1 - s < V2_NST - 2 ? nsteps - 1 - s : V2_NST - 2;
    if (diag) wait_later<V2_CPO, V2_NST - 2>(later);
    else wait_later<2 * V2_CPO, V2_NST - 2>(later);
    stage_barrier();
    // stage s + V2_NST - 1 goes into the buffer read in iteration s - 1; its copies go
    // between the first MFMAs so that a stalled copy issue does not leave the matrix core idle
    const bool more = s + V2_NST - 1 < nsteps;
    const short* sa = stage_a(s);
    const short* sb = diag ? sa : sa + V2_STAGE_HALFS;
#pragma unroll
    for (int kk = 0; kk < V2_BK / 16; ++kk) {
      half8 af[4], bf[V2_BFR];
#pragma unroll
      for (int a = 0; a < 4; ++a) af[a] = v2_frag(sa, wm * 128 + a * 32, kk * 16, lane);
#pragma unroll
      for (int b = 0; b < V2_BFR; ++b) bf[b] = v2_frag(sb, wn * 64 + b * 32, kk * 16, lane);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < V2_BFR; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
        const int part = kk * 4 + a;   // V2_BK / 4 slots per stage, the first 2 V2_CPO used
        if (more && part < 2 * V2_CPO && (part < V2_CPO || !diag)) issue_part(s + V2_NST - 1, part);
      }
    }
  }

  float* out = part + ((int64_t)split * tiles + tile) * (int64_t)TILE * TILE;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < V2_BFR; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * 64 + b * 32 + (lane & 31);
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
  const int64_t sstride = (int64_t)tiles * TILE * TILE;   // between the splits of one tile
  // four columns 4 tq .. 4 tq + 3 of rows ty4 + 16 q (q = 0..3) per thread, four splits per
  // step: 16 loads of 16 bytes in flight per lane; each element's sum keeps split order
  const int tq = threadIdx.x % 16, ty4 = threadIdx.x / 16;
  const float* pq = part + (int64_t)tile * TILE * TILE + (int64_t)(sa * 64) * TILE + sbk * 64 + 4 * tq;
  const bool h_vec = (d & 3) == 0 && ((reinterpret_cast<uintptr_t>(H) & 15) == 0);
  {
    floatx4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    int sp = 0;
    for (; sp + 4 <= splits; sp += 4) {
      floatx4 a[4][4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          a[q][k] = *reinterpret_cast<const floatx4*>(pq + (ty4 + 16 * q) * TILE + (sp + k) * sstride);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) v[q] += a[q][k];
    }
    for (; sp < splits; ++sp)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] += *reinterpret_cast<const floatx4*>(pq + (ty4 + 16 * q) * TILE + sp * sstride);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = ty4 + 16 * q;
      const floatx4 w = 2.0f * v[q];
      const int64_t i = r0 + rr, j0 = c0 + 4 * tq;
#pragma unroll
      for (int c = 0; c < 4; ++c) s[rr][4 * tq + c] = w[c];
      if (h_vec && i < d && j0 + 3 < d && (!diag || j0 + 3 <= i)) {
        floatx4* hp = reinterpret_cast<floatx4*>(H + i * d + j0);
        *hp = *hp + w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t j = j0 + c;
          if (i < d && j < d && (!diag || j <= i)) H[i * d + j] += w[c];
        }
      }
    }
  }
  __syncthreads();
  // mirror: H[c0 + rr][r0 + tx] += s[tx][rr] for entries strictly below the diagonal
  for (int rr = ty; rr < 64; rr += 4) {
    const int64_t i = c0 + rr, j = r0 + tx;  // upper-triangle position (i < j)
    if (i < d && j < d && (!diag || tx > rr)) H[i * d + j] += s[tx][rr];
  }
}

}  // namespace

HessPlan hessian_plan(int64_t d, int64_t n_tok, int64_t ldx, int x_dtype) {
  HessPlan p{};
  p.d = d;
  p.n_tok = n_tok;
  if (ldx < d) ldx = d;
  const int64_t nb = ceil_div(d, TILE);
  p.tiles = (int)(nb * (nb + 1) / 2);
  const int64_t nbp = ceil_div(nb, 4) * 4;
  p.padded_tiles = (int)(nbp * (nbp + 1) / 2);
  // Enough workgroups to fill 256 CUs with a short tail, each split >= 2048 tokens.
  const int64_t cus = 256;
  const int64_t min_tok = 2048;
  int best = 1;
  double best_cost = 1e30;
  const int64_t max_split = n_tok / min_tok > 1 ? n_tok / min_tok : 1;
  // one split's rows must stay below 2^30 bytes (32-bit buffer offsets)
  const int64_t elt = x_dtype == 0 ? 2 : 4;
  const int64_t min_split = ceil_div(n_tok * ldx * elt, (int64_t)1 << 30);
  // What matters is the number of full rounds of workgroups (136 tiles x 16 splits leaves a
  // half-empty ninth round, 15 splits fill exactly eight) against the partial tiles every
  // split writes and the reduction reads again.  That traffic is fixed per tile while a
  // tile's work grows with the token count, so its weight is 0.004 per split at 262144
  // tokens, scaled by 262144 / n_tok (fitted on MI355X at d = 4096 and 8192).
  const double per_split = 0.004 * 262144.0 / (double)(n_tok > 0 ? n_tok : 1);
  for (int64_t s = min_split; s <= max_split || s == min_split; ++s) {
    if (s > 64 && s > min_split) break;
    const int64_t wgs = p.tiles * s * (x_dtype == 0 ? 1 : 16);
    const double rounds = (double)ceil_div(wgs, cus);
    // time ~ rounds * work per workgroup (1/s), plus partial-tile traffic per split
    const double cost = rounds / (double)s * (x_dtype == 0 ? 1.0 : 1.0 / 16.0) + per_split * (double)s;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = (int)s;
    }
  }
  p.splits = best;
  int64_t tps = ceil_div(n_tok, best);
  tps = ceil_div(tps, 64) * 64;
  p.tok_per_split = tps > 0 ? tps : 64;
  p.ws_bytes = (size_t)p.splits * p.tiles * TILE * TILE * sizeof(float);
  return p;
}

hipError_t hessian_launch(const HessPlan& p, float* H, const void* X, int x_dtype, int64_t ldx,
                          void* ws, hipStream_t stream) {
  float* part = static_cast<float*>(ws);
  {
    ProfScope ps("hessian_mfma", stream);
    if (x_dtype == 0) {
      hipLaunchKernelGGL(hess_f16_lds, dim3(p.padded_tiles * p.splits), dim3(64 * V2_WAVES), 0, stream,
                         static_cast<const _Float16*>(X), ldx, p.d, p.n_tok, p.tok_per_split,
                         p.tiles, p.padded_tiles, p.splits, part);
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
