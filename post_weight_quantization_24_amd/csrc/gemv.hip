// Weight-only quantized linear layer over the packed output of the column solve:
//     y[b][r] = sum_c x[b][c] * s[r][c / g] * (code[r][c] - z[r][c / g])
// for a few fp16 activation rows x (page "量化": section GPTQ, per-channel INT4 weights for
// memory-bound single-batch inference; section AWQ, W4A16 with the dequantization inside the
// matrix product, so no fp16 weight matrix is ever written).
//
// Layout of the work:
//   * One wave per output row (a grid-stride loop over rows); lane l takes the runs of 32
//     consecutive codes l, l + 64, ...  A run is exactly `bits` 32-bit words of the row, so
//     every load is aligned and the lanes of a wave read consecutive bytes.  With g a
//     multiple of 32 a run lies in one group: one scale and one zero per run.  For 2- and
//     4-bit codes with at most four runs per lane (d_col <= 8192) all runs of a row (with
//     their scales and zeros) are requested together, the next row's while the current one is
//     reduced, and the first row's before the activations are staged.
//   * The grid is one round of resident workgroups (what the registers and the staged
//     activations let fit on the chip), each wave looping over rows.
//   * The activation rows are staged once per workgroup in LDS as fp16, piece-major.
//   * INT4: the nibbles k and k + 4 of a word land in the two halves of
//     (w >> 4k) & 0x000F000F; OR-ing 0x6400 into each half gives the fp16 values 1024 + q,
//     and subtracting 1024 + z leaves q - z exactly (|q - z| < 16).  v_dot2_f32_f16 then
//     multiplies the pair with (x_k, x_k+4) and accumulates in fp32, so x is staged in that
//     pair order.  Per run the fp32 dot of (q - z) and x is scaled once by s.
//   * INT2: the same with the codes j and j + 8 of a word: (w >> 8s) & (0x00030003 << 2t)
//     ORed with 0x6400 is the pair 1024 + 4^t q, one packed fma by 4^-t with -(1024 4^-t + z)
//     leaves q - z exactly, and v_dot2_f32_f16 takes (x_j, x_j+8), staged in that order.
//   * INT3: codes i and i + 16 of a run lie 48 bits apart, so the low halves of
//     (w >> 3i) over the run's low 64 bits and over its high 64 bits hold them at bits 0 and
//     16; masked and ORed with 0x6400 they are the pair 1024 + q, the packed subtract of
//     1024 + z leaves q - z, and v_dot2_f32_f16 takes (x_i, x_i+16), staged in that order.
//   * INT8: the codes are extracted from a 64-bit window of two words, converted to fp32 and
//     accumulated with fp32 fused multiply-adds, one run after the other.
//   * The 64 lane sums of a row are added by a butterfly, in a fixed order.

#include <map>
#include <mutex>
#include <utility>

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int MV_THREADS = 512;                  // 8 waves
constexpr int MV_WAVES = MV_THREADS / 64;
constexpr int MV_MAX_NB = 8;                     // activation rows per launch
constexpr size_t MV_LDS = 64 * 1024;             // staged x (at most)

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Position of column c inside its 8-column piece in the INT4 pair order: (x_8j+k, x_8j+k+4)
// at 8j + 2k, 8j + 2k + 1
__device__ __forceinline__ int pos4(int c) {
  const int k = c & 7;
  return (c & ~7) + ((k & 3) << 1) + (k >> 2);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// The runs of one row that belong to this lane (k = lane + 64 i < runs), with their scale and
// zero, all loads issued together.
template <int BITS, int RPL>
struct RowRuns {
  uint32_t w[RPL][BITS];
  float s[RPL];
  int z[RPL];
};

// Group of run k as (k * mul) >> shift, exact for k < 1024 runs and up to 1024 runs per group:
// one group per row (mul 0), a power of two 2^s runs per group (mul 1, shift s), otherwise
// mul = ceil(2^40 / runs per group) and shift 40 (the rounding error of mul is below 2^-30).
struct Grp {
  int n_groups;    // per row
  uint64_t mul;
  int shift;
};
__device__ __forceinline__ int group_of(const Grp& gp, int k) {
  return (int)(((uint64_t)(uint32_t)k * gp.mul) >> gp.shift);
}

template <int BITS, int RPL>
__device__ __forceinline__ void load_runs(RowRuns<BITS, RPL>& rr, const uint32_t* __restrict__ rowp,
                                          const float* __restrict__ srow,
                                          const uint8_t* __restrict__ zrow, const Grp& gp,
                                          int runs, int lane) {
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const int k = lane + 64 * i;
    if (k < runs) {
      const uint32_t* p = rowp + k * BITS;
      if constexpr (BITS == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        rr.w[i][0] = v.x; rr.w[i][1] = v.y; rr.w[i][2] = v.z; rr.w[i][3] = v.w;
      } else if constexpr (BITS == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        rr.w[i][0] = v.x; rr.w[i][1] = v.y;
      } else if constexpr (BITS == 8) {
        const uint4 v0 = reinterpret_cast<const uint4*>(p)[0], v1 = reinterpret_cast<const uint4*>(p)[1];
        rr.w[i][0] = v0.x; rr.w[i][1] = v0.y; rr.w[i][2] = v0.z; rr.w[i][3] = v0.w;
        rr.w[i][4] = v1.x; rr.w[i][5] = v1.y; rr.w[i][6] = v1.z; rr.w[i][7] = v1.w;
      } else {
#pragma unroll
        for (int j = 0; j < BITS; ++j) rr.w[i][j] = p[j];
      }
      const int gi = group_of(gp, k);
      rr.s[i] = srow[gi];
      rr.z[i] = zrow[gi];
    }
  }
}

// Activation rows to LDS, in the pair order of the code expansion: for 4-bit codes
// (x_k, x_k+4) within each 8-column piece, for 2-bit codes (x_j, x_j+8) within each
// 16-column block (two pieces), else natural.  16-byte pieces of 8 columns, four loads per
// thread in flight before the stores; the pair orders are shuffles of the pieces' dwords.
// Piece p of run k is stored at (p * runs + k) * 16 bytes, so the 64 lanes of a wave (runs
// k .. k + 63) read consecutive 16-byte slots: no bank conflicts.  Unaligned rows fall back to
// one element at a time.
__device__ __forceinline__ int pos2(int c) {   // 2-bit pair order inside a 32-column run
  const int r = c & 31, i = r >> 4, j = r & 15, kk = j & 7;
  return 16 * i + 8 * (kk >> 2) + 2 * (kk & 3) + (j >> 3);
}
__device__ __forceinline__ int pos3(int c) {   // 3-bit pair order: (x_i, x_i+16) of a run
  const int r = c & 31, i = r & 15;
  return 8 * (i >> 2) + 2 * (i & 3) + (r >> 4);
}
template <int MODE>
__device__ __forceinline__ void stage_x(_Float16* xs, const _Float16* __restrict__ x, int64_t ldx,
                                        int nb, int dc) {
  constexpr bool PAIRS = MODE == 4;
  const bool vec = ((reinterpret_cast<uintptr_t>(x) | (uintptr_t)(ldx * 2)) & 15) == 0;
  if (MODE == 3 && vec) {
    // a whole run (four pieces) per thread and step: (x_i, x_i+16) for i = 0..15, four pairs
    // per output piece
    const int per_row = dc / 32, runs_all = nb * per_row;
    for (int i = threadIdx.x; i < runs_all; i += MV_THREADS) {
      const int b = i / per_row, k = i - b * per_row;
      const uint4* src = reinterpret_cast<const uint4*>(x + b * ldx + 32 * k);
      const uint4 v[4] = {src[0], src[1], src[2], src[3]};
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {     // pieces hp and hp + 2 pair up
        const uint4 lo = v[hp], hi = v[hp + 2];
        uint4 o0, o1;
        o0.x = (lo.x & 0xffffu) | (hi.x << 16);
        o0.y = (lo.x >> 16) | (hi.x & 0xffff0000u);
        o0.z = (lo.y & 0xffffu) | (hi.y << 16);
        o0.w = (lo.y >> 16) | (hi.y & 0xffff0000u);
        o1.x = (lo.z & 0xffffu) | (hi.z << 16);
        o1.y = (lo.z >> 16) | (hi.z & 0xffff0000u);
        o1.z = (lo.w & 0xffffu) | (hi.w << 16);
        o1.w = (lo.w >> 16) | (hi.w & 0xffff0000u);
        *reinterpret_cast<uint4*>(xs + b * dc + 8 * ((2 * hp) * (dc / 32) + k)) = o0;
        *reinterpret_cast<uint4*>(xs + b * dc + 8 * ((2 * hp + 1) * (dc / 32) + k)) = o1;
      }
    }
  } else if (MODE == 2 && vec) {
    // two pieces (a 16-column block) per thread and step: (x_j, x_j+8) for j = 0..3 into the
    // first output piece, j = 4..7 into the second
    const int per_row = dc / 16, blocks = nb * per_row;
    for (int i = threadIdx.x; i < blocks; i += MV_THREADS) {
      const int b = i / per_row, c16 = i - b * per_row;
      const uint4 v0 = *reinterpret_cast<const uint4*>(x + b * ldx + 16 * c16);
      const uint4 v1 = *reinterpret_cast<const uint4*>(x + b * ldx + 16 * c16 + 8);
      uint4 o0, o1;
      o0.x = (v0.x & 0xffffu) | (v1.x << 16);
      o0.y = (v0.x >> 16) | (v1.x & 0xffff0000u);
      o0.z = (v0.y & 0xffffu) | (v1.y << 16);
      o0.w = (v0.y >> 16) | (v1.y & 0xffff0000u);
      o1.x = (v0.z & 0xffffu) | (v1.z << 16);
      o1.y = (v0.z >> 16) | (v1.z & 0xffff0000u);
      o1.z = (v0.w & 0xffffu) | (v1.w << 16);
      o1.w = (v0.w >> 16) | (v1.w & 0xffff0000u);
      const int k = c16 >> 1, p = 2 * (c16 & 1);          // run, first output piece
      *reinterpret_cast<uint4*>(xs + b * dc + 8 * (p * (dc / 32) + k)) = o0;
      *reinterpret_cast<uint4*>(xs + b * dc + 8 * ((p + 1) * (dc / 32) + k)) = o1;
    }
  } else if (vec) {
    const int per_row = dc / 8, pieces = nb * per_row;
    for (int i0 = threadIdx.x; i0 < pieces; i0 += 4 * MV_THREADS) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * MV_THREADS;
        if (i < pieces) {
          const int b = i / per_row, c8 = i - b * per_row;
          v[u] = *reinterpret_cast<const uint4*>(x + b * ldx + 8 * c8);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * MV_THREADS;
        if (i < pieces) {
          const int b = i / per_row, c8 = i - b * per_row;
          const int k = c8 >> 2, p = c8 & 3;          // run, piece of the run
          uint4 o = v[u];
          if (PAIRS) {   // halves (0..7) -> (0, 4), (1, 5), (2, 6), (3, 7)
            o.x = (v[u].x & 0xffffu) | (v[u].z << 16);
            o.y = (v[u].x >> 16) | (v[u].z & 0xffff0000u);
            o.z = (v[u].y & 0xffffu) | (v[u].w << 16);
            o.w = (v[u].y >> 16) | (v[u].w & 0xffff0000u);
          }
          *reinterpret_cast<uint4*>(xs + b * dc + 8 * (p * (dc / 32) + k)) = o;
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < nb * dc; i += MV_THREADS) {
      const int b = i / dc, c = i - b * dc;
      const int k = c >> 5;
      const int q = MODE == 2 ? pos2(c) : MODE == 3 ? pos3(c) : (c & 24) + (PAIRS ? pos4(c) & 7 : c & 7);
      xs[b * dc + 8 * ((q >> 3) * (dc / 32) + k) + (q & 7)] = x[b * ldx + c];
    }
  }
}

// Sum over one run of 32 codes (k) of (code - z) * x for every activation row, in fp32.
template <int BITS, int NB>
__device__ __forceinline__ void run_dot(const uint32_t (&w)[BITS], int z, const _Float16* xs,
                                        int dc, int k, float (&part)[NB]) {
  if constexpr (BITS == 4) {
    const _Float16 zh = (_Float16)(1024 + z);
    const half2v zz = {zh, zh};
    const uint32_t magic = 0x64006400u;   // fp16 1024 in both halves (a VGPR operand)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half2v q[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // (w >> 4 kk) & 0x000F000F | 0x64006400 in one v_and_or_b32 (the compiler emits an
        // and and an or); a pure register operation with no memory operand
        uint32_t t;
        __asm__("v_and_or_b32 %0, %1, %2, %3"
                : "=v"(t)
                : "v"(w[j] >> (4 * kk)), "s"(0x000F000Fu), "v"(magic));
        q[kk] = __builtin_bit_cast(half2v, t) - zz;         // (q_k - z, q_k+4 - z), exact
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + b * dc + 8 * (j * (dc / 32) + k));
        const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          part[b] = __builtin_amdgcn_fdot2(q[kk], __builtin_bit_cast(half2v, xa[kk]), part[b],
                                           false);
      }
    }
  } else if constexpr (BITS == 2) {
    // word i holds columns 16 i .. 16 i + 15 of the run.  For kk = 4 s + t, the codes kk and
    // kk + 8 sit in bits 8 s + 2 t (+ 16) of the word: masked in place and ORed with
    // 0x6400 they are the fp16 values 1024 + 4^t c, and one packed fma by 4^-t with
    // -(1024 4^-t + z) leaves c - z exactly (all values are small integers times powers of 2).
    const uint32_t magic = 0x64006400u;
    half2v scl[4], off[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const _Float16 sc = (_Float16)(1.0f / (float)(1 << (2 * t)));
      const _Float16 of = (_Float16)(-(1024.0f / (float)(1 << (2 * t))) - (float)z);
      scl[t] = half2v{sc, sc};
      off[t] = half2v{of, of};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      half2v q[8];
#pragma unroll
      for (int s8 = 0; s8 < 2; ++s8) {
        const uint32_t ws = w[i] >> (8 * s8);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint32_t h;
          __asm__("v_and_or_b32 %0, %1, %2, %3"
                  : "=v"(h)
                  : "v"(ws), "s"(0x00030003u << (2 * t)), "v"(magic));
          q[4 * s8 + t] = __builtin_bit_cast(half2v, h) * scl[t] + off[t];
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint4 xa = *reinterpret_cast<const uint4*>(xs + b * dc + 8 * ((2 * i) * (dc / 32) + k));
        const uint4 xb = *reinterpret_cast<const uint4*>(xs + b * dc + 8 * ((2 * i + 1) * (dc / 32) + k));
        const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          part[b] = __builtin_amdgcn_fdot2(q[kk], __builtin_bit_cast(half2v, xv[kk]), part[b],
                                           false);
      }
    }
  } else if constexpr (BITS == 3) {
    // code i of the run at bit 3 i of (w2:w1:w0); codes i and i + 16 are 48 bits apart, so
    // (w >> 3 i) of the low 64 bits has code i at bit 0 and (w >> 3 i) of the high 64 bits
    // code i + 16 at bit 16: their low and high halves, masked and ORed with 0x6400, are the
    // fp16 pair (1024 + q_i, 1024 + q_i+16), and one packed subtract of 1024 + z leaves
    // q - z exactly.
    const _Float16 zh = (_Float16)(1024 + z);
    const half2v zz = {zh, zh};
    const uint32_t magic = 0x64006400u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {            // output piece p: pairs i = 4 p .. 4 p + 3
      half2v q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * p + e, sh = 3 * i;
        const uint32_t lo = sh < 32 ? __builtin_amdgcn_alignbit(w[1], w[0], (uint32_t)sh)
                                    : __builtin_amdgcn_alignbit(w[2], w[1], (uint32_t)(sh - 32));
        const uint32_t hi = sh < 32 ? __builtin_amdgcn_alignbit(w[2], w[1], (uint32_t)sh)
                                    : w[2] >> (sh - 32);
        const uint32_t both = __builtin_amdgcn_perm(hi, lo, 0x07060100u);   // lo 16 | hi 16
        uint32_t t;
        __asm__("v_and_or_b32 %0, %1, %2, %3"
                : "=v"(t)
                : "v"(both), "s"(0x00070007u), "v"(magic));
        q[e] = __builtin_bit_cast(half2v, t) - zz;
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + b * dc + 8 * (p * (dc / 32) + k));
        const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          part[b] = __builtin_amdgcn_fdot2(q[e], __builtin_bit_cast(half2v, xa[e]), part[b],
                                           false);
      }
    }
  } else {
    const float zf = (float)z;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float qz[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        constexpr uint32_t mask = (1u << BITS) - 1u;
        const int bit = (8 * p + e) * BITS, wi = bit >> 5, sh = bit & 31;
        const uint32_t hi = wi + 1 < BITS ? w[wi + 1] : 0u;
        const uint64_t win = ((uint64_t)hi << 32) | w[wi];
        qz[e] = (float)((uint32_t)(win >> sh) & mask) - zf;
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + b * dc + 8 * (p * (dc / 32) + k));
        const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const half2v h = __builtin_bit_cast(half2v, xa[e >> 1]);
          part[b] = fmaf(qz[e], (float)h[e & 1], part[b]);
        }
      }
    }
  }
}

template <int BITS, int RPL, int NB>
__global__ void __launch_bounds__(MV_THREADS)
dequant_matvec(const uint32_t* __restrict__ qw, const float* __restrict__ scales,
               const uint8_t* __restrict__ zeros, int64_t d_row, int64_t d_col, Grp gp,
               const _Float16* __restrict__ x, int64_t ldx, float* __restrict__ y, int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) _Float16 xs[];   // nb rows of d_col
  const int dc = (int)d_col;
  const int lane = threadIdx.x & 63;
  const int64_t n_waves = (int64_t)gridDim.x * MV_WAVES;
  const int runs = dc / 32;
  const int64_t words = d_col * BITS / 32;          // per row
  int64_t r = (int64_t)blockIdx.x * MV_WAVES + (threadIdx.x >> 6);
  // 2- and 4-bit codes with at most 4 runs per lane: whole rows in registers (prefetched).
  // 8-bit codes and wider rows already give each lane several loads per row; 3-bit codes,
  // prefetched (71-145 VGPRs), measured -1 % to +4 % on MI355X.  They take the codes run by
  // run.
  constexpr bool PREFETCH = (BITS == 4 || BITS == 2) && RPL <= 4;

  // the first row's codes are requested before x is staged, so the two fetches overlap
  RowRuns<BITS, PREFETCH ? RPL : 1> rr;
  if constexpr (PREFETCH)
    if (r < d_row)
      load_runs<BITS, RPL>(rr, qw + r * words, scales + r * gp.n_groups, zeros + r * gp.n_groups, gp,
                           runs, lane);
  stage_x<BITS == 8 ? 0 : BITS>(xs, x, ldx, NB, dc);
  __syncthreads();

  for (; r < d_row; r += n_waves) {
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
    if constexpr (PREFETCH) {
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int k = lane + 64 * i;
        if (k >= runs) continue;
        float part[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) part[b] = 0.0f;
        run_dot<BITS, NB>(rr.w[i], rr.z[i], xs, dc, k, part);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = fmaf(rr.s[i], part[b], acc[b]);
      }
      // next row's codes in flight while this row's sums are reduced and stored
      const int64_t rn = r + n_waves;
      if (rn < d_row)
        load_runs<BITS, RPL>(rr, qw + rn * words, scales + rn * gp.n_groups,
                             zeros + rn * gp.n_groups, gp, runs, lane);
    } else {
      for (int k = lane; k < runs; k += 64) {
        uint32_t w[BITS];
        const uint32_t* p = qw + r * words + k * BITS;
#pragma unroll
        for (int j = 0; j < BITS; ++j) w[j] = p[j];
        const int64_t gi = r * gp.n_groups + group_of(gp, k);
        float part[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) part[b] = 0.0f;
        run_dot<BITS, NB>(w, zeros[gi], xs, dc, k, part);
        const float sc = scales[gi];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = fmaf(sc, part[b], acc[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = wave_sum(acc[b]);
      if (lane == 0) y[b * ldy + r] = v;
    }
  }
}

template <int BITS, int RPL, int NB>
hipError_t launch_nb(const uint32_t* qw, const float* scales, const uint8_t* zeros, int64_t d_row,
                     int64_t d_col, Grp g, const _Float16* x, int64_t ldx, float* y,
                     int64_t ldy, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(dequant_matvec<BITS, RPL, NB>);
  const size_t lds = (size_t)NB * d_col * sizeof(_Float16);
  // Per device, once (callers on several threads share it): the dynamic LDS limit is raised
  // and the CU count read; per device and LDS size, once: the workgroups that fit on a CU.
  static std::mutex mu;
  static bool attr[64] = {};
  static int cus[64] = {};
  static std::map<std::pair<int, size_t>, int> per_cu_of;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> lk(mu);
    if (!attr[dev]) {
      e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)MV_LDS);
      if (e != hipSuccess) return e;
      e = hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      attr[dev] = true;
    }
    const auto key = std::make_pair(dev, lds);
    const auto it = per_cu_of.find(key);
    if (it != per_cu_of.end()) {
      per_cu = it->second;
    } else {
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, MV_THREADS, lds);
      if (e != hipSuccess) return e;
      per_cu_of[key] = per_cu;
    }
  }
  // One round of resident workgroups, each wave looping over rows: the grid is what fits on
  // the chip at once (registers and the staged activations decide), so no partial second
  // round of workgroups starts after the first (INT4 with 4 runs per lane holds 71 VGPRs:
  // three 8-wave workgroups per CU, not four).
  const int64_t fit = (int64_t)(per_cu > 0 ? per_cu : 1) * (cus[dev] > 0 ? cus[dev] : 1);
  const int64_t want = ceil_div(d_row, (int64_t)MV_WAVES);
  const unsigned grid = (unsigned)(want < fit ? want : fit);
  hipLaunchKernelGGL((dequant_matvec<BITS, RPL, NB>), dim3(grid), dim3(MV_THREADS), lds, s, qw,
                     scales, zeros, d_row, d_col, g, x, ldx, y, ldy);
  return hipGetLastError();
}

template <int BITS, int RPL>
hipError_t launch_rpl(const uint32_t* qw, const float* scales, const uint8_t* zeros,
                      int64_t d_row, int64_t d_col, Grp g, const _Float16* x, int64_t ldx,
                      int nb, float* y, int64_t ldy, hipStream_t s) {
  switch (nb) {
    case 1: return launch_nb<BITS, RPL, 1>(qw, scales, zeros, d_row, d_col, g, x, ldx, y, ldy, s);
    case 2: return launch_nb<BITS, RPL, 2>(qw, scales, zeros, d_row, d_col, g, x, ldx, y, ldy, s);
    case 4: return launch_nb<BITS, RPL, 4>(qw, scales, zeros, d_row, d_col, g, x, ldx, y, ldy, s);
    case 8: return launch_nb<BITS, RPL, 8>(qw, scales, zeros, d_row, d_col, g, x, ldx, y, ldy, s);
    default: return hipErrorInvalidValue;
  }
}

// runs of 32 codes per lane: d_col / 2048 rounded up to 2, 4, 8 or 16 (d_col <= 32768)
template <int BITS>
hipError_t launch_bits(const uint32_t* qw, const float* scales, const uint8_t* zeros,
                       int64_t d_row, int64_t d_col, Grp g, const _Float16* x, int64_t ldx,
                       int nb, float* y, int64_t ldy, hipStream_t s) {
  const int64_t rpl = ceil_div(d_col, 2048);
  if (rpl <= 2) return launch_rpl<BITS, 2>(qw, scales, zeros, d_row, d_col, g, x, ldx, nb, y, ldy, s);
  if (rpl <= 4) return launch_rpl<BITS, 4>(qw, scales, zeros, d_row, d_col, g, x, ldx, nb, y, ldy, s);
  if (rpl <= 8) return launch_rpl<BITS, 8>(qw, scales, zeros, d_row, d_col, g, x, ldx, nb, y, ldy, s);
  return launch_rpl<BITS, 16>(qw, scales, zeros, d_row, d_col, g, x, ldx, nb, y, ldy, s);
}

}  // namespace

int64_t matvec_max_rows_per_launch(int64_t d_col) {
  const int64_t fit = (int64_t)(MV_LDS / sizeof(_Float16)) / d_col;
  return fit < MV_MAX_NB ? fit : MV_MAX_NB;
}

hipError_t matvec_launch(const uint32_t* qw, const float* scales, const uint8_t* zeros,
                         int64_t d_row, int64_t d_col, int bits, int group, const void* x,
                         int64_t n, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  const int64_t gsz = group == 0 ? d_col : group;
  Grp g;
  g.n_groups = (int)(d_col / gsz);
  const int64_t rpg = gsz / 32;   // runs per group (d_col <= 32768: at most 1024)
  if (g.n_groups == 1) {
    g.mul = 0;
    g.shift = 0;
  } else if ((rpg & (rpg - 1)) == 0) {
    g.mul = 1;
    g.shift = 0;
    while ((int64_t(1) << g.shift) < rpg) ++g.shift;
  } else {
    g.mul = (((uint64_t)1 << 40) + (uint64_t)rpg - 1) / (uint64_t)rpg;
    g.shift = 40;
  }
  const int64_t per = matvec_max_rows_per_launch(d_col);
  const _Float16* xh = static_cast<const _Float16*>(x);
  ProfScope ps("dequant_matvec", s);
  for (int64_t b0 = 0; b0 < n;) {
    // the largest of 8, 4, 2, 1 rows that is left and fits the LDS
    int nb = 8;
    while (nb > 1 && (nb > per || nb > n - b0)) nb >>= 1;
    hipError_t e;
    switch (bits) {
      case 2: e = launch_bits<2>(qw, scales, zeros, d_row, d_col, g, xh + b0 * ldx, ldx, nb, y + b0 * ldy, ldy, s); break;
      case 3: e = launch_bits<3>(qw, scales, zeros, d_row, d_col, g, xh + b0 * ldx, ldx, nb, y + b0 * ldy, ldy, s); break;
      case 4: e = launch_bits<4>(qw, scales, zeros, d_row, d_col, g, xh + b0 * ldx, ldx, nb, y + b0 * ldy, ldy, s); break;
      case 8: e = launch_bits<8>(qw, scales, zeros, d_row, d_col, g, xh + b0 * ldx, ldx, nb, y + b0 * ldy, ldy, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    b0 += nb;
  }
  return hipSuccess;
}

}  // namespace gptq
