// Product of fp16 activations with a packed layer on the fp16 matrix cores, group by group:
//     C[m][n] = sum_g s[n][g] * sum_{k in group g} A[m][k] * (code[n][k] - z[n][g])
// which is A W^T for the dequantized weights W^ = s (code - z) (page "量化", section GPTQ:
// the quantized layer's output; the format is the one the column solve writes).
//
// The integers code - z (|.| <= 255) are exact in fp16, and so is every product of one with
// an fp16 activation in the fp32 accumulator, so each group's sum rounds only in its fp32
// accumulation; the group sums are then scaled and added in fp32.  The codes are expanded
// once per call into an fp16 matrix [N x K] (code - z), which the tiles read like a plain
// fp16 operand.
//
// Requirements (checked by the callers): K a multiple of 32, g a multiple of 16 dividing K,
// A's rows 16-byte aligned (lda a multiple of 8).
//
// Tiles of 128 x 128 outputs per workgroup of four waves (2 x 2, 64 x 64 per wave: four
// 32 x 32 MFMA tiles), 64-wide K stages through LDS in two buffers (the next stage is loaded
// into registers while the current one is multiplied).  Rows of a stage are padded to 72
// halfs so the eight lanes that a 16-byte LDS read serves at once fall in distinct banks.

#include <type_traits>

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int QM = 128, QN = 128, QK = 64;
constexpr int LDR = QK + 8;                     // halfs per LDS row
constexpr int STAGE = QM * LDR;                 // halfs per operand stage

__global__ void __launch_bounds__(256)
expand_codes(const uint32_t* __restrict__ qweight, const uint8_t* __restrict__ zeros, int64_t N,
             int64_t K, int bits, int64_t g, _Float16* __restrict__ B) {
  const int64_t n = N * K;
  const int64_t words_per_row = K * bits / 32;
  const int64_t n_groups = K / g;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / K, c = i % K;
    const int64_t bit = c * bits;
    const uint32_t* wr = qweight + r * words_per_row;
    uint64_t two = wr[bit / 32];
    if ((bit % 32) + bits > 32) two |= (uint64_t)wr[bit / 32 + 1] << 32;
    const int code = (int)((uint32_t)(two >> (bit % 32)) & mask);
    B[i] = (_Float16)(float)(code - (int)zeros[r * n_groups + c / g]);
  }
}

// The same for 2-, 4- and 8-bit codes, one 32-bit word per thread: its 32 / BITS codes are
// consecutive columns of one group (g is a multiple of 16), so one zero point serves them,
// and they are written as one or two 16-byte (or one 8-byte) stores.
template <int BITS>
__global__ void __launch_bounds__(256)
expand_words(const uint32_t* __restrict__ qweight, const uint8_t* __restrict__ zeros, int64_t N,
             int64_t K, int64_t g, _Float16* __restrict__ B) {
  constexpr int PER = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int64_t wpr = K / PER;
  const int64_t n = N * wpr;
  const int64_t n_groups = K / g;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / wpr, c0 = (i - r * wpr) * PER;
    const uint32_t wv = qweight[i];
    const float z = (float)zeros[r * n_groups + c0 / g];
    _Float16 o[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = (_Float16)((float)((wv >> (BITS * k)) & MASK) - z);
    _Float16* dst = B + r * K + c0;
    if constexpr (PER == 16) {
      half8 a, b;
#pragma unroll
      for (int k = 0; k < 8; ++k) { a[k] = o[k]; b[k] = o[8 + k]; }
      reinterpret_cast<half8*>(dst)[0] = a;
      reinterpret_cast<half8*>(dst)[1] = b;
    } else if constexpr (PER == 8) {
      half8 a;
#pragma unroll
      for (int k = 0; k < 8; ++k) a[k] = o[k];
      *reinterpret_cast<half8*>(dst) = a;
    } else {
      typedef _Float16 half4 __attribute__((ext_vector_type(4)));
      half4 a;
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = o[k];
      *reinterpret_cast<half4*>(dst) = a;
    }
  }
}

__global__ void __launch_bounds__(256, 2)
qgemm_k(const _Float16* __restrict__ A, int64_t lda, int64_t M, const _Float16* __restrict__ B,
        int64_t N, int64_t K, const float* __restrict__ S, int64_t n_groups, int gsteps,
        float* __restrict__ C, int64_t ldc) {
  __shared__ _Float16 As[2 * STAGE];
  __shared__ _Float16 Bs[2 * STAGE];
  const int64_t tiles_m = (M + QM - 1) / QM;
  const int64_t tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = tm * QM, n0 = tn * QN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int li = lane & 31, lh = lane >> 5;

  // one stage of one operand: 128 rows x 64 halfs = 1024 16-byte pieces, 4 per thread
  half8 ra[4], rb[4];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int id = e * 256 + tid;
      const int row = id >> 3, kc = (id & 7) * 8;
      const half8 zero = {};
      const bool kin = k0 + kc < K;
      ra[e] = m0 + row < M && kin ? *reinterpret_cast<const half8*>(A + (m0 + row) * lda + k0 + kc) : zero;
      rb[e] = n0 + row < N && kin ? *reinterpret_cast<const half8*>(B + (n0 + row) * K + k0 + kc) : zero;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int id = e * 256 + tid;
      const int row = id >> 3, kc = (id & 7) * 8;
      *reinterpret_cast<half8*>(As + buf * STAGE + row * LDR + kc) = ra[e];
      *reinterpret_cast<half8*>(Bs + buf * STAGE + row * LDR + kc) = rb[e];
    }
  };

  floatx16 acc[2][2], part[2][2];
  const floatx16 zero16 = {};
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = zero16;

  // the scale of this lane's output column in each of its two N tiles, group grp
  const int64_t col0 = n0 + wn * 64 + li, col1 = col0 + 32;
  const float* s0 = S + (col0 < N ? col0 : N - 1) * n_groups;
  const float* s1 = S + (col1 < N ? col1 : N - 1) * n_groups;

  const int64_t nst = (K + QK - 1) / QK;     // K is a multiple of 32: the last stage may be half
  load(0);
  store(0);
  __syncthreads();
  int step = 0;
  int64_t grp = 0;
  for (int64_t st = 0; st < nst; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nst) load((st + 1) * QK);
    const _Float16* as = As + buf * STAGE;
    const _Float16* bs = Bs + buf * STAGE;
#pragma unroll
    for (int kk = 0; kk < QK / 16; ++kk) {
      if (st * QK + kk * 16 >= K) break;
      half8 af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = *reinterpret_cast<const half8*>(as + (wm * 64 + a * 32 + li) * LDR + kk * 16 + lh * 8);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bf[b] = *reinterpret_cast<const half8*>(bs + (wn * 64 + b * 32 + li) * LDR + kk * 16 + lh * 8);
      if (step == 0) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            part[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], zero16, 0, 0, 0);
      } else {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            part[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], part[a][b], 0, 0, 0);
      }
      if (++step == gsteps) {            // the group ends here: scale its sums into acc
        step = 0;
        const float sc0 = s0[grp], sc1 = s1[grp];
        ++grp;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            acc[a][0][c] += sc0 * part[a][0][c];
            acc[a][1][c] += sc1 * part[a][1][c];
          }
      }
    }
    if (st + 1 < nst) {
      store(buf ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + li;
      if (col >= N) continue;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int64_t row = m0 + wm * 64 + a * 32 + 8 * (c >> 2) + 4 * lh + (c & 3);
        if (row < M) C[row * ldc + col] = acc[a][b][c];
      }
    }
}

// ---------------------------------------------------------------------------------------
// The same product through a ring of three K stages filled by direct-to-LDS copies, for
// groups that are whole stages (g % 64 == 0, K % 64 == 0): every production layer.
// Eight waves in a 2 x 4 grid own 64 x 64 outputs each of a 128 x 256 tile.  A stage holds
// 128 rows of A and 256 rows of B, 64 halfs (128 bytes) per row, 48 KB; the copies of stage
// s + 2 are issued while stage s is multiplied, so loads run two stages ahead without
// staging registers.  In a row the 16-byte slots are XOR-swizzled by (row / 2) % 8, so the
// 16 rows that a fragment read serves at once fall in distinct banks.  Rows past M or N
// read as zero (the buffer ends there).

constexpr int DM = 128, DN = 256, DK = 64, DNST = 3;
constexpr int DROW = DK * 2;                              // bytes per row and stage
constexpr int DA_BYTES = DM * DROW, DB_BYTES = DN * DROW;
constexpr int DSTAGE = DA_BYTES + DB_BYTES;               // 48 KB
constexpr int DWAVES = 8;
constexpr int DCPW = (DM + DN) * DROW / 1024 / DWAVES;    // 1 KB copies per wave and stage: 6

typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dswz(int row, int slot) { return slot ^ ((row >> 1) & 7); }

// One wave-wide 1 KB copy global -> LDS: lane l's 16 bytes at buffer offset voff land at
// lds_base + 16 l.  No register output; the explicit vmcnt waits order the copies.
__device__ __forceinline__ void dcopy(rsrc_t rsrc, uint32_t lds_base, int voff) {
  __asm__ volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "s"(lds_base)
                   : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void dwait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// barrier without __syncthreads' fence (which would drain the copies meant to stay in flight)
__device__ __forceinline__ void dbarrier() {
  __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t nbytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane((uint32_t)nbytes);
  const rsrc_t r = {lo, hi & 0xffffu, n, 0x00020000u};
  return r;
}

__global__ void __launch_bounds__(64 * DWAVES, 1)
qgemm_dma(const _Float16* __restrict__ A, int64_t lda, int64_t M, const _Float16* __restrict__ B,
          int64_t N, int64_t K, const float* __restrict__ S, int64_t n_groups, int spg,
          float* __restrict__ C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) char lds[DNST * DSTAGE];
  const int64_t tiles_m = (M + DM - 1) / DM;
  const int64_t tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = tm * DM, n0 = tn * DN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int li = lane & 31, lh = lane >> 5;
  const int64_t rows_a = M - m0 < DM ? M - m0 : DM;
  const int64_t rows_b = N - n0 < DN ? N - n0 : DN;
  const rsrc_t ra = make_rsrc(A + m0 * lda, rows_a * lda * 2);
  const rsrc_t rb = make_rsrc(B + n0 * K, rows_b * K * 2);
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)lds);

  // copy c (0 .. DCPW - 1) of this wave for stage st: copy q = wave * DCPW + c covers rows
  // 8 q' .. 8 q' + 7 of A (q < 16, q' = q) or of B (q' = q - 16)
  auto issue = [&](int64_t st) {
    const uint32_t sbase = lds0 + (uint32_t)((st % DNST) * DSTAGE);
#pragma unroll
    for (int c = 0; c < DCPW; ++c) {
      const int q = wave * DCPW + c;
      const bool isa = q < DM / 8;
      const int qq = isa ? q : q - DM / 8;
      const int row = 8 * qq + (lane >> 3);
      const int lslot = dswz(row, lane & 7);
      const int64_t ld = isa ? lda : K;
      const int voff = (int)((row * ld + st * DK + 8 * lslot) * 2);
      dcopy(isa ? ra : rb, sbase + (isa ? 0u : (uint32_t)DA_BYTES) + (uint32_t)qq * 1024u, voff);
    }
  };

  floatx16 acc[2][2], part[2][2];
  const floatx16 zero16 = {};
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = part[a][b] = zero16;
  const int64_t col0 = n0 + wn * 64 + li, col1 = col0 + 32;
  const float* s0 = S + (col0 < N ? col0 : N - 1) * n_groups;
  const float* s1 = S + (col1 < N ? col1 : N - 1) * n_groups;
  float sc0 = s0[0], sc1 = s1[0];
  int64_t grp = 0;

  const int64_t nst = K / DK;
  issue(0);
  if (nst > 1) issue(1);
  for (int64_t st = 0; st < nst; ++st) {
    if (st + 1 < nst) dwait_vmcnt<DCPW>();
    else dwait_vmcnt<0>();
    dbarrier();
    if (st + 2 < nst) issue(st + 2);
    const char* sb = lds + (st % DNST) * DSTAGE;
    const bool fresh = st % spg == 0;
#pragma unroll
    for (int kk = 0; kk < DK / 16; ++kk) {
      const int lslot = 2 * kk + lh;
      half8 af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int row = wm * 64 + a * 32 + li;
        af[a] = *reinterpret_cast<const half8*>(sb + row * DROW + 16 * dswz(row, lslot));
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int row = wn * 64 + b * 32 + li;
        bf[b] = *reinterpret_cast<const half8*>(sb + DA_BYTES + row * DROW + 16 * dswz(row, lslot));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          part[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              af[a], bf[b], fresh && kk == 0 ? zero16 : part[a][b], 0, 0, 0);
    }
    if ((st + 1) % spg == 0) {            // the group ends with this stage
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          acc[a][0][c] += sc0 * part[a][0][c];
          acc[a][1][c] += sc1 * part[a][1][c];
        }
      ++grp;
      if (grp < n_groups) {
        sc0 = s0[grp];
        sc1 = s1[grp];
      }
    }
  }

#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + li;
      if (col >= N) continue;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int64_t row = m0 + wm * 64 + a * 32 + 8 * (c >> 2) + 4 * lh + (c & 3);
        if (row < M) C[row * ldc + col] = acc[a][b][c];
      }
    }
}

// ---------------------------------------------------------------------------------------
// The same product straight from the packed codes: dequantization inside the main loop (page
// "量化", section AWQ: the weight-only kernel unpacks the codes in the GEMM's main loop, so the
// weights cross HBM at b bits each).  Tiles, waves and the ring of three K stages are those
// of qgemm_dma; a stage of KD columns (64, or 128 for 4-bit codes in groups of 128 columns)
// holds 128 rows of A (fp16, 16-byte copies) and the 256 rows of packed codes of its columns
// (KD b / 8 bytes per row, dword copies): 24 KB for a 64-deep 4-bit stage instead of 48 KB,
// 48 KB for a 128-deep one.  The deeper stage halves the barriers per column of K (measured
// on MI355X at 2048 x 28672 x 8192: 1.44-1.47 ms against 1.50-1.54 ms).
//
// K order inside a stage: lane half h of an MFMA fragment (lanes 32 h .. 32 h + 31) takes the
// stage's columns (KD / 2) h .. (KD / 2) h + KD / 2 - 1 and step kk the eight columns
// (KD / 2) h + 8 kk .. + 7.  The sum over a stage's columns does not depend on which MFMA step
// and lane half a column goes to, as long as A and B agree; with this order each lane's codes
// of the stage are contiguous (KD b / 16 bytes: one or two 16-byte LDS reads for 4-bit codes)
// and are expanded in registers, 8 per step: 1024 + c is the fp16 with bits 0x6400 | c, and
// one packed fp16 add of -(1024 + z) gives c - z exactly.  Groups are whole stages.
//
// LDS layout of the codes: row r's dwords of the stage at r * KD b / 32 ..; 4-bit rows are
// permuted in 16-byte pieces (pk_pos) so that the 16 lanes that one LDS read cycle serves
// (rows r .. r + 15, the same piece) fall in distinct banks.

template <int BITS, int KD>
struct PackedCfg {
  static constexpr int A_ROW = KD * 2;                   // bytes of a row of A per stage
  static constexpr int A_BYTES = DM * A_ROW;
  static constexpr int SLOTS = KD / 8;                   // 16-byte slots per row of A
  static constexpr int RD = KD * BITS / 32;              // dwords of codes per row and stage
  static constexpr int B_BYTES = DN * RD * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_CPW = A_BYTES / 1024 / DWAVES;  // 1 KB copies of A per wave: KD / 32
  static constexpr int B_CPW = DN * RD / 64 / DWAVES;    // 256 B copies of B per wave
  static constexpr int CPW = A_CPW + B_CPW;
  static constexpr int CHUNK = RD / 2;                   // dwords of codes per lane and stage
  static_assert(KD == 64 || (KD == 128 && BITS == 4), "stage depths built");
};

// LDS slot of a row of A's 16-byte slot `slot`: 64-deep stages (128-byte rows, two to a bank
// row) XOR by (row / 2) % 8, 128-deep stages (one 256-byte row per bank row) by row % 16, so
// the 16 rows one read cycle serves fall in distinct banks (an involution)
template <int KD>
__device__ __forceinline__ int a_swz(int row, int slot) {
  return KD == 64 ? slot ^ ((row >> 1) & 7) : slot ^ (row & 15);
}

// LDS dword position of global dword j of row r's stage segment (an involution).  4-bit rows
// of a 64-deep stage are 32 bytes (8 to a bank row): the two 16-byte halves swap in rows with
// bit 3 set; of a 128-deep stage 64 bytes (4 to a bank row): the four 16-byte quarters are
// XORed with (row / 4) % 4.
template <int BITS, int KD>
__device__ __forceinline__ int pk_pos(int row, int j) {
  if constexpr (BITS == 4 && KD == 64) return j ^ (((row >> 3) & 1) << 2);
  if constexpr (BITS == 4 && KD == 128) return j ^ (((row >> 2) & 3) << 2);
  return j;
}

// One wave-wide copy of 64 dwords global -> LDS: lane l's dword at buffer offset voff lands at
// lds_base + 4 l.
__device__ __forceinline__ void dcopy4(rsrc_t rsrc, uint32_t lds_base, int voff) {
  __asm__ volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rsrc), "s"(lds_base)
                   : "memory", "m0");
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_pair(uint32_t lo, uint32_t hi) {
  return lo | (hi << 16) | 0x64006400u;
}

// (w & mask) | magic in one v_and_or_b32 (gfx9 VOP3 takes no literal: the mask comes from an
// SGPR, the magic from a VGPR).
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  __asm__("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
  return r;
}

__device__ __forceinline__ half2v as_h2(uint32_t u) {
  half2v h;
  __builtin_memcpy(&h, &u, 4);
  return h;
}

// Eight codes of step kk from the lane's chunk as fp16 (c - z), in the slot order of
// pk_slot_order: 4-bit codes come out as (c0, c4), (c1, c5), (c2, c6), (c3, c7) (a nibble and
// the one four places up share the halves of a dword: (w & 0x000F000F) | 0x64006400 is the
// pair 1024 + c; the odd nibbles sit 4 bits higher, 1024 + 16 c, and one packed FMA by 1/16
// brings them back), other widths in natural order.  Every value is a small integer, exact in
// fp16, and so is every step.
template <int BITS>
__device__ __forceinline__ half8 pk_expand(const uint32_t* ch, int kk, half2v nz, half2v nz16) {
  half2v h[4];
  if constexpr (BITS == 4) {
    const uint32_t w = ch[kk], w8 = w >> 8;
    const uint32_t magic = __builtin_amdgcn_readfirstlane(0x64006400u);
    const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    h[0] = as_h2(and_or(w, 0x000F000Fu, magic)) + nz;
    h[1] = as_h2(and_or(w, 0x00F000F0u, magic)) * sixteenth + nz16;
    h[2] = as_h2(and_or(w8, 0x000F000Fu, magic)) + nz;
    h[3] = as_h2(and_or(w8, 0x00F000F0u, magic)) * sixteenth + nz16;
  } else if constexpr (BITS == 8) {
    const uint32_t w0 = ch[2 * kk], w1 = ch[2 * kk + 1];
#pragma unroll
    for (int p = 0; p < 4; ++p) {  // bytes 2p, 2p + 1 of (w1:w0), each widened to a half
      const uint32_t sel = (2u * p) | (0x0Cu << 8) | ((2u * p + 1u) << 16) | (0x0Cu << 24);
      h[p] = as_h2(__builtin_amdgcn_perm(w1, w0, sel) | 0x64006400u) + nz;
    }
  } else {
    // window of the step's 8 BITS bits, from bit 8 BITS kk of the chunk
    constexpr int W = 8 * BITS;
    const int bit = W * kk, i = bit >> 5, sh = bit & 31;
    const uint32_t lo = ch[i];
    const uint32_t hi = (i + 1 < BITS) ? ch[i + 1] : 0u;
    const uint32_t win = sh ? __builtin_amdgcn_alignbit(hi, lo, (uint32_t)sh) : lo;
    constexpr uint32_t M = (1u << BITS) - 1u;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      h[p] = as_h2(pk_pair((win >> (BITS * 2 * p)) & M, (win >> (BITS * (2 * p + 1))) & M)) + nz;
  }
  half8 out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    out[2 * p] = h[p][0];
    out[2 * p + 1] = h[p][1];
  }
  return out;
}

// A's eight fp16 of one fragment, in the slot order of the B expansion: for 4-bit codes
// (a0, a4, a1, a5, a2, a6, a3, a7), else unchanged.
template <int BITS>
__device__ __forceinline__ half8 pk_slot_order(half8 a) {
  if constexpr (BITS == 4) {
    uint32_t d[4], o[4];
    __builtin_memcpy(d, &a, 16);
    o[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);   // a0, a4
    o[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);   // a1, a5
    o[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);   // a2, a6
    o[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);   // a3, a7
    half8 r;
    __builtin_memcpy(&r, o, 16);
    return r;
  } else {
    return a;
  }
}

template <int BITS, int KD>
__global__ void __launch_bounds__(64 * DWAVES, 1)
qgemm_packed(const _Float16* __restrict__ A, int64_t lda, int64_t M,
             const uint32_t* __restrict__ Q, const uint8_t* __restrict__ Z, int64_t N, int64_t K,
             const float* __restrict__ S, int64_t n_groups, int spg, float* __restrict__ C,
             int64_t ldc) {
  using P = PackedCfg<BITS, KD>;
  __shared__ __attribute__((aligned(16))) char lds[DNST * P::STAGE];
  const int64_t tiles_m = (M + DM - 1) / DM;
  const int64_t tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int64_t m0 = tm * DM, n0 = tn * DN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int li = lane & 31, lh = lane >> 5;
  const int64_t wpr = K * BITS / 32;                     // words per row of codes
  const int64_t rows_a = M - m0 < DM ? M - m0 : DM;
  const int64_t rows_b = N - n0 < DN ? N - n0 : DN;
  const rsrc_t ra = make_rsrc(A + m0 * lda, rows_a * lda * 2);
  const rsrc_t rb = make_rsrc(Q + n0 * wpr, rows_b * wpr * 4);
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)lds);

  // copies of stage st: A copy q covers rows (1024 / A_ROW) q ..; B copy q covers the stage's
  // LDS dwords 64 q .. 64 q + 63 of the code block
  auto issue = [&](int st, int slot) {
    const uint32_t sbase = lds0 + (uint32_t)(slot * P::STAGE);
#pragma unroll
    for (int c = 0; c < P::A_CPW; ++c) {
      const int q = wave * P::A_CPW + c;
      const int row = (1024 / P::A_ROW) * q + lane / P::SLOTS;
      const int voff = (int)((row * lda + st * KD + 8 * a_swz<KD>(row, lane % P::SLOTS)) * 2);
      dcopy(ra, sbase + (uint32_t)q * 1024u, voff);
    }
#pragma unroll
    for (int c = 0; c < P::B_CPW; ++c) {
      const int q = wave * P::B_CPW + c;
      const int L = 64 * q + lane;
      const int row = L / P::RD, jl = L % P::RD;
      const int voff = (int)((row * wpr + st * P::RD + pk_pos<BITS, KD>(row, jl)) * 4);
      dcopy4(rb, sbase + (uint32_t)P::A_BYTES + (uint32_t)q * 256u, voff);
    }
  };

  floatx16 acc[2][2], part[2][2];
  const floatx16 zero16 = {};
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = part[a][b] = zero16;
  const int64_t col0 = n0 + wn * 64 + li, col1 = col0 + 32;
  const int64_t c0 = (col0 < N ? col0 : N - 1) * n_groups, c1 = (col1 < N ? col1 : N - 1) * n_groups;
  float sc0 = S[c0], sc1 = S[c1];
  // -(1024 + z) and -(64 + z) for the two B rows of this lane, per group
  half2v nz[2], nz16[2];
  auto zero_points = [&](int64_t gi) {
    const float z0 = (float)Z[c0 + gi], z1 = (float)Z[c1 + gi];
    const _Float16 a0 = (_Float16)(-1024.0f - z0), a1 = (_Float16)(-1024.0f - z1);
    const _Float16 b0 = (_Float16)(-64.0f - z0), b1 = (_Float16)(-64.0f - z1);
    nz[0] = half2v{a0, a0};
    nz[1] = half2v{a1, a1};
    nz16[0] = half2v{b0, b0};
    nz16[1] = half2v{b1, b1};
  };
  zero_points(0);
  int64_t grp = 0;

  const int nst = (int)(K / KD);
  issue(0, 0);
  if (nst > 1) issue(1, 1);
  int slot = 0, gstep = 0;          // ring slot of stage st, stage index within its group
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) dwait_vmcnt<P::CPW>();
    else dwait_vmcnt<0>();
    dbarrier();
    if (st + 2 < nst) issue(st + 2, slot == 0 ? 2 : slot - 1);
    const char* sb = lds + slot * P::STAGE;
    const bool fresh = gstep == 0;
    // this lane's codes of the stage for its two B rows
    uint32_t ch[2][P::CHUNK];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int row = wn * 64 + b * 32 + li;
      const uint32_t* rb_l = reinterpret_cast<const uint32_t*>(sb + P::A_BYTES) + row * P::RD;
      if constexpr (BITS == 4) {
#pragma unroll
        for (int j = 0; j < P::CHUNK; j += 4) {
          const uint4 v = *reinterpret_cast<const uint4*>(rb_l + pk_pos<4, KD>(row, P::CHUNK * lh + j));
          ch[b][j] = v.x; ch[b][j + 1] = v.y; ch[b][j + 2] = v.z; ch[b][j + 3] = v.w;
        }
      } else if constexpr (BITS == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(rb_l + 8 * lh);
        const uint4 u = *reinterpret_cast<const uint4*>(rb_l + 8 * lh + 4);
        ch[b][0] = v.x; ch[b][1] = v.y; ch[b][2] = v.z; ch[b][3] = v.w;
        ch[b][4] = u.x; ch[b][5] = u.y; ch[b][6] = u.z; ch[b][7] = u.w;
      } else if constexpr (BITS == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(rb_l + 2 * lh);
        ch[b][0] = v.x; ch[b][1] = v.y;
      } else {
#pragma unroll
        for (int j = 0; j < BITS; ++j) ch[b][j] = rb_l[BITS * lh + j];
      }
    }
    auto step = [&](int kk, auto first) {
      const int lslot = (KD / 16) * lh + kk;
      half8 af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int row = wm * 64 + a * 32 + li;
        af[a] = pk_slot_order<BITS>(
            *reinterpret_cast<const half8*>(sb + row * P::A_ROW + 16 * a_swz<KD>(row, lslot)));
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) bf[b] = pk_expand<BITS>(ch[b], kk, nz[b], nz16[b]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          part[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              af[a], bf[b], decltype(first)::value ? zero16 : part[a][b], 0, 0, 0);
    };
    if (fresh) step(0, std::true_type{});
    else step(0, std::false_type{});
#pragma unroll
    for (int kk = 1; kk < KD / 16; ++kk) step(kk, std::false_type{});
    slot = slot == DNST - 1 ? 0 : slot + 1;
    if (++gstep == spg) {                  // the group ends with this stage
      gstep = 0;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          acc[a][0][c] += sc0 * part[a][0][c];
          acc[a][1][c] += sc1 * part[a][1][c];
        }
      ++grp;
      if (grp < n_groups) {
        sc0 = S[c0 + grp];
        sc1 = S[c1 + grp];
        zero_points(grp);
      }
    }
  }

#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + wn * 64 + b * 32 + li;
      if (col >= N) continue;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int64_t row = m0 + wm * 64 + a * 32 + 8 * (c >> 2) + 4 * lh + (c & 3);
        if (row < M) C[row * ldc + col] = acc[a][b][c];
      }
    }
}

}  // namespace

bool qgemm_packed_ok(int64_t K, int bits, int64_t g, int64_t lda) {
  return (bits == 2 || bits == 3 || bits == 4 || bits == 8) && K % DK == 0 && g % DK == 0 &&
         (int64_t)DM * lda * 2 < ((int64_t)1 << 31) &&
         (int64_t)DN * (K * bits / 8) < ((int64_t)1 << 31);
}

hipError_t qgemm_packed_f16(const _Float16* A, int64_t lda, int64_t M, const uint32_t* q,
                            const uint8_t* z, const float* S, int64_t N, int64_t K, int bits,
                            int64_t g, float* C, int64_t ldc, hipStream_t s,
                            const char* prof_name) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!qgemm_packed_ok(K, bits, g, lda)) return hipErrorInvalidValue;
  ProfScope ps(prof_name, s);
  const int64_t tiles = ceil_div(M, DM) * ceil_div(N, DN);
  const dim3 grid((unsigned)tiles), block(64 * DWAVES);
  const int spg = (int)(g / DK);
  // 4-bit codes with 128-column groups: 128-deep stages (48 KB, three in the ring), one
  // group per stage and half the barriers per column of K
  if (bits == 4 && K % 128 == 0 && g % 128 == 0) {
    hipLaunchKernelGGL((qgemm_packed<4, 128>), grid, block, 0, s, A, lda, M, q, z, N, K, S, K / g,
                       (int)(g / 128), C, ldc);
    return hipGetLastError();
  }
  switch (bits) {
    case 2: hipLaunchKernelGGL((qgemm_packed<2, 64>), grid, block, 0, s, A, lda, M, q, z, N, K, S, K / g, spg, C, ldc); break;
    case 3: hipLaunchKernelGGL((qgemm_packed<3, 64>), grid, block, 0, s, A, lda, M, q, z, N, K, S, K / g, spg, C, ldc); break;
    case 4: hipLaunchKernelGGL((qgemm_packed<4, 64>), grid, block, 0, s, A, lda, M, q, z, N, K, S, K / g, spg, C, ldc); break;
    default: hipLaunchKernelGGL((qgemm_packed<8, 64>), grid, block, 0, s, A, lda, M, q, z, N, K, S, K / g, spg, C, ldc); break;
  }
  return hipGetLastError();
}

void expand_codes_f16(const uint32_t* q, const uint8_t* z, int64_t N, int64_t K, int bits,
                      int64_t g, _Float16* B, hipStream_t s) {
  if (bits != 3) {
    const int64_t words = N * K * bits / 32;
    const int64_t wb = ceil_div(words, 256);
    const dim3 grid((unsigned)(wb < 16384 ? wb : 16384));
    if (bits == 4) hipLaunchKernelGGL(expand_words<4>, grid, dim3(256), 0, s, q, z, N, K, g, B);
    else if (bits == 2) hipLaunchKernelGGL(expand_words<2>, grid, dim3(256), 0, s, q, z, N, K, g, B);
    else hipLaunchKernelGGL(expand_words<8>, grid, dim3(256), 0, s, q, z, N, K, g, B);
    return;
  }
  const int64_t blocks = ceil_div(N * K, 256);
  hipLaunchKernelGGL(expand_codes, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0,
                     s, q, z, N, K, bits, g, B);
}

hipError_t qgemm_f16(const _Float16* A, int64_t lda, int64_t M, const _Float16* B, int64_t N,
                     int64_t K, const float* S, int64_t g, float* C, int64_t ldc, hipStream_t s,
                     const char* prof_name) {
  if (M <= 0 || N <= 0) return hipSuccess;
  ProfScope ps(prof_name, s);
  if (g % DK == 0 && K % DK == 0 && (int64_t)DM * lda * 2 < ((int64_t)1 << 31) &&
      (int64_t)DN * K * 2 < ((int64_t)1 << 31)) {
    const int64_t tiles = ceil_div(M, DM) * ceil_div(N, DN);
    hipLaunchKernelGGL(qgemm_dma, dim3((unsigned)tiles), dim3(64 * DWAVES), 0, s, A, lda, M, B, N, K,
                       S, K / g, (int)(g / DK), C, ldc);
    return hipGetLastError();
  }
  const int64_t tiles = ceil_div(M, QM) * ceil_div(N, QN);
  hipLaunchKernelGGL(qgemm_k, dim3((unsigned)tiles), dim3(256), 0, s, A, lda, M, B, N, K, S, K / g,
                     (int)(g / 16), C, ldc);
  return hipGetLastError();
}

}  // namespace gptq
