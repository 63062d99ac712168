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
//     multiple of 32 a run lies in one group: one scale and one zero per run.
//   * The activation rows are staged once per workgroup in LDS as fp16.
//   * INT4: the nibbles k and k + 4 of a word land in the two halves of
//     (w >> 4k) & 0x000F000F; OR-ing 0x6400 into each half gives the fp16 values 1024 + q,
//     and subtracting 1024 + z leaves q - z exactly (|q - z| < 16).  v_dot2_f32_f16 then
//     multiplies the pair with (x_k, x_k+4) and accumulates in fp32, so x is staged in that
//     pair order.  Per run the fp32 dot of (q - z) and x is scaled once by s.
//   * INT2, INT3, INT8: the codes are extracted from a 64-bit window of two words, converted
//     to fp32 and accumulated with fp32 fused multiply-adds.
//   * The 64 lane sums of a row are added by a butterfly, in a fixed order.

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int MV_THREADS = 1024;                 // 16 waves
constexpr int MV_WAVES = MV_THREADS / 64;
constexpr int MV_MAX_NB = 8;                     // activation rows per launch
constexpr size_t MV_LDS = 64 * 1024;             // staged x: two workgroups per CU

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// LDS position of column c in the INT4 pair order: (x_8j+k, x_8j+k+4) at 8j + 2k, 8j + 2k + 1
__device__ __forceinline__ int pos4(int c) {
  const int k = c & 7;
  return (c & ~7) + ((k & 3) << 1) + (k >> 2);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int BITS>
__global__ void __launch_bounds__(MV_THREADS)
dequant_matvec(const uint32_t* __restrict__ qw, const float* __restrict__ scales,
               const uint8_t* __restrict__ zeros, int64_t d_row, int64_t d_col, int64_t g,
               const _Float16* __restrict__ x, int64_t ldx, int nb, float* __restrict__ y,
               int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) _Float16 xs[];   // nb rows of d_col
  const int dc = (int)d_col;
  for (int i = threadIdx.x; i < nb * dc; i += MV_THREADS) {
    const int b = i / dc, c = i - b * dc;
    xs[b * dc + (BITS == 4 ? pos4(c) : c)] = x[b * ldx + c];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int64_t n_waves = (int64_t)gridDim.x * MV_WAVES;
  const int runs = dc / 32;
  const int64_t words = d_col * BITS / 32;          // per row
  const int64_t n_groups = d_col / g;
  for (int64_t r = (int64_t)blockIdx.x * MV_WAVES + (threadIdx.x >> 6); r < d_row; r += n_waves) {
    const uint32_t* row = qw + r * words;
    float acc[MV_MAX_NB];
#pragma unroll
    for (int b = 0; b < MV_MAX_NB; ++b) acc[b] = 0.0f;
#pragma unroll 2
    for (int k = lane; k < runs; k += 64) {
      const int64_t gi = (int64_t)k * 32 / g;
      const float s = scales[r * n_groups + gi];
      const int z = zeros[r * n_groups + gi];
      float part[MV_MAX_NB];
#pragma unroll
      for (int b = 0; b < MV_MAX_NB; ++b) part[b] = 0.0f;
      if constexpr (BITS == 4) {
        const uint4 wv = *reinterpret_cast<const uint4*>(row + 4 * (int64_t)k);
        const uint32_t wa[4] = {wv.x, wv.y, wv.z, wv.w};
        const _Float16 zh = (_Float16)(1024 + z);
        const half2v zz = {zh, zh};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          half2v q[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint32_t t = ((wa[j] >> (4 * kk)) & 0x000F000Fu) | 0x64006400u;
            q[kk] = __builtin_bit_cast(half2v, t) - zz;         // (q_k - z, q_k+4 - z), exact
          }
#pragma unroll
          for (int b = 0; b < MV_MAX_NB; ++b) {
            if (b < nb) {
              const uint4 xv = *reinterpret_cast<const uint4*>(xs + b * dc + 32 * k + 8 * j);
              const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
              for (int kk = 0; kk < 4; ++kk)
                part[b] = __builtin_amdgcn_fdot2(q[kk], __builtin_bit_cast(half2v, xa[kk]),
                                                 part[b], false);
            }
          }
        }
      } else {
        uint32_t wa[BITS + 1];
#pragma unroll
        for (int j = 0; j < BITS; ++j) wa[j] = row[(int64_t)k * BITS + j];
        wa[BITS] = 0u;
        const float zf = (float)z;
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          constexpr uint32_t mask = (1u << BITS) - 1u;
          const int bit = c * BITS, wi = bit >> 5, sh = bit & 31;
          const uint64_t win = ((uint64_t)wa[wi + 1] << 32) | wa[wi];
          const float qz = (float)((uint32_t)(win >> sh) & mask) - zf;
#pragma unroll
          for (int b = 0; b < MV_MAX_NB; ++b)
            if (b < nb) part[b] = fmaf(qz, (float)xs[b * dc + 32 * k + c], part[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < MV_MAX_NB; ++b) acc[b] = fmaf(s, part[b], acc[b]);
    }
#pragma unroll
    for (int b = 0; b < MV_MAX_NB; ++b) {
      if (b < nb) {
        const float v = wave_sum(acc[b]);
        if (lane == 0) y[b * ldy + r] = v;
      }
    }
  }
}

template <int BITS>
hipError_t launch_bits(const uint32_t* qw, const float* scales, const uint8_t* zeros,
                       int64_t d_row, int64_t d_col, int64_t g, const _Float16* x, int64_t ldx,
                       int nb, float* y, int64_t ldy, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(dequant_matvec<BITS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)MV_LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t want = ceil_div(d_row, (int64_t)MV_WAVES);
  const unsigned grid = (unsigned)(want < 512 ? want : 512);   // up to two per CU
  const size_t lds = (size_t)nb * d_col * sizeof(_Float16);
  hipLaunchKernelGGL(dequant_matvec<BITS>, dim3(grid), dim3(MV_THREADS), lds, s, qw, scales,
                     zeros, d_row, d_col, g, x, ldx, nb, y, ldy);
  return hipGetLastError();
}

}  // namespace

int64_t matvec_max_rows_per_launch(int64_t d_col) {
  const int64_t fit = (int64_t)(MV_LDS / sizeof(_Float16)) / d_col;
  return fit < MV_MAX_NB ? fit : MV_MAX_NB;
}

hipError_t matvec_launch(const uint32_t* qw, const float* scales, const uint8_t* zeros,
                         int64_t d_row, int64_t d_col, int bits, int group, const void* x,
                         int64_t n, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  const int64_t g = group == 0 ? d_col : group;
  const int64_t per = matvec_max_rows_per_launch(d_col);
  const _Float16* xh = static_cast<const _Float16*>(x);
  ProfScope ps("dequant_matvec", s);
  for (int64_t b0 = 0; b0 < n; b0 += per) {
    const int nb = (int)(n - b0 < per ? n - b0 : per);
    hipError_t e;
    switch (bits) {
      case 2: e = launch_bits<2>(qw, scales, zeros, d_row, d_col, g, xh + b0 * ldx, ldx, nb, y + b0 * ldy, ldy, s); break;
      case 3: e = launch_bits<3>(qw, scales, zeros, d_row, d_col, g, xh + b0 * ldx, ldx, nb, y + b0 * ldy, ldy, s); break;
      case 4: e = launch_bits<4>(qw, scales, zeros, d_row, d_col, g, xh + b0 * ldx, ldx, nb, y + b0 * ldy, ldy, s); break;
      case 8: e = launch_bits<8>(qw, scales, zeros, d_row, d_col, g, xh + b0 * ldx, ldx, nb, y + b0 * ldy, ldy, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gptq
