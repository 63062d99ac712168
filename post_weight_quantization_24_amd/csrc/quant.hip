// GPTQ column solve (page "量化", section GPTQ): columns in fixed left-to-right order;
// after quantizing column q every not-yet-quantized weight of the row moves by
// -(w_q - quant(w_q)) / [H^-1]_qq * H^-1_{:,q}, which through G = Cholesky(H^-1)^T is
//     e = (w_q - w^_q) / G_qq,   w_k -= e * G_qk  (k > q).
// Blocks of B columns: updates inside the block are immediate (quant_block), the columns
// right of the block get the batch update W[:, end:] -= E G[blk, end:] (fp32 MFMA GEMM);
// the batch updates of all blocks are grouped recursively by halves (solve, below).
//
// Quantizer (section 量化基础 of the same page; round and clip of the linear form on
// the m.youleyou.com introduction, section 四): code = clip(rne(w/s + z), 0, 2^b - 1),
// with (s, z) per row and group of g columns (granularity table on psvmc.cn), computed
// at the group's first column from the current weights.  Every decision that yields an
// integer is taken in float32 with IEEE division.
//
// quant_block layout: a wave holds 4 rows; each row is spread over a DPP row of 16
// lanes, lane c owning block columns c, c+16, c+32, ... in registers.  The B x B block
// of G sits in LDS, stored [q][slot][lane] and only for slots that can still change, so
// each lane reads its update coefficients conflict-free (the four rows of a wave read
// the same addresses).  Column q is quantized by its owner lane; its e reaches the
// other 15 lanes with one DPP row broadcast.

#include <mutex>
#include <utility>

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int LPR = 16;            // lanes per row
constexpr int ROWS_PER_WG = 16;    // 4 waves x 4 rows

__global__ void __launch_bounds__(256)
convert_w(const void* __restrict__ W, int w_dtype, int64_t n, float* __restrict__ Wc) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    Wc[i] = w_dtype == 0 ? (float)static_cast<const _Float16*>(W)[i]
                         : static_cast<const float*>(W)[i];
}
// The same in 16-byte pieces (W and Wc 16-byte aligned, n a multiple of 8): eight fp16 (two
// pieces of four fp32) weights per thread and step, as two 16-byte stores.
__global__ void __launch_bounds__(256)
convert_w16(const void* __restrict__ W, int w_dtype, int64_t n, float* __restrict__ Wc) {
  floatx4* out = reinterpret_cast<floatx4*>(Wc);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n / 8; i += (int64_t)gridDim.x * 256) {
    if (w_dtype == 0) {
      const half8 h = static_cast<const half8*>(W)[i];
      out[2 * i] = floatx4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
      out[2 * i + 1] = floatx4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
    } else {
      const floatx4* in = static_cast<const floatx4*>(W);
      out[2 * i] = in[2 * i];
      out[2 * i + 1] = in[2 * i + 1];
    }
  }
}

__global__ void __launch_bounds__(256) zero_f64(double* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.0;
}

struct Params {
  float s;
  float z;
  float y;   // RN(1/s): w/s is formed as RN(q0 + RN(w - q0 s) y) with q0 = RN(w y)
};

// (s, z) from the group's min and max (already including 0 for the asymmetric form).
__device__ __forceinline__ Params make_params(float mn, float mx, int bits, int sym) {
  const int maxq = (1 << bits) - 1;
  Params p;
  if (sym) {
    float amax = fmaxf(mx, -mn);
    if (amax == 0.0f) amax = 1.0f;
    p.s = __fdiv_rn(amax, (float)((1 << (bits - 1)) - 1));
    p.z = (float)(1 << (bits - 1));
  } else {
    float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
    if (lo == hi) {
      lo = -1.0f;
      hi = 1.0f;
    }
    p.s = __fdiv_rn(hi - lo, (float)maxq);
    const float zf = __fdiv_rn(-lo, p.s);
    p.z = fminf(fmaxf(__builtin_rintf(zf), 0.0f), (float)maxq);
  }
  p.y = __fdiv_rn(1.0f, p.s);
  return p;
}

// w / s correctly rounded (the same value as an IEEE division) from the correctly rounded
// reciprocal y: q0 = RN(w y) is within an ulp of w / s, r = w - q0 s is exact with an FMA,
// and one correction RN(q0 + r y) then gives RN(w / s) (Markstein's theorem on division
// with a correctly rounded reciprocal; also checked against exact rational arithmetic).
// Three dependent operations instead of the eleven of a general division.
__device__ __forceinline__ float div_by_scale(float w, const Params& p) {
  const float q0 = w * p.y;
  const float r = fmaf(-q0, p.s, w);
  return fmaf(r, p.y, q0);
}

// One wave per row: parameters of the group [c0, c0 + g) from the current weights.
__global__ void __launch_bounds__(256)
group_params(const float* __restrict__ Wc, int64_t d_row, int64_t d_col, int64_t c0, int64_t g,
             int bits, int sym, float* __restrict__ scales, uint8_t* __restrict__ zeros,
             int64_t n_groups) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d_row) return;
  const float* w = Wc + row * d_col + c0;
  float mn = 3.0e38f, mx = -3.0e38f;
  for (int64_t c = lane; c < g; c += 64) {
    const float x = w[c];
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  if (lane == 0) {
    const Params p = make_params(mn, mx, bits, sym);
    scales[row * n_groups + c0 / g] = p.s;
    zeros[row * n_groups + c0 / g] = (uint8_t)p.z;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// min / max over the 16 lanes of a DPP row (row_ror:8, 4, 2, 1)
__device__ __forceinline__ float row_min(float v) {
  v = fminf(v, dpp<0x128>(v));
  v = fminf(v, dpp<0x124>(v));
  v = fminf(v, dpp<0x122>(v));
  return fminf(v, dpp<0x121>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0x128>(v);
  v += dpp<0x124>(v);
  v += dpp<0x122>(v);
  return v + dpp<0x121>(v);
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<0x128>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x122>(v));
  return fmaxf(v, dpp<0x121>(v));
}

// LDS offset of row q of the compact G block: rows q in [16a, 16a+16) keep slots a..S-1.
template <int B>
__host__ __device__ constexpr int grow_off(int q) {
  constexpr int S = B / LPR;
  const int a = q / LPR;
  return LPR * LPR * (a * S - a * (a - 1) / 2) + (q - LPR * a) * LPR * (S - a);
}
template <int B>
constexpr int g_lds_floats() { return grow_off<B>(B); }

template <int B>
struct Row {
  static constexpr int S = B / LPR;
  float w[S];      // current weights of the owned columns (column s*16 + lane)
  uint32_t code[(S + 3) / 4];   // decided codes of the owned columns, one byte each
  float err[S];    // e of the owned columns, for the lazy update
  float gc[S];     // G_qk / G_qq of the current column q for the owned columns k
  float gn[S];     // the same for the next column (read one step ahead)
  Params p;
};

template <int B, int Q>
__device__ __forceinline__ void load_coef(Row<B>& r, const float* gl, int c) {
  constexpr int S = B / LPR;
  constexpr int A = Q / LPR;
  const float* gq = gl + grow_off<B>(Q);
#pragma unroll
  for (int s = A; s < S; ++s) r.gn[s] = gq[(s - A) * LPR + c];
}

template <int B, int Q>
__device__ __forceinline__ void quant_step(Row<B>& r, const float* gl, int c, int bits,
                                           int sym, int64_t g, int width, int64_t j0,
                                           float* __restrict__ scales, uint8_t* __restrict__ zeros,
                                           int64_t n_groups, int64_t row, bool row_ok) {
  constexpr int S = B / LPR;
  constexpr int A = Q / LPR;   // slot holding column Q
  constexpr int O = Q % LPR;   // owner lane
  const int maxq = (1 << bits) - 1;
  // this column's coefficients were read during the previous step; read the next ones now
#pragma unroll
  for (int s = A; s < S; ++s) r.gc[s] = r.gn[s];
  if (Q + 1 < B) load_coef<B, (Q + 1 < B ? Q + 1 : Q)>(r, gl, c);
  // keep later steps' LDS reads from being hoisted here (they would each hold a register)
  __asm__ volatile("" ::: "memory");
  // groups are multiples of 16 columns, so a group can only start at a multiple of 16
  if (O == 0 && g <= B && (Q % g) == 0 && Q < width) {
    // group [Q, Q + g) inside the block: min / max of the current values
    float mn = 3.0e38f, mx = -3.0e38f;
#pragma unroll
    for (int s = A; s < S; ++s) {
      const int col = s * LPR + c;
      if (col >= Q && col < Q + g) {
        mn = fminf(mn, r.w[s]);
        mx = fmaxf(mx, r.w[s]);
      }
    }
    mn = row_min(mn);
    mx = row_max(mx);
    r.p = make_params(mn, mx, bits, sym);
    if (c == 0 && row_ok) {
      const int64_t gi = (j0 + Q) / g;
      scales[row * n_groups + gi] = r.p.s;
      zeros[row * n_groups + gi] = (uint8_t)r.p.z;
    }
  }
  const float x = r.w[A];
  const float v = div_by_scale(x, r.p) + r.p.z;
  // clip to [0, maxq] in one v_med3 (the same value as max then min for every finite or
  // infinite v; finite weights never give a NaN here)
  const float code = __builtin_amdgcn_fmed3f(__builtin_rintf(v), 0.0f, (float)maxq);
  const float wq = r.p.s * (code - r.p.z);
  // d = w - w^ (e = d / G_qq is formed after the block; the stored G rows carry the 1/G_qq).
  // Columns past `width` need no mask here: their weights are 0, so d is finite, and their
  // staged coefficients and 1 / G_qq are 0, so d moves nothing and is never stored.
  const float dq = dpp<0x150 + O>(x - wq);  // row_newbcast: every lane takes the owner's d
  {                        // register selects, no memory traffic on the column chain
    constexpr int SH = 8 * (A % 4);
    const bool own = c == O;
    const uint32_t cw = (r.code[A / 4] & ~(0xffu << SH)) | ((uint32_t)code << SH);
    r.code[A / 4] = own ? cw : r.code[A / 4];
    r.err[A] = own ? dq : r.err[A];
  }
#pragma unroll
  for (int s = A; s < S; ++s) r.w[s] = fmaf(-dq, r.gc[s], r.w[s]);
}

template <int B, int... Qs>
__device__ __forceinline__ void quant_steps(Row<B>& r, const float* gl, int c,
                                            int bits, int sym, int64_t g, int width, int64_t j0,
                                            float* scales, uint8_t* zeros, int64_t n_groups,
                                            int64_t row, bool row_ok,
                                            std::integer_sequence<int, Qs...>) {
  (quant_step<B, Qs>(r, gl, c, bits, sym, g, width, j0, scales, zeros, n_groups, row, row_ok),
   ...);
}

template <int B>
__global__ void __launch_bounds__(256)
quant_block(const float* __restrict__ Wc, const float* __restrict__ G, int64_t d_row,
            int64_t d_col, int64_t j0, int width, int bits, int sym, int64_t g,
            float* __restrict__ scales, uint8_t* __restrict__ zeros, int64_t n_groups,
            uint32_t* __restrict__ qweight, float* __restrict__ E, double* __restrict__ err_sq) {
  constexpr int S = B / LPR;
  extern __shared__ float smem[];
  float* gl = smem;                          // compact G block
  float* rinv = smem + g_lds_floats<B>();    // 1 / G_qq
  uint8_t* cbuf = reinterpret_cast<uint8_t*>(rinv + B);  // codes [ROWS_PER_WG][B]

  const int c = threadIdx.x % LPR;
  const int rl = threadIdx.x / LPR;  // row within the workgroup
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_WG + rl;
  const bool row_ok = row < d_row;
  // This thread's weights first: their loads stay in flight while G is staged.
  Row<B> r;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int k = s * LPR + c;
    r.w[s] = (row_ok && k < width) ? Wc[row * d_col + j0 + k] : 0.0f;
  }
  float g_sc = 1.0f, g_z = 0.0f;
  if (g > B && row_ok) {
    const int64_t gi = j0 / g;
    g_sc = scales[row * n_groups + gi];
    g_z = (float)zeros[row * n_groups + gi];
  }

  // Stage G[j0 + q][j0 + s*16 + c] / G_qq for columns > q (0 elsewhere).  Thread (q0, c)
  // handles rows q = q0 + 16 i and reads their diagonal entries itself; row q keeps slots
  // i..S-1, so every index is known at compile time and the loads of all its rows (up to
  // eight) are in flight together.  1 / G_qq also goes to LDS for the epilogue.
  {
    const int q0 = threadIdx.x / LPR;
    const float* gsrc = G + (j0 + q0) * d_col + j0 + c;
    constexpr int RPC = S <= 8 ? S : 2;   // rows per chunk (bounded registers)
#pragma unroll
    for (int i0 = 0; i0 < S; i0 += RPC) {
      float v[RPC][S];
      float gd[RPC];
#pragma unroll
      for (int i = i0; i < i0 + RPC; ++i) {
        const int q = q0 + LPR * i;
        gd[i - i0] = q < width ? G[(j0 + q) * d_col + j0 + q] : 1.0f;
#pragma unroll
        for (int s = i; s < S; ++s) {
          const int k = s * LPR + c;
          v[i - i0][s] = (k > q && k < width && q < width)
                             ? gsrc[(int64_t)LPR * i * d_col + s * LPR] : 0.0f;
        }
      }
#pragma unroll
      for (int i = i0; i < i0 + RPC; ++i) {
        const int q = q0 + LPR * i;
        const float rq = q < width ? 1.0f / gd[i - i0] : 0.0f;
        if (c == 0) rinv[q] = rq;
        float* dst = gl + grow_off<B>(q);
#pragma unroll
        for (int s = i; s < S; ++s) dst[(s - i) * LPR + c] = v[i - i0][s] * rq;
      }
    }
  }

  if (g > B) {
    r.p.s = g_sc;
    r.p.z = g_z;
    r.p.y = __fdiv_rn(1.0f, g_sc);
  } else {
    r.p.s = 1.0f;
    r.p.z = 0.0f;
    r.p.y = 1.0f;
  }
#pragma unroll
  for (int s = 0; s < S; ++s) r.err[s] = 0.0f;
#pragma unroll
  for (int s = 0; s < (S + 3) / 4; ++s) r.code[s] = 0u;
  __syncthreads();
  load_coef<B, 0>(r, gl, c);

  quant_steps<B>(r, gl, c, bits, sym, g, width, j0, scales, zeros, n_groups, row, row_ok,
                 std::make_integer_sequence<int, B>{});

  // codes of the owned columns to LDS (for packing); e = d / G_qq to E (16 lanes per 64
  // bytes) and its squares summed over the row
  uint8_t* crow = cbuf + rl * B;
  float* erow = E + (row_ok ? row : 0) * d_col + j0;
  float esq = 0.0f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int k = s * LPR + c;
    crow[k] = (uint8_t)(r.code[s / 4] >> (8 * (s % 4)));
    const float e = r.err[s] * rinv[k];
    esq = fmaf(e, e, esq);
    if (row_ok && k < width) erow[k] = e;
  }
  esq = row_sum(esq);
  if (row_ok && c == 0 && err_sq) err_sq[row] += (double)esq;
  // pack: each lane assembles whole 32-bit words from the row's code bytes in LDS
  __syncthreads();
  if (row_ok) {
    const int nw = width * bits / 32;
    const int64_t words_per_row = d_col * bits / 32;
    uint32_t* out = qweight + row * words_per_row + j0 * bits / 32;
    for (int wi = c; wi < nw; wi += LPR) {
      const int b0 = wi * 32;
      const int col_lo = b0 / bits, col_hi = (b0 + 31) / bits;
      uint32_t word = 0;
      for (int col = col_lo; col <= col_hi; ++col) {
        const uint32_t code = cbuf[rl * B + col];
        const int sh = col * bits - b0;
        word |= sh >= 0 ? (code << sh) : (code >> (-sh));
      }
      out[wi] = word;
    }
  }
}

template <int B>
size_t quant_block_lds() {
  return (size_t)(g_lds_floats<B>() + B) * sizeof(float) + ROWS_PER_WG * B;
}

template <int B>
hipError_t launch_block(const QuantArgs& a, const float* Wc, float* E, int64_t j0, int width,
                        hipStream_t s) {
  // the dynamic LDS limit is raised once per device (callers on several threads share it)
  static std::mutex mu;
  static bool attr[64] = {};
  const size_t lds = quant_block_lds<B>();
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lk(mu);
    if (!attr[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(quant_block<B>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr[dev] = true;
    }
  }
  const int64_t g = a.group == 0 ? a.d_col : a.group;
  const int64_t n_groups = a.d_col / g;
  const int64_t grid = ceil_div(a.d_row, ROWS_PER_WG);
  hipLaunchKernelGGL(quant_block<B>, dim3((unsigned)grid), dim3(256), lds, s, Wc, a.G, a.d_row,
                     a.d_col, j0, width, a.bits, a.sym, g, a.scales, a.zeros, n_groups,
                     a.qweight, E, a.err_sq_rows);
  return hipGetLastError();
}

}  // namespace

size_t quant_ws_bytes(int64_t d_row, int64_t d_col, int block) {
  (void)block;
  // working copy of W and the errors E of every column, both d_row x d_col float32
  return 2 * align_up((size_t)d_row * d_col * sizeof(float), 256);
}

namespace {

// Columns [c0, c0 + n) with every update from the columns left of c0 already applied.
// The lazy batch update is applied recursively: after the left half of the range is
// quantized, its errors update the right half in one product (K = left width), so each
// weight is rewritten once per level (log2 of the block count) instead of once per block,
// and the products are large.  The sum of the products equals the per-block updates
// W[:, j+B:] -= E_j G[j:j+B, j+B:] of all blocks j.
hipError_t solve(const QuantArgs& a, float* Wc, float* E, int64_t c0, int64_t n, int64_t g,
                 int64_t n_groups, hipStream_t s) {
  hipError_t e;
  if (n <= a.block) {
    if (g > a.block && c0 % g == 0) {
      ProfScope ps("quant_group_params", s);
      hipLaunchKernelGGL(group_params, dim3((unsigned)ceil_div(a.d_row, 4)), dim3(256), 0, s, Wc,
                         a.d_row, a.d_col, c0, g, a.bits, a.sym, a.scales, a.zeros, n_groups);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    ProfScope ps("quant_block", s);
    switch (a.block) {
      case 32: return launch_block<32>(a, Wc, E, c0, (int)n, s);
      case 64: return launch_block<64>(a, Wc, E, c0, (int)n, s);
      case 128: return launch_block<128>(a, Wc, E, c0, (int)n, s);
      case 256: return launch_block<256>(a, Wc, E, c0, (int)n, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int64_t h = ceil_div(n, a.block) / 2 * a.block;
  if ((e = solve(a, Wc, E, c0, h, g, n_groups, s)) != hipSuccess) return e;
  // W[:, c0+h : c0+n] -= E[:, c0 : c0+h] G[c0 : c0+h, c0+h : c0+n]
  GemmArgs ga{a.d_row, n - h, h, E + c0, a.d_col, 0, 0,
              a.G + c0 * a.d_col + c0 + h, a.d_col, 0, 0,
              Wc + c0 + h, a.d_col, 0, -1.0f, 1.0f};
  if ((e = gemm_f32(ga, s, "lazy_gemm")) != hipSuccess) return e;
  return solve(a, Wc, E, c0 + h, n - h, g, n_groups, s);
}

}  // namespace

hipError_t quant_launch(const QuantArgs& a, void* ws, hipStream_t s) {
  hipError_t e;
  float* Wc = static_cast<float*>(ws);
  float* E = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                      align_up((size_t)a.d_row * a.d_col * sizeof(float), 256));
  const int64_t n = a.d_row * a.d_col;
  const int64_t g = a.group == 0 ? a.d_col : a.group;
  const int64_t n_groups = a.d_col / g;
  {
    ProfScope ps("quant_convert", s);
    const bool vec = n % 8 == 0 &&
                     ((reinterpret_cast<uintptr_t>(a.W) | reinterpret_cast<uintptr_t>(Wc)) & 15) == 0;
    if (vec) {
      const int64_t grid = ceil_div(n / 8, 256) < 8192 ? ceil_div(n / 8, 256) : 8192;
      hipLaunchKernelGGL(convert_w16, dim3((unsigned)grid), dim3(256), 0, s, a.W, a.w_dtype, n, Wc);
    } else {
      const int64_t grid = ceil_div(n, 256) < 4096 ? ceil_div(n, 256) : 4096;
      hipLaunchKernelGGL(convert_w, dim3((unsigned)grid), dim3(256), 0, s, a.W, a.w_dtype, n, Wc);
    }
    if (a.err_sq_rows) {
      const int64_t gz = ceil_div(a.d_row, 256) < 1024 ? ceil_div(a.d_row, 256) : 1024;
      hipLaunchKernelGGL(zero_f64, dim3((unsigned)gz), dim3(256), 0, s, a.err_sq_rows, a.d_row);
    }
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return solve(a, Wc, E, 0, a.d_col, g, n_groups, s);
}

}  // namespace gptq
