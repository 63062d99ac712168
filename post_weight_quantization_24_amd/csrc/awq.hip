// Activation-aware scale search (page "量化", section AWQ).  Input channels with large
// activations matter most; instead of keeping them in high precision, channel c of W is
// multiplied by s_c before quantization and the activations are divided by s_c, which leaves
// the product unchanged but puts those weights on more grid points.  s = s_X^alpha, where
// s_X is the mean magnitude of each channel over the calibration tokens, and alpha is chosen
// on a grid of n evenly spaced points of [0, 1] (n = 20 on the page) by the layer loss
//     L(alpha) = ||W X - Q(W diag s) diag(s)^-1 X||^2 = 1/2 sum_r D_r H D_r^T,
//     D = W - Q(W diag s) diag(s)^-1,   H = 2 X X^T (undamped),
// with Q the round-to-nearest quantizer (scale and zero point per row and group from the
// scaled weights; section 量化基础 of the same page).
//
// Per grid point: the scales (one thread per channel), W' = W s, its quantization and D in
// one pass over W (one wave per row and group), then the loss from half a product: H is
// symmetric, so 1/2 D H D^T = sum T .* D - 1/2 sum D^2 diag(H) with T = D U, U the upper
// triangle of H (the fp32 MFMA GEMM with a triangular operand mask), row sums in double.  The argmin stays on
// the device; a last pass quantizes at alpha*, and the codes are packed like the column
// solve's output.  Every decision that yields an integer is taken in float32 with IEEE
// division, the scales s in double and rounded to float32.

#include <cmath>
#include <mutex>

#include "gptq_internal.h"

// Scratch of the allocation-free magnitude sums (gptq_act_absmean_noalloc): the per-split
// partial sums, in an array the library owns for the life of the process, one copy per GPU.
// Its size covers every shape the call accepts (the planner keeps splits x d below
// 2^20 + d doubles for d <= 2^20), so no caller ever hits the limit in practice; the call
// still checks it.  Host code never passes the array's name to a kernel: it is a host-side
// stand-in, not a device address.  The device address comes from hipGetSymbolAddress, once
// per device.
static __device__ __align__(256) double scratch[(size_t)1 << 21];

namespace gptq {

namespace {

constexpr int AM_THREADS = 256;
constexpr int AM_WAVES = AM_THREADS / 64;

// Partial sums of |x| over one token range (blockIdx.y) for 64 * VEC consecutive channels
// (blockIdx.x): lane l owns VEC consecutive channels, wave w a quarter of the token range,
// and the four waves' sums are added in wave order.  Rows are 16-byte aligned, so whole
// vectors are aligned loads.
template <typename T>
__global__ void __launch_bounds__(AM_THREADS)
absmean_partial(const T* __restrict__ X, int64_t ldx, int64_t d, int64_t n_tok,
                int64_t tok_per_split, double* __restrict__ part) {
  constexpr int VEC = 16 / sizeof(T);
  typedef T vec_t __attribute__((ext_vector_type(VEC)));
  __shared__ double red[AM_WAVES][64][VEC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * VEC;
  const int64_t s0 = (int64_t)blockIdx.y * tok_per_split;
  const int64_t s1 = s0 + tok_per_split < n_tok ? s0 + tok_per_split : n_tok;
  const int64_t q = (s1 - s0 + AM_WAVES - 1) / AM_WAVES;
  const int64_t t0 = s0 + wave * q;
  const int64_t t1 = t0 + q < s1 ? t0 + q : s1;
  double acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0;
  if (c0 + VEC <= d) {
    // eight token rows in flight per lane, then their sums in token order
    constexpr int TU = 8;
    int64_t t = t0;
    for (; t + TU <= t1; t += TU) {
      vec_t v[TU];
#pragma unroll
      for (int u = 0; u < TU; ++u) v[u] = *reinterpret_cast<const vec_t*>(X + (t + u) * ldx + c0);
#pragma unroll
      for (int u = 0; u < TU; ++u)
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += fabs((double)(float)v[u][i]);
    }
    for (; t < t1; ++t) {
      const vec_t v = *reinterpret_cast<const vec_t*>(X + t * ldx + c0);
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[i] += fabs((double)(float)v[i]);
    }
  } else if (c0 < d) {
    for (int64_t t = t0; t < t1; ++t)
#pragma unroll
      for (int i = 0; i < VEC; ++i)
        if (c0 + i < d) acc[i] += fabs((double)(float)X[t * ldx + c0 + i]);
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) red[wave][lane][i] = acc[i];
  __syncthreads();
  if (wave != 0 || c0 >= d) return;
  double* out = part + (int64_t)blockIdx.y * d + c0;
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    double sum = red[0][lane][i];
#pragma unroll
    for (int w = 1; w < AM_WAVES; ++w) sum += red[w][lane][i];
    if (c0 + i < d) out[i] = sum;
  }
}

// sx_sum[c] += the sum over the splits: thread (w, l) of a workgroup adds the w-th quarter
// of the splits of channel 64 blockIdx.x + l in split order, then the quarters are added in
// order.
__global__ void __launch_bounds__(AM_THREADS)
absmean_reduce(const double* __restrict__ part, int splits, int64_t d, double* __restrict__ sx_sum) {
  __shared__ double red[AM_WAVES][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  const int per = (splits + AM_WAVES - 1) / AM_WAVES;
  const int a = wave * per, b = a + per < splits ? a + per : splits;
  double acc = 0.0;
  if (c < d) {
    int s = a;
    for (; s + 8 <= b; s += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(s + u) * d + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; s < b; ++s) acc += part[(int64_t)s * d + c];
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0 || c >= d) return;
  double sum = red[0][lane];
#pragma unroll
  for (int w = 1; w < AM_WAVES; ++w) sum += red[w][lane];
  sx_sum[c] += sum;
}

struct AbsPlan {
  int vec, gx, splits;
  int64_t tok_per_split;
};

AbsPlan absmean_plan(int64_t d, int64_t n_tok, int x_dtype) {
  AbsPlan p;
  p.vec = x_dtype == 0 ? 8 : 4;
  p.gx = (int)ceil_div(d, 64 * (int64_t)p.vec);
  // about 2048 workgroups, each over at least 256 tokens (64 per wave)
  int64_t s = ceil_div(2048, p.gx);
  const int64_t max_s = ceil_div(n_tok, 256);
  if (s > max_s) s = max_s;
  if (s > 65535) s = 65535;
  if (s < 1) s = 1;
  p.tok_per_split = ceil_div(n_tok, s);
  p.splits = (int)ceil_div(n_tok, p.tok_per_split);
  return p;
}

// s[c] = s_X[c]^alpha in double, rounded to float32; alpha = k / (n_grid - 1) with k = *best
// when best is given, else k = i.  A channel with s_X = 0 keeps s = 1.
__global__ void __launch_bounds__(256)
awq_scale(const double* __restrict__ sx_sum, int64_t n_tok, int64_t d, int i, int n_grid,
          const int* __restrict__ best, float* __restrict__ s) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  const int k = best ? *best : i;
  const double alpha = (double)k / (double)(n_grid - 1);
  const double m = sx_sum[c] / (double)n_tok;
  s[c] = m > 0.0 ? (float)pow(m, alpha) : 1.0f;
}

__device__ __forceinline__ float load_w(const void* W, int w_dtype, int64_t i) {
  return w_dtype == 0 ? (float)static_cast<const _Float16*>(W)[i] : static_cast<const float*>(W)[i];
}

__device__ __forceinline__ float wave_min(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wave per (row, group): W' = W s (float32), the group's scale and zero point from the
// range of W' (symmetric: max |x| / (2^(b-1) - 1), zero 2^(b-1); asymmetric: the range
// widened to include 0, scale range / (2^b - 1), zero rint(-min / scale); a degenerate
// range is [-1, 1]), code = clamp(rint(w' / scale + zero), 0, 2^b - 1), and
// D = W - scale (code - zero) / s.  codes, scales and zeros are written when given.
__global__ void __launch_bounds__(256)
awq_rtn(const void* __restrict__ W, int w_dtype, const float* __restrict__ s, int64_t d_row,
        int64_t d_col, int64_t g, int bits, int sym, float* __restrict__ D,
        uint8_t* __restrict__ codes, float* __restrict__ scales, uint8_t* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t n_groups = d_col / g;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= d_row * n_groups) return;
  const int64_t r = item / n_groups, gi = item % n_groups;
  const int64_t c0 = gi * g, row0 = r * d_col;
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t c = c0 + lane; c < c0 + g; c += 64) {
    const float wp = load_w(W, w_dtype, row0 + c) * s[c];
    mn = fminf(mn, wp);
    mx = fmaxf(mx, wp);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int maxq = (1 << bits) - 1;
  float sc, z;
  if (sym) {
    float amax = fmaxf(mx, -mn);
    if (amax == 0.0f) amax = 1.0f;
    sc = __fdiv_rn(amax, (float)((1 << (bits - 1)) - 1));
    z = (float)(1 << (bits - 1));
  } else {
    float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
    if (lo == hi) {
      lo = -1.0f;
      hi = 1.0f;
    }
    sc = __fdiv_rn(hi - lo, (float)maxq);
    z = fminf(fmaxf(rintf(__fdiv_rn(-lo, sc)), 0.0f), (float)maxq);
  }
  for (int64_t c = c0 + lane; c < c0 + g; c += 64) {
    const float w = load_w(W, w_dtype, row0 + c);
    const float wp = w * s[c];
    const float v = __fdiv_rn(wp, sc) + z;
    const float code = fminf(fmaxf(rintf(v), 0.0f), (float)maxq);
    const double w_eff = (double)sc * (double)(code - z) / (double)s[c];
    D[row0 + c] = (float)((double)w - w_eff);
    if (codes) codes[row0 + c] = (uint8_t)code;
  }
  if (scales && lane == 0) {
    scales[r * n_groups + gi] = sc;
    zeros[r * n_groups + gi] = (uint8_t)z;
  }
}

// Little-endian bit stream of b-bit codes per row (code c at bits [c b, c b + b) of the row),
// one 32-bit word per thread.
__global__ void __launch_bounds__(256)
pack_words(const uint8_t* __restrict__ codes, int64_t d_row, int64_t d_col, int bits,
           uint32_t* __restrict__ qweight) {
  const int64_t wpr = d_col * bits / 32;
  const int64_t n = d_row * wpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / wpr, k = i % wpr;
    const int64_t b0 = 32 * k;
    const uint8_t* cr = codes + r * d_col;
    uint64_t acc = 0;
    for (int64_t c = b0 / bits; c * bits < b0 + 32; ++c) {
      const int64_t sh = c * bits - b0;
      const uint64_t v = cr[c];
      acc |= sh >= 0 ? v << sh : v >> (-sh);
    }
    qweight[i] = (uint32_t)acc;
  }
}

// The first grid point with the smallest loss.
__global__ void argmin_first(const double* __restrict__ losses, int n, int* __restrict__ best) {
  if (threadIdx.x != 0) return;
  int b = 0;
  for (int i = 1; i < n; ++i)
    if (losses[i] < losses[b]) b = i;
  *best = b;
}

struct AwqWs {
  float* D;
  float* T;
  double* rows;
  float* s;
  uint8_t* codes;
  int* best;
};

AwqWs carve_awq(void* ws, int64_t d_row, int64_t d_col) {
  const size_t mat = align_up((size_t)d_row * d_col * sizeof(float), 256);
  char* p = static_cast<char*>(ws);
  AwqWs w;
  w.D = reinterpret_cast<float*>(p);
  w.T = reinterpret_cast<float*>(p + mat);
  p += 2 * mat;
  w.rows = reinterpret_cast<double*>(p);
  p += align_up((size_t)d_row * sizeof(double), 256);
  w.s = reinterpret_cast<float*>(p);
  p += align_up((size_t)d_col * sizeof(float), 256);
  w.codes = reinterpret_cast<uint8_t*>(p);
  p += align_up((size_t)d_row * d_col, 256);
  w.best = reinterpret_cast<int*>(p);
  return w;
}

}  // namespace

size_t absmean_ws_bytes(int64_t d, int64_t n_tok) {
  if (n_tok < 1) return 256;
  const AbsPlan p = absmean_plan(d, n_tok, 1);   // the f32 plan has the most splits
  const AbsPlan q = absmean_plan(d, n_tok, 0);
  const int splits = p.splits > q.splits ? p.splits : q.splits;
  return align_up((size_t)splits * d * sizeof(double), 256);
}

hipError_t absmean_launch(double* sx_sum, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                          int64_t ldx, void* ws, hipStream_t stream) {
  if (n_tok < 1) return hipSuccess;
  const AbsPlan p = absmean_plan(d, n_tok, x_dtype);
  double* part = static_cast<double*>(ws);
  ProfScope ps("absmean", stream);
  const dim3 grid((unsigned)p.gx, (unsigned)p.splits);
  if (x_dtype == 0)
    hipLaunchKernelGGL(absmean_partial<_Float16>, grid, dim3(AM_THREADS), 0, stream,
                       static_cast<const _Float16*>(X), ldx, d, n_tok, p.tok_per_split, part);
  else
    hipLaunchKernelGGL(absmean_partial<float>, grid, dim3(AM_THREADS), 0, stream,
                       static_cast<const float*>(X), ldx, d, n_tok, p.tok_per_split, part);
  hipLaunchKernelGGL(absmean_reduce, dim3((unsigned)ceil_div(d, 64)), dim3(AM_THREADS), 0,
                     stream, part, p.splits, d, sx_sum);
  return hipGetLastError();
}

size_t absmean_scratch_bytes() { return sizeof(scratch); }

namespace {
std::mutex g_scratch_mu;
constexpr int MAX_DEVICES = 64;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

// The device address of this device's copy of `scratch`, looked up on the first call on each
// device (with that device current) and kept.
hipError_t absmean_scratch_ptr(int device, void** out) {
  if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

size_t awq_ws_bytes(int64_t d_row, int64_t d_col) {
  return 2 * align_up((size_t)d_row * d_col * sizeof(float), 256) +
         align_up((size_t)d_row * sizeof(double), 256) +
         align_up((size_t)d_col * sizeof(float), 256) + align_up((size_t)d_row * d_col, 256) + 256;
}

hipError_t awq_launch(const AwqArgs& a, void* ws, hipStream_t stream) {
  const AwqWs w = carve_awq(ws, a.d_row, a.d_col);
  const int64_t g = a.group == 0 ? a.d_col : a.group;
  const int64_t items = a.d_row * (a.d_col / g);
  const dim3 sgrid((unsigned)ceil_div(a.d_col, 256)), rgrid((unsigned)ceil_div(items, 4));
  int* best = a.best ? a.best : w.best;
  hipError_t e;
  for (int i = 0; i < a.n_grid; ++i) {
    {
      ProfScope ps("awq_scale_rtn", stream);
      hipLaunchKernelGGL(awq_scale, sgrid, dim3(256), 0, stream, a.sx_sum, a.n_tok, a.d_col, i,
                         a.n_grid, nullptr, w.s);
      hipLaunchKernelGGL(awq_rtn, rgrid, dim3(256), 0, stream, a.W, a.w_dtype, w.s, a.d_row,
                         a.d_col, g, a.bits, a.sym, w.D, nullptr, nullptr, nullptr);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = loss_of_diff_upper(w.D, a.H, a.d_row, a.d_col, a.losses + i, nullptr, w.T, w.rows,
                                stream, "awq_gemm")) != hipSuccess)
      return e;
  }
  ProfScope ps("awq_scale_rtn", stream);
  hipLaunchKernelGGL(argmin_first, dim3(1), dim3(64), 0, stream, a.losses, a.n_grid, best);
  hipLaunchKernelGGL(awq_scale, sgrid, dim3(256), 0, stream, a.sx_sum, a.n_tok, a.d_col, 0,
                     a.n_grid, best, a.s_out);
  hipLaunchKernelGGL(awq_rtn, rgrid, dim3(256), 0, stream, a.W, a.w_dtype, a.s_out, a.d_row,
                     a.d_col, g, a.bits, a.sym, w.D, w.codes, a.scales, a.zeros);
  const int64_t words = a.d_row * (a.d_col * a.bits / 32);
  hipLaunchKernelGGL(pack_words, dim3((unsigned)(ceil_div(words, 256) < 8192 ? ceil_div(words, 256) : 8192)),
                     dim3(256), 0, stream, w.codes, a.d_row, a.d_col, a.bits, a.qweight);
  return hipGetLastError();
}

}  // namespace gptq
