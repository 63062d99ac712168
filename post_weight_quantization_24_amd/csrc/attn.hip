// The attention half of a decoder layer on quantized q/k/v_proj and o_proj (page
// "大模型常见的量化方式", section on the layers of a large model: the LLaMA layer with
// input_layernorm, self_attn, post_attention_layernorm and the MLP; the norms are not
// quantized).  Read as the LLaMA layer:
//   n1 = rmsnorm(x) gamma1,  q, k, v = float16(n1 W^T),  O = float16(attn(rope(q), rope(k), v)),
//   h  = float16(x + O W_o^T)
// with causal multi-head attention over heads of 128 channels, rotary embedding on the channel
// pairs (i, i + 64) with theta = 10000, and positions that restart at every sequence of
// seq_len tokens (tokens [0, seq_len), [seq_len, 2 seq_len), ... form the sequences).
//
// Every tensor a quantized sub-layer reads is stored in float16; the products run group by
// group on the fp16 matrix cores over the codes expanded to fp16 integers (qgemm.hip), the
// rotary angles and the norm are formed in float64, the attention itself in float32 with a
// running softmax.

#include <cmath>

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int HD = ATTN_HEAD_DIM;  // channels per head
constexpr int AQ = 64;             // queries per workgroup (16 per wave, 4 lanes per query)
constexpr int AK = 64;             // keys per LDS tile
constexpr int SLAB = AK * 32;      // floats per 32-channel slab of a tile
constexpr int64_t TOK_CHUNK = 8192;
constexpr double ROPE_THETA = 10000.0;

unsigned grid_of(int64_t n) {
  const int64_t g = ceil_div(n, 256);
  return (unsigned)(g < 16384 ? g : 16384);
}

// Tokens per product chunk: whole sequences, about TOK_CHUNK tokens.
int64_t chunk_tokens(int64_t n_tok, int64_t seq_len) {
  int64_t c = seq_len >= TOK_CHUNK ? seq_len : TOK_CHUNK / seq_len * seq_len;
  return c < n_tok ? c : n_tok;
}

// ------------------------------------------------------------------ rmsnorm
// One wave per token: sum of squares in float64 over 16-byte loads, then
// y = x / sqrt(mean + eps) * gamma in float64, rounded to float32 and then float16.
__global__ void __launch_bounds__(256)
rmsnorm_k(const _Float16* __restrict__ x, int64_t ldx, int64_t n_tok, int64_t d,
          const _Float16* __restrict__ gamma, double eps, _Float16* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tok) return;
  const _Float16* row = x + t * ldx;
  double ss = 0.0;
  for (int64_t c = lane * 8; c < d; c += 512) {
    const half8 v = *reinterpret_cast<const half8*>(row + c);
#pragma unroll
    for (int k = 0; k < 8; ++k) ss += (double)v[k] * (double)v[k];
  }
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const double r = sqrt(ss / (double)d + eps);
  _Float16* out = y + t * ldy;
  for (int64_t c = lane * 8; c < d; c += 512) {
    const half8 v = *reinterpret_cast<const half8*>(row + c);
    const half8 g = *reinterpret_cast<const half8*>(gamma + c);
    half8 o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (_Float16)(float)((double)v[k] / r * (double)g[k]);
    *reinterpret_cast<half8*>(out + c) = o;
  }
}

// ------------------------------------------------------------------ rotary embedding
// tab[p * 64 + i] = (cos, sin) of p * theta^(-2i/128), in float64.
__global__ void __launch_bounds__(256) rope_table(double2* __restrict__ tab, int64_t L) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= L * (HD / 2)) return;
  const int64_t p = idx / (HD / 2);
  const int i = (int)(idx % (HD / 2));
  const double inv = pow(ROPE_THETA, -(2.0 * i) / (double)HD);
  const double a = (double)p * inv;
  tab[idx] = make_double2(cos(a), sin(a));
}

// A [rows x 3d] holds X (W_q; W_k; W_v)^T for a chunk that starts at a sequence boundary.
// Each of q, k, v is rounded to float16 (the stored projection); q and k are then turned by
// the rotary embedding in float64 and kept in float32; v keeps its float16 value.
__global__ void __launch_bounds__(256)
qkv_rope(float* __restrict__ A, int64_t rows, int64_t d, int64_t L,
         const double2* __restrict__ tab) {
  const int64_t pairs = d / 2;
  const int64_t n = rows * pairs;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t r = idx / pairs, rem = idx % pairs;
    const int64_t h = rem / (HD / 2);
    const int i = (int)(rem % (HD / 2));
    const double2 cs = tab[(r % L) * (HD / 2) + i];
    float* a = A + r * 3 * d + h * HD + i;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float* p = a + m * d;
      const double u = (double)(float)(_Float16)p[0];
      const double w = (double)(float)(_Float16)p[HD / 2];
      p[0] = (float)(u * cs.x - w * cs.y);
      p[HD / 2] = (float)(w * cs.x + u * cs.y);
    }
    float* v = a + 2 * d;
    v[0] = (float)(_Float16)v[0];
    v[HD / 2] = (float)(_Float16)v[HD / 2];
  }
}

// ------------------------------------------------------------------ causal attention
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// sum over the four lanes of a quad (quad_perm [1,0,3,2] then [2,3,0,1])
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xB1>(v);
  return v + dpp<0x4E>(v);
}

// One workgroup per (sequence, 64-query tile, head) of a chunk.  Lane l of wave w serves
// query w*16 + l/4 and channels [32 (l%4), 32 (l%4) + 32) of the head: its slice of q, its
// slice of the output, partial dot products summed over the quad.  Key tiles of 64 keys are
// staged in LDS as four 32-channel slabs; within a key's 32 floats, slab s is rotated by 8 s
// floats, so the four addresses a wave reads at once fall in different banks.  The tiles run
// from the sequence start to the diagonal, with a running maximum and sum (the softmax of the
// whole row without holding it).
__global__ void __launch_bounds__(256)
attn_causal(const float* __restrict__ A, int64_t rows, int64_t d, int64_t L,
            _Float16* __restrict__ O, int64_t ldo) {
  __shared__ float Ks[4 * SLAB];
  __shared__ float Vs[4 * SLAB];
  const int64_t n_heads = d / HD;
  const int64_t n_seq = (rows + L - 1) / L;
  const int64_t n_qt = ((L < rows ? L : rows) + AQ - 1) / AQ;
  // the longest query tiles (most key tiles) first
  const int64_t b = blockIdx.x;
  const int64_t per_qt = n_heads * n_seq;
  const int64_t qt = n_qt - 1 - b / per_qt;
  const int64_t seq = (b % per_qt) / n_heads;
  const int64_t h = b % n_heads;
  const int64_t s0 = seq * L;
  const int64_t len = rows - s0 < L ? rows - s0 : L;
  if (qt * AQ >= len) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int qi = (tid >> 6) * 16 + (lane >> 2);
  const int sub = lane & 3;
  const int64_t ld = 3 * d;
  const bool valid = qt * AQ + qi < len;
  const int64_t rq = s0 + qt * AQ + qi;

  float q[32];
  {
    const float* src = A + (valid ? rq : s0) * ld + h * HD + sub * 32;
#pragma unroll
    for (int c = 0; c < 32; c += 4) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(src + c);
      q[c] = v[0]; q[c + 1] = v[1]; q[c + 2] = v[2]; q[c + 3] = v[3];
    }
  }
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)

  for (int64_t kt = 0; kt <= qt; ++kt) {
    __syncthreads();
    // stage keys [kt*64, kt*64 + 64) of the sequence: 2048 float4 of K and of V
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = e * 256 + tid;
      const int j = idx >> 5, c4 = idx & 31;
      const int slab = c4 >> 3, cc = (c4 & 7) * 4;
      const int64_t kj = kt * AK + j;
      floatx4 kv = {0.0f, 0.0f, 0.0f, 0.0f}, vv = {0.0f, 0.0f, 0.0f, 0.0f};
      if (kj < len) {
        const float* src = A + (s0 + kj) * ld + h * HD + c4 * 4;
        kv = *reinterpret_cast<const floatx4*>(src + d);
        vv = *reinterpret_cast<const floatx4*>(src + 2 * d);
      }
      const int at = slab * SLAB + j * 32 + ((cc + 8 * slab) & 31);
      *reinterpret_cast<floatx4*>(Ks + at) = kv;
      *reinterpret_cast<floatx4*>(Vs + at) = vv;
    }
    __syncthreads();

    // four groups of 16 keys, each folded into the running maximum and sum
    const float* ks = Ks + sub * SLAB;
    const float* vs = Vs + sub * SLAB;
    const int jmax = kt == qt ? qi : AK - 1;  // the last key at or before the query
#pragma unroll 1
    for (int j0 = 0; j0 < AK; j0 += 16) {
      if (j0 > jmax) break;
      float sc[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int j = j0 + jj;
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < 32; c += 4) {
          const floatx4 k4 = *reinterpret_cast<const floatx4*>(ks + j * 32 + ((c + 8 * sub) & 31));
          part += q[c] * k4[0] + q[c + 1] * k4[1] + q[c + 2] * k4[2] + q[c + 3] * k4[3];
        }
        sc[jj] = j <= jmax ? quad_sum(part) * scale : -INFINITY;
      }
      float mx = m_run;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, sc[jj]);
      const float corr = expf(m_run - mx);
      float psum = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        sc[jj] = expf(sc[jj] - mx);
        psum += sc[jj];
      }
      l_run = l_run * corr + psum;
      m_run = mx;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] *= corr;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int j = j0 + jj;
#pragma unroll
        for (int c = 0; c < 32; c += 4) {
          const floatx4 v4 = *reinterpret_cast<const floatx4*>(vs + j * 32 + ((c + 8 * sub) & 31));
          acc[c] += sc[jj] * v4[0];
          acc[c + 1] += sc[jj] * v4[1];
          acc[c + 2] += sc[jj] * v4[2];
          acc[c + 3] += sc[jj] * v4[3];
        }
      }
    }
  }
  if (!valid) return;
  _Float16* dst = O + rq * ldo + h * HD + sub * 32;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int c = 0; c < 32; c += 8) {
    half8 o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (_Float16)(acc[c + k] * inv);
    *reinterpret_cast<half8*>(dst + c) = o;
  }
}

// ------------------------------------------------------------------ residual
// Hout = float16(R + A) for a chunk of rows; A [rows x d_out] float32.
__global__ void __launch_bounds__(256)
residual_add(const float* __restrict__ A, int64_t rows, int64_t d_out,
             const _Float16* __restrict__ R, int64_t ldr, _Float16* __restrict__ Hout,
             int64_t ldh) {
  const int64_t n = rows * d_out;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / d_out, j = i % d_out;
    Hout[t * ldh + j] = (_Float16)((float)R[t * ldr + j] + A[i]);
  }
}

}  // namespace

hipError_t rmsnorm_launch(const _Float16* x, int64_t ldx, int64_t n_tok, int64_t d,
                          const _Float16* gamma, double eps, _Float16* y, int64_t ldy,
                          hipStream_t s) {
  ProfScope ps("block_elementwise", s);
  hipLaunchKernelGGL(rmsnorm_k, dim3((unsigned)ceil_div(n_tok, 4)), dim3(256), 0, s, x, ldx, n_tok,
                     d, gamma, eps, y, ldy);
  return hipGetLastError();
}

size_t attn_ws_bytes(int64_t n_tok, int64_t d, int64_t seq_len) {
  const int64_t t = chunk_tokens(n_tok, seq_len);
  const int64_t L = seq_len < n_tok ? seq_len : n_tok;
  return align_up((size_t)3 * d * d * sizeof(_Float16), 256) +
         align_up((size_t)t * 3 * d * sizeof(float), 256) +
         align_up((size_t)L * (HD / 2) * sizeof(double2), 256);
}

hipError_t attn_launch(const _Float16* X, int64_t n_tok, int64_t d, int64_t ldx,
                       const uint32_t* const pq[3], const float* const ps[3],
                       const uint8_t* const pz[3], int bits, int group, int64_t seq_len,
                       _Float16* O, int64_t ldo, void* ws, hipStream_t s) {
  const int64_t g = group == 0 ? d : group;
  const int64_t T = chunk_tokens(n_tok, seq_len);
  const int64_t L = seq_len < n_tok ? seq_len : n_tok;
  char* p = static_cast<char*>(ws);
  _Float16* Bint = reinterpret_cast<_Float16*>(p);
  p += align_up((size_t)3 * d * d * sizeof(_Float16), 256);
  float* A = reinterpret_cast<float*>(p);
  p += align_up((size_t)T * 3 * d * sizeof(float), 256);
  double2* tab = reinterpret_cast<double2*>(p);
  {
    ProfScope ps_("block_elementwise", s);
    for (int m = 0; m < 3; ++m) expand_codes_f16(pq[m], pz[m], d, d, bits, g, Bint + m * d * d, s);
    hipLaunchKernelGGL(rope_table, dim3((unsigned)ceil_div(L * (HD / 2), 256)), dim3(256), 0, s, tab, L);
  }
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int64_t t0 = 0; t0 < n_tok; t0 += T) {
    const int64_t rows = n_tok - t0 < T ? n_tok - t0 : T;
    // A[:, m d : (m + 1) d] = X W_m^T for q, k, v
    for (int m = 0; m < 3; ++m)
      if ((e = qgemm_f16(X + t0 * ldx, ldx, rows, Bint + m * d * d, d, d, ps[m], g, A + m * d, 3 * d,
                         s, "block_gemm")) != hipSuccess)
        return e;
    {
      ProfScope ps_("block_elementwise", s);
      hipLaunchKernelGGL(qkv_rope, dim3(grid_of(rows * d / 2)), dim3(256), 0, s, A, rows, d, L, tab);
    }
    const int64_t n_seq = ceil_div(rows, L);
    const int64_t n_qt = ceil_div(L < rows ? L : rows, AQ);
    {
      ProfScope ps_("attention", s);
      hipLaunchKernelGGL(attn_causal, dim3((unsigned)(n_qt * n_seq * (d / HD))), dim3(256), 0, s, A,
                         rows, d, L, O + t0 * ldo, ldo);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t residual_ws_bytes(int64_t n_tok, int64_t d_in, int64_t d_out) {
  const int64_t t = n_tok < TOK_CHUNK ? n_tok : TOK_CHUNK;
  return align_up((size_t)d_out * d_in * sizeof(_Float16), 256) +
         align_up((size_t)t * d_out * sizeof(float), 256);
}

hipError_t residual_launch(const _Float16* X, int64_t n_tok, int64_t d_in, int64_t ldx,
                           const _Float16* R, int64_t ldr, const uint32_t* q, const float* sc,
                           const uint8_t* z, int64_t d_out, int bits, int group, _Float16* Hout,
                           int64_t ldh, void* ws, hipStream_t s) {
  const int64_t g = group == 0 ? d_in : group;
  const int64_t T = n_tok < TOK_CHUNK ? n_tok : TOK_CHUNK;
  char* p = static_cast<char*>(ws);
  _Float16* Bint = reinterpret_cast<_Float16*>(p);
  p += align_up((size_t)d_out * d_in * sizeof(_Float16), 256);
  float* A = reinterpret_cast<float*>(p);
  {
    ProfScope ps_("block_elementwise", s);
    expand_codes_f16(q, z, d_out, d_in, bits, g, Bint, s);
  }
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int64_t t0 = 0; t0 < n_tok; t0 += T) {
    const int64_t rows = n_tok - t0 < T ? n_tok - t0 : T;
    if ((e = qgemm_f16(X + t0 * ldx, ldx, rows, Bint, d_out, d_in, sc, g, A, d_out, s,
                       "block_gemm")) != hipSuccess)
      return e;
    {
      ProfScope ps_("block_elementwise", s);
      hipLaunchKernelGGL(residual_add, dim3(grid_of(rows * d_out)), dim3(256), 0, s, A, rows, d_out,
                         R + t0 * ldr, ldr, Hout + t0 * ldh, ldh);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gptq
