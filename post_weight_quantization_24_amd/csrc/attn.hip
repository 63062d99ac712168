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
// One workgroup per (sequence, 128-query tile, head) of a chunk, on the fp32 matrix cores
// (v_mfma_f32_32x32x2f32: lane l gives A[l%32][l/32] and B[l/32][l%32] and holds
// C[8(c/4) + 4(l/32) + c%4][l%32] in register c).  Wave w takes the 32 queries
// w*32 .. w*32 + 31 of the tile; lane l serves query l%32 and keeps its channels
// 2s + l/32 (s = 0..63) of q in registers.
//   scores: S^T = K Q^T over 32-key blocks, 64 steps of 2 channels; each lane then holds 16
//     of its query's 32 scores and the lane l^32 the other 16, so the running maximum and sum
//     need one swap between the two;
//   output: O^T += V^T P^T, four 32-channel blocks; step c of a block takes the keys of score
//     register c (8(c/4) + c%4 and that + 4), so every lane's B operand is its own score
//     register and nothing moves between lanes.
// K and V tiles of 64 keys are staged in LDS: K as [key][even channels | odd channels] (a
// lane's 16-byte read gives four steps), V transposed as [channel][key] (four keys of a
// block step in one 16-byte read).  Rows are padded by 4 floats.
constexpr int MQ = 128, MK = 64;
constexpr int KLD = HD + 4, VLD = MK + 4;

__global__ void __launch_bounds__(256, 2)
attn_causal(const float* __restrict__ A, int64_t rows, int64_t d, int64_t L,
            _Float16* __restrict__ O, int64_t ldo) {
  __shared__ float Ks[MK * KLD];
  __shared__ float Vt[HD * VLD];
  const int64_t n_heads = d / HD;
  const int64_t n_seq = (rows + L - 1) / L;
  const int64_t n_qt = ((L < rows ? L : rows) + MQ - 1) / MQ;
  // the longest query tiles (most key tiles) first
  const int64_t b = blockIdx.x;
  const int64_t per_qt = n_heads * n_seq;
  const int64_t qt = n_qt - 1 - b / per_qt;
  const int64_t seq = (b % per_qt) / n_heads;
  const int64_t hd = b % n_heads;
  const int64_t s0 = seq * L;
  const int64_t len = rows - s0 < L ? rows - s0 : L;
  if (qt * MQ >= len) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const int64_t ld = 3 * d;
  const int64_t q0 = qt * MQ + w * 32;     // the wave's first query
  const int64_t qj = q0 + j;               // this lane's query

  float qreg[64];
  {
    const float* src = A + (s0 + (qj < len ? qj : len - 1)) * ld + hd * HD + h;
#pragma unroll
    for (int t = 0; t < 64; ++t) qreg[t] = src[2 * t];
  }
  floatx16 acc[4];
  const floatx16 zero16 = {};
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = zero16;
  float m_run = -INFINITY, l_run = 0.0f;
  const float scale = 0.08838834764831845f;  // 1 / sqrt(128)

  const int64_t last_q = qt * MQ + MQ - 1 < len - 1 ? qt * MQ + MQ - 1 : len - 1;
  for (int64_t kt = 0; kt * MK <= last_q; ++kt) {
    __syncthreads();
    // stage keys [kt*64, kt*64 + 64): thread takes key idx % 64 and channels 4 (idx / 64) + 0..3
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = e * 256 + tid;
      const int key = idx & 63, c4 = idx >> 6;
      const int64_t kj = kt * MK + key;
      floatx4 kv = {0.0f, 0.0f, 0.0f, 0.0f}, vv = {0.0f, 0.0f, 0.0f, 0.0f};
      if (kj < len) {
        const float* src = A + (s0 + kj) * ld + hd * HD + c4 * 4;
        kv = *reinterpret_cast<const floatx4*>(src + d);
        vv = *reinterpret_cast<const floatx4*>(src + 2 * d);
      }
      float* kr = Ks + key * KLD;
      kr[2 * c4] = kv[0];
      kr[2 * c4 + 1] = kv[2];
      kr[64 + 2 * c4] = kv[1];
      kr[64 + 2 * c4 + 1] = kv[3];
#pragma unroll
      for (int t = 0; t < 4; ++t) Vt[(c4 * 4 + t) * VLD + key] = vv[t];
    }
    __syncthreads();

#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int64_t kb = kt * MK + sub * 32;
      if (kb > q0 + 31) continue;             // every key after every query of the wave
      floatx16 S = zero16;
      const float* kp = Ks + (sub * 32 + j) * KLD + h * 64;
#pragma unroll
      for (int s4 = 0; s4 < 16; ++s4) {
        const floatx4 k4 = *reinterpret_cast<const floatx4*>(kp + 4 * s4);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(k4[t], qreg[4 * s4 + t], S, 0, 0, 0);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int64_t key = kb + 8 * (c >> 2) + 4 * h + (c & 3);
        S[c] = key <= qj ? S[c] * scale : -INFINITY;
        mx = fmaxf(mx, S[c]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      float ps = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        S[c] = expf(S[c] - m_new);
        ps += S[c];
      }
      ps += __shfl_xor(ps, 32);
      const float corr = expf(m_run - m_new);
      l_run = l_run * corr + ps;
      m_run = m_new;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[k][c] *= corr;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const float* vp = Vt + (blk * 32 + j) * VLD + sub * 32 + 4 * h;
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          const floatx4 v4 = *reinterpret_cast<const floatx4*>(vp + 8 * m4);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[blk] = __builtin_amdgcn_mfma_f32_32x32x2f32(v4[t], S[4 * m4 + t], acc[blk], 0, 0, 0);
        }
      }
    }
  }
  if (qj >= len) return;
  const float inv = 1.0f / l_run;
  _Float16* dst = O + (s0 + qj) * ldo + hd * HD;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk)
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      typedef _Float16 half4 __attribute__((ext_vector_type(4)));
      half4 o;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = (_Float16)(acc[blk][4 * m4 + t] * inv);
      *reinterpret_cast<half4*>(dst + blk * 32 + 8 * m4 + 4 * h) = o;
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
    const int64_t n_qt = ceil_div(L < rows ? L : rows, MQ);
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
