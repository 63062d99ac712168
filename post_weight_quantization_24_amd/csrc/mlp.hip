// The MLP of a decoder layer on quantized gate_proj and up_proj (page "大模型常见的量化方式",
// section on the layers of a large model: the LLaMA MLP with gate_proj, up_proj, down_proj;
// read as the LLaMA definition down(silu(gate x) * up x)):
//     Y = silu(X G^T) * (X U^T),  silu(a) = a / (1 + exp(-a)),
// written in float16 as down_proj's calibration input when a block is quantized layer by
// layer.  The codes of G and U are expanded once into fp16 integers (code - z); the tokens go
// through in chunks of 8192: both products group by group on the fp16 matrix cores
// (qgemm.hip), then silu and the product into float16.

#include <cmath>

#include "gptq_internal.h"

namespace gptq {

namespace {

constexpr int64_t MLP_CHUNK = 8192;   // tokens per product

// Y[t][j] = float16(silu(A[t][j]) * A[t][d_ff + j]) for the chunk's rows.
__global__ void __launch_bounds__(256)
mlp_act(const float* __restrict__ A, int64_t rows, int64_t d_ff, _Float16* __restrict__ Y,
        int64_t ldy) {
  const int64_t n = rows * d_ff;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / d_ff, j = i % d_ff;
    const float a = A[t * 2 * d_ff + j];
    const float b = A[t * 2 * d_ff + d_ff + j];
    Y[t * ldy + j] = (_Float16)(a / (1.0f + expf(-a)) * b);
  }
}

unsigned grid_of(int64_t n) {
  const int64_t g = ceil_div(n, 256);
  return (unsigned)(g < 16384 ? g : 16384);
}

}  // namespace

size_t mlp_ws_bytes(int64_t n_tok, int64_t d, int64_t d_ff) {
  const int64_t t = n_tok < MLP_CHUNK ? n_tok : MLP_CHUNK;
  return align_up((size_t)2 * d_ff * d * sizeof(_Float16), 256) +
         align_up((size_t)t * 2 * d_ff * sizeof(float), 256);
}

hipError_t mlp_launch(const void* X, int64_t n_tok, int64_t d, int64_t ldx,
                      const uint32_t* qg, const float* sg, const uint8_t* zg,
                      const uint32_t* qu, const float* su, const uint8_t* zu, int64_t d_ff,
                      int bits, int group, void* Y, int64_t ldy, void* ws, hipStream_t s) {
  const int64_t g = group == 0 ? d : group;
  char* p = static_cast<char*>(ws);
  _Float16* Bint = reinterpret_cast<_Float16*>(p);
  p += align_up((size_t)2 * d_ff * d * sizeof(_Float16), 256);
  float* A = reinterpret_cast<float*>(p);
  hipError_t e;
  {
    ProfScope ps("mlp_elementwise", s);
    expand_codes_f16(qg, zg, d_ff, d, bits, g, Bint, s);
    expand_codes_f16(qu, zu, d_ff, d, bits, g, Bint + d_ff * d, s);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const _Float16* Xh = static_cast<const _Float16*>(X);
  _Float16* Yh = static_cast<_Float16*>(Y);
  for (int64_t t0 = 0; t0 < n_tok; t0 += MLP_CHUNK) {
    const int64_t rows = n_tok - t0 < MLP_CHUNK ? n_tok - t0 : MLP_CHUNK;
    // A[:, :d_ff] = X G^T and A[:, d_ff:] = X U^T, group by group on the fp16 matrix cores
    if ((e = qgemm_f16(Xh + t0 * ldx, ldx, rows, Bint, d_ff, d, sg, g, A, 2 * d_ff, s,
                       "mlp_gemm")) != hipSuccess ||
        (e = qgemm_f16(Xh + t0 * ldx, ldx, rows, Bint + d_ff * d, d_ff, d, su, g, A + d_ff,
                       2 * d_ff, s, "mlp_gemm")) != hipSuccess)
      return e;
    {
      ProfScope ps("mlp_elementwise", s);
      hipLaunchKernelGGL(mlp_act, dim3(grid_of(rows * d_ff)), dim3(256), 0, s, A, rows, d_ff,
                         Yh + t0 * ldy, ldy);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gptq
