// Internal declarations shared by the HIP sources of libgptq (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- instrumentation
// Records HIP events around a launch when profiling is on (see gptq_profile_enable).
struct ProfScope {
  const char* name;
  hipStream_t stream;
  void* ev0;
  ProfScope(const char* n, hipStream_t s);
  ~ProfScope();
};

// ---------------------------------------------------------------- Hessian (hessian.hip)
// Lower-triangle tiles of 256x256, split over token ranges into partial tiles.
struct HessPlan {
  int64_t d, n_tok;
  int tiles;        // number of lower-triangle 256x256 tiles
  int padded_tiles; // the same for the block grid padded to a multiple of 4 blocks
  int splits;       // token ranges
  int64_t tok_per_split;
  size_t ws_bytes;
};
HessPlan hessian_plan(int64_t d, int64_t n_tok, int64_t ldx, int x_dtype);
hipError_t hessian_launch(const HessPlan& p, float* H, const void* X, int x_dtype, int64_t ldx,
                          void* ws, hipStream_t stream);

// ---------------------------------------------------------------- fp32 MFMA GEMM (gemm.hip)
// C[MxN] = alpha * op(A) op(B) + beta * C.
//   op(A)[m][k] = transA ? A[k*lda + m] : A[m*lda + k]
//   op(B)[k][n] = transB ? B[n*ldb + k] : B[k*ldb + n]
//   triA: 0 none, 1 op(A) upper (entries with k < m are zero), 2 lower (k > m zero)
//   triB: 0 none, 1 op(B) upper (k > n zero), 2 lower (k < n zero)
//   triC: 0 all of C, 1 only entries with m <= n are computed and written.
// Entries an operand mask declares zero are never read.  beta is 0 or 1.
struct GemmArgs {
  int64_t M, N, K;
  const float* A; int64_t lda; int transA; int triA;
  const float* B; int64_t ldb; int transB; int triB;
  float* C; int64_t ldc; int triC;
  float alpha, beta;
};
hipError_t gemm_f32(const GemmArgs& g, hipStream_t stream, const char* prof_name);
// Two independent products in one launch (op(A) = A for both; transB may differ).
hipError_t gemm_f32_pair(const GemmArgs& g1, const GemmArgs& g2, hipStream_t stream,
                         const char* prof_name);

// ---------------------------------------------------------------- prepare (prep.hip)
size_t prepare_ws_bytes(int64_t d);
hipError_t prepare_launch(const float* H, float* G, int64_t d, float damp_frac, void* ws,
                          hipStream_t stream);
// Device flag written by the prepare kernels: 0 ok, else 1 + first failing block row.
int* prepare_flag_ptr(void* ws, int64_t d);

// ---------------------------------------------------------------- column solve (quant.hip)
struct QuantArgs {
  const void* W; int w_dtype; int64_t d_row, d_col;
  const float* G;
  int bits, group, sym, block;
  uint32_t* qweight; float* scales; uint8_t* zeros; double* err_sq_rows;
};
size_t quant_ws_bytes(int64_t d_row, int64_t d_col, int block);
hipError_t quant_launch(const QuantArgs& a, void* ws, hipStream_t stream);

// ---------------------------------------------------------------- check (check.hip)
size_t check_ws_bytes(int64_t d_row, int64_t d_col);
hipError_t check_launch(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                        const void* W, int w_dtype, const float* H, int64_t d_row, int64_t d_col,
                        int bits, int group, double* loss, double* row_loss, float* W_hat,
                        int64_t* off_grid, void* ws, hipStream_t stream);

// The same loss for a symmetric H from half the product: T = D U with U the upper triangle
// of H (diagonal included), then sum_c T D - 1/2 sum_c D^2 H_cc per row.
hipError_t loss_of_diff_upper(const float* D, const float* H, int64_t d_row, int64_t d_col,
                              double* loss, double* row_loss, float* T, double* rows, hipStream_t s,
                              const char* prof_name);

// ---------------------------------------------------------------- AWQ scale search (awq.hip)
size_t absmean_ws_bytes(int64_t d, int64_t n_tok);
// The allocation-free variant's scratch: its size in bytes, and this device's address of it.
size_t absmean_scratch_bytes();
hipError_t absmean_scratch_ptr(int device, void** out);
hipError_t absmean_launch(double* sx_sum, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                          int64_t ldx, void* ws, hipStream_t stream);
size_t awq_ws_bytes(int64_t d_row, int64_t d_col);
struct AwqArgs {
  const void* W; int w_dtype; int64_t d_row, d_col;
  const float* H; const double* sx_sum; int64_t n_tok;
  int bits, group, sym, n_grid;
  uint32_t* qweight; float* scales; uint8_t* zeros; float* s_out; double* losses; int* best;
};
hipError_t awq_launch(const AwqArgs& a, void* ws, hipStream_t stream);

// ---------------------------------------------------------------- MLP block forward (mlp.hip)
size_t mlp_ws_bytes(int64_t n_tok, int64_t d, int64_t d_ff);
hipError_t mlp_launch(const void* X, int64_t n_tok, int64_t d, int64_t ldx,
                      const uint32_t* qg, const float* sg, const uint8_t* zg,
                      const uint32_t* qu, const float* su, const uint8_t* zu, int64_t d_ff,
                      int bits, int group, void* Y, int64_t ldy, void* ws, hipStream_t s);

// ---------------------------------------------------------------- packed-layer product (qgemm.hip)
// B[n][k] = code - z as fp16 for a packed layer [N x K]; C = A W^T group by group on the fp16
// matrix cores (A fp16 [M x K], rows 16-byte aligned; S the scales [N x K/g]; C fp32).
void expand_codes_f16(const uint32_t* q, const uint8_t* z, int64_t N, int64_t K, int bits,
                      int64_t g, _Float16* B, hipStream_t s);
// Product of fp16 A [M x K] with a packed layer [N x K] (codes, zeros, scales), dequantized
// inside the main loop; for bits 2/3/4/8, K and g multiples of 64 (qgemm_packed_ok).
bool qgemm_packed_ok(int64_t K, int bits, int64_t g, int64_t lda);
hipError_t qgemm_packed_f16(const _Float16* A, int64_t lda, int64_t M, const uint32_t* q,
                            const uint8_t* z, const float* S, int64_t N, int64_t K, int bits,
                            int64_t g, float* C, int64_t ldc, hipStream_t s,
                            const char* prof_name);
hipError_t qgemm_f16(const _Float16* A, int64_t lda, int64_t M, const _Float16* B, int64_t N,
                     int64_t K, const float* S, int64_t g, float* C, int64_t ldc, hipStream_t s,
                     const char* prof_name);

// ---------------------------------------------------------------- attention half (attn.hip)
constexpr int ATTN_HEAD_DIM = 128;
hipError_t rmsnorm_launch(const _Float16* x, int64_t ldx, int64_t n_tok, int64_t d,
                          const _Float16* gamma, double eps, _Float16* y, int64_t ldy,
                          hipStream_t s);
size_t attn_ws_bytes(int64_t n_tok, int64_t d, int64_t seq_len);
hipError_t attn_launch(const _Float16* X, int64_t n_tok, int64_t d, int64_t ldx,
                       const uint32_t* const pq[3], const float* const ps[3],
                       const uint8_t* const pz[3], int bits, int group, int64_t seq_len,
                       _Float16* O, int64_t ldo, void* ws, hipStream_t s);
size_t residual_ws_bytes(int64_t n_tok, int64_t d_in, int64_t d_out);
hipError_t residual_launch(const _Float16* X, int64_t n_tok, int64_t d_in, int64_t ldx,
                           const _Float16* R, int64_t ldr, const uint32_t* q, const float* sc,
                           const uint8_t* z, int64_t d_out, int bits, int group, _Float16* Hout,
                           int64_t ldh, void* ws, hipStream_t s);

// ---------------------------------------------------------------- weight-only product (gemv.hip)
// y[n x d_row] = x[n x d_col] (fp16) * W^T with W^ = s (code - z) read from the packed format.
int64_t matvec_max_rows_per_launch(int64_t d_col);
hipError_t matvec_launch(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                         int64_t d_row, int64_t d_col, int bits, int group, const void* x,
                         int64_t n, int64_t ldx, float* y, int64_t ldy, hipStream_t stream);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

}  // namespace gptq
