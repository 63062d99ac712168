/*
 * gptq.h - C ABI of the GPTQ layer-quantization library for AMD Instinct MI355X (gfx950).
 *
 * One linear layer W [d_row x d_col] (row = output channel, column = input channel) is
 * quantized column by column, following the GPTQ section of the page "量化"
 * (Quantization, dingiv.github.io/ai/compute/kernel/quantization):
 *   objective      argmin_W^ ||W X - W^ X||^2 over the calibration inputs X,
 *   Hessian        H = 2 X X^T,
 *   inverse factor G = Cholesky(H^-1)^T (upper triangular, G^T G = H^-1),
 *   compensation   after quantizing column q, every not-yet-quantized weight of the row
 *                  moves by -(w_q - quant(w_q)) / [H^-1]_qq * H^-1_{:,q}, read through G,
 *   order          fixed, left to right,
 *   blocks         B columns at a time; columns right of the block get one lazy batch
 *                  update (a matrix product) after the block.
 * The quantizer is the linear one of section "量化基础" on the same page
 * (x_q = round(x/s) symmetric, round(x/s + z) asymmetric) with the round-and-clip of
 * section "四、量化形式" of the LLM-quantization introduction on m.youleyou.com, at one
 * scale/zero pair per output row or per run of g input columns (granularity table of
 * the page "大模型常见的量化方式", psvmc.cn).
 *
 * Conventions for every call:
 *   - Matrices are row-major.  Tensor arguments are DEVICE pointers owned by the caller;
 *     the library keeps no pointer after a call returns and allocates no device memory.
 *     Scratch memory is the caller's workspace `ws` of at least the size returned by the
 *     matching *_workspace_size function (16-byte aligned).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All work is
 *     enqueued on it and the call returns without waiting, except gptq_prepare_hinv with
 *     a non-NULL `info`, which waits for the stream once to read the pivot flag.
 *   - Arguments are validated before any HIP call.  Errors are returned as negative codes;
 *     gptq_last_error() gives a message for the calling thread.  Nothing is written on a
 *     validation error.  No C++ exception crosses this interface.
 *   - Results are deterministic: repeated calls on the same inputs give identical bytes.
 */
#ifndef GPTQ_H
#define GPTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define GPTQ_OK 0
#define GPTQ_EINVAL (-1)  /* bad argument (null pointer, shape, alignment, spec)          */
#define GPTQ_ENOTSPD (-2) /* damped Hessian not positive definite (a pivot <= 0 or NaN)  */
#define GPTQ_EHIP (-3)    /* a HIP runtime call failed                                    */
#define GPTQ_ENOWS (-4)   /* workspace smaller than the size query returned               */

/* element types of W and X */
#define GPTQ_F16 0
#define GPTQ_F32 1

/* What to quantize to.
 *   bits       2, 3, 4 or 8: codes are stored in [0, 2^bits - 1].
 *   group      0: one (scale, zero) per output row ("per-channel");
 *              g > 0: one pair per run of g consecutive input columns of a row.
 *              g must divide d_col, and block % g == 0 or g % block == 0.
 *   sym        0: asymmetric, range [min(0, min x), max(0, max x)] of the group,
 *                 s = range / (2^bits - 1), z = round(-min / s);
 *              1: symmetric, s = max|x| / (2^(bits-1) - 1), z = 2^(bits-1)
 *                 (signed codes clipped to [-2^(bits-1), 2^(bits-1) - 1], stored + z).
 *              A group whose range is empty uses the range [-1, 1].
 *   block      B in {32, 64, 128, 256}: columns quantized with immediate updates
 *              before the lazy batch update of the columns to their right.
 *   damp_frac  lambda = damp_frac * mean(diag H) is added to diag H before inversion
 *              (the pages do not fix a damping; 0.01 is customary).
 * (s, z) are computed at the first column of each group from the weights as they are
 * at that moment (after the compensation from all earlier columns).  Codes are
 * clip(round_half_even(w / s + z), 0, 2^bits - 1), decided in float32 with IEEE
 * division; the dequantized weight is s * (code - z). */
typedef struct gptq_spec {
  int bits;
  int group;
  int sym;
  int block;
  float damp_frac;
} gptq_spec;

const char* gptq_version(void);
const char* gptq_strerror(int code);
/* Message of the last failed call on this thread ("" if none). */
const char* gptq_last_error(void);

/* ---------------------------------------------------------------- Hessian (a1)
 * H += 2 * X^T X, i.e. H[i][j] += 2 * sum_t X[t][i] * X[t][j]  (page "量化", GPTQ:
 * H = 2 X X^T with X as d x n_tok; here X is stored token-major).
 *   H      d x d float32, row-major, read and written in full (both triangles receive
 *          the same value, so a symmetric H stays exactly symmetric).  The caller
 *          zeroes H before the first chunk; calls on successive token chunks sum up.
 *   X      n_tok x d, row t = the layer input of token t, leading dimension ldx
 *          (elements) >= d.  x_dtype GPTQ_F16 (products exact, float32 accumulation)
 *          or GPTQ_F32.  X and ldx * element size must be 16-byte aligned.
 *   n_tok  >= 0; 0 is a no-op.
 *   ws     workspace of gptq_hessian_workspace_size(d, n_tok, ldx, x_dtype) bytes (the
 *          float32 partial tiles of the token ranges processed in parallel).
 * Errors: GPTQ_EINVAL, GPTQ_ENOWS, GPTQ_EHIP. */
size_t gptq_hessian_workspace_size(int64_t d, int64_t n_tok, int64_t ldx, int x_dtype);
int gptq_hessian_accumulate(float* H, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                            int64_t ldx, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- inverse factor (a2, a3)
 * G = Cholesky((H + lambda I)^-1)^T with lambda = damp_frac * mean(diag H): G is upper
 * triangular with positive diagonal and G^T G = (H + lambda I)^-1 (page "量化", GPTQ,
 * Cholesky reformulation).  Computed without forming the inverse: H + lambda I = U U^T
 * with U upper, then G = U^-1 (the same unique factor).
 *   H      d x d float32 symmetric; only its upper triangle is read.
 *   G      d x d float32 output; the strictly lower triangle is set to 0.  G == H
 *          (in place) is allowed.
 *   info   host pointer or NULL.  Non-NULL: the call waits for the stream, sets *info
 *          to 0 on success or to a positive value when a pivot was <= 0 or not finite,
 *          and then returns GPTQ_ENOTSPD (G is then undefined).  NULL: no wait and
 *          no check.
 * Errors: GPTQ_EINVAL (d < 1, damp_frac < 0 or not finite), GPTQ_ENOWS, GPTQ_ENOTSPD,
 * GPTQ_EHIP. */
size_t gptq_prepare_workspace_size(int64_t d);
int gptq_prepare_hinv(const float* H, float* G, int64_t d, float damp_frac, void* ws,
                      size_t ws_bytes, int64_t* info, void* stream);

/* Inspection of the blocked schedule that gptq_prepare_hinv runs on diagonal blocks of
 * 1024 to 2048 columns (host only: no HIP call, usable without a GPU).  The same factor
 * as above, taken in 128-column blocks from the bottom right (page "量化", GPTQ, Cholesky
 * reformulation, in blocked form): per block a leaf factor G_kk = U_kk^-1, the panel
 * U[0:c_k, k] = A[0:c_k, k] G_kk^T into a scratch matrix, the update of the next block's
 * column, and the trailing update; the blocks of G above the diagonal from a binary tree
 * over the blocks.  All on the caller's stream: each leaf is one workgroup of a launch
 * whose other workgroups run the previous block's trailing update and tiles of the tree
 * products whose inputs are complete.  When the block is the left half of a recursion node
 * with an r-column right half, the schedule also forms that node's Q = P G22 (P = A12 G22^T,
 * n x r; G22 the factored r-block right below and right of the block) in K chunks of 512
 * that start on G22's diagonal, beside the leaves.
 *   n, ld  block size and leading dimension of the matrix it sits in (ld >= n + r).
 *   r      columns of the node's right half whose Q comes along (0: none).
 *   out    NULL or cap records of GPTQ_PLAN_FIELDS int64 each.  Record 0: number of
 *          128-blocks, r, U-scratch floats, tree-scratch floats, number of launches.
 *          Then one record per launch in stream order:
 *            [0] kind (0 a leaf and/or tile ranges of up to six products in one launch,
 *                1 one whole product), [1] number of products, [2] 0,
 *            [3] leaf offset on the diagonal, [4] leaf size (0: no leaf),
 *            [5 + 21 j .. 26 + 21 j) product j: M, N, K, then for A, B and C the buffer
 *                (0 the matrix, offsets from the block's corner; 1 the U scratch, n x n;
 *                2 the tree scratch; 3 the node's P and 4 its Q, n x r with leading
 *                dimension r), offset and leading dimension, followed by transA,
 *                triA (after A), transB, triB (after B), triC (after C), alpha, beta, and
 *                the range [t0, t1) of its 64 x 64 tiles in the product's tile order (tile
 *                t is tile row t / tiles_per_row, column t % tiles_per_row; by columns
 *                instead when triB = 2, by columns from the last when triB = 1, by rows
 *                from the last when triA = 2).
 *          C = alpha op(A) op(B) + beta C with op(X) = X^T when transX; triA/triB 1 (2):
 *          op(X) is upper (lower) triangular, entries outside are zero and never read;
 *          triC 1: only entries on or above the diagonal of C are written.
 * Returns the number of records needed (written when cap suffices); GPTQ_EINVAL for n < 1,
 * n > 65536, r < 0, r > 65536 or ld < n + r. */
#define GPTQ_PLAN_FIELDS 160
int64_t gptq_prepare_plan(int64_t n, int64_t ld, int64_t r, int64_t* out, int64_t cap);

/* ---------------------------------------------------------------- column solve (a4-a7)
 * Quantizes W with GPTQ given G from gptq_prepare_hinv (page "量化", GPTQ: fixed order,
 * OBS compensation through G, blocks of spec->block columns with a lazy batch update).
 *   W         d_row x d_col, w_dtype GPTQ_F16 or GPTQ_F32, not modified (the working
 *             copy lives in the workspace).  d_col must be a multiple of 32.
 *   G         d_col x d_col float32 upper triangular (entries below the diagonal unused).
 *   qweight   d_row x (d_col * bits / 32) uint32 words: code (r, c) occupies bits
 *             [c*bits, c*bits + bits) of row r's little-endian bit stream.
 *   scales    d_row x n_groups float32, zeros d_row x n_groups uint8, with
 *             n_groups = 1 (group 0) or d_col / group.
 *   err_sq_rows  NULL or d_row doubles: receives sum_q e_q^2 per row, where
 *             e_q = (w_q - w^_q) / G_qq; equals Delta H_d Delta^T for Delta = W - W^.
 * Errors: GPTQ_EINVAL, GPTQ_ENOWS, GPTQ_EHIP. */
size_t gptq_quantize_workspace_size(int64_t d_row, int64_t d_col, const gptq_spec* spec);
int gptq_quantize_layer(const void* W, int w_dtype, int64_t d_row, int64_t d_col, const float* G,
                        const gptq_spec* spec, uint32_t* qweight, float* scales, uint8_t* zeros,
                        double* err_sq_rows, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- check (a8)
 * Dequantizes W^ = s * (code - z) and measures the layer objective of page "量化", GPTQ,
 * ||W X - W^ X||_F^2 = 1/2 * sum_r (W - W^)_r H (W - W^)_r^T with the undamped H.
 *   qweight/scales/zeros  as written by gptq_quantize_layer for the same spec and shape.
 *   W        the original weights; H the undamped d_col x d_col Hessian (symmetric, as
 *            gptq_hessian_accumulate writes it: only its upper triangle is read; the loss
 *            is formed from the half product T = D U, U that triangle, as
 *            sum_c T D - 1/2 sum_c D^2 H_cc per row, in double).
 *   loss     device pointer to 1 double (the objective above).
 *   row_loss NULL or device pointer to d_row doubles (each row's share).
 *   W_hat    NULL or device d_row x d_col float32 receiving the dequantized weights.
 *   off_grid device pointer to 1 int64: number of groups whose zero point lies outside
 *            [0, 2^bits - 1] or whose scale is not finite and positive.
 * Errors: GPTQ_EINVAL, GPTQ_ENOWS, GPTQ_EHIP. */
size_t gptq_check_workspace_size(int64_t d_row, int64_t d_col);
int gptq_dequant_check(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                       const void* W, int w_dtype, const float* H, int64_t d_row, int64_t d_col,
                       const gptq_spec* spec, double* loss, double* row_loss, float* W_hat,
                       int64_t* off_grid, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- weight-only product
 * Quantized linear layer over the packed output of gptq_quantize_layer, for a few fp16
 * activation rows (W4A16 and its 2/3/8-bit kin: page "量化", section AWQ, weights in 4 bits
 * and activations in fp16 with the dequantization inside the matrix product; section GPTQ,
 * per-channel INT4 weights for memory-bound single-batch inference):
 *     y[i][r] = sum_c x[i][c] * scales[r][c / g] * (code(r, c) - zeros[r][c / g])
 * with code(r, c) at bits [c*bits, c*bits + bits) of row r's little-endian bitstream in
 * qweight, exactly as gptq_quantize_layer writes it (g = d_col when group = 0).
 *   qweight  [d_row x d_col*bits/32] uint32, 16-byte aligned; scales [d_row x d_col/g]
 *            fp32; zeros [d_row x d_col/g] uint8.
 *   x        [n x d_col] fp16 (x_dtype must be GPTQ_F16), 4-byte aligned, row stride
 *            ldx >= d_col (rows 16-byte aligned are staged 16 bytes at a time, others one
 *            element at a time).
 *   y        [n x d_row] fp32 output, row stride ldy >= d_row.
 *   bits 2, 3, 4 or 8; group 0 (per-channel) or a multiple of 32 dividing d_col;
 *   d_col a multiple of 32 and at most 32768; 1 <= n <= 4096 (the rows are taken in groups
 *   whose fp16 copy fits 64 KB of LDS, at most 8 per launch).
 * Products are accumulated in fp32 (fp16 products of the exact integers q - z for 2 and 4
 * bits),
 * one run of 32 codes at a time, then over runs in a fixed order: deterministic.
 * Errors: GPTQ_EINVAL for NULL pointers, shapes, strides or alignment; GPTQ_EHIP. */
int gptq_dequant_matvec(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                        int64_t d_row, int64_t d_col, int bits, int group, const void* x,
                        int x_dtype, int64_t n, int64_t ldx, float* y, int64_t ldy,
                        void* stream);

/* ---------------------------------------------------------------- weight-only product, batched
 * The same product y = x W^T over the packed layer for many activation rows, on the fp16
 * matrix cores (page "量化", section AWQ: W4A16, INT4 weights with fp16 activations; section
 * GPTQ: the quantized layer's output).  Group by group:
 *     y[i][r] = sum_g s[r][g] * sum_{c in group g} x[i][c] * (code[r][c] - z[r][g]),
 * fp16 x times the exact integers code - z in fp32 sums, scaled and added in fp32.  When d_col
 * and the group size are multiples of 64 (per-channel: d_col a multiple of 64), the codes are
 * read packed and expanded in the product's main loop (page "量化", section AWQ: the
 * weight-only kernel dequantizes inside the GEMM loop), so the weights cross HBM at b bits
 * each and no workspace is used; other layouts (groups of 16 or 32) expand the codes into
 * the workspace as fp16 integers (d_row x d_col halfs) first.  The call pays off from a few
 * hundred activation rows on; gptq_dequant_matvec is the small-n path.
 *   qweight, scales, zeros  as gptq_quantize_layer writes them; d_col a multiple of 32;
 *            bits 2, 3, 4 or 8; group 0 or a multiple of 16 dividing d_col.
 *   x  [n x d_col] fp16, row stride d_col <= ldx <= 2^22, a multiple of 8, x 16-byte aligned;
 *      n >= 0.
 *   y  [n x d_row] float32 output, row stride ldy >= d_row (overwritten).
 *   Workspace: gptq_dequant_matmul_workspace_size(d_row, d_col, bits, group) bytes, 256-byte
 *      aligned; 0 (ws may be NULL) for the layouts read packed.
 * Errors: GPTQ_EINVAL, GPTQ_ENOWS, GPTQ_EHIP. */
size_t gptq_dequant_matmul_workspace_size(int64_t d_row, int64_t d_col, int bits, int group);
int gptq_dequant_matmul(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                        int64_t d_row, int64_t d_col, int bits, int group, const void* x, int64_t n,
                        int64_t ldx, float* y, int64_t ldy, void* ws, size_t ws_bytes,
                        void* stream);

/* ---------------------------------------------------------------- AWQ scale search
 * Activation-aware scales (page "量化", section AWQ): channel c of W is multiplied by
 * s_c = s_X[c]^alpha before round-to-nearest quantization and the layer's activations are
 * meant to be divided by s_c, where s_X is the mean magnitude of each input channel over
 * the calibration tokens; alpha is the point of the grid k / (n_grid - 1), k = 0..n_grid-1
 * (n_grid = 20 on the page), with the smallest layer loss
 *     L = ||W X - Q(W diag s) diag(s)^-1 X||_F^2 = 1/2 sum_r D_r H D_r^T,
 *     D = W - Q(W diag s) diag(s)^-1,  H = 2 X X^T undamped.
 * Q is round-to-nearest per row and group of the scaled weights, with the scale and zero
 * point rules of gptq_quantize_layer (no error compensation).
 *
 * gptq_act_absmean: sx_sum[c] += sum_t |X[t][c]| over n_tok token-major rows of X
 *   (x_dtype F16 or F32, row stride ldx >= d, X and its rows 16-byte aligned), in double.
 *   The caller zeroes sx_sum and may call once per chunk of tokens; the per-call order of
 *   the sums is fixed, so results are reproducible.  n_tok = 0 is a no-op.
 *   Workspace: gptq_act_absmean_workspace_size(d, n_tok) bytes, 256-byte aligned.
 * gptq_awq_search: s_X = sx_sum / n_tok (n_tok = the number of tokens summed).
 *   W       [d_row x d_col] F16 or F32, row-major (not modified).
 *   H       [d_col x d_col] float32 undamped Hessian of the same tokens (both triangles).
 *   spec    bits, group and sym as for gptq_quantize_layer (group 0 = per output row, else
 *           a multiple of 16 dividing d_col); block and damp_frac are not used.
 *   n_grid  2 .. 1000.
 *   Outputs (device): qweight [d_row x d_col*bits/32], scales and zeros [d_row x d_col/g]
 *           of Q(W diag s) at the chosen alpha, in gptq_quantize_layer's format (so
 *           gptq_dequant_matvec applies, with x divided by s); s_out [d_col] float32, the
 *           chosen s; losses [n_grid] double, L at every grid point; best NULL or 1 int32,
 *           the chosen grid index (the first smallest loss).
 *   Workspace: gptq_awq_workspace_size(d_row, d_col) bytes, 256-byte aligned.
 *   Nothing is read back to the host: the call is asynchronous on the stream.
 * Errors: GPTQ_EINVAL (shapes, spec, n_grid, NULL pointers, alignment), GPTQ_ENOWS,
 * GPTQ_EHIP. */
size_t gptq_act_absmean_workspace_size(int64_t d, int64_t n_tok);
int gptq_act_absmean(double* sx_sum, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                     int64_t ldx, void* ws, size_t ws_bytes, void* stream);
/* gptq_act_absmean_noalloc: gptq_act_absmean without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight calibration loops,
 * harnesses that forbid hipMalloc).  The same kernels and the same result bit for bit.
 *   Arguments as for gptq_act_absmean; the call runs on `stream`, which must belong to the
 *   current device (NULL: the current device's null stream).
 *   Scratch: the per-split partial sums live in a 16 MiB array the library holds on each GPU
 *   it runs on until the process ends (its address is looked up on the first call on a
 *   device).  Every shape the call accepts fits; a plan that would need more is rejected with
 *   GPTQ_EINVAL.  The call allocates nothing (no hipMalloc, no hipFree).
 *   Calls that overlap on one GPU (on different streams, or from several threads) share that
 *   array and race; serialize them.  Each call writes every partial sum it reads, so nothing
 *   needs clearing between calls.
 * Errors: GPTQ_EINVAL (as gptq_act_absmean; a stream of another device), GPTQ_EHIP. */
int gptq_act_absmean_noalloc(double* sx_sum, int64_t d, const void* X, int x_dtype,
                             int64_t n_tok, int64_t ldx, void* stream);
size_t gptq_awq_workspace_size(int64_t d_row, int64_t d_col);
int gptq_awq_search(const void* W, int w_dtype, int64_t d_row, int64_t d_col, const float* H,
                    const double* sx_sum, int64_t n_tok, const gptq_spec* spec, int n_grid,
                    uint32_t* qweight, float* scales, uint8_t* zeros, float* s_out,
                    double* losses, int32_t* best, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- MLP block forward
 * The input of down_proj when one decoder layer's MLP is quantized layer by layer (page
 * "大模型常见的量化方式", section on the layers of a large model: gate_proj, up_proj and
 * down_proj of the LLaMA MLP, read as down(silu(gate x) * up x)):
 *     Y[t][j] = float16( silu(sum_c X[t][c] G^[j][c]) * sum_c X[t][c] U^[j][c] ),
 *     silu(a) = a / (1 + exp(-a)),
 * with G^ and U^ dequantized from the packed gate_proj and up_proj as gptq_quantize_layer
 * writes them (both [d_ff x d], the same bits and group).  Products group by group on the
 * fp16 matrix cores (fp16 X times the exact integers code - z, fp32 sums scaled by s),
 * tokens in chunks of 8192.
 *   X    [n_tok x d] fp16 (x_dtype GPTQ_F16), row stride ldx >= d, a multiple of 8; X
 *        16-byte aligned.
 *   Y    [n_tok x d_ff] fp16 output, row stride ldy >= d_ff.
 *   d a multiple of 32; bits 2, 3, 4 or 8; group 0 or a multiple of 16 dividing d.
 *   Workspace: gptq_mlp_forward_workspace_size(n_tok, d, d_ff) bytes, 256-byte aligned
 *   (the codes expanded to fp16 integers and one chunk's float32 products).
 * Errors: GPTQ_EINVAL, GPTQ_ENOWS, GPTQ_EHIP. */
size_t gptq_mlp_forward_workspace_size(int64_t n_tok, int64_t d, int64_t d_ff);
int gptq_mlp_forward(const void* X, int x_dtype, int64_t n_tok, int64_t d, int64_t ldx,
                     const uint32_t* qgate, const float* sgate, const uint8_t* zgate,
                     const uint32_t* qup, const float* sup, const uint8_t* zup, int64_t d_ff,
                     int bits, int group, void* Y, int64_t ldy, void* ws, size_t ws_bytes,
                     void* stream);

/* ---------------------------------------------------------------- attention half of a block
 * The calibration inputs of q/k/v_proj and o_proj, and the residual that feeds the MLP, when
 * one decoder layer is quantized layer by layer (page "大模型常见的量化方式", section on the
 * layers of a large model: the LLaMA layer with input_layernorm, self_attn,
 * post_attention_layernorm and the MLP, the norms kept in float16).  Read as the LLaMA layer:
 *
 * gptq_rmsnorm: y[t][c] = float16( x[t][c] / sqrt(mean_c x[t][c]^2 + eps) * gamma[c] ),
 *   in float64 (rounded to float32, then float16).
 *   x, y [n_tok x d] fp16, row strides ldx, ldy >= d; gamma [d] fp16.  d, ldx and ldy
 *   multiples of 8; x, y and gamma 16-byte aligned; eps finite and >= 0.  In place (y == x,
 *   ldy == ldx) is allowed.  No workspace.
 *
 * gptq_attention_forward: O = float16( attention(rope(q), rope(k), v) ) with
 *   q, k, v = float16(X W^T) for the packed q_proj, k_proj and v_proj (each [d x d], the
 *   same bits and group, in gptq_quantize_layer's format; products group by group on the
 *   fp16 matrix cores as for gptq_mlp_forward).  Causal multi-head self-attention, heads of 128 channels (head h is channels
 *   [128 h, 128 h + 128)), softmax of q.k / sqrt(128) over the keys at or before the query.
 *   Rotary embedding: channels i and i + 64 of a head turn by pos * 10000^(-2i/128), angles
 *   in float64.  The tokens form independent sequences [0, seq_len), [seq_len, 2 seq_len),
 *   ...; pos counts from 0 in each; the last one may be shorter.
 *   X  [n_tok x d] fp16, row stride ldx >= d;  O [n_tok x d] fp16, ldo >= d; ldx and ldo
 *   multiples of 8, X and O 16-byte aligned.  d a multiple of 128; bits 2, 3, 4 or 8; group 0 or a
 *   multiple of 16 dividing d; 1 <= seq_len <= 2^20.
 *   Workspace: gptq_attention_forward_workspace_size(n_tok, d, seq_len) bytes, 256-byte
 *   aligned (the codes as fp16 integers, one chunk of whole sequences in float32, the angles).
 *
 * gptq_residual_linear: Hout = float16( R + X W^T ) for one packed layer W [d_out x d_in]
 *   (o_proj: X the attention output, R the block input).
 *   X [n_tok x d_in] fp16, ldx >= d_in a multiple of 8, X 16-byte aligned; R and Hout
 *   [n_tok x d_out] fp16, ldr, ldh >= d_out.
 *   d_in a multiple of 32; bits and group as above (group divides d_in).
 *   Workspace: gptq_residual_linear_workspace_size(n_tok, d_in, d_out) bytes, 256-byte aligned.
 *
 * All three are asynchronous on the stream; n_tok = 0 is a no-op.
 * Errors: GPTQ_EINVAL (shapes, strides, alignment, NULL pointers), GPTQ_ENOWS, GPTQ_EHIP. */
int gptq_rmsnorm(const void* x, int64_t n_tok, int64_t d, int64_t ldx, const void* gamma,
                 double eps, void* y, int64_t ldy, void* stream);
size_t gptq_attention_forward_workspace_size(int64_t n_tok, int64_t d, int64_t seq_len);
int gptq_attention_forward(const void* X, int64_t n_tok, int64_t d, int64_t ldx,
                           const uint32_t* qq, const float* sq, const uint8_t* zq,
                           const uint32_t* qk, const float* sk, const uint8_t* zk,
                           const uint32_t* qv, const float* sv, const uint8_t* zv, int bits,
                           int group, int64_t seq_len, void* O, int64_t ldo, void* ws,
                           size_t ws_bytes, void* stream);
size_t gptq_residual_linear_workspace_size(int64_t n_tok, int64_t d_in, int64_t d_out);
int gptq_residual_linear(const void* X, int64_t n_tok, int64_t d_in, int64_t ldx, const void* R,
                         int64_t ldr, const uint32_t* q, const float* s, const uint8_t* z,
                         int64_t d_out, int bits, int group, void* Hout, int64_t ldh, void* ws,
                         size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- instrumentation
 * Optional per-kernel timing with HIP events recorded on the caller's stream around
 * every launch of the named kernel family ("hessian_mfma", "hessian_reduce", "prep_leaf",
 * "prep_gemm", "quant_block", "lazy_gemm", "dequant_matvec", "absmean", "awq_scale_rtn",
 * "awq_gemm", "mlp_gemm", "mlp_elementwise", "block_gemm", "block_elementwise", "attention",
 * "dequant_expand", "dequant_matmul", "check", "check_gemm", ...).  Enabling costs two event
 * records per timed launch; gptq_profile_only(name) restricts timing to one family (NULL: all).
 * gptq_profile_read returns the number of timed launches and their summed duration in
 * milliseconds (waits for the recorded events).  For measurement, not for production. */
int gptq_profile_enable(int on);
int gptq_profile_only(const char* kernel);
int gptq_profile_reset(void);
int gptq_profile_read(const char* kernel, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_H */
