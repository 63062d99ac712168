// C ABI of libgptq: argument validation (before any HIP call), workspace checks, launch
// orchestration on the caller's stream, error codes and messages, and the optional
// per-kernel event timing.  The numerical work lives in hessian.hip, prep.hip,
// quant.hip, gemm.hip, check.hip, gemv.hip, awq.hip and mlp.hip.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>
#include <climits>

#include "gptq.h"
#include "gptq_internal.h"
#include "prep_plan.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(GPTQ_EHIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------- instrumentation
struct PendingEvent {
  std::string name;
  hipEvent_t e0, e1;
};
struct ProfTotal {
  int64_t launches = 0;
  double ms = 0.0;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_only;                // empty: every kernel family
std::vector<PendingEvent> g_pending;
std::vector<hipEvent_t> g_free_events;  // recycled, so a timed launch costs two records only
std::map<std::string, ProfTotal> g_totals;

hipEvent_t take_event() {   // caller holds g_prof_mu
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

void drain_pending() {
  for (auto& p : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.e1) == hipSuccess && hipEventElapsedTime(&ms, p.e0, p.e1) == hipSuccess) {
      auto& t = g_totals[p.name];
      t.launches += 1;
      t.ms += ms;
    }
    g_free_events.push_back(p.e0);
    g_free_events.push_back(p.e1);
  }
  g_pending.clear();
}

int check_spec(const gptq_spec* spec, int64_t d_col) {
  if (!spec) return fail(GPTQ_EINVAL, "spec is NULL");
  if (spec->bits != 2 && spec->bits != 3 && spec->bits != 4 && spec->bits != 8)
    return fail(GPTQ_EINVAL, "bits must be 2, 3, 4 or 8 (got %d)", spec->bits);
  if (spec->block != 32 && spec->block != 64 && spec->block != 128 && spec->block != 256)
    return fail(GPTQ_EINVAL, "block must be 32, 64, 128 or 256 (got %d)", spec->block);
  if (spec->sym != 0 && spec->sym != 1) return fail(GPTQ_EINVAL, "sym must be 0 or 1");
  if (spec->group < 0) return fail(GPTQ_EINVAL, "group must be >= 0");
  if (spec->group > 0) {
    if (spec->group % 16 != 0)
      return fail(GPTQ_EINVAL, "group must be a multiple of 16 (got %d)", spec->group);
    if (d_col % spec->group != 0)
      return fail(GPTQ_EINVAL, "group %d does not divide d_col %lld", spec->group, (long long)d_col);
    if (spec->block % spec->group != 0 && spec->group % spec->block != 0)
      return fail(GPTQ_EINVAL, "block %d and group %d must nest", spec->block, spec->group);
  }
  return GPTQ_OK;
}

int check_layer(int w_dtype, int64_t d_row, int64_t d_col) {
  if (w_dtype != GPTQ_F16 && w_dtype != GPTQ_F32) return fail(GPTQ_EINVAL, "w_dtype must be F16 or F32");
  if (d_row < 1 || d_row > (int64_t)1 << 30) return fail(GPTQ_EINVAL, "d_row out of range");
  if (d_col < 32 || d_col % 32 != 0 || d_col > (int64_t)1 << 20)
    return fail(GPTQ_EINVAL, "d_col must be a positive multiple of 32 (got %lld)", (long long)d_col);
  return GPTQ_OK;
}

int check_packed(int bits, int group, int64_t d) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_EINVAL, "bits must be 2, 3, 4 or 8 (got %d)", bits);
  if (group < 0 || (group > 0 && (group % 16 != 0 || d % group != 0)))
    return fail(GPTQ_EINVAL, "group must be 0 or a multiple of 16 dividing %lld (got %d)",
                (long long)d, group);
  return GPTQ_OK;
}

}  // namespace

namespace gptq {

ProfScope::ProfScope(const char* n, hipStream_t s) : name(n), stream(s), ev0(nullptr) {
  if (!g_prof_on) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_only.empty() && g_prof_only != n) return;
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) {
    g_free_events.push_back(e);
    return;
  }
  ev0 = e;
}

ProfScope::~ProfScope() {
  if (!ev0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t e1 = take_event();
  if (!e1 || hipEventRecord(e1, stream) != hipSuccess) {
    g_free_events.push_back(static_cast<hipEvent_t>(ev0));
    if (e1) g_free_events.push_back(e1);
    return;
  }
  g_pending.push_back({name, static_cast<hipEvent_t>(ev0), e1});
}

}  // namespace gptq

extern "C" {

const char* gptq_version(void) { return "gptq-mi355x 0.1.0 (gfx950)"; }

const char* gptq_strerror(int code) {
  switch (code) {
    case GPTQ_OK: return "ok";
    case GPTQ_EINVAL: return "invalid argument";
    case GPTQ_ENOTSPD: return "damped Hessian is not positive definite";
    case GPTQ_EHIP: return "HIP runtime error";
    case GPTQ_ENOWS: return "workspace too small";
    default: return "unknown error";
  }
}

const char* gptq_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------- Hessian
size_t gptq_hessian_workspace_size(int64_t d, int64_t n_tok, int64_t ldx, int x_dtype) {
  if (d < 1 || n_tok < 1 || ldx < d || (x_dtype != GPTQ_F16 && x_dtype != GPTQ_F32)) return 0;
  return gptq::hessian_plan(d, n_tok, ldx, x_dtype).ws_bytes;
}

int gptq_hessian_accumulate(float* H, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                            int64_t ldx, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (d < 1 || d > (int64_t)1 << 20) return fail(GPTQ_EINVAL, "d out of range (%lld)", (long long)d);
  if (n_tok < 0) return fail(GPTQ_EINVAL, "n_tok < 0");
  if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_F32) return fail(GPTQ_EINVAL, "x_dtype must be F16 or F32");
  if (!H) return fail(GPTQ_EINVAL, "H is NULL");
  if (n_tok == 0) return GPTQ_OK;
  if (!X) return fail(GPTQ_EINVAL, "X is NULL");
  if (ldx < d) return fail(GPTQ_EINVAL, "ldx (%lld) < d (%lld)", (long long)ldx, (long long)d);
  const size_t elt = x_dtype == GPTQ_F16 ? 2 : 4;
  if (!aligned(X, 16) || (ldx * (int64_t)elt) % 16 != 0)
    return fail(GPTQ_EINVAL, "X and its rows must be 16-byte aligned");
  const gptq::HessPlan p = gptq::hessian_plan(d, n_tok, ldx, x_dtype);
  if (!ws || ws_bytes < p.ws_bytes)
    return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", p.ws_bytes);
  if (!aligned(ws, 16)) return fail(GPTQ_EINVAL, "workspace must be 16-byte aligned");
  hipError_t e = gptq::hessian_launch(p, H, X, x_dtype, ldx, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_hessian_accumulate");
  return GPTQ_OK;
}

// ---------------------------------------------------------------- inverse factor
size_t gptq_prepare_workspace_size(int64_t d) {
  if (d < 1) return 0;
  return gptq::prepare_ws_bytes(d);
}

int gptq_prepare_hinv(const float* H, float* G, int64_t d, float damp_frac, void* ws,
                      size_t ws_bytes, int64_t* info, void* stream) {
  g_last_error.clear();
  if (d < 1 || d > (int64_t)1 << 20) return fail(GPTQ_EINVAL, "d out of range (%lld)", (long long)d);
  if (!H || !G) return fail(GPTQ_EINVAL, "H or G is NULL");
  if (!(damp_frac >= 0.0f) || !std::isfinite(damp_frac))
    return fail(GPTQ_EINVAL, "damp_frac must be finite and >= 0");
  const size_t need = gptq::prepare_ws_bytes(d);
  if (!ws || ws_bytes < need) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (!aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = gptq::prepare_launch(H, G, d, damp_frac, ws, s);
  if (e != hipSuccess) return hip_fail(e, "gptq_prepare_hinv");
  if (info) {
    *info = 0;
    int flag = INT_MAX;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "gptq_prepare_hinv sync");
    if ((e = hipMemcpy(&flag, gptq::prepare_flag_ptr(ws, d), sizeof(int), hipMemcpyDeviceToHost)) !=
        hipSuccess)
      return hip_fail(e, "gptq_prepare_hinv flag");
    if (flag != INT_MAX) {
      *info = flag;
      return fail(GPTQ_ENOTSPD, "damped Hessian not positive definite (pivot %d)", flag);
    }
  }
  return GPTQ_OK;
}

int64_t gptq_prepare_plan(int64_t n, int64_t ld, int64_t r, int64_t* out, int64_t cap) {
  g_last_error.clear();
  if (n < 1 || n > (int64_t)1 << 16 || r < 0 || r > (int64_t)1 << 16 || ld < n + r)
    return fail(GPTQ_EINVAL, "n, r or ld out of range");
  const gptq::plan::Plan p = gptq::plan::blocked_plan(n, ld, r);
  const int64_t need = (int64_t)p.ops.size() + 1;
  if (!out || cap < need) return need;
  static_assert(5 + 21 * gptq::plan::FUSED_TASKS <= GPTQ_PLAN_FIELDS, "record too short");
  int64_t* rec = out;
  for (int i = 0; i < GPTQ_PLAN_FIELDS; ++i) rec[i] = 0;
  rec[0] = p.nb; rec[1] = p.r; rec[2] = p.panel_floats; rec[3] = p.q_floats;
  rec[4] = (int64_t)p.ops.size();
  for (const gptq::plan::Op& o : p.ops) {
    rec += GPTQ_PLAN_FIELDS;
    for (int i = 0; i < GPTQ_PLAN_FIELDS; ++i) rec[i] = 0;
    rec[0] = o.kind; rec[1] = (int64_t)o.t.size(); rec[3] = o.off; rec[4] = o.n;
    for (size_t j = 0; j < o.t.size(); ++j) {
      const gptq::plan::Task& t = o.t[j];
      const gptq::plan::Gemm& g = t.g;
      const int64_t v[21] = {g.M, g.N, g.K, g.A.buf, g.A.off, g.A.ld, g.transA, g.triA,
                             g.B.buf, g.B.off, g.B.ld, g.transB, g.triB,
                             g.C.buf, g.C.off, g.C.ld, g.triC,
                             (int64_t)g.alpha, (int64_t)g.beta, t.t0, t.t1};
      for (int i = 0; i < 21; ++i) rec[5 + 21 * j + i] = v[i];
    }
  }
  return need;
}

// ---------------------------------------------------------------- column solve
size_t gptq_quantize_workspace_size(int64_t d_row, int64_t d_col, const gptq_spec* spec) {
  if (check_layer(GPTQ_F32, d_row, d_col) != GPTQ_OK || check_spec(spec, d_col) != GPTQ_OK) {
    g_last_error.clear();
    return 0;
  }
  return gptq::quant_ws_bytes(d_row, d_col, spec->block);
}

int gptq_quantize_layer(const void* W, int w_dtype, int64_t d_row, int64_t d_col, const float* G,
                        const gptq_spec* spec, uint32_t* qweight, float* scales, uint8_t* zeros,
                        double* err_sq_rows, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_layer(w_dtype, d_row, d_col)) != GPTQ_OK) return rc;
  if ((rc = check_spec(spec, d_col)) != GPTQ_OK) return rc;
  if (!W || !G || !qweight || !scales || !zeros)
    return fail(GPTQ_EINVAL, "W, G, qweight, scales and zeros must not be NULL");
  const size_t need = gptq::quant_ws_bytes(d_row, d_col, spec->block);
  if (!ws || ws_bytes < need) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (!aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  gptq::QuantArgs a{W, w_dtype, d_row, d_col, G, spec->bits, spec->group, spec->sym, spec->block,
                    qweight, scales, zeros, err_sq_rows};
  hipError_t e = gptq::quant_launch(a, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_quantize_layer");
  return GPTQ_OK;
}

// ---------------------------------------------------------------- check
size_t gptq_check_workspace_size(int64_t d_row, int64_t d_col) {
  if (check_layer(GPTQ_F32, d_row, d_col) != GPTQ_OK) {
    g_last_error.clear();
    return 0;
  }
  return gptq::check_ws_bytes(d_row, d_col);
}

int gptq_dequant_check(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                       const void* W, int w_dtype, const float* H, int64_t d_row, int64_t d_col,
                       const gptq_spec* spec, double* loss, double* row_loss, float* W_hat,
                       int64_t* off_grid, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_layer(w_dtype, d_row, d_col)) != GPTQ_OK) return rc;
  if ((rc = check_spec(spec, d_col)) != GPTQ_OK) return rc;
  if (!qweight || !scales || !zeros || !W || !H || !loss || !off_grid)
    return fail(GPTQ_EINVAL, "qweight, scales, zeros, W, H, loss and off_grid must not be NULL");
  const size_t need = gptq::check_ws_bytes(d_row, d_col);
  if (!ws || ws_bytes < need) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (!aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  hipError_t e = gptq::check_launch(qweight, scales, zeros, W, w_dtype, H, d_row, d_col, spec->bits,
                                    spec->group, loss, row_loss, W_hat, off_grid, ws,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_dequant_check");
  return GPTQ_OK;
}

int gptq_dequant_matvec(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                        int64_t d_row, int64_t d_col, int bits, int group, const void* x,
                        int x_dtype, int64_t n, int64_t ldx, float* y, int64_t ldy,
                        void* stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_layer(GPTQ_F16, d_row, d_col)) != GPTQ_OK) return rc;
  if (d_col > 32768) return fail(GPTQ_EINVAL, "d_col must be at most 32768 (got %lld)", (long long)d_col);
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_EINVAL, "bits must be 2, 3, 4 or 8 (got %d)", bits);
  if (group < 0 || (group > 0 && (group % 32 != 0 || d_col % group != 0)))
    return fail(GPTQ_EINVAL, "group must be 0 or a multiple of 32 dividing d_col (got %d)", group);
  if (x_dtype != GPTQ_F16) return fail(GPTQ_EINVAL, "x must be fp16 (GPTQ_F16)");
  if (n < 1 || n > 4096) return fail(GPTQ_EINVAL, "n must be in [1, 4096] (got %lld)", (long long)n);
  if (ldx < d_col || ldy < d_row) return fail(GPTQ_EINVAL, "ldx >= d_col and ldy >= d_row required");
  if (!qweight || !scales || !zeros || !x || !y)
    return fail(GPTQ_EINVAL, "qweight, scales, zeros, x and y must not be NULL");
  if (!aligned(qweight, 16) || !aligned(x, 4))
    return fail(GPTQ_EINVAL, "qweight must be 16-byte aligned and x 4-byte aligned");
  hipError_t e = gptq::matvec_launch(qweight, scales, zeros, d_row, d_col, bits, group, x, n, ldx,
                                     y, ldy, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_dequant_matvec");
  return GPTQ_OK;
}

size_t gptq_dequant_matmul_workspace_size(int64_t d_row, int64_t d_col, int bits, int group) {
  if (d_row < 1 || d_col < 32 || d_col % 32 != 0 || d_row > (int64_t)1 << 30 || d_col > (int64_t)1 << 20)
    return 0;
  const int64_t g = group == 0 ? d_col : group;
  if (gptq::qgemm_packed_ok(d_col, bits, g, d_col)) return 0;   // codes read in the main loop
  return gptq::align_up((size_t)d_row * d_col * sizeof(_Float16), 256);
}

int gptq_dequant_matmul(const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                        int64_t d_row, int64_t d_col, int bits, int group, const void* x, int64_t n,
                        int64_t ldx, float* y, int64_t ldy, void* ws, size_t ws_bytes,
                        void* stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_layer(GPTQ_F16, d_row, d_col)) != GPTQ_OK) return rc;
  if ((rc = check_packed(bits, group, d_col)) != GPTQ_OK) return rc;
  if (n < 0) return fail(GPTQ_EINVAL, "n < 0");
  if (ldx < d_col || ldx % 8 != 0 || ldy < d_row || ldx > (int64_t)1 << 22)
    return fail(GPTQ_EINVAL, "d_col <= ldx <= 2^22 (a multiple of 8) and ldy >= d_row required");
  if (n == 0) return GPTQ_OK;
  if (!qweight || !scales || !zeros || !x || !y)
    return fail(GPTQ_EINVAL, "qweight, scales, zeros, x and y must not be NULL");
  if (!aligned(x, 16)) return fail(GPTQ_EINVAL, "x must be 16-byte aligned");
  const size_t need = gptq_dequant_matmul_workspace_size(d_row, d_col, bits, group);
  if (need && (!ws || ws_bytes < need)) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (need && !aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  if (!need) {
    const int64_t g = group == 0 ? d_col : group;
    hipError_t e = gptq::qgemm_packed_f16(static_cast<const _Float16*>(x), ldx, n, qweight, zeros,
                                          scales, d_row, d_col, bits, g, y, ldy,
                                          static_cast<hipStream_t>(stream), "dequant_matmul");
    if (e != hipSuccess) return hip_fail(e, "gptq_dequant_matmul");
    return GPTQ_OK;
  }
  const int64_t g = group == 0 ? d_col : group;
  hipStream_t s = static_cast<hipStream_t>(stream);
  _Float16* B = static_cast<_Float16*>(ws);
  {
    gptq::ProfScope ps("dequant_expand", s);
    gptq::expand_codes_f16(qweight, zeros, d_row, d_col, bits, g, B, s);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess)
    e = gptq::qgemm_f16(static_cast<const _Float16*>(x), ldx, n, B, d_row, d_col, scales, g, y,
                        ldy, s, "dequant_matmul");
  if (e != hipSuccess) return hip_fail(e, "gptq_dequant_matmul");
  return GPTQ_OK;
}

// ---------------------------------------------------------------- AWQ scale search
size_t gptq_act_absmean_workspace_size(int64_t d, int64_t n_tok) {
  if (d < 1 || d > (int64_t)1 << 20 || n_tok < 0) return 0;
  return gptq::absmean_ws_bytes(d, n_tok);
}

int gptq_act_absmean(double* sx_sum, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                     int64_t ldx, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (d < 1 || d > (int64_t)1 << 20) return fail(GPTQ_EINVAL, "d out of range (%lld)", (long long)d);
  if (n_tok < 0) return fail(GPTQ_EINVAL, "n_tok < 0");
  if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_F32) return fail(GPTQ_EINVAL, "x_dtype must be F16 or F32");
  if (!sx_sum) return fail(GPTQ_EINVAL, "sx_sum is NULL");
  if (n_tok == 0) return GPTQ_OK;
  if (!X) return fail(GPTQ_EINVAL, "X is NULL");
  if (ldx < d) return fail(GPTQ_EINVAL, "ldx (%lld) < d (%lld)", (long long)ldx, (long long)d);
  const size_t elt = x_dtype == GPTQ_F16 ? 2 : 4;
  if (!aligned(X, 16) || (ldx * (int64_t)elt) % 16 != 0)
    return fail(GPTQ_EINVAL, "X and its rows must be 16-byte aligned");
  const size_t need = gptq::absmean_ws_bytes(d, n_tok);
  if (!ws || ws_bytes < need) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (!aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  hipError_t e = gptq::absmean_launch(sx_sum, d, X, x_dtype, n_tok, ldx, ws,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_act_absmean");
  return GPTQ_OK;
}

int gptq_act_absmean_noalloc(double* sx_sum, int64_t d, const void* X, int x_dtype,
                             int64_t n_tok, int64_t ldx, void* stream) {
  g_last_error.clear();
  if (d < 1 || d > (int64_t)1 << 20) return fail(GPTQ_EINVAL, "d out of range (%lld)", (long long)d);
  if (n_tok < 0) return fail(GPTQ_EINVAL, "n_tok < 0");
  if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_F32) return fail(GPTQ_EINVAL, "x_dtype must be F16 or F32");
  if (!sx_sum) return fail(GPTQ_EINVAL, "sx_sum is NULL");
  if (n_tok == 0) return GPTQ_OK;
  if (!X) return fail(GPTQ_EINVAL, "X is NULL");
  if (ldx < d) return fail(GPTQ_EINVAL, "ldx (%lld) < d (%lld)", (long long)ldx, (long long)d);
  const size_t elt = x_dtype == GPTQ_F16 ? 2 : 4;
  if (!aligned(X, 16) || (ldx * (int64_t)elt) % 16 != 0)
    return fail(GPTQ_EINVAL, "X and its rows must be 16-byte aligned");
  const size_t need = gptq::absmean_ws_bytes(d, n_tok);
  if (need > gptq::absmean_scratch_bytes())
    return fail(GPTQ_EINVAL, "needs %zu bytes of scratch, more than the %zu the library holds",
                need, gptq::absmean_scratch_bytes());
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "gptq_act_absmean_noalloc: hipGetDevice");
  if (st) {
    hipDevice_t sdev = -1;
    if ((e = hipStreamGetDevice(st, &sdev)) != hipSuccess)
      return hip_fail(e, "gptq_act_absmean_noalloc: hipStreamGetDevice");
    if (sdev != dev)
      return fail(GPTQ_EINVAL, "the stream belongs to device %d, the current device is %d",
                  (int)sdev, dev);
  }
  void* ws = nullptr;
  if ((e = gptq::absmean_scratch_ptr(dev, &ws)) != hipSuccess)
    return hip_fail(e, "gptq_act_absmean_noalloc: scratch address");
  e = gptq::absmean_launch(sx_sum, d, X, x_dtype, n_tok, ldx, ws, st);
  if (e != hipSuccess) return hip_fail(e, "gptq_act_absmean_noalloc");
  return GPTQ_OK;
}

size_t gptq_awq_workspace_size(int64_t d_row, int64_t d_col) {
  if (check_layer(GPTQ_F32, d_row, d_col) != GPTQ_OK) {
    g_last_error.clear();
    return 0;
  }
  return gptq::awq_ws_bytes(d_row, d_col);
}

int gptq_awq_search(const void* W, int w_dtype, int64_t d_row, int64_t d_col, const float* H,
                    const double* sx_sum, int64_t n_tok, const gptq_spec* spec, int n_grid,
                    uint32_t* qweight, float* scales, uint8_t* zeros, float* s_out,
                    double* losses, int32_t* best, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_layer(w_dtype, d_row, d_col)) != GPTQ_OK) return rc;
  if (!spec) return fail(GPTQ_EINVAL, "spec is NULL");
  if (spec->bits != 2 && spec->bits != 3 && spec->bits != 4 && spec->bits != 8)
    return fail(GPTQ_EINVAL, "bits must be 2, 3, 4 or 8 (got %d)", spec->bits);
  if (spec->sym != 0 && spec->sym != 1) return fail(GPTQ_EINVAL, "sym must be 0 or 1");
  if (spec->group < 0 || (spec->group > 0 && (spec->group % 16 != 0 || d_col % spec->group != 0)))
    return fail(GPTQ_EINVAL, "group must be 0 or a multiple of 16 dividing d_col (got %d)", spec->group);
  if (n_grid < 2 || n_grid > 1000) return fail(GPTQ_EINVAL, "n_grid must be in [2, 1000] (got %d)", n_grid);
  if (n_tok < 1) return fail(GPTQ_EINVAL, "n_tok must be >= 1");
  if (!W || !H || !sx_sum || !qweight || !scales || !zeros || !s_out || !losses)
    return fail(GPTQ_EINVAL, "W, H, sx_sum, qweight, scales, zeros, s_out and losses must not be NULL");
  const size_t need = gptq::awq_ws_bytes(d_row, d_col);
  if (!ws || ws_bytes < need) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (!aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  gptq::AwqArgs a{W, w_dtype, d_row, d_col, H, sx_sum, n_tok, spec->bits, spec->group, spec->sym,
                  n_grid, qweight, scales, zeros, s_out, losses, best};
  hipError_t e = gptq::awq_launch(a, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_awq_search");
  return GPTQ_OK;
}

// ---------------------------------------------------------------- MLP block forward
size_t gptq_mlp_forward_workspace_size(int64_t n_tok, int64_t d, int64_t d_ff) {
  if (n_tok < 1 || d < 32 || d_ff < 1 || d > (int64_t)1 << 20 || d_ff > (int64_t)1 << 20) return 0;
  return gptq::mlp_ws_bytes(n_tok, d, d_ff);
}

int gptq_mlp_forward(const void* X, int x_dtype, int64_t n_tok, int64_t d, int64_t ldx,
                     const uint32_t* qgate, const float* sgate, const uint8_t* zgate,
                     const uint32_t* qup, const float* sup, const uint8_t* zup, int64_t d_ff,
                     int bits, int group, void* Y, int64_t ldy, void* ws, size_t ws_bytes,
                     void* stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_layer(GPTQ_F16, d_ff, d)) != GPTQ_OK) return rc;
  if (x_dtype != GPTQ_F16) return fail(GPTQ_EINVAL, "X must be fp16 (GPTQ_F16)");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_EINVAL, "bits must be 2, 3, 4 or 8 (got %d)", bits);
  if (group < 0 || (group > 0 && (group % 16 != 0 || d % group != 0)))
    return fail(GPTQ_EINVAL, "group must be 0 or a multiple of 16 dividing d (got %d)", group);
  if (n_tok < 0) return fail(GPTQ_EINVAL, "n_tok < 0");
  if (n_tok == 0) return GPTQ_OK;
  if (ldx < d || ldy < d_ff) return fail(GPTQ_EINVAL, "ldx >= d and ldy >= d_ff required");
  if (ldx % 8 != 0) return fail(GPTQ_EINVAL, "ldx must be a multiple of 8");
  if (!X || !qgate || !sgate || !zgate || !qup || !sup || !zup || !Y)
    return fail(GPTQ_EINVAL, "X, the packed gate and up layers and Y must not be NULL");
  if (!aligned(X, 16)) return fail(GPTQ_EINVAL, "X must be 16-byte aligned");
  const size_t need = gptq::mlp_ws_bytes(n_tok, d, d_ff);
  if (!ws || ws_bytes < need) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (!aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  hipError_t e = gptq::mlp_launch(X, n_tok, d, ldx, qgate, sgate, zgate, qup, sup, zup, d_ff, bits,
                                  group, Y, ldy, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_mlp_forward");
  return GPTQ_OK;
}


int gptq_rmsnorm(const void* x, int64_t n_tok, int64_t d, int64_t ldx, const void* gamma,
                 double eps, void* y, int64_t ldy, void* stream) {
  g_last_error.clear();
  if (d < 8 || d % 8 != 0 || d > (int64_t)1 << 20)
    return fail(GPTQ_EINVAL, "d must be a positive multiple of 8 (got %lld)", (long long)d);
  if (n_tok < 0) return fail(GPTQ_EINVAL, "n_tok < 0");
  if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(GPTQ_EINVAL, "eps must be finite and >= 0");
  if (ldx < d || ldy < d || ldx % 8 != 0 || ldy % 8 != 0)
    return fail(GPTQ_EINVAL, "ldx and ldy must be >= d and multiples of 8");
  if (n_tok == 0) return GPTQ_OK;
  if (!x || !gamma || !y) return fail(GPTQ_EINVAL, "x, gamma and y must not be NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(gamma, 16))
    return fail(GPTQ_EINVAL, "x, y and gamma must be 16-byte aligned");
  hipError_t e = gptq::rmsnorm_launch(static_cast<const _Float16*>(x), ldx, n_tok, d,
                                      static_cast<const _Float16*>(gamma), eps,
                                      static_cast<_Float16*>(y), ldy,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_rmsnorm");
  return GPTQ_OK;
}

size_t gptq_attention_forward_workspace_size(int64_t n_tok, int64_t d, int64_t seq_len) {
  if (n_tok < 1 || d < gptq::ATTN_HEAD_DIM || d % gptq::ATTN_HEAD_DIM != 0 || d > (int64_t)1 << 16 ||
      seq_len < 1 || seq_len > (int64_t)1 << 20)
    return 0;
  return gptq::attn_ws_bytes(n_tok, d, seq_len);
}

int gptq_attention_forward(const void* X, int64_t n_tok, int64_t d, int64_t ldx,
                           const uint32_t* qq, const float* sq, const uint8_t* zq,
                           const uint32_t* qk, const float* sk, const uint8_t* zk,
                           const uint32_t* qv, const float* sv, const uint8_t* zv, int bits,
                           int group, int64_t seq_len, void* O, int64_t ldo, void* ws,
                           size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc;
  if (d < gptq::ATTN_HEAD_DIM || d % gptq::ATTN_HEAD_DIM != 0 || d > (int64_t)1 << 16)
    return fail(GPTQ_EINVAL, "d must be a positive multiple of %d (got %lld)", gptq::ATTN_HEAD_DIM,
                (long long)d);
  if ((rc = check_packed(bits, group, d)) != GPTQ_OK) return rc;
  if (seq_len < 1 || seq_len > (int64_t)1 << 20) return fail(GPTQ_EINVAL, "seq_len out of range");
  if (n_tok < 0) return fail(GPTQ_EINVAL, "n_tok < 0");
  if (ldx < d || ldo < d || ldo % 8 != 0 || ldx % 8 != 0)
    return fail(GPTQ_EINVAL, "ldx >= d, ldo >= d and both multiples of 8 required");
  if (n_tok == 0) return GPTQ_OK;
  if (!X || !qq || !sq || !zq || !qk || !sk || !zk || !qv || !sv || !zv || !O)
    return fail(GPTQ_EINVAL, "X, the packed q/k/v layers and O must not be NULL");
  if (!aligned(O, 16) || !aligned(X, 16)) return fail(GPTQ_EINVAL, "X and O must be 16-byte aligned");
  const size_t need = gptq::attn_ws_bytes(n_tok, d, seq_len);
  if (!ws || ws_bytes < need) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (!aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  const uint32_t* pq[3] = {qq, qk, qv};
  const float* ps[3] = {sq, sk, sv};
  const uint8_t* pz[3] = {zq, zk, zv};
  hipError_t e = gptq::attn_launch(static_cast<const _Float16*>(X), n_tok, d, ldx, pq, ps, pz,
                                   bits, group, seq_len, static_cast<_Float16*>(O), ldo, ws,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_attention_forward");
  return GPTQ_OK;
}

size_t gptq_residual_linear_workspace_size(int64_t n_tok, int64_t d_in, int64_t d_out) {
  if (n_tok < 1 || d_in < 32 || d_in % 32 != 0 || d_out < 1 || d_in > (int64_t)1 << 20 ||
      d_out > (int64_t)1 << 20)
    return 0;
  return gptq::residual_ws_bytes(n_tok, d_in, d_out);
}

int gptq_residual_linear(const void* X, int64_t n_tok, int64_t d_in, int64_t ldx, const void* R,
                         int64_t ldr, const uint32_t* q, const float* s, const uint8_t* z,
                         int64_t d_out, int bits, int group, void* Hout, int64_t ldh, void* ws,
                         size_t ws_bytes, void* stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_layer(GPTQ_F16, d_out, d_in)) != GPTQ_OK) return rc;
  if ((rc = check_packed(bits, group, d_in)) != GPTQ_OK) return rc;
  if (n_tok < 0) return fail(GPTQ_EINVAL, "n_tok < 0");
  if (ldx < d_in || ldr < d_out || ldh < d_out || ldx % 8 != 0)
    return fail(GPTQ_EINVAL, "ldx >= d_in (a multiple of 8), ldr >= d_out and ldh >= d_out required");
  if (n_tok == 0) return GPTQ_OK;
  if (!X || !R || !q || !s || !z || !Hout)
    return fail(GPTQ_EINVAL, "X, R, the packed layer and Hout must not be NULL");
  if (!aligned(X, 16)) return fail(GPTQ_EINVAL, "X must be 16-byte aligned");
  const size_t need = gptq::residual_ws_bytes(n_tok, d_in, d_out);
  if (!ws || ws_bytes < need) return fail(GPTQ_ENOWS, "workspace of %zu bytes needed", need);
  if (!aligned(ws, 256)) return fail(GPTQ_EINVAL, "workspace must be 256-byte aligned");
  hipError_t e = gptq::residual_launch(static_cast<const _Float16*>(X), n_tok, d_in, ldx,
                                       static_cast<const _Float16*>(R), ldr, q, s, z, d_out, bits,
                                       group, static_cast<_Float16*>(Hout), ldh, ws,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gptq_residual_linear");
  return GPTQ_OK;
}

// ---------------------------------------------------------------- instrumentation
int gptq_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return GPTQ_OK;
}

int gptq_profile_only(const char* kernel) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = kernel ? kernel : "";
  return GPTQ_OK;
}

int gptq_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending();
  g_totals.clear();
  return GPTQ_OK;
}

int gptq_profile_read(const char* kernel, int64_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return fail(GPTQ_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending();
  auto it = g_totals.find(kernel);
  *launches = it == g_totals.end() ? 0 : it->second.launches;
  *total_ms = it == g_totals.end() ? 0.0 : it->second.ms;
  return GPTQ_OK;
}

}  // extern "C"
