// C ABI of libswa: argument validation on the host, then kernel dispatch on the caller's stream.
// Declarations and the contract of every entry point are in include/swa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/swa.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SWA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SWA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared checks of (B, T, H, D, dtype); returns 0 or a status with the message set.
int check_shape(const char* fn, int B, int T, int H, int D, int dtype) {
  if (B < 1 || T < 1 || H < 1)
    return fail(SWA_ERR_INVALID_ARG, "%s: B, T, H must be >= 1 (got %d, %d, %d)", fn, B, T, H);
  if (dtype != SWA_F32 && dtype != SWA_BF16)
    return fail(SWA_ERR_INVALID_ARG, "%s: dtype must be SWA_F32 or SWA_BF16 (got %d)", fn, dtype);
  if (D != 64 && D != 128)
    return fail(SWA_ERR_UNSUPPORTED, "%s: head dim D must be 64 or 128 (got %d)", fn, D);
  const long long n = (long long)B * T * H * D;
  if (n >= (1LL << 31) / 2 || (long long)B * H * T >= (1LL << 31) / 2)
    return fail(SWA_ERR_UNSUPPORTED, "%s: B*T*H*D = %lld exceeds the supported index range", fn, n);
  return 0;
}

int need(const char* fn, const char* name, const void* p) {
  if (!p) return fail(SWA_ERR_INVALID_ARG, "%s: %s must not be NULL", fn, name);
  if (!aligned16(p)) return fail(SWA_ERR_ALIGN, "%s: %s must be 16-byte aligned", fn, name);
  return 0;
}

int opt(const char* fn, const char* name, const void* p) {
  if (p && !aligned16(p)) return fail(SWA_ERR_ALIGN, "%s: %s must be 16-byte aligned", fn, name);
  return 0;
}

int check_window_scale(const char* fn, int window, float scale, int T, int* w_out) {
  if (window == 0 || window < SWA_WINDOW_FULL)
    return fail(SWA_ERR_INVALID_ARG, "%s: window must be >= 1 or SWA_WINDOW_FULL (got %d)", fn,
                window);
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  *w_out = (window == SWA_WINDOW_FULL || window > T) ? T : window;
  return 0;
}

int check_ws(const char* fn, const void* workspace, size_t ws_bytes, int B, int T, int H, int D,
             int dtype) {
  const size_t need_ws = swa::bwd_workspace_bytes(B, T, H, D, dtype == SWA_BF16);
  if (!workspace || ws_bytes < need_ws)
    return fail(SWA_ERR_WORKSPACE, "%s: workspace of %zu bytes required (got %zu)", fn, need_ws,
                workspace ? ws_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SWA_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  return 0;
}

// Workspace of the stored-dS backward: the row terms, then (bf16) the dS^T chunks at the next
// 256-byte boundary. W is the clamped window (1..T).
size_t ds_ws_rowterm_bytes(int B, int T, int H, int D, int dtype) {
  return (swa::bwd_workspace_bytes(B, T, H, D, dtype == SWA_BF16) + 255) & ~(size_t)255;
}
size_t ds_ws_bytes(int B, int T, int H, int D, int W, int dtype) {
  const size_t rt = ds_ws_rowterm_bytes(B, T, H, D, dtype);
  return dtype == SWA_BF16 ? rt + swa::ds_buffer_bytes(B, T, H, W) : rt;
}

int check_ws_ds(const char* fn, const void* workspace, size_t ws_bytes, int B, int T, int H, int D,
                int W, int dtype) {
  const size_t need_ws = ds_ws_bytes(B, T, H, D, W, dtype);
  if (!workspace || ws_bytes < need_ws)
    return fail(SWA_ERR_WORKSPACE, "%s: workspace of %zu bytes required (got %zu; see "
                "swa_bwd_ds_workspace_size)", fn, need_ws, workspace ? ws_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SWA_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  return 0;
}

void* ds_part(void* workspace, int B, int T, int H, int D, int dtype) {
  return static_cast<char*>(workspace) + ds_ws_rowterm_bytes(B, T, H, D, dtype);
}

}  // namespace

#define SWA_TRY(expr)        \
  do {                       \
    int _st = (expr);        \
    if (_st) return _st;     \
  } while (0)

extern "C" {

const char* swa_last_error(void) { return g_last_error.c_str(); }

const char* swa_version(void) { return "swa 1.0 gfx950"; }

int rope_table(float* cos_sin, int T, int D, double base, void* stream) {
  const char* fn = "rope_table";
  SWA_TRY(need(fn, "cos_sin", cos_sin));
  if (T < 1) return fail(SWA_ERR_INVALID_ARG, "%s: T must be >= 1", fn);
  if (D != 64 && D != 128) return fail(SWA_ERR_UNSUPPORTED, "%s: D must be 64 or 128", fn);
  if (!(std::isfinite(base) && base > 0.0))
    return fail(SWA_ERR_INVALID_ARG, "%s: base must be finite and > 0", fn);
  return hip_status(swa::launch_rope_table(cos_sin, T, D, base, (hipStream_t)stream), fn);
}

int rope_qknorm_fwd(const void* q, const void* k, const float* cos_sin, void* qn, void* kn, int B,
                    int T, int H, int D, float eps, swa_dtype dtype, void* stream) {
  const char* fn = "rope_qknorm_fwd";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "cos_sin", cos_sin)); SWA_TRY(need(fn, "kn", kn));
  if ((q == nullptr) != (qn == nullptr))
    return fail(SWA_ERR_INVALID_ARG, "%s: q and qn must be given together (both NULL: k only)", fn);
  if (q) { SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "qn", qn)); }
  if (!(std::isfinite(eps) && eps >= 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  if ((q && (qn == q || qn == k || kn == q)) || kn == k)
    return fail(SWA_ERR_INVALID_ARG, "%s: outputs may not alias inputs", fn);
  return hip_status(swa::launch_rope_qknorm_fwd(q, k, cos_sin, qn, kn, B, T, H, D, eps,
                                                dtype == SWA_BF16, (hipStream_t)stream), fn);
}

int rope_qknorm_bwd(const void* q, const void* k, const float* cos_sin, const void* dqn,
                    const void* dkn, void* dq, void* dk, int B, int T, int H, int D, float eps,
                    swa_dtype dtype, void* stream) {
  const char* fn = "rope_qknorm_bwd";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "cos_sin", cos_sin));
  SWA_TRY(need(fn, "dkn", dkn)); SWA_TRY(need(fn, "dk", dk));
  if ((q == nullptr) != (dqn == nullptr) || (q == nullptr) != (dq == nullptr))
    return fail(SWA_ERR_INVALID_ARG,
                "%s: q, dqn and dq must be given together (all NULL: k only)", fn);
  if (q) { SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "dqn", dqn)); SWA_TRY(need(fn, "dq", dq)); }
  if (!(std::isfinite(eps) && eps >= 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  return hip_status(swa::launch_rope_qknorm_bwd(q, k, cos_sin, dqn, dkn, dq, dk, B, T, H, D, eps,
                                                dtype == SWA_BF16, (hipStream_t)stream), fn);
}

// Value-embedding table mode arguments of the gate calls (no AttnShape there).
static int check_ve_ids(const char* fn, const int* ve_ids, int ve_rows, int H, int D) {
  if (!ve_ids) {
    if (ve_rows != 0) return fail(SWA_ERR_INVALID_ARG, "%s: ve_rows must be 0 without ve_ids", fn);
    return ok();
  }
  if (ve_rows < 1) return fail(SWA_ERR_INVALID_ARG, "%s: ve_rows must be >= 1 with ve_ids", fn);
  if ((long long)ve_rows * H * D >= (1LL << 40))
    return fail(SWA_ERR_UNSUPPORTED, "%s: value-embedding table too large", fn);
  return ok();
}

int ve_gate_v(const void* x, int ldx, const float* Wg, float* gate, const void* v, const void* ve,
              const int* ve_ids, int ve_rows, void* v_eff, int B, int T, int H, int D,
              swa_dtype dtype, void* stream) {
  const char* fn = "ve_gate_v";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  if (!x || !Wg || !gate) return fail(SWA_ERR_INVALID_ARG, "%s: x, Wg and gate are required", fn);
  if (ldx < SWA_GATE_CHANNELS) return fail(SWA_ERR_INVALID_ARG, "%s: ldx must be >= 32", fn);
  const int nset = (v != nullptr) + (ve != nullptr) + (v_eff != nullptr);
  if (nset != 0 && nset != 3)
    return fail(SWA_ERR_INVALID_ARG, "%s: v, ve, v_eff must be all set or all NULL", fn);
  if (nset == 3) {
    SWA_TRY(need(fn, "v", v)); SWA_TRY(need(fn, "ve", ve)); SWA_TRY(need(fn, "v_eff", v_eff));
  }
  if (ve_ids && nset == 0)
    return fail(SWA_ERR_INVALID_ARG, "%s: ve_ids needs v, ve and v_eff", fn);
  SWA_TRY(check_ve_ids(fn, ve_ids, ve_rows, H, D));
  return hip_status(swa::launch_ve_gate(x, ldx, Wg, gate, v, ve, ve_ids, ve_rows, v_eff, B, T, H,
                                        D, dtype == SWA_BF16, (hipStream_t)stream), fn);
}

int ve_gate_dv(const void* dv_eff, const void* ve, const int* ve_ids, int ve_rows,
               const float* gate, void* dve, float* dgate, int B, int T, int H, int D,
               swa_dtype dtype, void* stream) {
  const char* fn = "ve_gate_dv";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "dv_eff", dv_eff)); SWA_TRY(need(fn, "ve", ve));
  SWA_TRY(need(fn, "gate", gate)); SWA_TRY(need(fn, "dve", dve));
  SWA_TRY(need(fn, "dgate", dgate));
  SWA_TRY(check_ve_ids(fn, ve_ids, ve_rows, H, D));
  return hip_status(swa::launch_ve_gate_dv(dv_eff, ve, ve_ids, ve_rows, gate, dve, dgate, B, T, H,
                                           D, dtype == SWA_BF16, (hipStream_t)stream), fn);
}

size_t ve_gate_v_bwd_workspace_size(int B, int T, int H) {
  if (B < 1 || T < 1 || H < 1 || H > SWA_GATE_MAX_HEADS) return 0;
  return swa::gate_bwd_workspace_bytes(B, T, H);
}

int ve_gate_v_bwd(const void* x, int ldx, const float* Wg, const float* gate, const float* dgate,
                  float* dWg, void* dx32, void* workspace, size_t ws_bytes, int B, int T, int H,
                  swa_dtype dtype, void* stream) {
  const char* fn = "ve_gate_v_bwd";
  SWA_TRY(check_shape(fn, B, T, H, 64, dtype));
  if (!x || !Wg || !gate || !dgate || !dWg)
    return fail(SWA_ERR_INVALID_ARG, "%s: x, Wg, gate, dgate and dWg are required", fn);
  if (ldx < SWA_GATE_CHANNELS) return fail(SWA_ERR_INVALID_ARG, "%s: ldx must be >= 32", fn);
  if (H > SWA_GATE_MAX_HEADS)
    return fail(SWA_ERR_UNSUPPORTED, "%s: at most %d heads", fn, SWA_GATE_MAX_HEADS);
  if (!workspace) return fail(SWA_ERR_WORKSPACE, "%s: workspace is required", fn);
  if (!aligned16(workspace))
    return fail(SWA_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  if (ws_bytes < swa::gate_bwd_workspace_bytes(B, T, H))
    return fail(SWA_ERR_WORKSPACE, "%s: workspace of %zu bytes is smaller than the %zu needed", fn,
                ws_bytes, swa::gate_bwd_workspace_bytes(B, T, H));
  return hip_status(swa::launch_ve_gate_bwd(x, ldx, Wg, gate, dgate, dWg, dx32, workspace, B, T, H,
                                            dtype == SWA_BF16, (hipStream_t)stream), fn);
}

int swa_doc_bounds(const int* doc_id, int* doc_bounds, int B, int T, void* stream) {
  const char* fn = "swa_doc_bounds";
  SWA_TRY(need(fn, "doc_id", doc_id));
  SWA_TRY(need(fn, "doc_bounds", doc_bounds));
  if (B < 1 || T < 1) return fail(SWA_ERR_INVALID_ARG, "%s: B and T must be >= 1", fn);
  if ((long long)B * T >= (1LL << 30))
    return fail(SWA_ERR_UNSUPPORTED, "%s: B*T exceeds the supported index range", fn);
  if (doc_bounds == doc_id) return fail(SWA_ERR_INVALID_ARG, "%s: doc_bounds may not alias doc_id", fn);
  return hip_status(swa::launch_doc_bounds(doc_id, doc_bounds, B, T, (hipStream_t)stream), fn);
}

// Value-embedding table mode: with ve_ids, ve is a (ve_rows, H*D) table indexed by the token
// ids and the backward's dve is its float gradient; without, ve_rows must be 0.
static int check_ve_table(const char* fn, const void* ve, const int* ve_ids, int ve_rows, int H,
                          int D, swa::AttnShape* a) {
  if (!ve_ids) {
    if (ve_rows != 0) return fail(SWA_ERR_INVALID_ARG, "%s: ve_rows must be 0 without ve_ids", fn);
    return ok();
  }
  if (!ve) return fail(SWA_ERR_INVALID_ARG, "%s: ve_ids needs ve and gate", fn);
  SWA_TRY(check_ve_ids(fn, ve_ids, ve_rows, H, D));
  a->ve_ids = ve_ids;
  a->ve_rows = ve_rows;
  return ok();
}

int swa_fwd(const void* q, const void* k, const void* v, const void* ve, const float* gate,
            const int* ve_ids, int ve_rows, const int* doc_bounds, void* o, float* lse, int B,
            int T, int H, int D, int window, float scale, swa_dtype dtype, void* stream) {
  const char* fn = "swa_fwd";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "v", v));
  SWA_TRY(need(fn, "o", o)); SWA_TRY(need(fn, "lse", lse));
  if ((ve == nullptr) != (gate == nullptr))
    return fail(SWA_ERR_INVALID_ARG, "%s: ve and gate must be given together", fn);
  SWA_TRY(opt(fn, "ve", ve)); SWA_TRY(opt(fn, "doc_bounds", doc_bounds));
  swa::AttnShape a{B, T, H, D, 0, scale};
  a.bounds = doc_bounds;
  SWA_TRY(check_ve_table(fn, ve, ve_ids, ve_rows, H, D, &a));
  SWA_TRY(check_window_scale(fn, window, scale, T, &a.window));
  return hip_status(swa::launch_fwd(a, q, k, v, ve, gate, o, lse, dtype == SWA_BF16,
                                    (hipStream_t)stream), fn);
}

int swa_fwd_qnorm(const void* q, const float* cos_sin, float eps, const void* k, const void* v,
                  const void* ve, const float* gate, const int* ve_ids, int ve_rows,
                  const int* doc_bounds, void* qn, void* o, float* lse, int B, int T, int H, int D,
                  int window, float scale, swa_dtype dtype, void* stream) {
  const char* fn = "swa_fwd_qnorm";
  if (dtype != SWA_BF16)
    return fail(SWA_ERR_UNSUPPORTED, "%s: the fused query prologue is bfloat16 only", fn);
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "cos_sin", cos_sin)); SWA_TRY(need(fn, "k", k));
  SWA_TRY(need(fn, "v", v)); SWA_TRY(need(fn, "qn", qn)); SWA_TRY(need(fn, "o", o));
  SWA_TRY(need(fn, "lse", lse));
  if (!(std::isfinite(eps) && eps >= 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  if (qn == q || qn == k || qn == v || qn == o)
    return fail(SWA_ERR_INVALID_ARG, "%s: qn may not alias q, k, v or o", fn);
  if ((ve == nullptr) != (gate == nullptr))
    return fail(SWA_ERR_INVALID_ARG, "%s: ve and gate must be given together", fn);
  SWA_TRY(opt(fn, "ve", ve)); SWA_TRY(opt(fn, "doc_bounds", doc_bounds));
  swa::AttnShape a{B, T, H, D, 0, scale};
  a.bounds = doc_bounds;
  SWA_TRY(check_ve_table(fn, ve, ve_ids, ve_rows, H, D, &a));
  SWA_TRY(check_window_scale(fn, window, scale, T, &a.window));
  const swa::QNorm qnorm{q, cos_sin, eps, qn};
  return hip_status(swa::launch_fwd(a, nullptr, k, v, ve, gate, o, lse, true,
                                    (hipStream_t)stream, &qnorm), fn);
}

size_t swa_bwd_workspace_size(int B, int T, int H, int D, swa_dtype dtype) {
  if (B < 1 || T < 1 || H < 1 || (D != 64 && D != 128)) return 0;
  return swa::bwd_workspace_bytes(B, T, H, D, dtype == SWA_BF16);
}

// Every argument of a backward call except the workspace.
static int check_bwd_args(const char* fn, const void* q, const void* k, const void* v,
                          const void* ve, const float* gate, const int* ve_ids, int ve_rows,
                          const int* doc_bounds, const void* o, const float* lse, const void* dO,
                          const void* dq, const void* dk, const void* dv, const void* dve,
                          const float* dgate, int B, int T, int H, int D, int window, float scale,
                          swa_dtype dtype, swa::AttnShape* a) {
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "v", v));
  if (o) SWA_TRY(need(fn, "o", o));
  SWA_TRY(need(fn, "lse", lse)); SWA_TRY(need(fn, "dO", dO));
  SWA_TRY(need(fn, "dq", dq)); SWA_TRY(need(fn, "dk", dk)); SWA_TRY(need(fn, "dv", dv));
  const bool g = gate != nullptr;
  if ((ve != nullptr) != g)
    return fail(SWA_ERR_INVALID_ARG, "%s: ve and gate must be given together", fn);
  if (g != (dve != nullptr) || g != (dgate != nullptr))
    return fail(SWA_ERR_INVALID_ARG, "%s: dve and dgate are required with the gate, NULL without", fn);
  SWA_TRY(opt(fn, "ve", ve)); SWA_TRY(opt(fn, "dve", dve));
  SWA_TRY(opt(fn, "doc_bounds", doc_bounds));
  *a = swa::AttnShape{B, T, H, D, 0, scale};
  a->bounds = doc_bounds;
  SWA_TRY(check_ve_table(fn, ve, ve_ids, ve_rows, H, D, a));
  return check_window_scale(fn, window, scale, T, &a->window);
}

static int check_bwd(const char* fn, const void* q, const void* k, const void* v, const void* ve,
                     const float* gate, const int* ve_ids, int ve_rows, const int* doc_bounds,
                     const void* o, const float* lse, const void* dO,
                     const void* dq, const void* dk, const void* dv, const void* dve,
                     const float* dgate, const void* workspace, size_t ws_bytes, int B, int T,
                     int H, int D, int window, float scale, swa_dtype dtype, swa::AttnShape* a) {
  SWA_TRY(check_bwd_args(fn, q, k, v, ve, gate, ve_ids, ve_rows, doc_bounds, o, lse, dO, dq, dk,
                         dv, dve, dgate, B, T, H, D, window, scale, dtype, a));
  return check_ws(fn, workspace, ws_bytes, B, T, H, D, dtype);
}

int swa_bwd(const void* q, const void* k, const void* v, const void* ve, const float* gate,
            const int* ve_ids, int ve_rows, const int* doc_bounds, const void* o, const float* lse,
            const void* dO, void* dq, void* dk, void* dv, void* dve, float* dgate, void* workspace,
            size_t ws_bytes, int B, int T, int H, int D, int window, float scale, swa_dtype dtype,
            void* stream) {
  const char* fn = "swa_bwd";
  swa::AttnShape a;
  SWA_TRY(need(fn, "o", o));
  SWA_TRY(check_bwd(fn, q, k, v, ve, gate, ve_ids, ve_rows, doc_bounds, o, lse, dO, dq, dk, dv, dve,
                    dgate, workspace, ws_bytes, B, T, H, D, window, scale, dtype, &a));
  const bool bf = dtype == SWA_BF16;
  const hipStream_t s = (hipStream_t)stream;
  // dQ first: it also writes the row terms that the key-major dK/dV kernel reads
  hipError_t e = swa::launch_bwd_dq_rowterms(a, q, k, v, ve, gate, o, lse, dO, dq, workspace, bf, s);
  if (e == hipSuccess)
    e = swa::launch_bwd_dkdv(a, q, k, v, ve, gate, lse, dO, dk, dv, dve, dgate, workspace, bf, s);
  return hip_status(e, fn);
}

size_t swa_bwd_ds_workspace_size(int B, int T, int H, int D, int window, swa_dtype dtype) {
  if (B < 1 || T < 1 || H < 1 || (D != 64 && D != 128)) return 0;
  if (window == 0 || window < SWA_WINDOW_FULL) return 0;
  const int W = (window == SWA_WINDOW_FULL || window > T) ? T : window;
  return ds_ws_bytes(B, T, H, D, W, dtype);
}

int swa_bwd_ds(const void* q, const void* k, const void* v, const void* ve, const float* gate,
               const int* ve_ids, int ve_rows, const int* doc_bounds, const void* o,
               const float* lse, const void* dO, void* dq, void* dk, void* dv, void* dve,
               float* dgate, void* workspace, size_t ws_bytes, int B, int T, int H, int D,
               int window, float scale, swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_ds";
  swa::AttnShape a;
  SWA_TRY(need(fn, "o", o));
  SWA_TRY(check_bwd_args(fn, q, k, v, ve, gate, ve_ids, ve_rows, doc_bounds, o, lse, dO, dq, dk,
                         dv, dve, dgate, B, T, H, D, window, scale, dtype, &a));
  SWA_TRY(check_ws_ds(fn, workspace, ws_bytes, B, T, H, D, a.window, dtype));
  const bool bf = dtype == SWA_BF16;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (!bf) {
    // float32: the recomputing kernels (no dS is stored)
    e = swa::launch_bwd_dq_rowterms(a, q, k, v, ve, gate, o, lse, dO, dq, workspace, bf, s);
    if (e == hipSuccess)
      e = swa::launch_bwd_dkdv(a, q, k, v, ve, gate, lse, dO, dk, dv, dve, dgate, workspace, bf, s);
    return hip_status(e, fn);
  }
  void* ds = ds_part(workspace, B, T, H, D, dtype);
  e = swa::launch_bwd_pre(a, o, dO, lse, workspace, bf, s);
  if (e == hipSuccess)
    e = swa::launch_bwd_dkdv(a, q, k, v, ve, gate, lse, dO, dk, dv, dve, dgate, workspace, bf, s,
                             ds);
  if (e == hipSuccess) e = swa::launch_dq_from_ds(a, k, ds, dq, s);
  return hip_status(e, fn);
}

int swa_bwd_dkdv_ds(const void* q, const void* k, const void* v, const void* ve,
                    const float* gate, const int* ve_ids, int ve_rows, const int* doc_bounds,
                    const float* lse, const void* dO, void* dk, void* dv, void* dve, float* dgate,
                    void* workspace, size_t ws_bytes, int B, int T, int H, int D, int window,
                    float scale, swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_dkdv_ds";
  swa::AttnShape a;
  if (dtype != SWA_BF16)
    return fail(SWA_ERR_UNSUPPORTED, "%s: the stored-dS stages are bfloat16 only", fn);
  // dq is not used by this stage; dk stands in for it in the shared checks
  SWA_TRY(check_bwd_args(fn, q, k, v, ve, gate, ve_ids, ve_rows, doc_bounds, nullptr, lse, dO, dk,
                         dk, dv, dve, dgate, B, T, H, D, window, scale, dtype, &a));
  SWA_TRY(check_ws_ds(fn, workspace, ws_bytes, B, T, H, D, a.window, dtype));
  return hip_status(swa::launch_bwd_dkdv(a, q, k, v, ve, gate, lse, dO, dk, dv, dve, dgate,
                                         workspace, true, (hipStream_t)stream,
                                         ds_part(workspace, B, T, H, D, dtype)), fn);
}

int swa_bwd_dq_ds(const void* k, const int* doc_bounds, void* dq, void* workspace,
                  size_t ws_bytes, int B, int T, int H, int D, int window, float scale,
                  swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_dq_ds";
  if (dtype != SWA_BF16)
    return fail(SWA_ERR_UNSUPPORTED, "%s: the stored-dS stages are bfloat16 only", fn);
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "dq", dq));
  SWA_TRY(opt(fn, "doc_bounds", doc_bounds));
  swa::AttnShape a{B, T, H, D, 0, scale};
  a.bounds = doc_bounds;
  SWA_TRY(check_window_scale(fn, window, scale, T, &a.window));
  SWA_TRY(check_ws_ds(fn, workspace, ws_bytes, B, T, H, D, a.window, dtype));
  return hip_status(swa::launch_dq_from_ds(a, k, ds_part(workspace, B, T, H, D, dtype), dq,
                                           (hipStream_t)stream), fn);
}

int swa_bwd_dq_ds_qnorm(const void* k, const int* doc_bounds, const void* q,
                        const float* cos_sin, float eps, void* dq, void* workspace,
                        size_t ws_bytes, int B, int T, int H, int D, int window, float scale,
                        swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_dq_ds_qnorm";
  if (dtype != SWA_BF16)
    return fail(SWA_ERR_UNSUPPORTED, "%s: the stored-dS stages are bfloat16 only", fn);
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "cos_sin", cos_sin));
  SWA_TRY(need(fn, "dq", dq));
  SWA_TRY(opt(fn, "doc_bounds", doc_bounds));
  if (!(std::isfinite(eps) && eps >= 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  if (dq == q || dq == k) return fail(SWA_ERR_INVALID_ARG, "%s: dq may not alias q or k", fn);
  swa::AttnShape a{B, T, H, D, 0, scale};
  a.bounds = doc_bounds;
  SWA_TRY(check_window_scale(fn, window, scale, T, &a.window));
  SWA_TRY(check_ws_ds(fn, workspace, ws_bytes, B, T, H, D, a.window, dtype));
  const swa::QNorm qnorm{q, cos_sin, eps, nullptr};
  return hip_status(swa::launch_dq_from_ds(a, k, ds_part(workspace, B, T, H, D, dtype), dq,
                                           (hipStream_t)stream, &qnorm), fn);
}

int swa_bwd_preprocess(const void* o, const void* dO, const float* lse, void* workspace,
                       size_t ws_bytes, int B, int T, int H, int D, swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_preprocess";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "o", o)); SWA_TRY(need(fn, "dO", dO)); SWA_TRY(need(fn, "lse", lse));
  SWA_TRY(check_ws(fn, workspace, ws_bytes, B, T, H, D, dtype));
  swa::AttnShape a{B, T, H, D, T, 1.f};
  return hip_status(swa::launch_bwd_pre(a, o, dO, lse, workspace, dtype == SWA_BF16, (hipStream_t)stream), fn);
}

int swa_bwd_dkdv(const void* q, const void* k, const void* v, const void* ve, const float* gate,
                 const int* ve_ids, int ve_rows, const int* doc_bounds, const float* lse,
                 const void* dO, void* dk, void* dv, void* dve, float* dgate, void* workspace,
                 size_t ws_bytes, int B, int T, int H, int D, int window, float scale,
                 swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_dkdv";
  swa::AttnShape a;
  // dq is not used by this stage; dk stands in for it in the shared checks
  SWA_TRY(check_bwd(fn, q, k, v, ve, gate, ve_ids, ve_rows, doc_bounds, nullptr, lse, dO, dk, dk, dv,
                    dve, dgate, workspace, ws_bytes, B, T, H, D, window, scale, dtype, &a));
  return hip_status(swa::launch_bwd_dkdv(a, q, k, v, ve, gate, lse, dO, dk, dv, dve, dgate,
                                         workspace, dtype == SWA_BF16, (hipStream_t)stream), fn);
}

int swa_bwd_dq(const void* q, const void* k, const void* v, const void* ve, const float* gate,
               const int* ve_ids, int ve_rows, const int* doc_bounds, const float* lse,
               const void* dO, void* dq, void* workspace, size_t ws_bytes, int B, int T, int H,
               int D, int window, float scale, swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_dq";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "v", v));
  SWA_TRY(need(fn, "lse", lse)); SWA_TRY(need(fn, "dO", dO)); SWA_TRY(need(fn, "dq", dq));
  if ((ve != nullptr) != (gate != nullptr))
    return fail(SWA_ERR_INVALID_ARG, "%s: ve and gate must be given together", fn);
  SWA_TRY(opt(fn, "ve", ve)); SWA_TRY(opt(fn, "doc_bounds", doc_bounds));
  swa::AttnShape a{B, T, H, D, 0, scale};
  a.bounds = doc_bounds;
  SWA_TRY(check_ve_table(fn, ve, ve_ids, ve_rows, H, D, &a));
  SWA_TRY(check_window_scale(fn, window, scale, T, &a.window));
  SWA_TRY(check_ws(fn, workspace, ws_bytes, B, T, H, D, dtype));
  return hip_status(swa::launch_bwd_dq(a, q, k, v, ve, gate, lse, dO, dq, workspace,
                                       dtype == SWA_BF16, (hipStream_t)stream), fn);
}

int swa_bwd_dq_rowterms(const void* q, const void* k, const void* v, const void* ve,
                        const float* gate, const int* ve_ids, int ve_rows, const int* doc_bounds,
                        const void* o, const float* lse, const void* dO, void* dq,
                        void* workspace, size_t ws_bytes, int B, int T, int H, int D, int window,
                        float scale, swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_dq_rowterms";
  swa::AttnShape a;
  SWA_TRY(need(fn, "o", o));
  // dk, dv, dve, dgate are not used by this stage; dq and lse stand in for them in the shared
  // checks
  SWA_TRY(check_bwd(fn, q, k, v, ve, gate, ve_ids, ve_rows, doc_bounds, o, lse, dO, dq, dq, dq,
                    gate ? dq : nullptr, gate ? lse : nullptr, workspace, ws_bytes, B, T, H, D,
                    window, scale, dtype, &a));
  return hip_status(swa::launch_bwd_dq_rowterms(a, q, k, v, ve, gate, o, lse, dO, dq, workspace,
                                                dtype == SWA_BF16, (hipStream_t)stream), fn);
}

// ---- fp8 forward variant

static int check_fp8_scale(const char* fn, const char* name, float s) {
  if (!(std::isfinite(s) && s > 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: %s must be finite and > 0", fn, name);
  if (!std::isfinite(1.0f / s))
    return fail(SWA_ERR_INVALID_ARG, "%s: 1/%s is not finite", fn, name);
  return ok();
}

int rope_qknorm_fwd_fp8(const void* q, const void* k, const float* cos_sin, void* q8, void* k8,
                        int B, int T, int H, int D, float eps, swa_dtype dtype, void* stream) {
  const char* fn = "rope_qknorm_fwd_fp8";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "cos_sin", cos_sin));
  SWA_TRY(need(fn, "q8", q8)); SWA_TRY(need(fn, "k8", k8));
  if (!(std::isfinite(eps) && eps >= 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  return hip_status(swa::launch_rope_qknorm_fwd_fp8(q, k, cos_sin, q8, k8, B, T, H, D, eps,
                                                    dtype == SWA_BF16, (hipStream_t)stream), fn);
}

size_t swa_fp8_v_bytes(int B, int T, int H, int D) {
  if (B < 1 || T < 1 || H < 1 || (D != 64 && D != 128)) return 0;
  return swa::fp8_v_bytes(B, T, H, D);
}

int swa_fp8_pack(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                 float v_scale, void* q8, void* k8, void* v8t, int B, int T, int H, int D,
                 swa_dtype dtype, void* stream) {
  const char* fn = "swa_fp8_pack";
  SWA_TRY(check_shape(fn, B, T, H, D, dtype));
  if ((q == nullptr) != (q8 == nullptr) || (k == nullptr) != (k8 == nullptr) ||
      (v == nullptr) != (v8t == nullptr))
    return fail(SWA_ERR_INVALID_ARG, "%s: each of (q, q8), (k, k8), (v, v8t) must be both set "
                "or both NULL", fn);
  if (!q && !k && !v) return fail(SWA_ERR_INVALID_ARG, "%s: nothing to pack", fn);
  if (q) {
    SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "q8", q8));
    SWA_TRY(check_fp8_scale(fn, "q_scale", q_scale));
  }
  if (k) {
    SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "k8", k8));
    SWA_TRY(check_fp8_scale(fn, "k_scale", k_scale));
  }
  if (v) {
    SWA_TRY(need(fn, "v", v)); SWA_TRY(need(fn, "v8t", v8t));
    SWA_TRY(check_fp8_scale(fn, "v_scale", v_scale));
  }
  return hip_status(swa::launch_fp8_pack(q, k, v, 1.0f / q_scale, 1.0f / k_scale, 1.0f / v_scale,
                                         q8, k8, v8t, B, T, H, D, dtype == SWA_BF16,
                                         (hipStream_t)stream), fn);
}

int swa_fwd_fp8(const void* q8, const void* k8, const void* v8t, float q_scale, float k_scale,
                float v_scale, const int* doc_bounds, void* o, float* lse, int B, int T, int H,
                int D, int window, float scale, void* stream) {
  const char* fn = "swa_fwd_fp8";
  SWA_TRY(check_shape(fn, B, T, H, D, SWA_BF16));
  SWA_TRY(need(fn, "q8", q8)); SWA_TRY(need(fn, "k8", k8)); SWA_TRY(need(fn, "v8t", v8t));
  SWA_TRY(need(fn, "o", o)); SWA_TRY(need(fn, "lse", lse));
  SWA_TRY(opt(fn, "doc_bounds", doc_bounds));
  SWA_TRY(check_fp8_scale(fn, "q_scale", q_scale));
  SWA_TRY(check_fp8_scale(fn, "k_scale", k_scale));
  SWA_TRY(check_fp8_scale(fn, "v_scale", v_scale));
  swa::AttnShape a{B, T, H, D, 0, scale};
  a.bounds = doc_bounds;
  SWA_TRY(check_window_scale(fn, window, scale, T, &a.window));
  return hip_status(swa::launch_fwd_fp8(a, q8, k8, v8t, q_scale * k_scale, v_scale, o, lse,
                                        (hipStream_t)stream), fn);
}

// ---- sliding-window decoding from a ring K/V cache

static int check_decode_shape(const char* fn, int B, int H, int D, int cap, int dtype) {
  if (B < 1 || H < 1 || cap < 1)
    return fail(SWA_ERR_INVALID_ARG, "%s: B, H and the cache capacity must be >= 1", fn);
  if (dtype != SWA_F32 && dtype != SWA_BF16)
    return fail(SWA_ERR_INVALID_ARG, "%s: dtype must be SWA_F32 or SWA_BF16 (got %d)", fn, dtype);
  if (D != 64 && D != 128)
    return fail(SWA_ERR_UNSUPPORTED, "%s: head dim D must be 64 or 128 (got %d)", fn, D);
  if ((long long)B * cap * H * D >= (1LL << 40) || (long long)B * H >= (1LL << 24))
    return fail(SWA_ERR_UNSUPPORTED, "%s: sizes exceed the supported range", fn);
  return 0;
}

static int decode_window(const char* fn, int window, int cap, int* w_out) {
  if (window == SWA_WINDOW_FULL) window = cap;
  if (window < 1 || window > cap)
    return fail(SWA_ERR_INVALID_ARG,
                "%s: window must be in [1, cache capacity %d] or SWA_WINDOW_FULL (got %d)", fn,
                cap, window);
  *w_out = window;
  return 0;
}

int swa_decode_prologue(const void* q, const void* k, const void* v, const float* cos_sin,
                        int table_rows, const int* pos, void* qn, void* k_cache, void* v_cache,
                        int B, int H, int D, int cap, float eps, swa_dtype dtype, void* stream) {
  const char* fn = "swa_decode_prologue";
  SWA_TRY(check_decode_shape(fn, B, H, D, cap, dtype));
  SWA_TRY(need(fn, "q", q)); SWA_TRY(need(fn, "k", k)); SWA_TRY(need(fn, "v", v));
  SWA_TRY(need(fn, "cos_sin", cos_sin)); SWA_TRY(need(fn, "pos", pos)); SWA_TRY(need(fn, "qn", qn));
  SWA_TRY(need(fn, "k_cache", k_cache)); SWA_TRY(need(fn, "v_cache", v_cache));
  if (table_rows < 1) return fail(SWA_ERR_INVALID_ARG, "%s: table_rows must be >= 1", fn);
  if (!(std::isfinite(eps) && eps >= 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  return hip_status(swa::launch_decode_prologue(q, k, v, cos_sin, table_rows, pos, qn, k_cache,
                                                v_cache, B, H, D, cap, eps, dtype == SWA_BF16,
                                                (hipStream_t)stream), fn);
}

size_t swa_decode_workspace_size(int B, int H, int D, int cap, int window) {
  if (B < 1 || H < 1 || cap < 1 || (D != 64 && D != 128)) return 0;
  if (window == SWA_WINDOW_FULL) window = cap;
  if (window < 1 || window > cap) return 0;
  return swa::decode_workspace_bytes(B, H, D, window);
}

int swa_decode(const void* qn, const void* k_cache, const void* v_cache, const int* pos, void* o,
               float* lse, void* workspace, size_t ws_bytes, int B, int H, int D, int cap,
               int window, float scale, swa_dtype dtype, void* stream) {
  const char* fn = "swa_decode";
  SWA_TRY(check_decode_shape(fn, B, H, D, cap, dtype));
  SWA_TRY(need(fn, "qn", qn)); SWA_TRY(need(fn, "k_cache", k_cache));
  SWA_TRY(need(fn, "v_cache", v_cache)); SWA_TRY(need(fn, "pos", pos));
  SWA_TRY(need(fn, "o", o)); SWA_TRY(need(fn, "lse", lse));
  int w = 0;
  SWA_TRY(decode_window(fn, window, cap, &w));
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(SWA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  const size_t need_ws = swa::decode_workspace_bytes(B, H, D, w);
  if (!workspace || ws_bytes < need_ws)
    return fail(SWA_ERR_WORKSPACE, "%s: workspace of %zu bytes required (got %zu)", fn, need_ws,
                workspace ? ws_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SWA_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  return hip_status(swa::launch_decode(qn, k_cache, v_cache, pos, o, lse, workspace, B, H, D, cap,
                                       w, scale, dtype == SWA_BF16, (hipStream_t)stream), fn);
}

// ---------------------------------------------------------------------------------------------
// swa_bwd_noalloc: the backward on a scratch area inside the library's code object instead of a
// caller workspace, for callers that cannot allocate device memory. The area is a static device
// array, so each GPU the library runs on holds its own copy at its own address, resolved once
// per device with hipGetSymbolAddress and cached; host code never uses the array's name as an
// address (on the host it names a stand-in, not device memory). Nothing in it has to start at
// zero: every row term the kernels read is written earlier in the same call (the rows, then the
// zeroed slack behind them).
// ---------------------------------------------------------------------------------------------
}  // extern "C"

static __device__ __align__(256) unsigned char scratch[SWA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

// Device address of `scratch` on the current device (resolved on the first call per device).
int scratch_on_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SWA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(SWA_ERR_UNSUPPORTED, "%s: device %d beyond the %d devices the scratch table holds",
                fn, dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SWA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  e != hipSuccess ? hipGetErrorString(e) : "null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}
}  // namespace

extern "C" {

int swa_bwd_noalloc(const void* q, const void* k, const void* v, const void* ve,
                    const float* gate, const int* ve_ids, int ve_rows, const int* doc_bounds,
                    const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    void* dve, float* dgate, int B, int T, int H, int D, int window, float scale,
                    swa_dtype dtype, void* stream) {
  const char* fn = "swa_bwd_noalloc";
  swa::AttnShape a;
  SWA_TRY(need(fn, "o", o));
  SWA_TRY(check_bwd_args(fn, q, k, v, ve, gate, ve_ids, ve_rows, doc_bounds, o, lse, dO, dq, dk,
                         dv, dve, dgate, B, T, H, D, window, scale, dtype, &a));
  const bool bf = dtype == SWA_BF16;
  const size_t need_ws = swa::bwd_workspace_bytes(B, T, H, D, bf);
  if (need_ws > (size_t)SWA_NOALLOC_SCRATCH_BYTES)
    return fail(SWA_ERR_WORKSPACE,
                "%s: B*H*T = %lld rows need %zu bytes of scratch, more than the %zu bytes the "
                "library holds (SWA_NOALLOC_SCRATCH_BYTES); call swa_bwd with a workspace",
                fn, (long long)B * H * T, need_ws, (size_t)SWA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  SWA_TRY(scratch_on_current_device(fn, &ws));
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = swa::launch_bwd_dq_rowterms(a, q, k, v, ve, gate, o, lse, dO, dq, ws, bf, s);
  if (e == hipSuccess)
    e = swa::launch_bwd_dkdv(a, q, k, v, ve, gate, lse, dO, dk, dv, dve, dgate, ws, bf, s);
  return hip_status(e, fn);
}

}  // extern "C"
