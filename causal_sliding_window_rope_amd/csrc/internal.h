// Host-side launchers of the libswa kernels (called by the C ABI in api.hip after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace swa {

struct AttnShape {
  int B, T, H, D;
  int window;   // already clamped: 1 <= window <= T
  float scale;
  const int* bounds = nullptr;   // optional per-token document [start, end), (B, T, 2) int32
  // optional value-embedding table: ve is then (ve_rows, H*D) and token (b, t) uses row
  // ve_ids[b*T + t]; the backward then adds gate * dv into a float (ve_rows, H*D) gradient
  const int* ve_ids = nullptr;
  int ve_rows = 0;
};

// The query half of the RoPE -> RMS QK-norm prologue run inside an attention kernel: q is the
// raw (B,T,H,D) input, cs the rope_table angles, eps the norm's epsilon; qn (the forward) is
// where the normalised rows go.
struct QNorm {
  const void* q;
  const float* cs;
  float eps;
  void* qn;
};

// Longest-first block order for small full-causal grids. With window >= T the work of a block
// grows with its position along the sequence, and a grid of a few workgroups per slot ends on a
// long tail when the blocks of one head are issued together. When the per-head tiles that the
// blocks re-read (2 D-wide bf16 rows per position) of all heads an XCD holds fit in its 4 MiB
// L2, the kernels instead issue, on each XCD, the largest block of every head first, then the
// second largest, and so on. Larger grids keep one head's blocks together for L2 reuse.
inline bool lpt_order(const AttnShape& a) {
  const long bh = (long)a.B * a.H;
  return a.window >= a.T && a.bounds == nullptr && bh % 8 == 0 &&
         (bh / 8) * a.T * a.D * 4 <= (4l << 20);
}

hipError_t launch_doc_bounds(const int* doc_id, int* bounds, int B, int T, hipStream_t s);

hipError_t launch_rope_table(float* cos_sin, int T, int D, double base, hipStream_t s);
hipError_t launch_rope_qknorm_fwd(const void* q, const void* k, const float* cs, void* qn, void* kn,
                                  int B, int T, int H, int D, float eps, bool bf16, hipStream_t s);
hipError_t launch_rope_qknorm_bwd(const void* q, const void* k, const float* cs, const void* dqn,
                                  const void* dkn, void* dq, void* dk, int B, int T, int H, int D,
                                  float eps, bool bf16, hipStream_t s);

hipError_t launch_ve_gate(const void* x, int ldx, const float* Wg, float* gate, const void* v,
                          const void* ve, const int* ids, int ve_rows, void* v_eff, int B, int T,
                          int H, int D, bool bf16, hipStream_t s);
hipError_t launch_ve_gate_dv(const void* dv, const void* ve, const int* ids, int ve_rows,
                             const float* gate, void* dve, float* dgate, int B, int T, int H,
                             int D, bool bf16, hipStream_t s);
hipError_t launch_rope_qknorm_fwd_fp8(const void* q, const void* k, const float* cs, void* q8,
                                      void* k8, int B, int T, int H, int D, float eps, bool bf16,
                                      hipStream_t s);
size_t fp8_v_bytes(int B, int T, int H, int D);
hipError_t launch_fp8_pack(const void* q, const void* k, const void* v, float q_inv, float k_inv,
                           float v_inv, void* q8, void* k8, void* v8t, int B, int T, int H,
                           int D, bool bf16, hipStream_t s);
hipError_t launch_fwd_fp8(const AttnShape& a, const void* q8, const void* k8, const void* v8t,
                          float qk_scale, float v_scale, void* o, float* lse, hipStream_t s);
size_t gate_bwd_workspace_bytes(int B, int T, int H);
hipError_t launch_ve_gate_bwd(const void* x, int ldx, const float* Wg, const float* gate,
                              const float* dgate, float* dWg, void* dx32, void* ws, int B, int T,
                              int H, bool bf16, hipStream_t s);

// qnorm: NULL, or (bf16 only) q is ignored and the kernel normalises the raw rows qnorm->q
// itself, writing them to qnorm->qn (bitwise what rope_qknorm_fwd writes).
hipError_t launch_fwd(const AttnShape& a, const void* q, const void* k, const void* v,
                      const void* ve, const float* gate, void* o, float* lse, bool bf16,
                      hipStream_t s, const QNorm* qnorm = nullptr);

size_t bwd_workspace_bytes(int B, int T, int H, int D, bool bf16);
// Backward in three stages on one workspace: row terms (-delta, -lse*log2e), dK/dV (key-block
// major), dQ (query-block major).
hipError_t launch_bwd_pre(const AttnShape& a, const void* o, const void* dO, const float* lse,
                          void* ws, bool bf16, hipStream_t s);
// ds: nullptr, or (bf16 only) the dS^T buffer of dsbuf.h, which the kernel then also fills.
hipError_t launch_bwd_dkdv(const AttnShape& a, const void* q, const void* k, const void* v,
                           const void* ve, const float* gate, const float* lse, const void* dO,
                           void* dk, void* dv, void* dve, float* dgate, void* ws, bool bf16,
                           hipStream_t s, void* ds = nullptr);
// dq = scale * dS K from the dS^T buffer the dK/dV kernel stored (bf16 only).
size_t ds_buffer_bytes(int B, int T, int H, int window);
// qnorm: NULL, or dq is the gradient w.r.t. the raw rows qnorm->q (the query prologue's
// backward applied to this kernel's bf16 dq_hat, bitwise what rope_qknorm_bwd gives).
hipError_t launch_dq_from_ds(const AttnShape& a, const void* k, const void* ds, void* dq,
                             hipStream_t s,
                             const QNorm* qnorm = nullptr);
hipError_t launch_bwd_dq(const AttnShape& a, const void* q, const void* k, const void* v,
                         const void* ve, const float* gate, const float* lse, const void* dO,
                         void* dq, void* ws, bool bf16, hipStream_t s);
// dQ that also computes the row terms from O, dO and lse and stores them in the workspace
// (bf16: inside the dQ kernel; float32: the preprocess kernel, then dQ).
hipError_t launch_bwd_dq_rowterms(const AttnShape& a, const void* q, const void* k,
                                  const void* v, const void* ve, const float* gate,
                                  const void* o, const float* lse, const void* dO, void* dq,
                                  void* ws, bool bf16, hipStream_t s);
hipError_t launch_dq_bf16(const AttnShape& a, const void* q, const void* k, const void* v,
                          const void* ve, const float* gate, const void* dO, float* nlse2,
                          float* ndelta, const void* o, const float* lse, void* dq,
                          hipStream_t s);

// Sliding-window decoding from a ring K/V cache (one new token per sequence).
int decode_splits(int B, int H, int window);
size_t decode_workspace_bytes(int B, int H, int D, int window);
hipError_t launch_decode_prologue(const void* q, const void* k, const void* v, const float* cs,
                                  int rows, const int* pos, void* qn, void* kc, void* vc, int B,
                                  int H, int D, int cap, float eps, bool bf16, hipStream_t s);
hipError_t launch_decode(const void* qn, const void* kc, const void* vc, const int* pos, void* o,
                         float* lse, void* ws, int B, int H, int D, int cap, int window,
                         float scale, bool bf16, hipStream_t s);

}  // namespace swa
