/*
 * swa.h — C ABI of the MI355X (gfx950) causal sliding-window attention library (libswa.so).
 *
 * What it computes (the attention core of the nanochat / nanoGPT GPT-2 training step):
 *
 *   prologue   q_hat = RMSNorm(RoPE(q)), k_hat = RMSNorm(RoPE(k))
 *              ("从4万美元到73美元：GPT-2复现的成本革命", intelliparadigm.com, §2.2: q and k are
 *              normalised after RoPE; §2.1: the norm has no learnable gamma/beta)
 *   gate       v_eff = v + 2*sigmoid(x[:, :, :32] @ Wg) * ve   (optional; lanjinlin.com.cn
 *              repost of the same write-up, "3. Value Embeddings")
 *   attention  s_ij = scale * q_hat_i . k_hat_j for max(0, i-W+1) <= j <= i, softmax over j,
 *              O_i = sum_j P_ij v_eff_j, lse_i = log sum_j exp(s_ij)
 *              ("GPT-2 124M 复现", notes.cassieliang.com, §3: scaled dot product, causal
 *              lower-triangular mask including the diagonal, softmax over keys; §19: tiled
 *              online softmax, exact, backward by recomputation; intelliparadigm.com §3.2:
 *              per-layer windows of 1024 or 2048 tokens)
 *
 * Conventions shared by every entry point
 *   - Tensors are device pointers to contiguous arrays in the native (B, T, H, D) layout
 *     ("从4万美元到73美元" §3.1): element (b, t, h, d) at ((b*T + t)*H + h)*D + d.
 *     lse and delta are (B, H, T); gate and dgate are (B, T, H); ve is (B, T, H*D) with
 *     channel h*D + d feeding head h; x is (B, T, ldx) of which channels 0..31 are read.
 *   - Positions are 0..T-1 in every sequence b; sequences never attend to one another.
 *   - dtype selects the storage type of q, k, v, o, dO, dq, dk, dv, ve, dve, x and dx32:
 *     SWA_F32 (float) or SWA_BF16 (bfloat16). lse, gate, dgate, Wg, dWg, cos_sin and the
 *     workspace are always float32. Arithmetic is float32; the bf16 attention contractions
 *     run on bf16 MFMA with float32 accumulation.
 *   - Head dim D must be 64 or 128. window W >= 1 counts keys including the query itself;
 *     W >= T or W == SWA_WINDOW_FULL is plain causal attention.
 *   - Ownership: the caller allocates and owns every buffer, including workspaces sized by
 *     the *_workspace_size queries. The library allocates no device memory and keeps no
 *     state between calls beyond the thread-local error message.
 *   - Execution: work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and never synchronised. Outputs are valid once the stream has reached that point.
 *   - Errors: every call validates all arguments on the host before any launch and returns
 *     a swa_status; on a non-zero status nothing was enqueued (except SWA_ERR_HIP, where a
 *     launch failed) and swa_last_error() describes the problem. No C++ exception crosses
 *     the ABI. Device pointers must be 16-byte aligned (128-bit vector access).
 *   - Gradients are overwritten, never accumulated into (except the value-embedding table
 *     gradient of swa_bwd / swa_bwd_dkdv / ve_gate_dv in the table mode, see there).
 */
#ifndef SWA_H_
#define SWA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SWA_F32 = 0, SWA_BF16 = 1 } swa_dtype;

typedef enum {
  SWA_OK = 0,
  SWA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad window/scale/eps/dtype */
  SWA_ERR_UNSUPPORTED = 2, /* D not 64 or 128, sizes beyond 32-bit index range */
  SWA_ERR_ALIGN = 3,       /* a device pointer is not 16-byte aligned */
  SWA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the query returns */
  SWA_ERR_HIP = 5          /* a kernel launch failed (message has the HIP error string) */
} swa_status;

#define SWA_WINDOW_FULL (-1)
#define SWA_GATE_CHANNELS 32
/* Most heads ve_gate_v_bwd handles (its LDS staging holds 128 rows of dz per block). */
#define SWA_GATE_MAX_HEADS 64

/* Text of the last non-zero status returned on the calling thread ("" if none). */
const char* swa_last_error(void);

/* Library version string, e.g. "swa 1.0 gfx950". */
const char* swa_version(void);

/*
 * rope_table — RoPE angle table (setup; once per (T, D, base)).
 * Writes cos_sin[(t*(D/2) + i)*2 + 0] = cos(t*theta_i), [...+1] = sin(t*theta_i) with
 * theta_i = base^(-2i/D), i < D/2, t < T; angles are formed and evaluated in float64 and
 * stored as float32. The rotation convention ("NanoGPT Speedrun：大模型训练效率的极限竞速指南",
 * kongchang.com, "模型架构层面的改进": a position-dependent rotation of q and k; the pages
 * give no formula) is rotate-half: pair (i, i + D/2) turns by +t*theta_i.
 *   cos_sin: device, T*D floats, written.   T >= 1, D in {64, 128}, base > 0 finite.
 */
int rope_table(float* cos_sin, int T, int D, double base, void* stream);

/*
 * rope_qknorm_fwd — fused prologue for q and k in one launch
 * ("从4万美元到73美元" §2.2, §2.1):
 *   u = RoPE_t(x) over all D dims;  x_hat = u / sqrt(mean_d u^2 + eps).
 * The 1/sqrt(D) score scale is not applied here; swa_fwd/swa_bwd take it as `scale`.
 *   q, k   : device (B,T,H,D) dtype, read.         qn, kn: device (B,T,H,D) dtype, written.
 *   cos_sin: device table from rope_table(T, D).   eps >= 0 finite.
 * qn/kn may not alias q/k. q and qn may both be NULL: then only k is processed (for callers
 * that run the query half inside swa_fwd_qnorm).
 */
int rope_qknorm_fwd(const void* q, const void* k, const float* cos_sin, void* qn, void* kn,
                    int B, int T, int H, int D, float eps, swa_dtype dtype, void* stream);

/*
 * rope_qknorm_bwd — backward of the prologue, for q and k in one launch.
 * Recomputes u and r = (mean u^2 + eps)^(-1/2) from the raw input, then
 *   du = r * (dx_hat - x_hat * (x_hat . dx_hat) / D);   dx = RoPE_t^T(du) (rotation by -t*theta).
 *   q, k  : device (B,T,H,D) dtype, the raw pre-RoPE inputs, read.
 *   dqn, dkn: device (B,T,H,D) dtype, gradients w.r.t. q_hat, k_hat, read.
 *   dq, dk: device (B,T,H,D) dtype, written (may alias dqn/dkn).
 * q, dqn and dq may all be NULL: then only k is processed (for callers that run the query half
 * inside swa_bwd_dq_ds_qnorm).
 */
int rope_qknorm_bwd(const void* q, const void* k, const float* cos_sin, const void* dqn,
                    const void* dkn, void* dq, void* dk, int B, int T, int H, int D, float eps,
                    swa_dtype dtype, void* stream);

/*
 * ve_gate_v — value-embedding gate (lanjinlin.com.cn repost, "3. Value Embeddings"):
 *   gate[b,t,h] = 2 * sigmoid(sum_{c<32} x[b,t,c] * Wg[c,h])   (range (0, 2)).
 * Optionally materialises v_eff = v + gate * ve (pass v, ve, v_eff all non-NULL, or all
 * NULL); swa_fwd / swa_bwd then run on v_eff without the gate and ve_gate_dv closes the
 * backward. This is the faster route on MI355X; swa_fwd / swa_bwd can instead take (ve, gate)
 * and form v_eff inside their V-tile loads.
 *   x   : device (B,T,ldx) dtype, ldx >= 32 (elements), read.    Wg: device (32,H) float, read.
 *   gate: device (B,T,H) float, written.
 *   v, ve: (B,T,H,D) and (B,T,H*D) dtype, read.   v_eff: (B,T,H,D) dtype, written.
 *   ve_ids, ve_rows: NULL and 0, or the table mode as in swa_fwd: ve is a (ve_rows, H*D) table
 *   and token (b,t) reads row ve_ids[b*T + t] (an id outside [0, ve_rows): zero row).
 */
int ve_gate_v(const void* x, int ldx, const float* Wg, float* gate, const void* v,
              const void* ve, const int* ve_ids, int ve_rows, void* v_eff, int B, int T, int H,
              int D, swa_dtype dtype, void* stream);

/*
 * ve_gate_dv — backward of v_eff = v + gate * ve through ve and the gate, from
 *   dv_eff = the dv that swa_bwd returns when it ran on a materialised v_eff
 *   (lanjinlin.com.cn repost, "3. Value Embeddings"; dv itself is dv_eff):
 *   dve = gate * dv_eff;   dgate[b,t,h] = sum_d dv_eff[b,t,h,d] * ve[b,t,h*D + d].
 *   dv_eff: (B,T,H,D) dtype, read.  ve: as given to ve_gate_v.  gate: (B,T,H) float, read.
 *   dve: (B,T,H*D) dtype, written; in the table mode (ve_ids non-NULL) the table's gradient, a
 *   (ve_rows, H*D) FLOAT array ACCUMULATED into with float atomics (the caller zeroes it; its
 *   bits depend on the order of the atomics).   dgate: (B,T,H) float, written.
 */
int ve_gate_dv(const void* dv_eff, const void* ve, const int* ve_ids, int ve_rows,
               const float* gate, void* dve, float* dgate, int B, int T, int H, int D,
               swa_dtype dtype, void* stream);

/* Bytes of workspace ve_gate_v_bwd needs: 32*H float partial sums per chunk of 128 rows of the
 * B*T rows. 0 for invalid sizes (or H > SWA_GATE_MAX_HEADS). */
size_t ve_gate_v_bwd_workspace_size(int B, int T, int H);

/*
 * ve_gate_v_bwd — backward of the gate given dgate = dL/dgate (B,T,H) float (from swa_bwd
 *   or ve_gate_dv):
 *   dz = dgate * gate * (1 - gate/2);  dWg[c,h] = sum_{b,t} x[b,t,c] dz[b,t,h] (overwritten);
 *   dx32[b,t,c] = sum_h dz[b,t,h] Wg[c,h]   (optional; dx32 NULL skips it).
 * dWg is reduced in two passes with a fixed order (bitwise repeatable): partial sums of each
 * chunk of 128 rows into the workspace, then the chunks in order. H <= SWA_GATE_MAX_HEADS.
 *   dx32: device (B,T,32) dtype, written.
 *   workspace: device, >= ve_gate_v_bwd_workspace_size() bytes, 16-byte aligned, clobbered.
 */
int ve_gate_v_bwd(const void* x, int ldx, const float* Wg, const float* gate,
                  const float* dgate, float* dWg, void* dx32, void* workspace, size_t ws_bytes,
                  int B, int T, int H, swa_dtype dtype, void* stream);

/*
 * swa_doc_bounds — document segments of packed rows ("从4万美元到73美元" §6.1: BOS-aligned rows
 *   hold several documents; per-document attention is the variable-length attention that §7 of
 *   the same page, "避坑指南", lists among the ideas tried). A document is a maximal run of equal ids along a row; for each token
 *   the call writes doc_bounds[(b*T + t)*2 + 0] = first position of its run and [... + 1] = one
 *   past the last. Computed once per batch; every attention call of the step can reuse it.
 *   doc_id: device (B,T) int32, read.   doc_bounds: device (B,T,2) int32, written.
 */
int swa_doc_bounds(const int* doc_id, int* doc_bounds, int B, int T, void* stream);

/*
 * swa_fwd — causal sliding-window attention forward ("GPT-2 124M 复现" §3, §19).
 *   s_ij = scale * q_i . k_j for max(0, i-W+1) <= j <= i; lse_i = log sum_j exp(s_ij);
 *   O_i = sum_j exp(s_ij - lse_i) v_eff_j, v_eff = v (+ gate * ve when ve and gate are given).
 *   q, k, v: device (B,T,H,D) dtype (normally qn, kn from rope_qknorm_fwd), read.
 *   ve, gate: both NULL, or ve (B,T,H*D) dtype and gate (B,T,H) float, read.
 *   ve_ids, ve_rows: NULL and 0, or the value-embedding table mode (lanjinlin.com.cn repost,
 *   "3. Value Embeddings": the per-layer value embedding is a lookup of the token ids): ve is
 *   then a (ve_rows, H*D) dtype table and token (b,t) uses row ve_ids[b*T + t] (device (B,T)
 *   int32, read), gathered inside the kernels' V-row loads; an id outside [0, ve_rows) reads
 *   as a zero row. Needs ve and gate.
 *   o  : device (B,T,H,D) dtype, written.     lse: device (B,H,T) float, natural log, written.
 *   doc_bounds: NULL, or swa_doc_bounds' output for this batch: then a token also sees only
 *   keys of its own document (j >= start of i's run), on top of the causal window.
 *   scale: finite, > 0 (1/sqrt(D) for this model).
 */
int swa_fwd(const void* q, const void* k, const void* v, const void* ve, const float* gate,
            const int* ve_ids, int ve_rows, const int* doc_bounds, void* o, float* lse, int B,
            int T, int H, int D, int window, float scale, swa_dtype dtype, void* stream);

/*
 * swa_fwd_qnorm — swa_fwd with the query half of the prologue run inside the attention kernel
 *   (bfloat16 only; SWA_ERR_UNSUPPORTED for float32): each workgroup normalises its own query
 *   rows (RoPE then RMS norm, "从4万美元到73美元" §2.2, §2.1, as rope_qknorm_fwd) before its
 *   key loop, so q_hat is formed without a separate pass over q.
 *   q: device (B,T,H,D) bf16, the RAW queries, read.   cos_sin, eps: as rope_qknorm_fwd.
 *   k: the normalised keys (rope_qknorm_fwd with q = NULL).   qn: device (B,T,H,D) bf16,
 *   written: the normalised queries, bitwise what rope_qknorm_fwd writes (the backward needs
 *   them). o, lse: bitwise what swa_fwd(qn, k, ...) writes. Other arguments as swa_fwd;
 *   qn may not alias q, k, v or o.
 */
int swa_fwd_qnorm(const void* q, const float* cos_sin, float eps, const void* k, const void* v,
                  const void* ve, const float* gate, const int* ve_ids, int ve_rows,
                  const int* doc_bounds, void* qn, void* o, float* lse, int B, int T, int H, int D,
                  int window, float scale, swa_dtype dtype, void* stream);

/* Bytes of workspace swa_bwd needs: the row terms -delta and -lse*log2(e), each (B,H,T) float32,
 * 256-byte aligned inside the block and followed by 512 bytes of slack. */
size_t swa_bwd_workspace_size(int B, int T, int H, int D, swa_dtype dtype);

/*
 * swa_bwd — backward of swa_fwd with score recomputation ("GPT-2 124M 复现" §19).
 *   P = exp(s - lse); dv_eff = P^T dO; dP = dO v_eff^T; delta_i = dO_i . O_i;
 *   dS = P * (dP - delta); dq = scale dS k; dk = scale dS^T q. Outputs are bitwise repeatable.
 *   With the gate: dv = dv_eff, dve = gate * dv_eff, dgate = sum_d dv_eff * ve.
 *   q, k, v, ve, gate, ve_ids, ve_rows, doc_bounds: as given to swa_fwd.
 *   o, lse: swa_fwd's outputs.   dO: (B,T,H,D) dtype.
 *   dq, dk, dv: device (B,T,H,D) dtype, written.
 *   dve (B,T,H*D) dtype and dgate (B,T,H) float: written when the gate is used (both
 *   required then), must be NULL otherwise.
 *   In the table mode dve is instead the table's gradient, a (ve_rows, H*D) FLOAT array that
 *   is ACCUMULATED into (sum over the tokens of each id of gate * dv_eff, float atomics):
 *   the caller zeroes it (or passes a running gradient), and its bits depend on the order of
 *   the atomics (every other output stays bitwise repeatable). dgate uses the table row.
 *   workspace: device, >= swa_bwd_workspace_size() bytes, 256-byte aligned, clobbered.
 */
int swa_bwd(const void* q, const void* k, const void* v, const void* ve, const float* gate,
            const int* ve_ids, int ve_rows, const int* doc_bounds, const void* o, const float* lse,
            const void* dO, void* dq, void* dk, void* dv, void* dve, float* dgate, void* workspace,
            size_t ws_bytes, int B, int T, int H, int D, int window, float scale, swa_dtype dtype,
            void* stream);

/*
 * The backward with the score gradient stored ("GPT-2 124M 复现" §19: the backward recomputes
 * S and P from the saved row statistics; here that recomputation runs once, in the dK/dV
 * kernel, and the bf16 dS it forms for dK is kept in the workspace for dq = scale * dS k).
 * Same results as swa_bwd up to float rounding order, bitwise repeatable (no atomics).
 *
 * swa_bwd_ds_workspace_size — bytes of its workspace: swa_bwd's row terms rounded up to 256
 *   bytes, then (bf16) the dS chunks: B*H*nkb*min(nkb, (W + 126)/128 + 1) * 32 KiB with
 *   nkb = ceil(T/128) and W the window clamped to T (d24 layer, B=16, H=12, T=2048: 0.91 GB at
 *   W = 1024, 1.61 GB at W = 2048). window as in swa_bwd; 0 for invalid sizes or windows. For
 *   float32 nothing is stored and no chunk bytes are added.
 */
size_t swa_bwd_ds_workspace_size(int B, int T, int H, int D, int window, swa_dtype dtype);

/*
 * swa_bwd_ds — swa_bwd on that workspace (device, >= swa_bwd_ds_workspace_size() bytes for
 *   this window, 256-byte aligned, clobbered). bf16: row terms (as swa_bwd_preprocess), then
 *   dK/dV storing dS, then dq from the stored dS. float32: the recomputing kernels of swa_bwd.
 *   Other arguments and outputs as swa_bwd.
 */
int swa_bwd_ds(const void* q, const void* k, const void* v, const void* ve, const float* gate,
               const int* ve_ids, int ve_rows, const int* doc_bounds, const void* o,
               const float* lse, const void* dO, void* dq, void* dk, void* dv, void* dve,
               float* dgate, void* workspace, size_t ws_bytes, int B, int T, int H, int D,
               int window, float scale, swa_dtype dtype, void* stream);

/*
 * Stages of swa_bwd_ds (bfloat16 only; SWA_ERR_UNSUPPORTED for float32), one workspace sized by
 * swa_bwd_ds_workspace_size for the same sizes and window, in this order on one stream:
 *   swa_bwd_preprocess (the row terms; it uses the first swa_bwd_workspace_size bytes),
 *   swa_bwd_dkdv_ds — swa_bwd_dkdv that also stores dS (arguments as swa_bwd_dkdv),
 *   swa_bwd_dq_ds   — dq = scale * dS k from the stored dS: k (B,T,H,D) bf16 read, doc_bounds
 *                     as given to the other stages (NULL or the same), dq (B,T,H,D) written.
 */
int swa_bwd_dkdv_ds(const void* q, const void* k, const void* v, const void* ve,
                    const float* gate, const int* ve_ids, int ve_rows, const int* doc_bounds,
                    const float* lse, const void* dO, void* dk, void* dv, void* dve, float* dgate,
                    void* workspace, size_t ws_bytes, int B, int T, int H, int D, int window,
                    float scale, swa_dtype dtype, void* stream);
int swa_bwd_dq_ds(const void* k, const int* doc_bounds, void* dq, void* workspace,
                  size_t ws_bytes, int B, int T, int H, int D, int window, float scale,
                  swa_dtype dtype, void* stream);

/*
 * swa_bwd_dq_ds_qnorm — swa_bwd_dq_ds followed, inside the same kernel, by the query half of
 *   the prologue's backward (rope_qknorm_bwd): each workgroup turns its dq_hat rows (rounded
 *   to bf16 as swa_bwd_dq_ds stores them) into the gradient w.r.t. the raw queries.
 *   q: device (B,T,H,D) bf16, the RAW queries, read.   cos_sin, eps: as rope_qknorm_bwd.
 *   dq: device (B,T,H,D) bf16, written: bitwise what rope_qknorm_bwd computes for q from
 *   swa_bwd_dq_ds's output. dq may not alias q or k. Other arguments as swa_bwd_dq_ds.
 */
int swa_bwd_dq_ds_qnorm(const void* k, const int* doc_bounds, const void* q,
                        const float* cos_sin, float eps, void* dq, void* workspace,
                        size_t ws_bytes, int B, int T, int H, int D, int window, float scale,
                        swa_dtype dtype, void* stream);

/* Bytes of device scratch that swa_bwd_noalloc holds per GPU (its largest workspace). */
#define SWA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * swa_bwd_noalloc — swa_bwd for callers that cannot allocate device memory: code being captured
 *   into a HIP graph, tight serving loops, harnesses that forbid allocation. Same arguments,
 *   kernels and results as swa_bwd (bitwise), without workspace and ws_bytes: the row terms go
 *   to a static device array inside the library (SWA_NOALLOC_SCRATCH_BYTES per GPU, held until
 *   the process ends), so B*H*T is limited to the sizes whose swa_bwd_workspace_size() fits it
 *   (B*H*T <= 2,097,024 rows); larger sizes return SWA_ERR_WORKSPACE before anything is
 *   enqueued. The call allocates nothing; its first call on a device resolves the array's
 *   address there (hipGetSymbolAddress) with that device current, so call it with the
 *   stream's device current. Every call on one GPU shares that GPU's array: calls that can
 *   overlap on one GPU (other streams, other host threads) race and must be ordered by the
 *   caller; calls in order on one stream are safe. Nothing in the array needs to start at zero.
 */
int swa_bwd_noalloc(const void* q, const void* k, const void* v, const void* ve,
                    const float* gate, const int* ve_ids, int ve_rows, const int* doc_bounds,
                    const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    void* dve, float* dgate, int B, int T, int H, int D, int window, float scale,
                    swa_dtype dtype, void* stream);

/*
 * The stages of the backward, for callers that schedule or time them separately. Both orders
 * give the same results up to the rounding of delta (the one-call swa_bwd runs the first):
 *   (1) swa_bwd_dq_rowterms, then swa_bwd_dkdv;
 *   (2) swa_bwd_preprocess, then swa_bwd_dkdv and swa_bwd_dq in either order.
 * One stream, one workspace, the same sizes and dtype throughout.
 *
 * swa_bwd_preprocess — the row terms -delta_i = -dO_i . O_i and -lse_i * log2(e) into the
 *   workspace (stored negated: the bf16 kernels start their accumulators from them).
 */
int swa_bwd_preprocess(const void* o, const void* dO, const float* lse, void* workspace,
                       size_t ws_bytes, int B, int T, int H, int D, swa_dtype dtype, void* stream);

/*
 * swa_bwd_dkdv — the key-block-major part of the recomputing backward (arguments as swa_bwd,
 *   without o and dq): writes dk, dv (and dve, dgate with the gate). Needs the workspace
 *   filled by swa_bwd_preprocess or swa_bwd_dq_rowterms.
 */
int swa_bwd_dkdv(const void* q, const void* k, const void* v, const void* ve, const float* gate,
                 const int* ve_ids, int ve_rows, const int* doc_bounds, const float* lse,
                 const void* dO, void* dk, void* dv, void* dve, float* dgate, void* workspace,
                 size_t ws_bytes, int B, int T, int H, int D, int window, float scale,
                 swa_dtype dtype, void* stream);

/*
 * swa_bwd_dq — the query-block-major part: recomputes the scores per query block and writes
 *   dq = scale * dS k directly (no atomics; bitwise repeatable). Needs the workspace filled by
 *   swa_bwd_preprocess. May run before, after or concurrently with swa_bwd_dkdv.
 */
int swa_bwd_dq(const void* q, const void* k, const void* v, const void* ve, const float* gate,
               const int* ve_ids, int ve_rows, const int* doc_bounds, const float* lse,
               const void* dO, void* dq, void* workspace, size_t ws_bytes, int B, int T, int H,
               int D, int window, float scale, swa_dtype dtype, void* stream);

/*
 * swa_bwd_dq_rowterms — swa_bwd_dq that computes the row terms itself from o, lse and dO (the
 *   bf16 kernel: in its prologue, from the dO row it already holds and the O row) and stores
 *   them in the workspace for a following swa_bwd_dkdv, in place of swa_bwd_preprocess.
 *   Arguments as swa_bwd without dk, dv, dve, dgate.
 */
int swa_bwd_dq_rowterms(const void* q, const void* k, const void* v, const void* ve,
                        const float* gate, const int* ve_ids, int ve_rows, const int* doc_bounds,
                        const void* o, const float* lse, const void* dO, void* dq,
                        void* workspace, size_t ws_bytes, int B, int T, int H, int D, int window,
                        float scale, swa_dtype dtype, void* stream);

/*
 * Sliding-window decoding from a K/V cache ("GPT-2 124M 复现" §7: generation that keeps the
 * past keys and values instead of recomputing every prefix position). One new token per
 * sequence b at position pos[b] >= 0; a decoding step computes row pos[b] of the training
 * forward. The cache of a sequence is a ring of `cap` slots in the native layout
 * (B, cap, H, D): position j lives in slot j mod cap, so cap >= the longest context means no
 * wrap, and cap >= window suffices for a sliding window.
 */

/*
 * fp8 forward variant ("NanoGPT Speedrun：大模型训练效率的极限竞速指南", kongchang.com, section
 * "工程与硬件优化", its paragraph on bf16 and fp8: fp8 can double matrix throughput over bf16
 * and needs finer calibration (scales) to stay accurate).
 * Format: OCP e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
 * infinities, largest finite 448, S.1111.111 = NaN), the format gfx950's fp8 MFMA reads.
 * Calibration: one float32 scale per tensor, x ~= scale * e4m3 value.
 *
 * swa_fp8_v_bytes — bytes of the packed V operand: B*H*D*Tp with Tp = T rounded up to 64.
 */
size_t swa_fp8_v_bytes(int B, int T, int H, int D);

/*
 * swa_fp8_pack — quantise q, k, v (dtype, (B,T,H,D), normally q_hat, k_hat from
 *   rope_qknorm_fwd and v or v_eff) to e4m3 codes of x / scale: a float32 multiply by the
 *   float32 reciprocal of the scale, then round to nearest even, saturating finite values
 *   beyond 448 (and infinities) to +-448; NaN stays NaN. Each pair (q, q8), (k, k8), (v, v8t)
 *   is either both set or both NULL (at least one set).
 *   q8, k8: device (B,T,H,D) bytes, written.   v8t: device, swa_fp8_v_bytes() bytes, written:
 *   per (b, h) a D x Tp byte matrix (row d = dimension d, V transposed), in which every block
 *   of 64 keys starting at 64t stores key 64t + 32kb + 8a + 4g + c at column
 *   64t + 32g + 16kb + 4a + c (kb, g in {0,1}; a, c in 0..3): the order in which the forward
 *   kernel's probabilities leave its score accumulators. Keys >= T are 0.
 *   Scales: finite, > 0, with a finite reciprocal. q_hat and k_hat need no calibration: their
 *   entries are bounded by sqrt(D) < 448, so scale 1 keeps them in range.
 */
int swa_fp8_pack(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                 float v_scale, void* q8, void* k8, void* v8t, int B, int T, int H, int D,
                 swa_dtype dtype, void* stream);

/*
 * rope_qknorm_fwd_fp8 — rope_qknorm_fwd writing q_hat, k_hat directly as e4m3 codes at scale 1
 *   (float32 results rounded once to nearest even; every entry of a normalised row is below
 *   sqrt(D) in magnitude, so no saturation occurs). Feeds swa_fwd_fp8 (q_scale = k_scale = 1)
 *   without a separate quantisation pass. Arguments as rope_qknorm_fwd; q8, k8: device
 *   (B,T,H,D) bytes, written.
 */
int rope_qknorm_fwd_fp8(const void* q, const void* k, const float* cos_sin, void* q8, void* k8,
                        int B, int T, int H, int D, float eps, swa_dtype dtype, void* stream);

/*
 * swa_fwd_fp8 — swa_fwd on fp8 operands: s_ij = scale * q_scale * k_scale * (q8_i . k8_j) on
 *   the e4m3 values (exact products, float32 accumulation), online softmax in float32,
 *   probabilities rounded to e4m3 as the PV operand (the running reference keeps them <= 2^8),
 *   O = v_scale * sum_j P_ij v8_j / l_i in float32, stored as bf16. lse from the float32 sums.
 *   q8, k8, v8t, scales: as written by swa_fp8_pack.   doc_bounds: as for swa_fwd.
 *   o: device (B,T,H,D) bf16, written.   lse: device (B,H,T) float, natural log, written.
 *   Forward only: the backward of this variant is not provided.
 */
int swa_fwd_fp8(const void* q8, const void* k8, const void* v8t, float q_scale, float k_scale,
                float v_scale, const int* doc_bounds, void* o, float* lse, int B, int T, int H,
                int D, int window, float scale, void* stream);

/*
 * swa_decode_prologue — RoPE at angle pos[b] * theta_i and the RMS QK-norm of the new q and k
 *   (as rope_qknorm_fwd at row pos[b]); writes qn and stores the normalised k and the raw v in
 *   slot pos[b] mod cap of the caches.
 *   q, k, v: device (B,H,D) dtype, read.   qn: device (B,H,D) dtype, written.
 *   cos_sin: rope_table(table_rows, D) output; positions outside [0, table_rows) give NaN in qn
 *   and leave the caches untouched.   pos: device (B) int32, read.
 *   k_cache, v_cache: device (B,cap,H,D) dtype, one slot per sequence written.
 */
int swa_decode_prologue(const void* q, const void* k, const void* v, const float* cos_sin,
                        int table_rows, const int* pos, void* qn, void* k_cache, void* v_cache,
                        int B, int H, int D, int cap, float eps, swa_dtype dtype, void* stream);

/* Bytes of workspace swa_decode needs for these sizes (0 for invalid arguments). */
size_t swa_decode_workspace_size(int B, int H, int D, int cap, int window);

/*
 * swa_decode — the new query of each sequence attends to positions max(0, p-W+1) .. p of its
 *   cache (p = pos[b]); o (B,H,D) dtype and lse (B,H) float (natural log) are written.
 *   window: 1 <= W <= cap, or SWA_WINDOW_FULL (= cap).   scale: finite, > 0.
 *   pos[b] < 0 gives NaN for that sequence. workspace: >= swa_decode_workspace_size() bytes,
 *   256-byte aligned, clobbered.
 */
int swa_decode(const void* qn, const void* k_cache, const void* v_cache, const int* pos, void* o,
               float* lse, void* workspace, size_t ws_bytes, int B, int H, int D, int cap,
               int window, float scale, swa_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H_ */
