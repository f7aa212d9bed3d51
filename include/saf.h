/*
 * saf.h -- C ABI of libsaf.so: the fused mixed-head causal attention layer of Selective Attention
 * Freezing (SAF) on AMD Instinct MI355X (gfx950).
 *
 * Citations name the page and the section / equation / table on it:
 *   [Notes]      "When Can Attention Heads Be Statically Defined?：中文精读笔记" (close-reading notes
 *                on arXiv 2609.34650v1).
 *   [Paper page] "When Can Attention Heads Be Statically Defined?" (abstract, captions, tables).
 *
 * The layer ([Notes §二.4, Fig. 2]): per layer, some heads are "replaced".  An ordinary head computes
 *     O = softmax_causal(s Q K^T) V,  s = 1/sqrt(d) by default                        [Notes §一]
 * A replaced head has no query or key; its fixed causal pattern is rebuilt from two length-T
 * vectors, an absolute-position preference a and a relative-distance preference r,
 *     P(i,j) = exp(a[j] + r[i-j]) / Z(i)  for j <= i,  0 for j > i,
 *     Z(i)   = sum_{k<=i} exp(a[k] + r[i-k])                         [Notes §二.3, Eq.(3)]
 * (0-based: a[j] is the preference for key position j, r[delta] for distance delta = i - j) and
 * mixes the current values: O = P V.  Both kinds run in one launch.  In the backward pass an
 * ordinary head gets the full softmax gradient (dQ, dK, dV); a replaced head only dV = P^T dO,
 * because a and r are frozen buffers and the output does not depend on its Q or K
 * ([Notes §二.4]).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major [B][H][T][d] (batch, head, position, channel) in the element type
 *    `dt`: SAF_F32 (fp32 everywhere) or SAF_BF16 (bf16 storage, fp32 accumulation inside).  Per-row
 *    statistics (lse) are fp32 [B][H][T].  a and r are fp32 [H][pat_len] (only the rows of
 *    replaced heads are read; positions 0..T-1 of each row are used, so a pattern fitted at a
 *    longer length serves shorter inputs: row i depends on positions <= i only).
 *  - All tensor pointers are DEVICE pointers on the current HIP device, 16-byte aligned, allocated
 *    and owned by the caller.  `replaced` is a HOST array of H bytes (nonzero = replaced head).
 *  - `ws` is a caller-owned device workspace of at least the size returned by the matching
 *    *_workspace_size() call (256-byte aligned); the library never allocates device memory and
 *    holds no pointer after returning.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns without waiting;
 *    outputs are valid once the stream has completed, and inputs must stay unchanged until then.
 *  - `scale` <= 0 selects 1/sqrt(d).  It applies to ordinary heads only (a and r are logits as
 *    they stand).
 *  - Supported: d in {64, 128}; 1 <= H <= 256; T <= 65536; B >= 0.  B == 0 or T == 0 is an empty
 *    call: SAF_OK, nothing enqueued, pointers not inspected.
 *  - Errors: every call returns a status and never aborts.  Arguments are checked BEFORE any HIP
 *    call, so a call that returns SAF_ERR_INVALID_ARG or SAF_ERR_UNSUPPORTED has enqueued nothing
 *    and written nothing.  A failed launch returns SAF_ERR_HIP.  saf_last_error() gives the text
 *    of the calling thread's last non-OK status.
 *  - The Q and K slices of replaced heads are never read (they may hold anything, NaN included),
 *    nor are the a / r rows of ordinary heads.
 */
#ifndef SAF_H_
#define SAF_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAF_OK = 0,
  SAF_ERR_INVALID_ARG = 1, /* a null / misaligned pointer, a size out of range, a short workspace */
  SAF_ERR_UNSUPPORTED = 2, /* a valid request this build does not serve (d not in {64,128}, ...) */
  SAF_ERR_HIP = 3          /* a HIP launch failed; the HIP error text is in saf_last_error()     */
} saf_status;

typedef enum { SAF_F32 = 0, SAF_BF16 = 1 } saf_dtype;

/* Bytes of device workspace each call needs (0 for an empty call, SIZE_MAX if the sizes are out of
 * range).  The sizes depend on the shapes only. */
size_t saf_attn_fwd_workspace_size(int B, int H, int T, int d);
size_t saf_attn_bwd_workspace_size(int B, int H, int T, int d);
size_t saf_calibrate_workspace_size(int N, int H, int T, int d);
/* A larger backward workspace with which saf_attn_bwd / saf_attn_bwd_gqa keep the ordinary heads'
 * dS = P o (dP - delta) between their two kernels instead of forming S and dP a second time for dQ
 * (three products per entry become one).  It applies to bf16 at d = 128 without grouped key/value
 * heads (Hkv = H) and with at least one ordinary head (n_replaced < H); the extra room is
 * 2 * B * (H - n_replaced) * n32 (n32 + 1) / 2 * 1024 bytes, n32 = ceil(T / 32) (bf16 32 x 32
 * subtiles on or below the diagonal: about B * (H - n_replaced) * T^2 bytes).  Returns
 * saf_attn_bwd_workspace_size(B, H, T, d) where the path does not apply, 0 for an empty call and
 * SIZE_MAX for sizes out of range or an unknown dtype. */
size_t saf_attn_bwd_ds_workspace_size(saf_dtype dt, int B, int H, int Hkv, int T, int d, int n_replaced);

/*
 * Prepared fixed pattern (optional).                            [Notes §二.3, Eq.(3); §二.4]
 * The replaced heads' pattern is stored as a and r plus the row normaliser Z(i), which does not
 * depend on the input, so it can be formed once when a pattern is installed instead of on every
 * call.  saf_pattern_prepare fills `pattern` (device memory of saf_pattern_size(H, pat_len)
 * bytes, 256-byte aligned, caller-owned) for every position < pat_len of the replaced heads'
 * rows of a and r ([H][pat_len] fp32 device).  The result may be passed to saf_attn_fwd and
 * saf_attn_bwd with the same replaced mask, a, r and pat_len, for any T <= pat_len; it must not be
 * modified while such calls are in flight.  Errors as below; nothing is enqueued on error.
 */
size_t saf_pattern_size(int H, int pat_len);
saf_status saf_pattern_prepare(int H, const uint8_t* replaced, const float* a, const float* r,
                               int pat_len, void* pattern, size_t pattern_bytes,
                               hipStream_t stream);

/*
 * Forward of the mixed layer.                                  [Notes §二.4, Fig. 2; Eq.(3)]
 *   q, k, v : [B][H][T][d] dt     o : [B][H][T][d] dt (written)
 *   lse     : [B][H][T] fp32 (written): for an ordinary head the natural-log logsumexp of the
 *             scaled causal scores of row i; for a replaced head log Z(i) (the same for every b).
 *             The backward pass reads it back.
 *   replaced: [H] host bytes;  a, r : [H][pat_len] fp32 device, pat_len >= T.
 *   pattern : NULL, or a pattern prepared by saf_pattern_prepare for (H, replaced, a, r, pat_len);
 *             with NULL the call prepares what it needs in its workspace (for length T).
 */
saf_status saf_attn_fwd(saf_dtype dt, int B, int H, int T, int d, const void* q, const void* k,
                        const void* v, const uint8_t* replaced, const float* a, const float* r,
                        int pat_len, const void* pattern, float scale, void* o, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of the mixed layer, given dout = dL/dO and the forward's o and lse.   [Notes §二.4]
 *   ordinary head: dq, dk, dv of softmax attention;
 *   replaced head: dv = P^T dout, and dq = dk = 0 (written as zeros).  No gradient for a or r.
 *   q, k, v, o, dout : [B][H][T][d] dt;   lse : [B][H][T] fp32 as written by saf_attn_fwd for
 *   the same q, k, v, replaced, a, r, scale;   dq, dk, dv : [B][H][T][d] dt (written).
 *   pattern : as for saf_attn_fwd (NULL or prepared).
 * Two kernels follow a row-statistic pass: a key-block kernel (dK, dV) and a query-block kernel
 * (dQ).  With ws_bytes >= saf_attn_bwd_ds_workspace_size(...) for this call's shapes and number of
 * replaced heads (bf16, d = 128, Hkv = H), the key-block kernel stores dS in the workspace and the
 * query-block kernel, launched after it on `stream`, reads it (not while the overlap option below
 * is enabled); otherwise the query-block kernel forms S and dP again.  Both paths give the same
 * values up to the order of fp32 additions.
 */
saf_status saf_attn_bwd(saf_dtype dt, int B, int H, int T, int d, const void* q, const void* k,
                        const void* v, const void* o, const void* dout, const float* lse,
                        const uint8_t* replaced, const float* a, const float* r, int pat_len,
                        const void* pattern, float scale, void* dq, void* dk, void* dv, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/*
 * Grouped key/value heads (GQA): H query heads share Hkv key/value heads, query head h reading
 * K, V head h / (H / Hkv); Hkv must divide H.                  [Notes §二.4; Paper page Table 26]
 * A replaced head skips only its queries and keys of the score path: it still reads the V of its
 * group.  saf_attn_fwd / saf_attn_bwd are these calls with Hkv = H.
 *   q, o, dout, dq : [B][H][T][d] dt;   k, v, dk, dv : [B][Hkv][T][d] dt.
 *   dk, dv of a key/value head are the sums over the query heads of its group (replaced heads add
 *   to dv only; dk is zero when every head of the group is replaced).  Other arguments, the
 *   workspaces and errors are those of saf_attn_fwd / saf_attn_bwd.
 */
saf_status saf_attn_fwd_gqa(saf_dtype dt, int B, int H, int Hkv, int T, int d, const void* q,
                            const void* k, const void* v, const uint8_t* replaced, const float* a,
                            const float* r, int pat_len, const void* pattern, float scale, void* o,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t stream);
saf_status saf_attn_bwd_gqa(saf_dtype dt, int B, int H, int Hkv, int T, int d, const void* q,
                            const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, const uint8_t* replaced, const float* a,
                            const float* r, int pat_len, const void* pattern, float scale, void* dq,
                            void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * saf_attn_bwd without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Arguments,
 * results and errors are those of saf_attn_bwd (Hkv = H).  The workspace (the delta rows, and the
 * prepared pattern when `pattern` is NULL) lives in a device array owned by the library, 16 MiB
 * per device, allocated when the library is loaded and held until the process ends; the call
 * itself allocates nothing.  Shapes whose saf_attn_bwd_workspace_size exceeds 16 MiB (B*H*T*4
 * bytes of delta plus, without a prepared pattern, about 12*H*T bytes) return SAF_ERR_UNSUPPORTED
 * with nothing enqueued.  The backward-overlap option is not used on this path (its side stream
 * would be created on first use).  Every call on a device uses that device's one array: calls
 * that may run at the same time on one device (other streams, other threads) race and must be
 * ordered by the caller.  Each call writes every part of the array it reads.
 */
saf_status saf_attn_bwd_noalloc(saf_dtype dt, int B, int H, int T, int d, const void* q,
                                const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, const uint8_t* replaced, const float* a,
                                const float* r, int pat_len, const void* pattern, float scale,
                                void* dq, void* dk, void* dv, hipStream_t stream);

/*
 * Gradient with respect to the replaced heads' pattern, for a pattern that is trained instead of
 * frozen ([Paper page] Table 14, "trainable mean"; saf_attn_bwd treats a and r as frozen).
 * With P(i,j) = exp(a[j] + r[i-j]) / Z(i) on j <= i ([Notes §二.3, Eq.(3)]), G(i,j) = dout_i . v_j
 * and delta_i = dout_i . o_i:
 *   dT(i,j) = P(i,j) (G(i,j) - delta_i),  da[j] = sum_b sum_{i>=j} dT(i,j),
 *   dr[k] = sum_b sum_i dT(i, i-k).
 *   v, o, dout : [B][H][T][d] dt;  lse : [B][H][T] fp32 as written by saf_attn_fwd;
 *   replaced, a, r, pat_len, pattern : as for saf_attn_fwd.
 *   da, dr : [H][pat_len] fp32 device (written for the replaced heads' rows, summed over the
 *            batch; zeros at positions T .. pat_len-1; rows of ordinary heads are not touched).
 * The result is bitwise repeatable.  With no replaced head nothing is enqueued.
 * Workspace: saf_attn_bwd_pattern_workspace_size(B, H, T, d) bytes, 256-byte aligned.
 */
size_t saf_attn_bwd_pattern_workspace_size(int B, int H, int T, int d);
saf_status saf_attn_bwd_pattern(saf_dtype dt, int B, int H, int T, int d, const void* v,
                                const void* o, const void* dout, const float* lse,
                                const uint8_t* replaced, const float* a, const float* r, int pat_len,
                                const void* pattern, float* da, float* dr, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/*
 * Calibration statistics over N sequences.                       [Notes §二.1, Eq.(1)]
 *   q, k : [N][H][T][d] dt, the queries and keys of the N calibration sequences; the maps
 *          A^(n) = softmax_causal(s Q^(n) K^(n)T) are formed tile by tile and never stored.
 *   ahat : [H][T][T] fp32 (written): the mean map (1/N) sum_n A^(n), zeros above the diagonal.
 *   svar : [H] fp64 (written): sum_n ||A^(n) - ahat||_F^2 / ((N-1) T^2), every one of the T^2
 *          entries counted.  N >= 2.
 *   skl  : [H] fp64 (written) or NULL (not computed): the row-wise forward-KL score, the mean over
 *          sequences n and rows i of KL(A^(n)_i || ahat_i) in nats ([Notes §二.1] names this
 *          alternative selector without a formula; this is its plainest reading).
 */
saf_status saf_calibrate(saf_dtype dt, int N, int H, int T, int d, const void* q, const void* k,
                         float scale, float* ahat, double* svar, double* skl, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * Compact fit of fixed patterns to target maps.                     [Notes §二.3, Eq.(3)]
 * For each of H heads, a and r (length T) with P(i,j) = exp(a[j] + r[i-j]) / Z(i) minimising the
 * row-wise cross-entropy to the target, averaged over rows:
 *   L = -(1/T) sum_i sum_{j<=i} ahat(i,j) ln P(i,j),
 * by `steps` Adam updates (step size lr; moment rates 0.9 and 0.999, eps 1e-8, bias corrections)
 * from a = r = 0 (the uniform causal pattern).  The notes fit each candidate with 400 steps and
 * accept it when the mean row KL is at most 0.2 nat; neither the step size nor the starting point is
 * given there (0.1 and zero are this library's reading).
 *   ahat : [H][T][T] fp32 device, e.g. saf_calibrate's output (rows need not sum exactly to 1;
 *          entries above the diagonal are not read).
 *   a, r : [H][T] fp32 device (written): the fitted logits.
 *   kl   : [H] fp64 device (written): mean row KL(ahat_i || P_i) = L + (1/T) sum ahat ln ahat.
 *   loss : [H] fp64 device (written) or NULL: L.
 * The arithmetic is fp64 (the marginals of ahat, the normalisers, the gradient and Adam; the
 * entropy term of kl takes fp32 logarithms of the entries, an error of at most 2^-21 ln T); a pass
 * over ahat forms its column, row and distance sums once, then every step costs three length-T
 * causal convolutions per head.  Workspace: saf_fit_pattern_workspace_size(H, T) bytes, 256-byte
 * aligned.  T = 0 is a no-op.
 */
size_t saf_fit_pattern_workspace_size(int H, int T);
saf_status saf_fit_pattern(int H, int T, const float* ahat, int steps, double lr, float* a,
                           float* r, double* kl, double* loss, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * Head selection across a whole model.                             [Notes §二.1]
 *   score    : [L][H] host fp64, one score per head of each of L layers (s_var, or s_kl); lower
 *              means the head is easier to replace by a fixed pattern.  NaN is rejected.
 *   accepted : [L][H] host bytes or NULL.  A zero marks a candidate whose compact fit failed the
 *              acceptance test ([Notes §二.3]: mean row KL above 0.2 nat); it is skipped and the
 *              next head in order is taken.  NULL accepts every head.
 *   ratio    : replacement ratio r in [0, 1]; k = round(r L H) heads are selected, halves rounded
 *              to even.
 *   replaced : [L][H] host bytes (written): 1 for the selected heads, the first k accepted heads of
 *              the ascending order of score, equal scores ordered by (layer, head).
 *   n_selected : (written) the number selected, fewer than k only when fewer heads are accepted.
 * Host memory only; makes no HIP call.
 */
saf_status saf_select_heads(int L, int H, const double* score, const uint8_t* accepted,
                            double ratio, uint8_t* replaced, int* n_selected);

/* Text of the calling thread's last non-OK status ("" if none).  Valid until the thread's next
 * call into the library. */
const char* saf_last_error(void);

/*
 * Overlap inside the backward (off by default; per host thread).  When enabled, saf_attn_bwd and
 * saf_attn_bwd_gqa run the query-block kernel on a second stream of the current device (created on
 * first use, kept for the thread's life, default priority) beside the key-block kernel: both depend
 * only on the preprocess and write disjoint outputs.  The fork and join are event record / wait
 * pairs on the caller's stream (a graph capture of that stream records them), so the call keeps its
 * stream semantics and its results are bitwise those of the call without overlap and with a
 * workspace of saf_attn_bwd_workspace_size bytes (the stored-dS path, which orders the two
 * kernels, is not taken while overlap is enabled).  Faster where the two kernels leave each
 * other's tails idle (e.g. half the heads replaced at 8K context); per-kernel durations from
 * saf_trace_* then overlap.
 */
saf_status saf_set_backward_overlap(int enable);

/*
 * Per-kernel timing (off by default), for profiling a layer from the host.
 * saf_trace_begin(ev, capacity): until saf_trace_end(), every kernel that a call made on this
 * thread launches is bracketed by hipEventRecord(ev[i].start) / hipEventRecord(ev[i].stop) on that
 * call's stream, filling ev[0], ev[1], ... in launch order and setting ev[i].name to a static
 * string naming the kernel.  Launches beyond `capacity` are not recorded.  The caller creates the
 * events (hipEventCreate, on the current device) and owns them and the array; the library only
 * records into them.  saf_trace_end() stops recording and returns the number of entries filled.
 * Errors: SAF_ERR_INVALID_ARG if ev is NULL or capacity < 1.  A failed event record makes the
 * traced call return SAF_ERR_HIP.
 */
typedef struct {
  const char* name;
  hipEvent_t start;
  hipEvent_t stop;
} saf_kernel_event;

saf_status saf_trace_begin(saf_kernel_event* ev, int capacity);
int saf_trace_end(void);

#ifdef __cplusplus
}
#endif

#endif /* SAF_H_ */
