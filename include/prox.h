/*
 * prox.h -- C ABI of libprox, the MI355X (gfx950) implementation of the Prox
 * two-stage sparse SwiGLU FFN decode step.
 *
 * Method: "Prox: Training-Free FFN Activation Sparsity via Approximate
 * Intermediate-Channel Salience in LLMs" (arXiv 2607.27591).
 *   Stage 1 (Sec. 4.1, m_x and u~/h~ equations): keep the inputs with
 *     |x_i| >= threshold, run the INT4 proxy up/gate projections over those
 *     rows only, and form s~ = (x W~up) . SiLU(x W~gate).
 *   Mask (App. A.6, top-k equation): the k channels of largest |s~|, ties to
 *     the lower index, shared by all three projections.
 *   Stage 2 (Sec. 4.1, Stage 2 equations): exact up/gate over the selected
 *     channels with the full x, s = u . SiLU(g), then y = s W_down over the
 *     selected rows.
 *
 * Conventions shared by every call:
 *  - All pointers to tensors are DEVICE pointers owned by the caller; the
 *    library allocates no device memory.  `stream` is a hipStream_t (NULL =
 *    the null stream); every call only enqueues work on it and never
 *    synchronizes the host.
 *  - Element type of weights, x and y is the layer's dtype (PROX_F32 or
 *    PROX_BF16, bf16 = IEEE-754 binary32 truncated to its top 16 bits).
 *  - Weights are given in the paper's x.W layout (Sec. 2.1):
 *      w_up, w_gate: [d_model][d_ff] row-major; w_down: [d_ff][d_model].
 *  - Arguments are validated on the host before anything is enqueued; a
 *    rejected call enqueues nothing.  Errors: PROX_EINVAL (bad argument),
 *    PROX_EUNSUPPORTED (valid but unsupported shape), PROX_EHIP (a HIP call
 *    or launch failed).  prox_last_error() describes the last failure of the
 *    calling thread.
 *  - A layer's workspace is reused by every call on that layer.  Layers of
 *    any shapes may share one workspace buffer as large as the largest of
 *    their workspace_bytes: its synchronisation block (tickets, flags,
 *    counters, the status word) sits at offset 0 with a size fixed for the
 *    largest supported shape, and everything past it is scratch that each
 *    call writes before it reads.  Calls that share a layer or a workspace
 *    must be ordered on one stream.
 */
#ifndef PROX_H_
#define PROX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PROX_OK = 0,
  PROX_EINVAL = -1,
  PROX_EUNSUPPORTED = -2,
  PROX_EHIP = -3
} prox_status;

typedef enum { PROX_F32 = 0, PROX_BF16 = 1 } prox_dtype;

/* Gate activation of the gated FFN: SwiGLU, SiLU(z) = z / (1 + e^-z) (the
 * pages' FFN, Sec. 2.1), or GeGLU with the tanh form of GELU,
 * 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) (Gemma-3 style models,
 * evaluated in Sec. 5).  Both the proxy state s~ and the exact state s use
 * the layer's activation.                                                  */
typedef enum { PROX_ACT_SILU = 0, PROX_ACT_GELU_TANH = 1 } prox_activation;

/* Kernel path of batch-1 forwards: one persistent kernel that takes Stage 1,
 * the top-k select, Stage 2 up/gate and Stage 2 down items in dependency
 * order (the default), or four kernels, one per phase.                     */
typedef enum { PROX_PATH_PERSISTENT = 0, PROX_PATH_MULTI = 1 } prox_path;

/* Arithmetic form of a batched (2..8 token) step: PROX_FORM_AUTO picks the
 * measured faster one (Stage 1: matrix cores from 2 tokens for bf16 layers
 * whose G is a multiple of 64, else vector ALU; Stage 2 up/gate: vector ALU).
 * PROX_FORM_VALU / PROX_FORM_MFMA force one (MFMA: bf16 layers only).       */
typedef enum { PROX_FORM_AUTO = 0, PROX_FORM_VALU = 1, PROX_FORM_MFMA = 2 } prox_form;

/* Shape of one FFN layer, and the kernel choices made for it at prepare time.
 *   d_model     input/output width, at most 16384, a multiple of group_size
 *               and of 512 (bf16) or 256 (f32); batch * d_model activations
 *               must fit in 160 KiB
 *   d_ff        intermediate width, 1..32768
 *   group_size  G, rows per INT4 proxy scale group: 64, 128 or 256
 *   dtype       prox_dtype of weights, x and y
 *   max_batch   largest batch a forward call may pass, 1..8
 *   activation  prox_activation (0: SiLU, the default)
 *   path        prox_path of batch-1 forwards (0: the persistent kernel)
 *   batch_stage1, batch_upgate
 *               prox_form of the Stage 1 proxy GEMV and of the Stage 2
 *               up/gate GEMV for batches of 2..8 tokens (0: automatic)
 * A zero-initialised prox_shape with the first five fields set is the
 * default configuration.                                                    */
typedef struct {
  int d_model;
  int d_ff;
  int group_size;
  int dtype;
  int max_batch;
  int activation;
  int path;
  int batch_stage1;
  int batch_upgate;
} prox_shape;

/* Opaque host-side handle: shape, launch plan and the caller's buffers. */
typedef struct prox_layer prox_layer;

/* Bytes the caller must allocate (device memory, 256-byte aligned) for:
 *   weights_bytes   relaid exact weights (up/gate channel-major, down row-major)
 *   proxy_bytes     packed INT4 proxy codes and their float32 scales, plus
 *                   one word of layer state that batch-1 top-k calls update
 *                   (a guess of the next cut, used for scheduling only); bf16
 *                   layers with max_batch >= 2 (G a multiple of 64, d_model of 32)
 *                   hold the codes a second time, 8 rows of one column per
 *                   word, for the matrix-core Stage 1 of several tokens
 *   workspace_bytes the synchronisation block plus per-call scratch (partial
 *                   sums, |s~|, masks, s values)
 * Pure host function.  PROX_EINVAL on a null pointer or an invalid shape,
 * PROX_EUNSUPPORTED on a shape outside the limits above.                    */
prox_status prox_query_sizes(const prox_shape *shape, size_t *weights_bytes,
                             size_t *proxy_bytes, size_t *workspace_bytes);

/* Bytes of the synchronisation block at offset 0 of every workspace: the
 * same for every shape (sized for the largest supported one), so layers of
 * different shapes can share a workspace; workspace_bytes includes it.     */
size_t prox_sync_block_bytes(void);

/* Build a layer (Sec. 4.3: the INT4 proxy of W_up and W_gate is computed once
 * and stays resident).  Enqueues on `stream`:
 *   - relayout: W_up and W_gate transposed to channel-major rows (channel j's
 *     up row followed by its gate row), W_down kept row-major in chunks of
 *     256 output columns ([d_model/256][d_ff][256]);
 *   - quantization: per group g of G input rows and per column j,
 *     scale = max|W[i][j]| / 7 (float32), code = clamp(rint(W / scale), -7, 7)
 *     (float32 divide, ties to even; an all-zero group has scale 0, codes 0),
 *     stored as 4-bit (code + 8), packed along j per input row;
 *   - zeroing of the workspace's synchronisation block.
 * Source weights must stay valid until the stream has run these kernels.
 * The three buffers belong to the caller and must outlive the layer.
 * On success *out receives a handle to free with prox_destroy_layer.        */
prox_status prox_prepare_layer(const prox_shape *shape, const void *w_up,
                               const void *w_gate, const void *w_down,
                               void *weights_buf, void *proxy_buf,
                               void *workspace_buf, void *stream,
                               prox_layer **out);

/* Read back a prepared layer's INT4 codes (as signed int8 [d_model][d_ff], in
 * the paper's layout) and scales (float32 [d_model/G][d_ff]) into caller
 * device buffers.  Inspection only (used to check the quantizer bit for bit). */
prox_status prox_export_proxy(const prox_layer *layer, int matrix /*0 up, 1 gate*/,
                              int8_t *codes, float *scales, void *stream);

/* One token: y = Prox-FFN(x) (batch 1, the decode hot path).  Runs as one
 * persistent kernel whose work-groups take Stage 1, top-k, Stage 2 up/gate
 * and Stage 2 down items in dependency order (a layer prepared with
 * path = PROX_PATH_MULTI runs four kernels instead).  The persistent kernel
 * assumes that all of its work-groups are resident together (its grid is
 * sized from the occupancy of the device); work running concurrently on
 * other streams can break that, and its bounded waits then give up: the
 * workspace status (prox_read_status) has bit 0 set and y is invalid.
 *   x          [d_model] layer dtype
 *   threshold  tau of the Stage 1 input mask; an input survives iff
 *              |x_i| >= threshold (so threshold <= 0 keeps every input and
 *              +inf keeps none); NaN -> PROX_EINVAL
 *   k          channels kept by the Stage 2 mask, 0 <= k <= d_ff (k = 0
 *              gives y = 0, k = d_ff the dense result)
 *   y          [d_model] layer dtype (written, never read)                  */
prox_status prox_ffn_forward(const prox_layer *layer, const void *x,
                             float threshold, int k, void *y, void *stream);

/* prox_ffn_forward for callers that cannot allocate device memory or run
 * allocating routines (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, but the
 * per-call scratch (partial sums, |s~|, masks, tickets, flags) lives in one
 * static device array of the library, 8 MiB per GPU (every GPU the library
 * runs on holds its own copy until the process ends), instead of the layer's
 * workspace.  The layer's weights and proxy buffers are read as usual.  The
 * call allocates nothing (no hipMalloc/hipFree, no allocating library
 * routine); on its first use on a device it takes the array's device address
 * and zeroes its synchronisation block with a fill kernel on `stream`.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads)
 * race.  The status word of these calls stays in the array (it is not read
 * back by prox_read_status).  Errors as prox_ffn_forward, plus
 * PROX_EUNSUPPORTED when the layer's batch-1 scratch exceeds 8 MiB (shapes
 * above 8192 x 28672).                                                      */
prox_status prox_ffn_forward_noalloc(const prox_layer *layer, const void *x,
                                     float threshold, int k, void *y, void *stream);

/* `batch` independent tokens (1 <= batch <= max_batch), x and y [batch][d_model].
 * Each token gets its own input mask and its own top-k mask; the union of
 * the masks decides which weight rows are streamed, and every token's s is
 * zero outside its own mask, so the result equals `batch` batch-1 calls.   */
prox_status prox_ffn_forward_batch(const prox_layer *layer, const void *x,
                                   int batch, float threshold, int k, void *y,
                                   void *stream);

/* Intermediate results of a forward call, for verification.  Every pointer
 * is a caller device buffer or NULL (not written).                           */
typedef struct {
  int32_t *n1;       /* [batch]            surviving inputs per token          */
  int32_t *idx;      /* [batch][d_model]   survivors, ascending               */
  float *s_abs;      /* [batch][d_ff]      |s~| of the INT4 proxy             */
  int32_t *sel;      /* [batch][d_ff]      selected channels, ascending (k used) */
  float *s_sel;      /* [batch][d_ff]      exact s of sel[b][t] at t (k used) */
  int32_t *n_union;  /* [1]                size of the union of the masks     */
  int32_t *union_idx;/* [d_ff]             the union, ascending               */
  int32_t *status;   /* [1]  the workspace status word of this call alone (see
                        prox_read_status); the debug entries clear it before
                        the call                                             */
  int32_t *n_sel;    /* [1]  number of kept channels (batch-1 persistent kernel:
                        k for top-k, the count for the threshold mask)      */
} prox_debug;

/* prox_ffn_forward_batch plus a copy of its intermediate results into `dbg`. */
prox_status prox_ffn_forward_debug(const prox_layer *layer, const void *x,
                                   int batch, float threshold, int k, void *y,
                                   const prox_debug *dbg, void *stream);

/* Workspace status.  Every forward on the persistent kernel ORs its error
 * bits into a sticky status word of the layer's workspace (shared by every
 * layer prepared on that workspace); no forward entry clears it.
 *   bit 0 (1)  a bounded wait timed out: the outputs of the calls since the
 *              last read are invalid (a work-group was not resident, see
 *              prox_ffn_forward, or a wait limit set with prox_set_wait_limit
 *              was too small);
 *   bit 1 (2)  the top-k select took its slow exact path (massive exact ties
 *              of |s~| around the k-th value); results valid.
 * Enqueues on `stream` one kernel that copies the word into `status` (device
 * int32) and clears it; when bit 0 was set it also resets the workspace's
 * synchronisation block (tickets, flags, counters, histogram), so the next
 * call starts clean.  No host synchronisation; read `status` after the stream
 * has run it.  PROX_EINVAL on NULL arguments.                              */
prox_status prox_read_status(const prox_layer *layer, int32_t *status, void *stream);

/* Poll limit of the persistent kernel's bounded waits for this layer (the
 * default, 4194304 polls, is seconds: only a work-group that never runs
 * reaches it).  A wait that reaches it sets bit 0 of the workspace status and
 * lets its work item finish with whatever data it has (the kernel always
 * exits).  For tests of the error path.  PROX_EINVAL on a NULL layer.       */
prox_status prox_set_wait_limit(prox_layer *layer, uint32_t polls);

/* Batch-1 forward with the calibrated Stage 2 threshold of Sec. 4.1 instead
 * of the per-token top-k: channel j is kept iff |s~_j| >= threshold_s (|s~|
 * in float32), so the number of kept channels varies per token.  Stage 1 is
 * as in prox_ffn_forward (input mask |x_i| >= threshold_x, INT4 proxy).  Runs
 * on the persistent kernel without its select phase: each Stage 2 item
 * starts as soon as the Stage 1 tile holding its channels is done.
 * Errors: PROX_EINVAL for a NaN threshold or bad pointers; PROX_EUNSUPPORTED
 * for a layer prepared with path = PROX_PATH_MULTI.                                 */
prox_status prox_ffn_forward_ts(const prox_layer *layer, const void *x,
                                float threshold_x, float threshold_s, void *y,
                                void *stream);

/* prox_ffn_forward_ts plus its intermediate results: n1, idx, s_abs, sel (the
 * kept channels, ascending, up to d_ff), s_sel (their exact s), n_sel (their
 * count) and status; n_union and union_idx are not written.                 */
prox_status prox_ffn_forward_ts_debug(const prox_layer *layer, const void *x,
                                      float threshold_x, float threshold_s,
                                      void *y, const prox_debug *dbg,
                                      void *stream);

/* Dense SwiGLU FFN on the same relaid weights (Sec. 2.1), the baseline:
 * y = (x W_up . SiLU(x W_gate)) W_down for `batch` tokens.                   */
prox_status prox_dense_ffn_forward(const prox_layer *layer, const void *x,
                                   int batch, void *y, void *stream);

/* A decode stack of n_layers FFN layers of one shape on a float32 residual
 * stream r [batch][d_model] (updated in place): for each layer l,
 *   x = cast(r / sqrt(mean(r^2) + eps)) (RMSNorm with unit gain),
 *   y = Prox-FFN_l(x, thresholds[l], k) (or the dense FFN when k < 0),
 *   r = r + y.
 * thresholds is a HOST array [n_layers].  The layers may share one workspace. */
prox_status prox_stack_forward(const prox_layer *const *layers, int n_layers,
                               const float *thresholds, int k, float *resid,
                               int batch, float eps, void *stream);

/* prox_stack_forward with the Stage 2 threshold mask of every layer (batch
 * 1): x = cast(RMSNorm(r)), y = Prox-FFN_l(x) with |x_i| >= thresholds_x[l]
 * and |s~_j| >= thresholds_s[l], r = r + y.  Both threshold arrays are HOST
 * arrays [n_layers].  PROX_EUNSUPPORTED if a layer was prepared with
 * path = PROX_PATH_MULTI.                                                          */
prox_status prox_stack_forward_ts(const prox_layer *const *layers, int n_layers,
                                  const float *thresholds_x,
                                  const float *thresholds_s, float *resid,
                                  float eps, void *stream);

/* The stack's normalization alone: x = cast(r / sqrt(mean(r^2) + eps)) for
 * `batch` (1..8) rows of the float32 residual r [batch][d_model], written in
 * the layer dtype.  Used to collect layer inputs for threshold calibration
 * (each layer's tau is a quantile of |x| over calibration tokens that went
 * through the already-calibrated layers before it).                         */
prox_status prox_rmsnorm(const prox_layer *layer, const float *resid, int batch,
                         float eps, void *x, void *stream);

/* Instrumented forms of prox_ffn_forward_batch and prox_dense_ffn_forward,
 * for measurement.  `events` holds n_events caller-created hipEvent_t; one is
 * recorded on `stream` before the first kernel and one after each kernel, so
 * consecutive pairs bracket the kernels in launch order:
 *   sparse: Stage 1 proxy, top-k (which also forms the union of the masks
 *           when batch > 1), Stage 2 up/gate, Stage 2 down
 *                                               (at least 5 events needed)
 *   dense:  up/gate, down                        (at least 3 events needed)
 * *n_recorded receives the number of events recorded.  Same results as the
 * plain calls; no host synchronization.                                      */
prox_status prox_ffn_forward_profiled(const prox_layer *layer, const void *x,
                                      int batch, float threshold, int k, void *y,
                                      void *const *events, int n_events,
                                      int *n_recorded, void *stream);
prox_status prox_dense_ffn_forward_profiled(const prox_layer *layer,
                                            const void *x, int batch, void *y,
                                            void *const *events, int n_events,
                                            int *n_recorded, void *stream);

/* Timeline of one batch-1 forward on the persistent kernel (the default path
 * of prox_ffn_forward for k > 0), for performance work.  The launch takes
 * work items by ticket: counts[0..3] (host) receive the number of Stage 1
 * items, select items (1), Stage 2 up/gate items (ceil(k/8)) and Stage 2 down
 * items; their sum is the ticket count.  With trace == NULL only counts are
 * written.  Otherwise trace (device, [trace_items >= tickets][4] u64) receives
 * per ticket: start, end of its wait for earlier items, end (ticks of the
 * 100 MHz GPU real-time clock) and the work-group that ran it in the low 32
 * bits of the 4th word, its phase (1..4: Stage 1, select, up/gate, down) in
 * the high 32 bits.  y is the
 * same as prox_ffn_forward's.  PROX_EUNSUPPORTED when the layer runs the
 * multi-kernel path (path = PROX_PATH_MULTI).                       */
prox_status prox_ffn_forward_traced(const prox_layer *layer, const void *x,
                                   float threshold, int k, void *y,
                                   unsigned long long *trace, int trace_items,
                                   int *counts, void *stream);

/* Stage 1 alone (Sec. 4.1: input mask |x_i| >= threshold and the INT4 proxy
 * GEMV of W_up and W_gate with the activation epilogue) for one token, on
 * the multi-kernel path's Stage 1 kernel.  s_abs (device float [d_ff]) may be
 * NULL: the result then stays in the layer workspace.  Used to time the INT4
 * proxy GEMV against prox_sparse_gemv (the ratio alpha of Sec. 4.2).        */
prox_status prox_stage1(const prox_layer *layer, const void *x, float threshold,
                        float *s_abs, void *stream);

/* Input-sparse bf16 GEMV of both gate projections, the full-precision
 * counterpart of Stage 1 (the FP16 GEMV at the same input sparsity that
 * App. A.3 times against the INT4 proxy):
 *   u_j = sum over i with |x_i| >= threshold of x_i W_up[i][j], likewise g,
 * float32 accumulation.  w_up, w_gate: bf16 [d_model][d_ff] row-major (x.W
 * layout, the caller's tensors, read in place); x bf16 [d_model]; u, g float
 * [d_ff].  d_model a multiple of 64 (<= 16384), d_ff a multiple of 8
 * (<= 32768).  workspace: device, 256-byte aligned,
 * prox_sparse_gemv_workspace_bytes(d_model, d_ff) bytes, zeroed before its
 * first use (every call leaves it zeroed); calls sharing it must not overlap. */
size_t prox_sparse_gemv_workspace_bytes(int d_model, int d_ff);
prox_status prox_sparse_gemv(const void *w_up, const void *w_gate, int d_model,
                             int d_ff, const void *x, float threshold, float *u,
                             float *g, void *workspace, void *stream);

/* Release a handle (host memory only; the caller's buffers are untouched). */
void prox_destroy_layer(prox_layer *layer);

/* Text of the calling thread's last error ("" if none). */
const char *prox_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PROX_H_ */
