// C ABI of libprox (declared in include/prox.h): argument checks, buffer
// layout and the launch sequence of the Prox FFN step.
//
// Method: "Prox: Training-Free FFN Activation Sparsity via Approximate
// Intermediate-Channel Salience in LLMs" (arXiv 2607.27591).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <stdlib.h>

#include <new>
#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/prox.h"
#include "prox_internal.h"

struct prox_layer {
  prox::Plan plan;
  prox::Bufs bufs;
};

// Scratch of prox_ffn_forward_noalloc: one static device array per GPU
// (every GPU the library runs on holds its own copy until the process ends),
// standing in for the caller's workspace.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): it
// uses the device address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[prox::kNoAllocScratchBytes];

namespace {

thread_local std::string g_err;

prox_status fail(prox_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
prox_status fail(prox_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

prox_status hip_fail(hipError_t e, const char *what) {
  return fail(PROX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

prox_status check_shape(const prox_shape *sh) {
  if (!sh) return fail(PROX_EINVAL, "shape is NULL");
  if (sh->d_model <= 0 || sh->d_ff <= 0 || sh->group_size <= 0 || sh->max_batch <= 0)
    return fail(PROX_EINVAL, "shape sizes must be positive (d_model=%d d_ff=%d G=%d max_batch=%d)",
                sh->d_model, sh->d_ff, sh->group_size, sh->max_batch);
  if (sh->dtype != PROX_F32 && sh->dtype != PROX_BF16)
    return fail(PROX_EINVAL, "unknown dtype %d", sh->dtype);
  if (sh->activation != PROX_ACT_SILU && sh->activation != PROX_ACT_GELU_TANH)
    return fail(PROX_EINVAL, "unknown activation %d", sh->activation);
  if (sh->path != PROX_PATH_PERSISTENT && sh->path != PROX_PATH_MULTI)
    return fail(PROX_EINVAL, "unknown path %d", sh->path);
  for (int f : {sh->batch_stage1, sh->batch_upgate})
    if (f != PROX_FORM_AUTO && f != PROX_FORM_VALU && f != PROX_FORM_MFMA)
      return fail(PROX_EINVAL, "unknown batch form %d", f);
  if (sh->d_model % sh->group_size != 0)
    return fail(PROX_EINVAL, "d_model (%d) is not a multiple of group_size (%d)",
                sh->d_model, sh->group_size);
  if (sh->group_size != 64 && sh->group_size != 128 && sh->group_size != 256)
    return fail(PROX_EUNSUPPORTED, "group_size must be 64, 128 or 256 (got %d)", sh->group_size);
  const int dm_mult = sh->dtype == PROX_BF16 ? 512 : 256;
  if (sh->d_model % dm_mult != 0)
    return fail(PROX_EUNSUPPORTED, "d_model must be a multiple of %d for this dtype (got %d)",
                dm_mult, sh->d_model);
  if (sh->d_model > prox::kMaxDmodel)
    return fail(PROX_EUNSUPPORTED, "d_model above %d is not supported (got %d)",
                prox::kMaxDmodel, sh->d_model);
  if (sh->d_ff > prox::kMaxDff)
    return fail(PROX_EUNSUPPORTED, "d_ff above %d is not supported (got %d)", prox::kMaxDff,
                sh->d_ff);
  if (sh->max_batch > prox::kMaxBatch)
    return fail(PROX_EUNSUPPORTED, "max_batch above %d is not supported (got %d)",
                prox::kMaxBatch, sh->max_batch);
  if (sh->batch_upgate == PROX_FORM_MFMA && sh->dtype != PROX_BF16)
    return fail(PROX_EUNSUPPORTED, "the matrix-core up/gate form needs bf16 weights");
  if (sh->batch_stage1 == PROX_FORM_MFMA &&
      (sh->dtype != PROX_BF16 || sh->group_size % 64 != 0 || sh->max_batch < 2))
    return fail(PROX_EUNSUPPORTED,
                "the matrix-core Stage 1 needs bf16 weights, G a multiple of 64 and max_batch >= 2");
  // Byte offsets inside the weight buffers are 32-bit.
  const size_t esz = sh->dtype == PROX_BF16 ? 2 : 4;
  if ((size_t)sh->d_ff * 2 * sh->d_model * esz >= (1ull << 32))
    return fail(PROX_EUNSUPPORTED, "up/gate weights above 4 GiB are not supported");
  return PROX_OK;
}

// Point the per-call buffers of a layer into the workspace at ws.
void bind_workspace(const prox::Layout &lay, char *ws, prox::Bufs &b) {
  b.part = (float *)(ws + lay.o_part);
  b.tile_cnt = (unsigned *)(ws + lay.o_tile_cnt);
  b.drows = (int *)(ws + lay.o_drows);
  b.dcnt = (int *)(ws + lay.o_dcnt);
  b.sabs = (float *)(ws + lay.o_sabs);
  b.sel = (int *)(ws + lay.o_sel);
  b.selw = (unsigned *)(ws + lay.o_selw);
  b.ssp = (float *)(ws + lay.o_ssp);
  b.uni = (int *)(ws + lay.o_uni);
  b.nuni = (int *)(ws + lay.o_nuni);
  b.umask = (uint8_t *)(ws + lay.o_umask);
  b.ypart = (float *)(ws + lay.o_ypart);
  b.col_cnt = (unsigned *)(ws + lay.o_col_cnt);
  b.ucnt = (unsigned *)(ws + lay.o_ucnt);
  b.sync = (unsigned *)(ws + lay.o_sync);
  b.xbuf = ws + lay.o_xbuf;
  b.ybuf = ws + lay.o_ybuf;
}

prox::Plan plan_of(const prox_shape *sh) {
  prox::PlanChoice ch;
  ch.path = sh->path;
  ch.batch_stage1 = sh->batch_stage1;
  ch.batch_upgate = sh->batch_upgate;
  return prox::make_plan(sh->d_model, sh->d_ff, sh->group_size, sh->dtype == PROX_BF16,
                         sh->max_batch, sh->activation, ch);
}

}  // namespace

namespace prox {

Plan make_plan(int d_model, int d_ff, int G, int bf16, int max_batch, int act,
               const PlanChoice &ch) {
  Plan p{};
  p.act = act;
  p.d_model = d_model;
  p.d_ff = d_ff;
  p.G = G;
  p.bf16 = bf16;
  p.max_batch = max_batch;
  p.esz = bf16 ? 2 : 4;
  p.ngroups = d_model / G;
  p.ntile = (d_ff + kTile - 1) / kTile;
  p.nchunk = (d_model / 64 + 7) / 8;  // proxy work-groups per tile (8 slices of 64 rows)
  p.ncol = d_model / kDownCols;
  int nrc = 512 / p.ncol;
  if (nrc < 1) nrc = 1;
  if (nrc > 64) nrc = 64;
  p.nrc = nrc;
  p.upgate_cap = 4096;
  p.use_fused = fused_supported(p) && ch.path == PROX_PATH_PERSISTENT;
  p.batch_mfma = ch.batch_upgate == PROX_FORM_MFMA;
  // Stage 1 of several tokens on the matrix cores unless the vector form is
  // asked for (measured faster from 2 tokens, although at 2 the vector
  // kernel reads only the rows the union of the input masks keeps: 8B 67.1
  // against 69.5 us, 70B 182.6 against 183.5-187.1 us per 2-token step).
  const bool mfma_ok = bf16 && G % 64 == 0 && d_model % 32 == 0;
  if (ch.batch_stage1 != PROX_FORM_VALU && mfma_ok && max_batch >= 2)
    p.proxy_mfma = 2;
  else
    p.proxy_mfma = 0;
  p.wait_limit = kDefaultWaitLimit;
  return p;
}

size_t sync_block_bytes() {
  size_t o = align256(fused_sync_words() * sizeof(unsigned));
  o = align256(o + (size_t)(kMaxDff / kTile) * sizeof(unsigned));
  o = align256(o + (size_t)(kMaxDmodel / kDownCols) * sizeof(unsigned));
  o = align256(o + sizeof(unsigned));
  return o;
}

Layout make_layout(const Plan &p) {
  Layout L{};
  const size_t B = (size_t)p.max_batch;
  const size_t wug = (size_t)p.d_ff * 2 * p.d_model * p.esz;
  L.o_wd = align256(wug);
  L.weights = align256(L.o_wd + (size_t)p.d_ff * p.d_model * p.esz);
  const size_t pq = (size_t)p.ntile * p.d_model * kTileBytes;
  L.o_psc = align256(pq);
  L.o_pred = align256(L.o_psc + (size_t)p.ntile * p.ngroups * 512 * sizeof(float));
  L.o_pq2 = L.o_pred + 256;
  L.proxy = L.o_pq2 + (p.proxy_mfma ? align256(pq) : 0);
  // The synchronisation block (fixed size, see sync_block_bytes).
  size_t o = 0;
  L.o_sync = o;      o = align256(o + fused_sync_words() * sizeof(unsigned));
  L.o_tile_cnt = o;  o = align256(o + (size_t)(kMaxDff / kTile) * sizeof(unsigned));
  L.o_col_cnt = o;   o = align256(o + (size_t)(kMaxDmodel / kDownCols) * sizeof(unsigned));
  L.o_ucnt = o;      o = align256(o + sizeof(unsigned));
  L.hdr = o;
  // Per-call scratch.
  L.o_part = o;      o = align256(o + (size_t)p.ntile * p.nchunk * B * 512 * sizeof(float));
  L.o_sabs = o;      o = align256(o + B * p.d_ff * sizeof(float));
  L.o_sel = o;       o = align256(o + B * p.d_ff * sizeof(int));
  L.o_selw = o;      o = align256(o + B * ((p.d_ff + 31) / 32) * sizeof(unsigned));
  L.o_ssp = o;       o = align256(o + ((B + 3) & ~(size_t)3) * p.d_ff * sizeof(float));
  L.o_uni = o;       o = align256(o + (size_t)p.d_ff * sizeof(int));
  L.o_nuni = o;      o = align256(o + sizeof(int));
  L.o_umask = o;     o = align256(o + (size_t)p.d_ff);
  const size_t yrows = std::max((size_t)p.nrc * B, (size_t)fused_ypart_rows(p));
  L.o_ypart = o;     o = align256(o + yrows * p.d_model * sizeof(float));
  L.o_xbuf = o;      o = align256(o + B * p.d_model * p.esz);
  L.o_ybuf = o;      o = align256(o + B * p.d_model * p.esz);
  L.o_drows = o;     o = align256(o + B * p.d_model * sizeof(int));
  L.o_dcnt = o;      o = align256(o + B * (p.d_model / 64) * sizeof(int));
  L.workspace = o;
  return L;
}

}  // namespace prox

namespace {

// Optional instrumentation: caller-owned HIP events recorded on the launch
// stream before the first kernel and after each kernel of a call.
struct EventLog {
  void *const *ev;
  int cap;
  int n;
  hipError_t mark(hipStream_t s) {
    if (!ev) return hipSuccess;
    if (n >= cap) return hipErrorInvalidValue;
    return hipEventRecord((hipEvent_t)ev[n++], s);
  }
};

// Stage 1, top-k and Stage 2 for `batch` tokens; writes y.  lists: the
// top-k kernel also writes the per-token lists (batch > 1); dbg: the Stage 1
// kernel writes its survivor lists (b.drows / b.dcnt), and with k = 0 (no
// kernel on the path) Stage 1 runs alone to give them.
prox_status run_forward(const prox_layer *L, const void *x, int batch, float tau,
                        int k, void *y, float *resid, hipStream_t s,
                        EventLog *log = nullptr, bool lists = false, bool dbg = false) {
  const prox::Plan &p = L->plan;
  const prox::Bufs &b = L->bufs;
  EventLog none{nullptr, 0, 0};
  EventLog &lg = log ? *log : none;
  hipError_t e;
  if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
  if (k == 0) {
    if (dbg && (e = prox::launch_proxy(p, b, x, batch, tau, s, true)) != hipSuccess)
      return hip_fail(e, "stage 1 proxy kernel");
    e = prox::launch_zero_y(p, y, batch, s);
    if (e != hipSuccess) return hip_fail(e, "zero output");
    if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
    return PROX_OK;  // y = 0 adds nothing to the residual
  }
  if (batch == 1 && p.use_fused) {
    prox::FusedOpts o;
    o.dbg = dbg;
    if ((e = prox::launch_fused(p, b, x, tau, k, y, resid, s, o)) != hipSuccess)
      return hip_fail(e, "fused kernel");
    if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
    return PROX_OK;
  }
  if ((e = prox::launch_proxy(p, b, x, batch, tau, s, dbg)) != hipSuccess)
    return hip_fail(e, "stage 1 proxy kernel");
  if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
  // Several tokens: Stage 2 runs over the union of the tokens' masks, taken
  // from their mask words by the Stage 2 kernels themselves (mode 3); the
  // matrix-core up/gate form reads a union list (mode 1), which the top-k
  // launch then builds, as it does for the debug entry.  The per-token lists
  // are written only when asked for.
  const int mode = batch == 1 ? 0 : (p.bf16 && p.batch_mfma ? 1 : 3);
  if ((e = prox::launch_topk(p, b, batch, k, batch == 1 || lists, mode == 1 || lists, s)) !=
      hipSuccess)
    return hip_fail(e, "top-k kernel");
  if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = prox::launch_upgate(p, b, x, batch, mode, k, s)) != hipSuccess)
    return hip_fail(e, "stage 2 up/gate kernel");
  if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = prox::launch_down(p, b, batch, mode, k, y, resid, s)) != hipSuccess)
    return hip_fail(e, "stage 2 down kernel");
  if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
  return PROX_OK;
}

prox_status run_dense(const prox_layer *L, const void *x, int batch, void *y,
                      float *resid, hipStream_t s, EventLog *log = nullptr) {
  const prox::Plan &p = L->plan;
  EventLog none{nullptr, 0, 0};
  EventLog &lg = log ? *log : none;
  hipError_t e;
  if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = prox::launch_upgate(p, L->bufs, x, batch, 2, p.d_ff, s)) != hipSuccess)
    return hip_fail(e, "dense up/gate kernel");
  if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = prox::launch_down(p, L->bufs, batch, 2, p.d_ff, y, resid, s)) != hipSuccess)
    return hip_fail(e, "dense down kernel");
  if ((e = lg.mark(s)) != hipSuccess) return hip_fail(e, "event record");
  return PROX_OK;
}

prox_status check_forward_args(const prox_layer *L, const void *x, int batch,
                               float tau, int k, const void *y) {
  if (!L) return fail(PROX_EINVAL, "layer is NULL");
  if (!x || !y) return fail(PROX_EINVAL, "x and y must be non-NULL device pointers");
  if (!aligned(x, 16) || !aligned(y, 16))
    return fail(PROX_EINVAL, "x and y must be 16-byte aligned");
  if (batch < 1 || batch > L->plan.max_batch)
    return fail(PROX_EINVAL, "batch %d outside [1, max_batch=%d]", batch, L->plan.max_batch);
  if (isnan(tau)) return fail(PROX_EINVAL, "threshold is NaN");
  if ((size_t)batch * L->plan.d_model * L->plan.esz > prox::kMaxLds)
    return fail(PROX_EUNSUPPORTED, "batch * d_model activations exceed the %zu-byte LDS budget",
                prox::kMaxLds);
  if (k < 0 || k > L->plan.d_ff)
    return fail(PROX_EINVAL, "k=%d outside [0, d_ff=%d]", k, L->plan.d_ff);
  return PROX_OK;
}

// The scratch array's device address on the current device, taken once per
// device (with the device current) and kept; its synchronisation block is
// zeroed on `s` by the first call on each device (a fill kernel).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

prox_status scratch_for_current_device(hipStream_t s, char **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PROX_EUNSUPPORTED, "device %d above the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PROX_EHIP, "hipGetSymbolAddress(scratch) gave a null address");
    // tickets, flags, counters and the status word start at zero
    e = prox::launch_zero_bytes(p, prox::sync_block_bytes(), s);
    if (e != hipSuccess) return hip_fail(e, "scratch clear kernel");
    g_scratch_ptr[dev] = p;
  }
  *out = (char *)g_scratch_ptr[dev];
  return PROX_OK;
}

}  // namespace

extern "C" {

const char *prox_last_error(void) { return g_err.c_str(); }

size_t prox_sync_block_bytes(void) { return prox::sync_block_bytes(); }

prox_status prox_query_sizes(const prox_shape *shape, size_t *weights_bytes,
                             size_t *proxy_bytes, size_t *workspace_bytes) {
  g_err.clear();
  prox_status st = check_shape(shape);
  if (st != PROX_OK) return st;
  if (!weights_bytes || !proxy_bytes || !workspace_bytes)
    return fail(PROX_EINVAL, "output size pointers must be non-NULL");
  const prox::Plan p = plan_of(shape);
  const prox::Layout L = prox::make_layout(p);
  *weights_bytes = L.weights;
  *proxy_bytes = L.proxy;
  *workspace_bytes = L.workspace;
  return PROX_OK;
}

prox_status prox_prepare_layer(const prox_shape *shape, const void *w_up,
                               const void *w_gate, const void *w_down,
                               void *weights_buf, void *proxy_buf,
                               void *workspace_buf, void *stream,
                               prox_layer **out) {
  g_err.clear();
  prox_status st = check_shape(shape);
  if (st != PROX_OK) return st;
  if (!out) return fail(PROX_EINVAL, "out is NULL");
  *out = nullptr;
  if (!w_up || !w_gate || !w_down || !weights_buf || !proxy_buf || !workspace_buf)
    return fail(PROX_EINVAL, "weight and buffer pointers must be non-NULL");
  if (!aligned(weights_buf, 256) || !aligned(proxy_buf, 256) || !aligned(workspace_buf, 256))
    return fail(PROX_EINVAL, "weights/proxy/workspace buffers must be 256-byte aligned");
  const size_t ea = shape->dtype == PROX_BF16 ? 2 : 4;
  if (!aligned(w_up, ea) || !aligned(w_gate, ea) || !aligned(w_down, ea))
    return fail(PROX_EINVAL, "source weights must be aligned to their element size");
  prox_layer *L = new (std::nothrow) prox_layer;
  if (!L) return fail(PROX_EINVAL, "out of host memory");
  L->plan = plan_of(shape);
  const prox::Layout lay = prox::make_layout(L->plan);
  char *wb = (char *)weights_buf, *pb = (char *)proxy_buf, *ws = (char *)workspace_buf;
  prox::Bufs &b = L->bufs;
  b.wug = wb;
  b.wd = wb + lay.o_wd;
  b.pq = (uint8_t *)pb;
  b.psc = (float *)(pb + lay.o_psc);
  b.pred = (unsigned *)(pb + lay.o_pred);
  b.pq2 = L->plan.proxy_mfma ? (unsigned *)(pb + lay.o_pq2) : nullptr;
  bind_workspace(lay, ws, b);
  hipError_t e = prox::launch_prepare(L->plan, b, w_up, w_gate, w_down, (hipStream_t)stream);
  // the synchronisation block (tickets, flags, counters, status) and the
  // layer's cut guess start at zero
  if (e == hipSuccess) e = hipMemsetAsync(ws, 0, lay.hdr, (hipStream_t)stream);
  if (e == hipSuccess) e = hipMemsetAsync(b.pred, 0, sizeof(unsigned), (hipStream_t)stream);
  if (e != hipSuccess) {
    delete L;
    return hip_fail(e, "prepare kernels");
  }
  *out = L;
  return PROX_OK;
}

prox_status prox_export_proxy(const prox_layer *layer, int matrix, int8_t *codes,
                              float *scales, void *stream) {
  g_err.clear();
  if (!layer || !codes || !scales) return fail(PROX_EINVAL, "NULL argument");
  if (matrix != 0 && matrix != 1) return fail(PROX_EINVAL, "matrix must be 0 (up) or 1 (gate)");
  hipError_t e = prox::launch_export_proxy(layer->plan, layer->bufs, matrix, codes, scales,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "export kernel");
  return PROX_OK;
}

prox_status prox_ffn_forward(const prox_layer *layer, const void *x, float threshold,
                             int k, void *y, void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, 1, threshold, k, y);
  if (st != PROX_OK) return st;
  return run_forward(layer, x, 1, threshold, k, y, nullptr, (hipStream_t)stream);
}

prox_status prox_ffn_forward_noalloc(const prox_layer *layer, const void *x, float threshold,
                                     int k, void *y, void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, 1, threshold, k, y);
  if (st != PROX_OK) return st;
  // the layer's batch-1 per-call buffers, laid out in the static scratch
  prox_layer L = *layer;
  L.plan.max_batch = 1;
  const prox::Layout lay = prox::make_layout(L.plan);
  if (lay.workspace > prox::kNoAllocScratchBytes)
    return fail(PROX_EUNSUPPORTED,
                "the layer needs %zu bytes of per-call scratch; the static scratch holds %zu",
                lay.workspace, prox::kNoAllocScratchBytes);
  hipStream_t s = (hipStream_t)stream;
  char *ws = nullptr;
  if ((st = scratch_for_current_device(s, &ws)) != PROX_OK) return st;
  bind_workspace(lay, ws, L.bufs);
  return run_forward(&L, x, 1, threshold, k, y, nullptr, s);
}

prox_status prox_ffn_forward_batch(const prox_layer *layer, const void *x, int batch,
                                   float threshold, int k, void *y, void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, batch, threshold, k, y);
  if (st != PROX_OK) return st;
  return run_forward(layer, x, batch, threshold, k, y, nullptr, (hipStream_t)stream);
}

prox_status prox_ffn_forward_debug(const prox_layer *layer, const void *x, int batch,
                                   float threshold, int k, void *y, const prox_debug *dbg,
                                   void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, batch, threshold, k, y);
  if (st != PROX_OK) return st;
  if (!dbg) return fail(PROX_EINVAL, "dbg is NULL");
  if ((dbg->n1 != nullptr) != (dbg->idx != nullptr))
    return fail(PROX_EINVAL, "n1 and idx must be given together");
  hipStream_t s = (hipStream_t)stream;
  const prox::Plan &p = layer->plan;
  const prox::Bufs &b = layer->bufs;
  hipError_t e = hipSuccess;
  if (dbg->status &&
      (e = hipMemsetAsync(b.sync + prox::kFusedErrWord, 0, sizeof(unsigned), s)) != hipSuccess)
    return hip_fail(e, "clear status");
  const bool surv = dbg->idx != nullptr;
  st = run_forward(layer, x, batch, threshold, k, y, nullptr, s, nullptr, true, surv);
  if (st != PROX_OK) return st;
  if (dbg->status &&
      (e = hipMemcpyAsync(dbg->status, b.sync + prox::kFusedErrWord, sizeof(unsigned),
                          hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return hip_fail(e, "copy status");
  // the survivors as the Stage 1 kernel itself decided them
  if (surv && (e = prox::launch_survivors(p, b, batch, dbg->n1, dbg->idx, s)) != hipSuccess)
    return hip_fail(e, "survivor list kernel");
  const size_t nf = (size_t)batch * p.d_ff;
  if (k > 0) {
    if (dbg->s_abs &&
        (e = hipMemcpyAsync(dbg->s_abs, b.sabs, nf * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "copy |s~|");
    if (batch == 1 && p.use_fused) {
      // the persistent kernel keeps per-range masks and s by channel
      int *selp = dbg->sel ? (int *)dbg->sel : b.sel;
      if ((dbg->sel || dbg->s_sel || dbg->n_sel) &&
          (e = prox::launch_fused_list(p, b, k, selp, (float *)dbg->s_sel, (int *)dbg->n_sel,
                                       s)) != hipSuccess)
        return hip_fail(e, "list kernel");
      return PROX_OK;
    }
    if (dbg->sel &&
        (e = hipMemcpyAsync(dbg->sel, b.sel, nf * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "copy sel");
    if (batch == 1 && dbg->s_sel &&
        (e = hipMemcpyAsync(dbg->s_sel, b.ssp, nf * 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "copy s");
    if (batch > 1) {
      if (dbg->n_union &&
          (e = hipMemcpyAsync(dbg->n_union, b.nuni, 4, hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return hip_fail(e, "copy union size");
      if (dbg->union_idx &&
          (e = hipMemcpyAsync(dbg->union_idx, b.uni, (size_t)p.d_ff * 4,
                              hipMemcpyDeviceToDevice, s)) != hipSuccess)
        return hip_fail(e, "copy union");
      // s is kept as [channel][token] (mode 3) or [union position][token]
      // (mode 1), row stride nbp: copied out token-major by union position
      if (dbg->s_sel &&
          (e = prox::launch_union_s(p, b, batch, !(p.bf16 && p.batch_mfma), (float *)dbg->s_sel,
                                    s)) != hipSuccess)
        return hip_fail(e, "copy s");
    }
  }
  return PROX_OK;
}

prox_status prox_read_status(const prox_layer *layer, int32_t *status, void *stream) {
  g_err.clear();
  if (!layer || !status) return fail(PROX_EINVAL, "layer and status are required");
  if (!aligned(status, 4)) return fail(PROX_EINVAL, "status must be 4-byte aligned");
  hipError_t e = prox::launch_read_status(layer->plan, layer->bufs, (int *)status,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "status kernel");
  return PROX_OK;
}

prox_status prox_set_wait_limit(prox_layer *layer, uint32_t polls) {
  g_err.clear();
  if (!layer) return fail(PROX_EINVAL, "layer is NULL");
  layer->plan.wait_limit = polls;
  return PROX_OK;
}

static prox_status check_ts_args(const prox_layer *layer, const void *x, float threshold_x,
                                 float threshold_s, const void *y) {
  prox_status st = check_forward_args(layer, x, 1, threshold_x, 0, y);
  if (st != PROX_OK) return st;
  if (isnan(threshold_s)) return fail(PROX_EINVAL, "threshold_s is NaN");
  if (!layer->plan.use_fused)
    return fail(PROX_EUNSUPPORTED,
                "the Stage 2 threshold mask runs on the persistent kernel only (layer prepared "
                "with path = PROX_PATH_MULTI)");
  return PROX_OK;
}

prox_status prox_ffn_forward_ts(const prox_layer *layer, const void *x, float threshold_x,
                                float threshold_s, void *y, void *stream) {
  g_err.clear();
  prox_status st = check_ts_args(layer, x, threshold_x, threshold_s, y);
  if (st != PROX_OK) return st;
  prox::FusedOpts o;
  o.ts_mode = true;
  o.tau_s = threshold_s;
  hipError_t e = prox::launch_fused(layer->plan, layer->bufs, x, threshold_x, 0, y, nullptr,
                                    (hipStream_t)stream, o);
  if (e != hipSuccess) return hip_fail(e, "fused kernel");
  return PROX_OK;
}

prox_status prox_ffn_forward_ts_debug(const prox_layer *layer, const void *x, float threshold_x,
                                      float threshold_s, void *y, const prox_debug *dbg,
                                      void *stream) {
  g_err.clear();
  prox_status st = check_ts_args(layer, x, threshold_x, threshold_s, y);
  if (st != PROX_OK) return st;
  if (!dbg) return fail(PROX_EINVAL, "dbg is NULL");
  if ((dbg->n1 != nullptr) != (dbg->idx != nullptr))
    return fail(PROX_EINVAL, "n1 and idx must be given together");
  hipStream_t s = (hipStream_t)stream;
  const prox::Plan &p = layer->plan;
  const prox::Bufs &b = layer->bufs;
  hipError_t e = hipSuccess;
  if (dbg->status &&
      (e = hipMemsetAsync(b.sync + prox::kFusedErrWord, 0, sizeof(unsigned), s)) != hipSuccess)
    return hip_fail(e, "clear status");
  prox::FusedOpts o;
  o.ts_mode = true;
  o.tau_s = threshold_s;
  o.dbg = dbg->idx != nullptr;
  if ((e = prox::launch_fused(p, b, x, threshold_x, 0, y, nullptr, s, o)) != hipSuccess)
    return hip_fail(e, "fused kernel");
  if (dbg->status &&
      (e = hipMemcpyAsync(dbg->status, b.sync + prox::kFusedErrWord, sizeof(unsigned),
                          hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return hip_fail(e, "copy status");
  // the survivors as the persistent kernel's Stage 1 items decided them
  if (dbg->idx && (e = prox::launch_survivors(p, b, 1, dbg->n1, dbg->idx, s)) != hipSuccess)
    return hip_fail(e, "survivor list kernel");
  if (dbg->s_abs && (e = hipMemcpyAsync(dbg->s_abs, b.sabs, (size_t)p.d_ff * 4,
                                        hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return hip_fail(e, "copy |s~|");
  int *selp = dbg->sel ? (int *)dbg->sel : b.sel;
  if ((dbg->sel || dbg->s_sel || dbg->n_sel) &&
      (e = prox::launch_fused_list(p, b, p.d_ff, selp, (float *)dbg->s_sel, (int *)dbg->n_sel,
                                   s)) != hipSuccess)
    return hip_fail(e, "list kernel");
  return PROX_OK;
}

prox_status prox_stage1(const prox_layer *layer, const void *x, float threshold, float *s_abs,
                        void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, 1, threshold, 0, x);
  if (st != PROX_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = prox::launch_proxy(layer->plan, layer->bufs, x, 1, threshold, s);
  if (e != hipSuccess) return hip_fail(e, "stage 1 proxy kernel");
  if (s_abs && (e = hipMemcpyAsync(s_abs, layer->bufs.sabs, (size_t)layer->plan.d_ff * 4,
                                   hipMemcpyDeviceToDevice, s)) != hipSuccess)
    return hip_fail(e, "copy |s~|");
  return PROX_OK;
}

size_t prox_sparse_gemv_workspace_bytes(int d_model, int d_ff) {
  if (d_model <= 0 || d_ff <= 0) return 0;
  return prox::sgemv_workspace_bytes(d_model, d_ff);
}

prox_status prox_sparse_gemv(const void *w_up, const void *w_gate, int d_model, int d_ff,
                             const void *x, float threshold, float *u, float *g, void *workspace,
                             void *stream) {
  g_err.clear();
  if (!w_up || !w_gate || !x || !u || !g || !workspace)
    return fail(PROX_EINVAL, "all pointers are required");
  if (d_model <= 0 || d_model % 64 != 0 || d_model > prox::kMaxDmodel)
    return fail(PROX_EINVAL, "d_model must be a positive multiple of 64, at most %d",
                prox::kMaxDmodel);
  if (d_ff <= 0 || d_ff % 8 != 0 || d_ff > prox::kMaxDff)
    return fail(PROX_EINVAL, "d_ff must be a positive multiple of 8, at most %d", prox::kMaxDff);
  if ((size_t)d_model * d_ff * 2 > 0xffffffffull)
    return fail(PROX_EUNSUPPORTED, "one weight matrix must be below 4 GiB");
  if (isnan(threshold)) return fail(PROX_EINVAL, "threshold is NaN");
  if (!aligned(w_up, 16) || !aligned(w_gate, 16) || !aligned(x, 16) || !aligned(workspace, 256))
    return fail(PROX_EINVAL, "weights and x must be 16-byte, workspace 256-byte aligned");
  hipError_t e = prox::launch_sgemv(w_up, w_gate, d_model, d_ff, x, threshold, u, g, workspace,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sparse gemv kernel");
  return PROX_OK;
}

prox_status prox_dense_ffn_forward(const prox_layer *layer, const void *x, int batch,
                                   void *y, void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, batch, 0.0f, 0, y);
  if (st != PROX_OK) return st;
  return run_dense(layer, x, batch, y, nullptr, (hipStream_t)stream);
}

prox_status prox_stack_forward(const prox_layer *const *layers, int n_layers,
                               const float *thresholds, int k, float *resid, int batch,
                               float eps, void *stream) {
  g_err.clear();
  if (!layers || n_layers <= 0 || !resid)
    return fail(PROX_EINVAL, "layers, n_layers > 0 and resid are required");
  if (k >= 0 && !thresholds) return fail(PROX_EINVAL, "thresholds are required when k >= 0");
  if (!(eps >= 0.0f)) return fail(PROX_EINVAL, "eps must be >= 0");
  if (!aligned(resid, 16)) return fail(PROX_EINVAL, "resid must be 16-byte aligned");
  const prox::Plan &p0 = layers[0] ? layers[0]->plan : prox::Plan{};
  for (int l = 0; l < n_layers; ++l) {
    const prox_layer *L = layers[l];
    if (!L) return fail(PROX_EINVAL, "layer %d is NULL", l);
    if (L->plan.d_model != p0.d_model || L->plan.bf16 != p0.bf16)
      return fail(PROX_EINVAL, "layer %d has a different d_model or dtype", l);
    if (batch < 1 || batch > L->plan.max_batch)
      return fail(PROX_EINVAL, "batch %d outside [1, max_batch] of layer %d", batch, l);
    if (k > L->plan.d_ff) return fail(PROX_EINVAL, "k=%d above d_ff of layer %d", k, l);
    if (k >= 0 && isnan(thresholds[l])) return fail(PROX_EINVAL, "threshold %d is NaN", l);
  }
  hipStream_t s = (hipStream_t)stream;
  for (int l = 0; l < n_layers; ++l) {
    const prox_layer *L = layers[l];
    hipError_t e;
    if (batch == 1 && k > 0 && L->plan.use_fused && prox::fused_norm_supported(L->plan)) {
      // one launch per layer: the persistent kernel forms x = RMSNorm(r)
      // itself, then adds y to r
      prox::FusedOpts o;
      o.norm_r = resid;
      o.eps = eps;
      o.xout = L->bufs.xbuf;
      e = prox::launch_fused(L->plan, L->bufs, L->bufs.xbuf, thresholds[l], k, L->bufs.ybuf,
                             resid, s, o);
      if (e != hipSuccess) return hip_fail(e, "fused kernel");
      continue;
    }
    e = prox::launch_rmsnorm(L->plan, resid, batch, eps, L->bufs.xbuf, s);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel");
    prox_status st = (k < 0) ? run_dense(L, L->bufs.xbuf, batch, L->bufs.ybuf, resid, s)
                             : run_forward(L, L->bufs.xbuf, batch, thresholds[l], k,
                                           L->bufs.ybuf, resid, s);
    if (st != PROX_OK) return st;
  }
  return PROX_OK;
}

prox_status prox_stack_forward_ts(const prox_layer *const *layers, int n_layers,
                                  const float *thresholds_x, const float *thresholds_s,
                                  float *resid, float eps, void *stream) {
  g_err.clear();
  if (!layers || n_layers <= 0 || !resid || !thresholds_x || !thresholds_s)
    return fail(PROX_EINVAL, "layers, n_layers > 0, both threshold arrays and resid are required");
  if (!(eps >= 0.0f)) return fail(PROX_EINVAL, "eps must be >= 0");
  if (!aligned(resid, 16)) return fail(PROX_EINVAL, "resid must be 16-byte aligned");
  const prox::Plan &p0 = layers[0] ? layers[0]->plan : prox::Plan{};
  for (int l = 0; l < n_layers; ++l) {
    const prox_layer *L = layers[l];
    if (!L) return fail(PROX_EINVAL, "layer %d is NULL", l);
    if (L->plan.d_model != p0.d_model || L->plan.bf16 != p0.bf16)
      return fail(PROX_EINVAL, "layer %d has a different d_model or dtype", l);
    if (!L->plan.use_fused)
      return fail(PROX_EUNSUPPORTED, "layer %d was prepared with path = PROX_PATH_MULTI", l);
    if (isnan(thresholds_x[l]) || isnan(thresholds_s[l]))
      return fail(PROX_EINVAL, "threshold of layer %d is NaN", l);
  }
  hipStream_t s = (hipStream_t)stream;
  for (int l = 0; l < n_layers; ++l) {
    const prox_layer *L = layers[l];
    hipError_t e;
    prox::FusedOpts o;
    o.ts_mode = true;
    o.tau_s = thresholds_s[l];
    if (prox::fused_norm_supported(L->plan)) {
      o.norm_r = resid;  // x = RMSNorm(r) formed inside the one launch
      o.eps = eps;
      o.xout = L->bufs.xbuf;
    } else if ((e = prox::launch_rmsnorm(L->plan, resid, 1, eps, L->bufs.xbuf, s)) !=
               hipSuccess) {
      return hip_fail(e, "rmsnorm kernel");
    }
    e = prox::launch_fused(L->plan, L->bufs, L->bufs.xbuf, thresholds_x[l], 0, L->bufs.ybuf, resid,
                           s, o);
    if (e != hipSuccess) return hip_fail(e, "fused kernel");
  }
  return PROX_OK;
}

prox_status prox_ffn_forward_profiled(const prox_layer *layer, const void *x, int batch,
                                      float threshold, int k, void *y,
                                      void *const *events, int n_events, int *n_recorded,
                                      void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, batch, threshold, k, y);
  if (st != PROX_OK) return st;
  if (!events || n_events < 5 || !n_recorded)
    return fail(PROX_EINVAL, "events (at least 5) and n_recorded are required");
  EventLog lg{events, n_events, 0};
  st = run_forward(layer, x, batch, threshold, k, y, nullptr, (hipStream_t)stream, &lg);
  *n_recorded = lg.n;
  return st;
}

prox_status prox_ffn_forward_traced(const prox_layer *layer, const void *x, float threshold,
                                   int k, void *y, unsigned long long *trace, int trace_items,
                                   int *counts, void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, 1, threshold, k, y);
  if (st != PROX_OK) return st;
  const prox::Plan &p = layer->plan;
  if (!p.use_fused) return fail(PROX_EUNSUPPORTED, "the layer does not use the persistent kernel");
  if (k == 0) return fail(PROX_EINVAL, "k = 0 launches no persistent kernel");
  if (!counts) return fail(PROX_EINVAL, "counts is NULL");
  const int n_p1 = p.ntile * p.nchunk, n_p3 = prox::fused_p3_items(p);
  const int total = prox::fused_items(p, false);
  counts[0] = n_p1;
  counts[1] = 1;
  counts[2] = n_p3;
  counts[3] = total - n_p1 - 1 - n_p3;
  if (!trace) return PROX_OK;  // size query
  if (trace_items < total)
    return fail(PROX_EINVAL, "trace holds %d items, the launch has %d", trace_items, total);
  if (!aligned(trace, 16)) return fail(PROX_EINVAL, "trace must be 16-byte aligned");
  prox::FusedOpts o;
  o.trace = trace;
  hipError_t e = prox::launch_fused(p, layer->bufs, x, threshold, k, y, nullptr,
                                    (hipStream_t)stream, o);
  if (e != hipSuccess) return hip_fail(e, "fused kernel");
  return PROX_OK;
}

prox_status prox_dense_ffn_forward_profiled(const prox_layer *layer, const void *x,
                                            int batch, void *y, void *const *events,
                                            int n_events, int *n_recorded, void *stream) {
  g_err.clear();
  prox_status st = check_forward_args(layer, x, batch, 0.0f, 0, y);
  if (st != PROX_OK) return st;
  if (!events || n_events < 3 || !n_recorded)
    return fail(PROX_EINVAL, "events (at least 3) and n_recorded are required");
  EventLog lg{events, n_events, 0};
  st = run_dense(layer, x, batch, y, nullptr, (hipStream_t)stream, &lg);
  *n_recorded = lg.n;
  return st;
}

prox_status prox_rmsnorm(const prox_layer *layer, const float *resid, int batch, float eps,
                         void *x, void *stream) {
  g_err.clear();
  if (!layer || !resid || !x) return fail(PROX_EINVAL, "layer, resid and x are required");
  if (batch < 1 || batch > prox::kMaxBatch)
    return fail(PROX_EINVAL, "batch %d outside [1, %d]", batch, prox::kMaxBatch);
  if (!(eps >= 0.0f)) return fail(PROX_EINVAL, "eps must be >= 0");
  hipError_t e = prox::launch_rmsnorm(layer->plan, resid, batch, eps, x, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel");
  return PROX_OK;
}

void prox_destroy_layer(prox_layer *layer) { delete layer; }

}  // extern "C"
