// Internal declarations shared by the kernel and ABI translation units of
// libprox.  Not part of the public interface (include/prox.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace prox {

// Proxy (Stage 1) column tile: 256 intermediate channels.  For one tile and
// one input row the INT4 codes of W_up (128 bytes) and W_gate (128 bytes) sit
// side by side, so a surviving row is one contiguous 256-byte read and a
// pruned row is skipped whole.
constexpr int kTile = 256;
constexpr int kTileBytes = 256;
// Output columns handled by one down-projection work-group.
constexpr int kDownCols = 256;
constexpr int kMaxBatch = 8;
constexpr int kMaxDff = 32768;
constexpr int kMaxDmodel = 16384;
// LDS a work-group may hold (gfx950: 160 KiB per compute unit).
constexpr size_t kMaxLds = 160 * 1024;
// Threads of a work-group that normalizes one residual row (RMSNorm); the
// persistent kernel normalizes with the same count, hence the same bits.
constexpr int kRmsThreads = 512;

// Device buffers of one layer (all owned by the caller).
struct Bufs {
  // weights_buf
  void *wug;       // [d_ff][2][d_model] dtype: channel j's up row, then gate row
  void *wd;        // [d_model/256][d_ff][256] dtype: W_down in 256-column chunks
  // proxy_buf
  uint8_t *pq;     // [ntile][d_model][256] bytes: (code + 8) nibbles, up | gate
  unsigned *pq2;   // [ntile][d_model/8][512] words: the same codes, 8 rows of one
                   //     proxy column per word (proxy_mfma layers only)
  float *psc;      // [ntile][ngroups][2][256] float32 scales
  unsigned *pred;  // [1] layer state kept across calls: b* of the last batch-1
                   //     top-k call + 1 (0: none), a guess of the next cut
  // workspace_buf
  float *part;     // [ntile][nchunk][batch][512]   Stage 1 partial sums
  unsigned *tile_cnt;  // [ntile]                  Stage 1 arrival counters
  float *sabs;     // [batch][d_ff]                 |s~|
  int *sel;        // [batch][d_ff]                 top-k channels, ascending
  unsigned *selw;  // [batch][ceil(d_ff/32)]        the same masks as bit words
  float *ssp;      // [d_ff][nbp]                   exact s by list position and token
                   //   (nbp = 1 for one token, else batch rounded up to 4)
  int *uni;        // [d_ff]                        union of the masks
  int *nuni;       // [1]
  uint8_t *umask;  // [d_ff]                        token bits per union entry
  float *ypart;    // [nrc][batch][d_model]         Stage 2 down partial sums
  unsigned *col_cnt;  // [ncol]                    Stage 2 arrival counters
  unsigned *ucnt;  // [1]                           top-k work-groups done (several tokens)
  unsigned *sync;  // fused kernel: tickets, flags, histogram, masks (fused_sync_words)
  void *xbuf;      // [batch][d_model] dtype         stack: normalized input
  void *ybuf;      // [batch][d_model] dtype         stack: layer output
  int *drows;      // [batch][d_model]               debug: Stage 1 survivors per 64-row slice
  int *dcnt;       // [batch][d_model / 64]          debug: their counts
};

struct Plan {
  int d_model, d_ff, G, bf16, max_batch;
  int esz;          // bytes per element
  int ngroups;      // d_model / G
  int ntile;        // ceil(d_ff / 256)
  int nchunk;       // ceil(d_model / 512): proxy work-groups per tile
  int ncol;         // d_model / 256
  int nrc;          // row chunks of the down projection
  int upgate_cap;   // max work-groups of the up/gate kernel
  int use_fused;    // batch-1 forwards run the persistent fused kernel
  int act;          // gate activation: 0 SiLU, 1 GELU (tanh form)
  int batch_mfma;   // bf16 batches of 2..8 tokens: up/gate on MFMA (default: VALU dot2)
  int proxy_mfma;   // bf16 batches of 2..8 tokens: Stage 1 on MFMA over pq2 (0: VALU)
  unsigned wait_limit;  // polls before a bounded wait of the persistent kernel gives up
};

// Kernel choices of a layer (the prox_shape fields beyond the sizes).
struct PlanChoice {
  int path = 0;          // 0 persistent kernel for batch 1, 1 four kernels
  int batch_stage1 = 0;  // 0 auto, 1 VALU, 2 MFMA
  int batch_upgate = 0;  // 0 auto (VALU), 1 VALU, 2 MFMA
};
constexpr unsigned kDefaultWaitLimit = 1u << 22;

// Workspace: the synchronisation block first, at a fixed size for the
// largest supported shape (so layers of any shapes can share one workspace:
// everything a launch expects to find zero, or leaves for the next launch,
// is in it), then per-call scratch that every call writes before it reads.
struct Layout {
  size_t weights, proxy, workspace;
  size_t o_wd, o_psc, o_pred, o_pq2;
  size_t o_sync, o_tile_cnt, o_col_cnt, o_ucnt, hdr;  // synchronisation block
  size_t o_part, o_sabs, o_sel, o_selw, o_ssp, o_uni, o_nuni, o_umask, o_ypart, o_xbuf,
      o_ybuf, o_drows, o_dcnt;
};

Plan make_plan(int d_model, int d_ff, int G, int bf16, int max_batch, int act,
               const PlanChoice &ch = PlanChoice());
Layout make_layout(const Plan &p);
// Bytes of the synchronisation block at the start of every workspace.
size_t sync_block_bytes();

// Kernel launchers (prox_kernels.hip).  Each returns hipSuccess or the launch
// error.  `batch` is the number of tokens (1..kMaxBatch).
hipError_t launch_prepare(const Plan &p, const Bufs &b, const void *w_up,
                          const void *w_gate, const void *w_down,
                          hipStream_t s);
hipError_t launch_export_proxy(const Plan &p, const Bufs &b, int matrix,
                               int8_t *codes, float *scales, hipStream_t s);
// dbg: the Stage 1 kernel also writes each token's survivors per 64-row
// slice (the m_x decision it took) into b.drows / b.dcnt.
hipError_t launch_proxy(const Plan &p, const Bufs &b, const void *x, int batch,
                        float tau, hipStream_t s, bool dbg = false);
// lists: the per-token lists (sel); union_list (several tokens): the union
// list uni / nuni / umask, built by the last work-group (mode 1 of Stage 2
// and the debug entry need it; mode 3 does not).
hipError_t launch_topk(const Plan &p, const Bufs &b, int batch, int k, bool lists,
                       bool union_list, hipStream_t s);
// mode: 0 = one token over sel, 1 = batch over the union list, 2 = dense,
// 3 = batch over the tokens' mask words (no union list; s by channel; the
// VALU forms only)
hipError_t launch_upgate(const Plan &p, const Bufs &b, const void *x, int batch,
                         int mode, int n, hipStream_t s);
hipError_t launch_down(const Plan &p, const Bufs &b, int batch, int mode, int n,
                       void *y, float *resid, hipStream_t s);
// The per-slice survivor lists a Stage 1 kernel wrote (b.drows, b.dcnt)
// assembled into n1[batch] and the ascending idx[batch][d_model].
hipError_t launch_survivors(const Plan &p, const Bufs &b, int batch, int *n1, int *idx,
                            hipStream_t s);
// Debug: out[t][p] = s of token t at union entry p (0 past the union), from
// b.ssp kept by channel (mode 3) or by union position (mode 1).
hipError_t launch_union_s(const Plan &p, const Bufs &b, int batch, bool by_channel, float *out,
                          hipStream_t s);
// Copy the workspace status word to *out and clear it; after a timed-out
// wait (bit 0) also reset the synchronisation block and the layer's cut guess.
hipError_t launch_read_status(const Plan &p, const Bufs &b, int *out, hipStream_t s);
hipError_t launch_rmsnorm(const Plan &p, const float *resid, int batch,
                          float eps, void *x, hipStream_t s);
hipError_t launch_zero_y(const Plan &p, void *y, int batch, hipStream_t s);
// Zero `bytes` (a multiple of 4) at p with a fill kernel.
hipError_t launch_zero_bytes(void *p, size_t bytes, hipStream_t s);

// Size of the static device scratch of prox_ffn_forward_noalloc: the
// batch-1 per-call buffers of layers up to the 70B shape (8192 x 28672).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;

// The batch-1 step as one persistent kernel (prox_fused.hip).
bool fused_supported(const Plan &p);
size_t fused_sync_words();  // words of the fused kernel's block (for the largest shape)
int fused_ypart_rows(const Plan &p);  // partial-y rows the fused kernel needs
// trace: optional [fused_items][4] u64 timeline (start, wait end, end,
// block | phase << 32).  ts_mode: Stage 2 mask |s~| >= tau_s instead of top-k
// (k is then unused).
// norm: when norm.r is set, x is not read; the kernel forms x = RMSNorm(r)
// itself (batch 1, x of at most 32 KiB, bit-identical to launch_rmsnorm) and
// writes it to norm.xout.
struct FusedOpts {
  unsigned long long *trace = nullptr;
  bool ts_mode = false;
  float tau_s = 0.0f;
  const float *norm_r = nullptr;  // RMSNorm input (float32 residual), or null
  float eps = 0.0f;
  void *xout = nullptr;           // where the normalized x is written
  bool dbg = false;               // Stage 1 survivor lists into b.drows / b.dcnt
};
hipError_t launch_fused(const Plan &p, const Bufs &b, const void *x, float tau, int k, void *y,
                        float *resid, hipStream_t s, const FusedOpts &o = FusedOpts());
// Can launch_fused normalize x itself for this layer?
bool fused_norm_supported(const Plan &p);
int fused_items(const Plan &p, bool ts_mode);
int fused_p3_items(const Plan &p);

// Input-sparse bf16 GEMV of the up and gate projections (prox_sgemv.hip).
size_t sgemv_workspace_bytes(int d_model, int d_ff);
hipError_t launch_sgemv(const void *w_up, const void *w_gate, int d_model, int d_ff, const void *x,
                        float tau, float *u, float *g, void *workspace, hipStream_t s);
// After a fused forward: the ascending kept-channel list and its exact s (at
// most cap entries each; ssel and count may be null; count gets the number
// of kept channels).
hipError_t launch_fused_list(const Plan &p, const Bufs &b, int cap, int *sel, float *ssel,
                             int *count, hipStream_t s);
// Words between two control words of the fused kernel (one 256-byte line each).
#ifndef PROX_SYNC_STRIDE
#define PROX_SYNC_STRIDE 64
#endif
constexpr int kSyncStride = PROX_SYNC_STRIDE;
constexpr int kFusedErrWord = 4 * kSyncStride;  // index of the sticky error word in Bufs::sync

}  // namespace prox
