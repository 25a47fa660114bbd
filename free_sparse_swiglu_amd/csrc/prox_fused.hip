// The batch-1 Prox FFN step as one persistent kernel for CDNA4 (gfx950).
//
// Method: "Prox: Training-Free FFN Activation Sparsity via Approximate
// Intermediate-Channel Salience in LLMs" (arXiv 2607.27591): Sec. 4.1
// (Stage 1 input mask and INT4 proxy, Stage 2 exact sparse computation),
// Sec. 4.3 (fused kernels), App. A.6 (top-k mask).
//
// Four dependent phases run inside one launch, so HBM never drains between
// them:
//   P1  Stage 1 proxy, one item per (256-column tile, 512-row chunk); the
//       last item of a tile also adds the tile's digit-1 counts of |s~| to a
//       global histogram;
//   P2  the top-k threshold (one item): the histogram gives the digit-1 bin
//       b* of the k-th key, which is published at once; the keys in that bin
//       then give the exact k-th key T and the tie cutoff J;
//   P3  Stage 2 up/gate + SwiGLU, one item per 32 consecutive channels: the
//       channels with digit 1 above b* (selected whatever T is) and those in
//       bin b* (about twice as many as will be kept), so nothing waits for T.
//       Once the layer has run a top-k call, an item does not wait for b*
//       either: as soon as its Stage 1 tile is done it computes every channel
//       above the previous call's b* (a guess of the cut kept per layer),
//       then, when b* is out, any channel of digit 1 >= b* that
//       the guess missed.  The guess moves work earlier; it never changes
//       which channels are kept or any value;
//   P4  Stage 2 down projection, one item per (512 channels, 256 columns):
//       with T and J known, the kept channels of the range, ascending, give a
//       partial y; the last item of a column chunk adds the partials in range
//       order.
// The selection of channel j is: |s~_j| > T, or |s~_j| = T and j <= J (the
// lowest-index channels win ties), which keeps exactly k channels.
//
// Items are numbered (tickets) in exactly that order.  The grid never exceeds
// the number of work-groups the GPU holds at once, so every work-group is
// resident; work-group b starts on ticket b (a Stage 1 item) and then takes
// tickets from a global counter.  An item only ever waits for items with
// smaller tickets (P2 for all of P1, P3 for its P1 tile and P2, P4 for P2 and
// the P3 items of its range); those are held by running work-groups, and P1 items wait
// for nothing, so the schedule cannot deadlock.  Every wait is bounded.  Data
// passed between work-groups goes through agent-coherent accesses
// (xstore/xload, sc1 buffer loads).  The flags of consecutive launches
// alternate between two halves of the sync words, each launch clearing the
// half it does not use (the select clears the histogram as soon as it has
// read it).  A P4 item waits for the s of each channel it lists itself: a
// Stage 1 item marks its tile's s as not yet computed before the tile's
// arrival, and the P3 item's store of s is the signal (no P3 flag and no
// wait for its stores to land).
#include <atomic>
#include <type_traits>

#include "prox_device.h"

namespace prox {

// Sync words at the start of the fused workspace block.  Each control word
// and each tile flag sits on its own 256-byte line (kSyncStride words), so
// that polling one flag does not contend with the atomics on another.
//
// Every per-launch word comes twice, as two halves: words 0 (and 1) of its
// line for launches of parity 0, words 2 (and 3) for parity 1.  A launch
// works in the half of its parity, whose words are all zero when it starts,
// and each of its work-groups clears a small share of the other half (the
// previous launch's) as it leaves, rather than the last one resetting every
// word on its way out.  The parity is bit 31 of the ticket count, which
// the last draw of a launch resets with the bit flipped (and of a word of its
// own, which the work-groups that start without a draw read).
enum : int {
  kSyncTicket = 0 * kSyncStride,  // ticket draws (bits 0..30) and the launch parity (bit 31)
  kSyncTiles = 1 * kSyncStride,   // P1 tiles finished
  kSyncSelect = 2 * kSyncStride,  // one 64-bit word: T (low), J + 1 (high; 0 until published);
                                  // T, J of the last top-k launch at +4, +5 (kept)
  kSyncInv = 3 * kSyncStride,     // in-kernel RMSNorm: bits of 1/rms(r) once known (0 before)
  kSyncErr = 4 * kSyncStride,     // sticky error bits (1: a wait timed out, 2: select fallback used)
  kSyncBin = 5 * kSyncStride,     // b* + 1 once published (0 before)
  kSyncPar = 6 * kSyncStride,     // the launch parity again (bit 31), read by the first items
  kSyncCtl = 7 * kSyncStride      // control words end here (the tile flags follow)
};
static_assert(kSyncErr == kFusedErrWord, "error word index");

constexpr int kFW = 8;             // waves per work-group
constexpr int kFT = kFW * 64;      // threads per work-group
constexpr int kWaveCand = 192;     // top-k candidates per wave held in LDS (fast path)
constexpr int kPreSlots = 28;      // key slots the select can hold in LDS: d_ff <= 28 * 512
constexpr int kMaxPer = 64;        // key slots per thread: d_ff <= 64 * 512
constexpr int kGroups = kMaxPer * kFW;  // groups of 64 channels: d_ff <= 512 * 64
constexpr int kKC = 32;            // key slots loaded per round of a select pass
constexpr int kP3Ch = 32;          // channels per P3 item (at most 64: one per lane of a mask)
constexpr int kP4Ch = 512;         // channels per P4 item (kP4Ch / kP3Ch P3 items)
constexpr int kSelBits = 16;       // buffer-load aux bit: sc1 (agent-coherent)
constexpr unsigned kSNone = 0xffffffffu;  // s of a channel not yet computed in this launch (a NaN)

struct FusedArgs {
  const uint8_t *pq;
  const float *psc;
  const void *wug;
  uint32_t wug_bytes;
  const void *wd;
  int d_model, d_ff, G, ngroups, ntile, nchunk, ncol, nrange;
  const void *x;
  float tau;
  int k;
  void *y;
  float *resid;
  float *part;
  float *sabs;
  float *sdense;    // [d_ff] exact s of each kept channel (others stale)
  float *ypart;
  unsigned *col_cnt;
  unsigned *sync;
  unsigned *tflag;  // per P1 tile t, on line t: word t * kSyncStride = |s~| written,
                    // the next word = chunks arrived (stays at nchunk); offset by the
                    // launch's half
  unsigned *ghist;  // [2048] digit-1 histogram of |s~| (zero between launches)
  unsigned *gmask;  // [n_p3][4] per P3 item: 64-bit masks of the channels above bin b*
                    // and of those in it (low word first)
  unsigned *pred;   // per layer, kept across calls: b* of the last top-k call + 1 (0: none)
  const float *rnorm;  // when set: x = RMSNorm(rnorm) (float32 residual), formed here
  float eps;
  void *xout;          // ... and written here by the tile-0 Stage 1 items
  int ts_mode;      // 1: Stage 2 mask |s~| >= tau_s instead of top-k (no P2)
  int act;          // gate activation (gate_act)
  float tau_s;
  int n_p1, n_p2, n_p3, n_p4;
  unsigned long long *trace;  // optional per-ticket timeline (nullptr: off)
  unsigned wlim;    // polls before a bounded wait gives up
  int *drows, *dcnt;  // debug: Stage 1 survivors per 64-row slice (nullptr: off)
};

// The select's result: T and J + 1 as one agent-coherent 64-bit word (J + 1
// is never 0, so a nonzero high half means published).
__device__ __forceinline__ void xstore_tj(unsigned *w, unsigned T, int J) {
  const unsigned long long v = (unsigned long long)T | ((unsigned long long)(unsigned)(J + 1) << 32);
  __hip_atomic_store((unsigned long long *)w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Bounded wait for it (like wait_geq): *T, *J receive the values.
__device__ __forceinline__ void wait_tj(const unsigned *w, unsigned *err, unsigned *T, unsigned *J,
                                        unsigned limit) {
  unsigned n = 0;
  unsigned long long v;
  while (((v = __hip_atomic_load((const unsigned long long *)w, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT)) >> 32) == 0ull) {
    __builtin_amdgcn_s_sleep(1);
    if (++n > limit) {
      atomicOr(err, 1u);
      break;
    }
  }
  *T = (unsigned)v;
  *J = (unsigned)(v >> 32) - 1u;
}


// Bounded wait of a whole wave until every lane's flag is >= 1 (lanes with
// nothing to wait for pass their own satisfied flag).
__device__ __forceinline__ void wave_wait_flags(const unsigned *f, unsigned *err, unsigned limit) {
  unsigned n = 0;
  while (!__all(xload_u(f) >= 1u)) {
    __builtin_amdgcn_s_sleep(1);
    if (++n > limit) {
      if ((threadIdx.x & 63) == 0) atomicOr(err, 1u);
      break;
    }
  }
}

// ---------------------------------------------------------------------------
// LDS of each phase (one union per work-group)
// ---------------------------------------------------------------------------
struct P1Smem {
  float red[kFW][512];
  __attribute__((aligned(16))) int rl[kFW][64 + 48];
  __attribute__((aligned(16))) float xc[kFW][64 + 48];
};
template <bool SEL>
struct P2Smem {
  // the small arrays first (LDS offsets below 64 KiB fit the instructions)
  unsigned ccnt[kFW];
  unsigned wt[16];
  unsigned misc[8];
  unsigned h[2048];
  unsigned ck[kFW * kWaveCand];  // candidate keys (per-wave lists)
  int ci[kFW * kWaveCand];       // candidate channels
  unsigned ceq[kGroups];         // per group of 64 channels: keys equal to T
  unsigned keys[SEL ? kPreSlots * kFT : 1];  // |s~| bits of channel j at j (top-k instances)
};
struct P3Smem {
  u4 x[2048];  // x when d_model * element size <= 32 KB
  float ured[2 * kP3Ch];  // dot product of each unit (row) of the item
  unsigned key[kP3Ch];    // |s~| bits of the item's channels
  unsigned lo, bstar;
};
// P4 rows (bf16, 512 bytes each) taken straight into LDS ahead of the wait,
// beyond the first batch held in registers: in the top-k instances as many
// as their LDS (sized by the select's keys) holds anyway; the threshold-mask
// instances grow theirs for 80 (measured: worth the larger LDS).
template <bool SEL>
constexpr int kP4LdsRows = SEL ? 128 : 80;
template <bool SEL>
struct P4Smem {
  unsigned wcnt[kFW];
  unsigned bstar;
  unsigned tj[2];      // T and J of the select
  float red[kFW][kDownCols];
  int rs[kP4Ch];       // listed channels
  unsigned rk[kP4Ch];  // their keys
  float sv[kP4Ch];     // their s (0 when below the cut)
  u2 rows[kP4LdsRows<SEL>][64];
};

// All of the kernel's LDS as one object, the small words first: LDS
// instructions encode offsets below 64 KiB, and a word placed past the
// 80 KB union would need an address register wherever it is used.
template <bool SEL>
struct FusedShared {
  unsigned hw;  // word offset of the launch's half in each sync line: 2 x parity
  // wave partial sums of the RMSNorm reduction (block_inv_rms); a work-group
  // of kRmsThreads, like the standalone RMSNorm kernel, gives the same bits
  float rms_part[kFW];
  // timeline stamp of the current item: when its wait for earlier items
  // ended (thread 0 only; 100 MHz s_memrealtime clock)
  unsigned long long twait;
  int ticket, flag;
  float inv;  // in-kernel RMSNorm: 1/rms(r) of the first Stage 1 item, until published
  unsigned ibits;  // in-kernel RMSNorm: the published 1/rms(r), read by an up/gate item
  union {
    P1Smem p1;
    P2Smem<SEL> p2;
    P3Smem p3;
    P4Smem<SEL> p4;
  } u;
};
static_assert(kFT == kRmsThreads, "RMSNorm reduction order");
// SEL: the instance runs the top-k select (the threshold-mask instances
// leave it out and keep the key array out of LDS).
template <bool SEL>
__shared__ FusedShared<SEL> g_fs;

template <bool SEL>
__device__ __forceinline__ void stamp_wait(const FusedArgs &a) {
  if (a.trace) g_fs<SEL>.twait = __builtin_amdgcn_s_memrealtime();
}

// |s~| of tile column col from the tile's partial sums (nchunk chunks of
// [256 up | 256 gate] floats), added in chunk order.  The tile epilogue and
// the P3 items both call this, so they get the same bits.
__device__ __forceinline__ float tile_key(const float *tp, int col, int nchunk, int act) {
  const float u = xsum_strided(&tp[col], nchunk, 512);
  const float g = xsum_strided(&tp[256 + col], nchunk, 512);
  return fabsf(u * gate_act(g, act));
}

// ---------------------------------------------------------------------------
// P1: Stage 1 for one (tile, chunk) item.  Same arithmetic as proxy_kernel
// (see there): one wave per 64-row slice, survivors by ballot, nibble pairs
// decoded under the bf16 exponent byte for bf16 layers.
// ---------------------------------------------------------------------------
// Share `q` of `nq` of the words of half `hw` that a launch may set (the
// other half of the running launch: the previous launch used it and the next
// one will): the control words and the tile flags.
constexpr int kMaxTiles = kMaxDff / kTile;
constexpr int kHalfWords = 5 + 2 * kMaxTiles;
__device__ __forceinline__ void clear_half_share(const FusedArgs &a, unsigned hw, int q, int nq) {
  const int per = (kHalfWords + nq - 1) / nq;
  for (int i = threadIdx.x; i < per; i += kFT) {
    const int e = q * per + i;
    if (e >= kHalfWords) break;
    unsigned *w;
    if (e < 5)
      w = &a.sync[e == 0 ? kSyncTiles : e == 1 ? kSyncSelect : e == 2 ? kSyncSelect + 1
                                      : e == 3 ? kSyncInv : kSyncBin];
    else
      w = &a.tflag[((e - 5) >> 1) * kSyncStride + ((e - 5) & 1)];
    xstore_u(w + hw, 0u);
  }
}

// The half of the launch is known by the partial-sum barrier: from the parity
// word `pw` that the work-group loaded as its first item started (`resolve`;
// the load is waited for only here) or from an earlier draw.
template <bool BF16, bool NORM, bool SEL>
__device__ __forceinline__ void p1_item(const FusedArgs &a, int item, P1Smem &sm, int *s_flag,
                                        unsigned pw, bool resolve) {
  constexpr int U = 16;
  // Work-group b runs on XCD b % 8.  With a multiple of 8 tiles, the chunks
  // of a tile go to one XCD: the chunks of one index then no longer all sit
  // on one XCD, whose Stage 1 items ran 2.5 us behind the others (the tiles'
  // codes are 1 MB apart, so one chunk index of every tile fell on the same
  // memory interleave).
  int t, chunk;
  if ((a.ntile & 7) == 0) {
    const int j = item >> 3;
    t = 8 * (j / a.nchunk) + (item & 7);
    chunk = j % a.nchunk;
  } else {
    chunk = item % a.nchunk;
    t = item / a.nchunk;
  }
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sl = chunk * kFW + wv;
  const int nsl = a.d_model >> 6;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  float inv = 1.0f;
  float rv = 0.0f;  // NORM: r of this thread's row of the chunk, chunk * 512 + tid
  if constexpr (NORM) {
    // loaded with the RMS pass's loads, not after it
    rv = a.rnorm[min(chunk * kFT + (int)threadIdx.x, a.d_model - 1)];
    inv = block_inv_rms<kFT>(a.rnorm, a.d_model, a.eps, g_fs<SEL>.rms_part);
    // for the Stage 2 items, which scale r by it without reducing again
    // (published at the partial-sum barrier, where the half is known)
    if (item == 0 && threadIdx.x == 0) g_fs<SEL>.inv = inv;
  }
  if (sl < nsl) {
    // the slice's scales first, so that their latency hides behind the rest
    const int g = (sl * 64) / a.G;
    const float4 *sp =
        (const float4 *)(a.psc + ((size_t)t * a.ngroups + g) * 512 + (size_t)lane * 8);
    const float4 s0 = sp[0], s1 = sp[1];
    float xl;
    uint64_t un;
    if constexpr (NORM) {
      // x_i = RMSNorm(r)_i in the layer dtype, as launch_rmsnorm stores it
      const int row = sl * 64 + lane;  // = chunk * 512 + tid
      xl = round_elem<BF16>(rv * inv);
      un = __ballot(fabsf(xl) >= a.tau);
      if (t == 0 && a.xout) st_elem<BF16>(a.xout, row, xl);
    } else {
      un = slice_mask<BF16>(a.x, (size_t)sl * 64, a.tau, xl);
    }
    if (a.drows && t == 0) export_slice(a.drows, a.dcnt, sl, un);
    const float xm = ((un >> lane) & 1ull) ? xl : 0.0f;
    const float xsum = wave_sum(xm);
    const int cnt = (int)__popcll(un);
    if ((un >> lane) & 1ull) {
      const int pos = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(un >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((unsigned)un, 0u));
      sm.rl[wv][pos] = lane;
      sm.xc[wv][pos] = xm;
    }
    if (lane < 3 * U) {
      sm.rl[wv][cnt + lane] = 0;
      sm.xc[wv][cnt + lane] = 0.0f;
    }
    __builtin_amdgcn_wave_barrier();

    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(a.pq + (size_t)t * a.d_model * kTileBytes, (uint32_t)a.d_model * kTileBytes);
    const uint32_t voff = (uint32_t)lane * 4u;
    const uint32_t sbase = (uint32_t)sl * 64u * kTileBytes;
    auto fetch = [&](int base, uint32_t (&w)[U]) {
#pragma unroll
      for (int q = 0; q < U / 4; ++q) {
        const int4 r4 = *(const int4 *)&sm.rl[wv][base + 4 * q];
        const int rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane(rr[e]);
          w[4 * q + e] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, sbase + row * kTileBytes, kNT);
        }
      }
    };
    uint32_t nib_mask;
    asm volatile("s_mov_b32 %0, 0x0f0f0f0f" : "=s"(nib_mask));
    auto consume = [&](int base, const uint32_t (&w)[U]) {
#pragma unroll
      for (int q = 0; q < U / 4; ++q) {
        const float4 x4 = *(const float4 *)&sm.xc[wv][base + 4 * q];
        if constexpr (BF16) {
          const uint32_t xp[2] = {
              (__float_as_uint(x4.x) >> 16) | (__float_as_uint(x4.y) & 0xffff0000u),
              (__float_as_uint(x4.z) >> 16) | (__float_as_uint(x4.w) & 0xffff0000u)};
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t wa = w[4 * q + 2 * h], wb = w[4 * q + 2 * h + 1];
            const uint32_t la = wa & nib_mask, ha = (wa >> 4) & nib_mask;
            const uint32_t lb = wb & nib_mask, hb = (wb >> 4) & nib_mask;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t sel = (uint32_t)i | 0x0c00u | ((uint32_t)(4 + i) << 16) | 0x0c000000u;
              const uint32_t pl = __builtin_amdgcn_perm(lb, la, sel) | 0x43004300u;
              const uint32_t ph = __builtin_amdgcn_perm(hb, ha, sel) | 0x43004300u;
              acc[2 * i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pl), as_bf16x2(xp[h]),
                                                          acc[2 * i], false);
              acc[2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ph), as_bf16x2(xp[h]),
                                                              acc[2 * i + 1], false);
            }
          }
        } else {
          const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wcur = w[4 * q + e];
            const uint32_t lo = wcur & nib_mask, hi = (wcur >> 4) & nib_mask;
            const float n[8] = {(float)(lo & 0xffu), (float)(hi & 0xffu),
                                (float)((lo >> 8) & 0xffu), (float)((hi >> 8) & 0xffu),
                                (float)((lo >> 16) & 0xffu), (float)((hi >> 16) & 0xffu),
                                (float)(lo >> 24), (float)(hi >> 24)};
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = fmaf(xs[e], n[c], acc[c]);
          }
        }
      }
    };
    uint32_t wa[U], wb[U];
    fetch(0, wa);
    for (int base = 0; base < cnt; base += 2 * U) {
      fetch(base + U, wb);
      consume(base, wa);
      fetch(base + 2 * U, wa);
      if (base + U < cnt) consume(base + U, wb);
    }
    const float off = BF16 ? 136.0f : 8.0f;
    const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = sc[c] * (acc[c] - off * xsum);
  }

  float4 *rp = (float4 *)&sm.red[wv][lane * 8];
  rp[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  rp[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (resolve && threadIdx.x == 0) g_fs<SEL>.hw = (pw >> 31) * 2u;
  __syncthreads();
  const unsigned hw = g_fs<SEL>.hw;
  if (NORM && item == 0 && threadIdx.x == 0)
    xstore_u(&a.sync[kSyncInv + hw], __float_as_uint(g_fs<SEL>.inv));
  // s of the tile's channels is marked not yet computed (before the tile's
  // arrival, so before any up/gate item of the tile can store it)
  if (chunk == 0 && threadIdx.x < kTile && t * kTile + (int)threadIdx.x < a.d_ff)
    xstore_u((unsigned *)&a.sdense[t * kTile + threadIdx.x], kSNone);
  // ... and so is this item's share of the down items' partial sums, long
  // before any down item stores one
  {
    const int tot = a.nrange * a.d_model;
    const int per = (tot + a.n_p1 - 1) / a.n_p1;
    const int e1 = min(tot, item * per + per);
    for (int e = item * per + (int)threadIdx.x; e < e1; e += kFT)
      xstore_u((unsigned *)&a.ypart[e], kSNone);
  }
  float *part = a.part + ((size_t)t * a.nchunk + chunk) * 512;
  {
    const int e = threadIdx.x;
    float v = sm.red[0][e];
#pragma unroll
    for (int q = 1; q < kFW; ++q) v += sm.red[q][e];
    xstore(&part[e], v);
  }
  // The tile's counter stays at nchunk once every chunk is in: P3 items wait
  // on it (until the half is cleared for its next use).
  if (!arrive_count(&a.tflag[t * kSyncStride + hw + 1], (unsigned)a.nchunk, s_flag)) return;
  __builtin_amdgcn_s_setprio(3);  // the tile epilogue gates the select and P3: issue first

  // Tile epilogue: |s~| = |u~ * SiLU(g~)| of the tile's 256 channels, and the
  // tile's counts of digit 1 (bits 30..20 of |s~|) added to the global
  // histogram (the partials in LDS are consumed, so it holds the counts).
  unsigned *h = (unsigned *)&sm.red[0][0];
  for (int i = threadIdx.x; i < 2048; i += kFT) h[i] = 0u;
  __syncthreads();
  const float *tp = a.part + (size_t)t * a.nchunk * 512;
  if (threadIdx.x < 256) {
    const int col = threadIdx.x;
    const float v = tile_key(tp, col, a.nchunk, a.act);
    const int j = t * kTile + col;
    if (j < a.d_ff) {
      xstore(&a.sabs[j], v);
      if (!a.ts_mode) atomicAdd(&h[__float_as_uint(v) >> 20], 1u);
    }
  }
  __syncthreads();
  if (!a.ts_mode) {
    for (int i = threadIdx.x; i < 2048; i += kFT) {
      const unsigned c = h[i];
      if (c) __hip_atomic_fetch_add(&a.ghist[i], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    xstore_u(&a.tflag[t * kSyncStride + hw], 1u);
    __hip_atomic_fetch_add(&a.sync[kSyncTiles + hw], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------------------
// P2: the top-k threshold (App. A.6, top-k equation), ties to the lower index.
// ---------------------------------------------------------------------------
// |s~| >= 0, so its float32 bits order like the value; digit 1 = bits 30..20,
// digit 2 = bits 19..9, digit 3 = bits 8..0.  Channel j is read by thread
// j % 512 in slot j / 512 and belongs to group j / 64 (one wave, one slot).
// Fast path:
//   0. while Stage 1 runs, the keys of every finished tile are copied
//      straight into LDS (d_ff <= kPreSlots * 512; larger layers copy them
//      after the histogram, kPreSlots slots at a time);
//   1. the global digit-1 histogram (built by the P1 tile epilogues) gives
//      the bin b* of the k-th largest key; b* is published for P3;
//   2. one pass over the keys in LDS gathers those with digit 1 = b*
//      (typically a few hundred) in per-wave LDS lists;
//   3. two radix steps over the gathered keys give the k-th key T and the
//      number kk of keys equal to T that are kept;
//   4. the tie cutoff J: the channel of the kk-th key equal to T in index
//      order (every key equal to T was gathered); J = d_ff - 1 when all of
//      them are kept, the usual case.
// Fallback (a wave gathers more than kWaveCand keys, e.g. massive exact
// ties): the radix steps over all keys.

// All waves: bins [NB - (t+1)*BPL, NB - t*BPL) belong to thread t (from the
// top).  Finds the bin holding the kk-th largest; 2 barriers.
template <int NBINS, typename H>
__device__ __forceinline__ void pick_bin_all(H hist, unsigned kk, unsigned *wt, unsigned *out) {
  constexpr int BPL = NBINS / kFT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hi = NBINS - 1 - tid * BPL;
  unsigned c[BPL], sum = 0;
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    c[i] = hist(hi - i);
    sum += c[i];
  }
  const unsigned incl = wave_incl_scan_dpp(sum);
  if (lane == 63) wt[w] = incl;
  __syncthreads();
  unsigned above = incl - sum;
#pragma unroll
  for (int q = 0; q < kFW; ++q) above += (q < w) ? wt[q] : 0u;
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    if (above < kk && above + c[i] >= kk) {
      out[0] = (unsigned)(hi - i);
      out[1] = kk - above;
    }
    above += c[i];
  }
  __syncthreads();
}

template <bool SEL>
__device__ __forceinline__ void p2_select(const FusedArgs &a, P2Smem<SEL> &sm) {
  // The select is on the critical path and shares its CU with P3 waves that
  // mostly wait on memory: its waves issue first.
  __builtin_amdgcn_s_setprio(3);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = a.d_ff;
  const int per = (n + kFT - 1) / kFT;
  const unsigned k = (unsigned)a.k;
  const unsigned hw = g_fs<SEL>.hw;
  // Keys in flight before the last tile is done: when every key fits the
  // LDS array (per <= kPreSlots) and every tile flag one lane (ntile <= 64),
  // each wave polls all tile flags at once and, slot by slot, copies the keys
  // of its slots whose tiles are done straight into LDS.  The keys of the
  // last tile then travel with the histogram instead of after b*.  Slot m of
  // wave w holds channels m * 512 + 64 w + lane, all in tile 2 m + w / 4
  // (the slots past d_ff read 0).
  const bool pre = per <= kPreSlots && a.ntile <= 64;
  if (pre) {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.sabs, (uint32_t)n * 4u);
    const uint32_t koff = (uint32_t)tid * 4u;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const unsigned *fl = &a.tflag[min(lane, a.ntile - 1) * kSyncStride + hw];
    uint64_t done = 0ull;  // tiles seen done (bit t), wave-uniform
    unsigned spins = 0;
#pragma unroll 1
    for (int m = 0; m < per; ++m) {
      const int tm = min(2 * m + (wu >> 2), a.ntile - 1);
      // Poll only while this slot's tile is not known to be done (a poll
      // waits for this wave's earlier copies too).
      while (!((done >> tm) & 1ull) && spins <= a.wlim) {
        const uint64_t b = __ballot(xload_u(fl) >= 1u);
        // scalar (no VGPR to wait on); readfirstlane returns int: widen unsigned
        done = ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
               (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
        if (!((done >> tm) & 1ull)) {
          __builtin_amdgcn_s_sleep(1);
          spins = __builtin_amdgcn_readfirstlane(spins + 1u);
        }
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void *)&sm.keys[m * kFT + wu * 64], 4, koff,
          (uint32_t)(m * kFT) * 4u, 0, kSelBits);
    }
    // Then the digit-1 histogram, complete once every tile is done: each
    // wave polls on until it has seen all of them and copies its share of
    // the bins (four blocks of 64) into LDS, without waiting for the others.
    const uint64_t all = a.ntile == 64 ? ~0ull : (1ull << a.ntile) - 1ull;
    while ((done & all) != all && spins <= a.wlim) {
      const uint64_t b = __ballot(xload_u(fl) >= 1u);
      done = ((uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
             (uint64_t)(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
      if ((done & all) != all) {
        __builtin_amdgcn_s_sleep(1);
        spins = __builtin_amdgcn_readfirstlane(spins + 1u);
      }
    }
    if (spins > a.wlim && lane == 0) atomicOr(&a.sync[kSyncErr], 1u);
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.ghist, 2048u * 4u);
#pragma unroll
    for (int q = 0; q < 2048 / kFT; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rh, (__attribute__((address_space(3))) void *)&sm.h[q * kFT + wu * 64], 4, koff,
          (uint32_t)(q * kFT) * 4u, 0, kSelBits);
  } else if (threadIdx.x == 0) {
    wait_geq(&a.sync[kSyncTiles + hw], (unsigned)a.ntile, &a.sync[kSyncErr], a.wlim);
  }
  if (threadIdx.x == 0) stamp_wait<SEL>(a);
  __syncthreads();
  // Keys of slots [e0, e0 + kKC): unconditional loads (indices clamped into
  // range) so that they all stay in flight; callers mask j >= n themselves.
  auto load_keys = [&](int e0, unsigned (&kc)[kKC]) {
#pragma unroll
    for (int m = 0; m < kKC; ++m) {
      const int j = min((e0 + m) * kFT + tid, n - 1);
      kc[m] = __float_as_uint(xload(&a.sabs[j]));
    }
  };
  if (!pre)
    for (int i = tid; i < 2048; i += kFT) sm.h[i] = xload_u(&a.ghist[i]);
  for (int i = tid; i < kGroups; i += kFT) sm.ceq[i] = 0u;
  wait_vmem();  // what went straight into LDS, too
  // The histogram is in LDS and nothing else reads it: clear it for the next
  // launch here rather than at the exit.
  for (int i = tid; i < 2048; i += kFT) xstore_u(&a.ghist[i], 0u);
  __syncthreads();

  // 1. the digit-1 bin of the k-th key, published at once.
  pick_bin_all<2048>([&](int b) { return sm.h[b]; }, k, sm.wt, &sm.misc[2]);
  const unsigned bstar = sm.misc[2];
  unsigned kk = sm.misc[3];
  if (tid == 0) {
    xstore_u(&a.sync[kSyncBin + hw], bstar + 1u);
    xstore_u(a.pred, bstar + 1u);  // the next call's guess of the cut bin
  }
  unsigned T;

  // 2. candidates at b*, from the keys in LDS (kPreSlots slots per round;
  // one round, already copied, on the early path).
  unsigned cbase = 0u;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  for (int e0 = 0; e0 < per; e0 += kPreSlots) {
    if (!pre) {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.sabs, (uint32_t)n * 4u);
#pragma unroll 1
      for (int m = 0; m < min(kPreSlots, per - e0); ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void *)&sm.keys[m * kFT + wu * 64], 4,
            (uint32_t)tid * 4u, (uint32_t)((e0 + m) * kFT) * 4u, 0, kSelBits);
      wait_vmem();
    }
    // Each thread marks its candidate slots in a bit mask (all LDS reads in
    // flight at once, no branches); one wave scan places them.
    static_assert(kPreSlots <= 32, "one mask bit per slot");
    unsigned msk = 0u;
#pragma unroll
    for (int m0 = 0; m0 < kPreSlots; m0 += kPreSlots / 2) {
      unsigned kv[kPreSlots / 2];
#pragma unroll
      for (int m = 0; m < kPreSlots / 2; ++m) kv[m] = sm.keys[(m0 + m) * kFT + tid];
#pragma unroll
      for (int m = 0; m < kPreSlots / 2; ++m)
        msk |= (unsigned)((e0 + m0 + m < per) & ((e0 + m0 + m) * kFT + tid < n) &
                          ((kv[m] >> 20) == bstar)) << (m0 + m);
    }
    const unsigned cnt = (unsigned)__popc(msk);
    const unsigned incl = wave_incl_scan_dpp(cnt);
    unsigned pos = cbase + incl - cnt;
    cbase += (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
    while (msk) {
      const int m = __builtin_ctz(msk);
      msk &= msk - 1u;
      if (pos < (unsigned)kWaveCand) {
        sm.ck[w * kWaveCand + pos] = sm.keys[m * kFT + tid];
        sm.ci[w * kWaveCand + pos] = (e0 + m) * kFT + tid;
      }
      ++pos;
    }
  }
  if (lane == 0) sm.ccnt[w] = cbase;
  __syncthreads();
  bool fast = true;
#pragma unroll
  for (int q = 0; q < kFW; ++q) fast = fast && sm.ccnt[q] <= (unsigned)kWaveCand;
  // candidate slot i (of kFW * kWaveCand) in use?
  auto cand = [&](int i) { return (unsigned)(i % kWaveCand) < sm.ccnt[i / kWaveCand]; };
  if (fast) {
    // 3. digits 2 and 3 over the candidates.
    for (int i = tid; i < 2048; i += kFT) sm.h[i] = 0u;
    __syncthreads();
    for (int i = tid; i < kFW * kWaveCand; i += kFT)
      if (cand(i)) atomicAdd(&sm.h[(sm.ck[i] >> 9) & 2047u], 1u);
    __syncthreads();
    pick_bin_all<2048>([&](int b) { return sm.h[b]; }, kk, sm.wt, &sm.misc[2]);
    const unsigned p2 = (bstar << 11) | sm.misc[2];
    kk = sm.misc[3];
    __syncthreads();
    for (int i = tid; i < 512; i += kFT) sm.h[i] = 0u;
    __syncthreads();
    for (int i = tid; i < kFW * kWaveCand; i += kFT)
      if (cand(i) && (sm.ck[i] >> 9) == p2) atomicAdd(&sm.h[sm.ck[i] & 511u], 1u);
    __syncthreads();
    pick_bin_all<512>([&](int b) { return sm.h[b]; }, kk, sm.wt, &sm.misc[2]);
    T = (p2 << 9) | sm.misc[2];
    kk = sm.misc[3];
    // keys equal to T, per group
    for (int i = tid; i < kFW * kWaveCand; i += kFT)
      if (cand(i) && sm.ck[i] == T) atomicAdd(&sm.ceq[sm.ci[i] >> 6], 1u);
  } else {
    // Fallback: radix over all keys (digits 11, 11, 9 bits), then the equal
    // counts per group.
    if (tid == 0) atomicOr(&a.sync[kSyncErr], 2u);
    unsigned prefix = 0u, pmask = 0u;
    kk = k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = pass == 0 ? 20 : (pass == 1 ? 9 : 0);
      const unsigned nb = pass == 2 ? 512u : 2048u;
      __syncthreads();
      for (int i = tid; i < 2048; i += kFT) sm.h[i] = 0u;
      __syncthreads();
      for (int e0 = 0; e0 < per; e0 += kKC) {
        unsigned kc[kKC];
        load_keys(e0, kc);
#pragma unroll
        for (int m = 0; m < kKC; ++m)
          if (e0 + m < per && (e0 + m) * kFT + tid < n && (kc[m] & pmask) == prefix)
            atomicAdd(&sm.h[(kc[m] >> sh) & (nb - 1u)], 1u);
      }
      __syncthreads();
      if (pass < 2)
        pick_bin_all<2048>([&](int b) { return sm.h[b]; }, kk, sm.wt, &sm.misc[2]);
      else
        pick_bin_all<512>([&](int b) { return sm.h[b]; }, kk, sm.wt, &sm.misc[2]);
      prefix |= sm.misc[2] << sh;
      pmask |= (nb - 1u) << sh;
      kk = sm.misc[3];
    }
    T = prefix;
    for (int e0 = 0; e0 < per; e0 += kKC) {
      unsigned kc[kKC];
      load_keys(e0, kc);
#pragma unroll
      for (int m = 0; m < kKC; ++m) {
        const int e = e0 + m;
        if (e < per) {
          const uint64_t me = __ballot(e * kFT + tid < n && kc[m] == T);
          if (lane == 0) sm.ceq[e * kFW + w] = (unsigned)__popcll(me);
        }
      }
    }
  }
  __syncthreads();

  // 4. tie cutoff (wave 0): the group holding the kk-th equal key, then the
  // lane inside it.
  if (w == 0) {
    constexpr int CPL = kGroups / 64;
    const int ng = per * kFW;
    unsigned ce[CPL], se = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int g = lane * CPL + i;
      ce[i] = g < ng ? sm.ceq[g] : 0u;
      se += ce[i];
    }
    const unsigned incl = wave_incl_scan_dpp(se);
    const unsigned total = __builtin_amdgcn_readlane(incl, 63);
    int J = n - 1;
    if (total > kk) {
      // group g* with eq-before < kk <= eq-before + ce, and kk's rank in it
      unsigned eb = incl - se;
      int gsel = -1;
      unsigned rin = 0;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        if (eb < kk && eb + ce[i] >= kk) {
          gsel = lane * CPL + i;
          rin = kk - eb;  // 1-based
        }
        eb += ce[i];
      }
      const uint64_t who = __ballot(gsel >= 0);
      const int src = who ? (int)__builtin_ctzll(who) : 0;
      const int g = max(__builtin_amdgcn_readlane(gsel, src), 0);
      const unsigned r1 = __builtin_amdgcn_readlane(rin, src);
      const int j = (g << 6) + lane;
      const unsigned key = __float_as_uint(xload(&a.sabs[min(j, n - 1)]));
      const uint64_t me = __ballot(j < n && key == T);
      const unsigned rank = __builtin_amdgcn_mbcnt_hi((unsigned)(me >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((unsigned)me, 0u));
      const uint64_t hit = __ballot(((me >> lane) & 1ull) && rank + 1u == r1);
      J = (who && hit) ? (g << 6) + (int)__builtin_ctzll(hit) : n - 1;
    }
    // T and J go out in one 64-bit store, which is also the flag: a waiter
    // gets both with the load that sees it, and nothing here waits for an
    // earlier store to land first.
    if (lane == 0) {
      // a copy that outlives the launch's reset, for the list kernel
      xstore_u(&a.sync[kSyncSelect + 4], T);
      xstore_u(&a.sync[kSyncSelect + 5], (unsigned)J);
      xstore_tj(&a.sync[kSyncSelect + hw], T, J);
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------------------
// P3: Stage 2a for 32 consecutive channels (Sec. 4.1, Stage 2 equations):
// for each kept channel, its exact up/gate rows (contiguous 2*d_model
// elements), dot2 with x, s = u * SiLU(g), stored by channel.  The kept
// channels are dealt to the 8 waves in ascending order.
// ---------------------------------------------------------------------------
// CH 16-byte steps of one row (byte offset base in the up/gate weights) in
// flight, then their dot products with x (from LDS when xs is given, else
// from global memory).
template <bool BF16, int CH>
__device__ __forceinline__ void p3_pass(const FusedArgs &a, const u4 *xs, __amdgpu_buffer_rsrc_t rs,
                                        uint32_t base, int m0, int lane, float &acc) {
  u4 w[CH];
#pragma unroll
  for (int m = 0; m < CH; ++m) {
    const uint32_t off = (uint32_t)((m0 + m) * 64 + lane) * 16u;
    w[m] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, base, kNT);
  }
  if (xs) {
#pragma unroll
    for (int m = 0; m < CH; ++m) acc = dot16<BF16>(w[m], xs[(m0 + m) * 64 + lane], acc);
  } else {
    u4 xr[CH];
#pragma unroll
    for (int m = 0; m < CH; ++m) xr[m] = ((const u4 *)a.x)[(m0 + m) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < CH; ++m) acc = dot16<BF16>(w[m], xr[m], acc);
  }
}

// Dot product of x with one whole row of the up/gate weights.  One 16-byte
// step covers 64 lanes x 16 bytes of a row; d_model * ESZ is a multiple of
// 1024, so the steps tile the row exactly.  A pass keeps 4 steps (4 KB per
// wave) in flight: P3 runs while Stage 1, the select and P4 wait on chains
// of dependent memory round trips, and every byte P3 keeps in flight
// lengthens those round trips without adding bandwidth (HBM is already
// saturated).  Measured at 8B: 2 rows x 8 KB per wave 46.0 us, 1 row x 8 KB
// 45.0 us, 1 row x 4 KB 44.3 us, 1 row x 2 KB 45.6 us.
template <bool BF16>
__device__ __forceinline__ float p3_row(const FusedArgs &a, const u4 *xs, uint32_t base, int lane) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.wug, a.wug_bytes);
  const int nstep = (int)(((uint32_t)a.d_model * (BF16 ? 2u : 4u)) >> 10);
  float acc = 0.0f;
  int m0 = 0;
  for (; m0 + 4 <= nstep; m0 += 4) p3_pass<BF16, 4>(a, xs, rs, base, m0, lane, acc);
  if (m0 + 2 <= nstep) {
    p3_pass<BF16, 2>(a, xs, rs, base, m0, lane, acc);
    m0 += 2;
  }
  if (m0 < nstep) p3_pass<BF16, 1>(a, xs, rs, base, m0, lane, acc);
  return wave_sum(acc);
}

// The i-th set bit (0-based) of a wave-uniform mask, found by all lanes.
__device__ __forceinline__ int nth_bit(uint64_t m, int i, int lane) {
  const unsigned r = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
  const uint64_t hit = __ballot(((m >> lane) & 1ull) && r == (unsigned)i);
  return (int)__builtin_ctzll(hit);
}

template <bool BF16, bool NORM, bool SEL>
__device__ __forceinline__ void p3_item(const FusedArgs &a, int item, P3Smem &sm) {
  const unsigned hw = g_fs<SEL>.hw;
  // every launch has P3 items: they clear the other half between them (off
  // the Stage 1 chains, and long before the item's own flag)
  clear_half_share(a, hw ^ 2u, item, a.n_p3);
  const int c0 = item * kP3Ch;
  // x to LDS when it fits (every item reads it, so it is L2-resident), before
  // the wait: it does not depend on Stage 1.
  const uint32_t rowb = (uint32_t)a.d_model * (BF16 ? 2u : 4u);
  const u4 *xs = nullptr;
  if (rowb <= sizeof(sm.x)) {
    if constexpr (NORM) {
      // x = RMSNorm(r) in the layer dtype, 16 bytes per step, with the
      // 1/rms(r) that the first Stage 1 item published (the same bits as a
      // reduction here; 1/rms > 0, so 0 means not yet).  The threshold-mask
      // instances load the residual of each thread's first step together
      // with that word (in the top-k instances those registers spill).
      constexpr int EPS16 = BF16 ? 8 : 4;
      const int nst = (int)(rowb >> 4);
      float r0[EPS16];
      if constexpr (!SEL) {
        const int i0 = min((int)threadIdx.x, nst - 1);
#pragma unroll
        for (int q = 0; q < EPS16; ++q) r0[q] = a.rnorm[(size_t)i0 * EPS16 + q];
      }
      // read by thread 0 and shared through LDS (a work-group-wide vote
      // would keep all three thread coordinates live through the kernel)
      if (threadIdx.x == 0) {
        unsigned ib = xload_u(&a.sync[kSyncInv + hw]);
        if (ib == 0u) {
          wait_geq(&a.sync[kSyncInv + hw], 1u, &a.sync[kSyncErr], a.wlim);
          ib = xload_u(&a.sync[kSyncInv + hw]);
        }
        g_fs<SEL>.ibits = ib;
      }
      __syncthreads();
      const float inv = __uint_as_float(g_fs<SEL>.ibits);
      auto put = [&](int i, const float *r) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (BF16)
            w[q] = (uint32_t)f32_to_bf16(r[2 * q] * inv) |
                   ((uint32_t)f32_to_bf16(r[2 * q + 1] * inv) << 16);
          else
            w[q] = __float_as_uint(r[q] * inv);
        }
        sm.x[i] = u4{w[0], w[1], w[2], w[3]};
      };
      int i1 = threadIdx.x;
      if constexpr (!SEL) {
        if (i1 < nst) put(i1, r0);
        i1 += kFT;
      }
      for (int i = i1; i < nst; i += kFT) put(i, a.rnorm + (size_t)i * EPS16);
    } else {
      for (int i = threadIdx.x; i < (int)(rowb >> 4); i += kFT) sm.x[i] = ((const u4 *)a.x)[i];
    }
    xs = sm.x;
  }
  // What to compute first.  Threshold: |s~| >= tau_s, once the item's Stage 1
  // tile is done.  Top-k: every channel whose digit 1 is at least the b* of
  // the layer's previous call (a guess of the cut, which moves little from
  // token to token), also as soon as the tile is done, so Stage 2 overlaps the
  // rest of Stage 1 and the select; once b* is out, whatever the guess missed
  // (digit 1 >= b*).  With no guess yet: digit 1 >= b*, after b*.  Only the
  // timing depends on the guess, never the result.  (Measured at 8B: one bin
  // lower 0.3 us slower; one bin higher within 0.1 us on a single layer but
  // 0.6 us slower per layer in the 32-layer stack; a start 1/16 to 1/4 octave
  // below the previous call's k-th key slower.)
  if (threadIdx.x == 0) {
    unsigned lo = 0u;
    const unsigned pb = a.ts_mode ? 0u : xload_u(a.pred);
    if (a.ts_mode || pb >= 2u) {
      // every chunk of the item's Stage 1 tile has stored its partial sums
      // (the item forms its keys from them, rather than waiting for the
      // tile epilogue to publish them)
      wait_geq(&a.tflag[(c0 / kTile) * kSyncStride + hw + 1], (unsigned)a.nchunk, &a.sync[kSyncErr],
               a.wlim);
      lo = pb >= 2u ? pb - 1u : 0u;
    } else {
      wait_geq(&a.sync[kSyncBin + hw], 1u, &a.sync[kSyncErr], a.wlim);
      lo = xload_u(&a.sync[kSyncBin + hw]) - 1u;
    }
    sm.lo = lo;
    stamp_wait<SEL>(a);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = a.d_ff;
  const int j = c0 + lane;
  const bool valid = lane < kP3Ch && j < n;
  // |s~| of the item's channels (the bits the tile epilogue stores in sabs),
  // formed by wave 0 and shared through LDS
  static_assert(kTile % kP3Ch == 0, "a P3 item lies in one Stage 1 tile");
  if (wv == 0 && lane < kP3Ch)
    sm.key[lane] = __float_as_uint(
        tile_key(a.part + (size_t)(c0 / kTile) * a.nchunk * 512, (c0 % kTile) + lane, a.nchunk, a.act));
  __syncthreads();
  const unsigned key = sm.key[min(lane, kP3Ch - 1)];
  const unsigned d1 = key >> 20;
  // Two passes: the first set, then (top-k) what b* adds to it.  Each
  // computes s of the channels of the wave-uniform mask cm, stored by
  // channel.  Work units are rows: unit 2m is the up row, unit 2m + 1 the gate
  // row of the m-th channel of cm.  Wave w takes units w, w + 8, ..., one at a
  // time, so every wave streams about the same number of bytes.
  uint64_t cm = a.ts_mode ? __ballot(valid && __uint_as_float(key) >= a.tau_s)
                          : __ballot(valid && d1 >= sm.lo);
  uint64_t dm = cm, bm = 0ull;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (a.ts_mode) break;
      // top-k: selected whatever T is (digit 1 > b*) / decided later by T
      // and J (digit 1 = b*, computed before T is known so nothing here
      // waits for the select)
      if (threadIdx.x == 0) {
        wait_geq(&a.sync[kSyncBin + hw], 1u, &a.sync[kSyncErr], a.wlim);
        sm.bstar = xload_u(&a.sync[kSyncBin + hw]) - 1u;
      }
      __syncthreads();
      const unsigned bstar = sm.bstar;
      const uint64_t done = cm;
      dm = __ballot(valid && d1 > bstar);
      bm = __ballot(valid && d1 == bstar);
      cm = (dm | bm) & ~done;
      if (!cm) break;
    }
    __syncthreads();  // x staged; ured free
    const int nu = 2 * (int)__popcll(cm);
    auto unit_base = [&](int u) {
      const int ch = c0 + nth_bit(cm, u >> 1, lane);
      return ((uint32_t)ch * 2u + (uint32_t)(u & 1)) * rowb;
    };
    for (int u = wv; u < nu; u += kFW) {
      const float r = p3_row<BF16>(a, xs, unit_base(u), lane);
      if (lane == 0) sm.ured[u] = r;
    }
    __syncthreads();
    if (wv == 0 && ((cm >> lane) & 1ull)) {
      const unsigned m = __builtin_amdgcn_mbcnt_hi((unsigned)(cm >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((unsigned)cm, 0u));
      xstore(&a.sdense[c0 + lane], sm.ured[2 * m] * gate_act(sm.ured[2 * m + 1], a.act));
    }
  }
  if (threadIdx.x == 0) {
    xstore_u(&a.gmask[4 * item], (unsigned)dm);
    xstore_u(&a.gmask[4 * item + 1], (unsigned)(dm >> 32));
    xstore_u(&a.gmask[4 * item + 2], (unsigned)bm);
    xstore_u(&a.gmask[4 * item + 3], (unsigned)(bm >> 32));
  }

}

// ---------------------------------------------------------------------------
// P4: Stage 2b for one (range of 512 channels, 256-column chunk) item (Sec.
// 4.1, Stage 2 equations; Sec. 3.1 weighted-sum view): the range's kept
// channels, ascending, each scaled by its s; the last item of a column chunk
// adds the range partials in range order.  The rows of every channel that
// may be kept (digit 1 >= b*) start loading before the range's P3 items and
// the select are done; a bin-b* channel below the cut gets s = 0.
// ---------------------------------------------------------------------------
template <bool BF16, bool SEL>
__device__ __forceinline__ void p4_item(const FusedArgs &a, int item, P4Smem<SEL> &sm, int *s_flag) {
  const unsigned hw = g_fs<SEL>.hw;
  // rows per wave per batch: 10 rows x 512 B; 20 measured 0.5 us slower at 8B
  // (more bytes in flight behind which the dependent round trips queue)
  constexpr int U = BF16 ? 10 : 8;
  constexpr int ESZ = BF16 ? 2 : 4;
  const int r = item / a.ncol, cc = item % a.ncol;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.d_ff;
  // 1. b* (top-k) or the range's Stage 1 tiles (threshold), then the range's
  // channels that may be kept (top-k: digit 1 >= b*, the kept ones and the
  // bin-b* ones that may drop; threshold: |s~| >= tau_s), ascending, with
  // their keys.
  if (a.ts_mode) {
    if (tid < 64) {
      constexpr int TPR = kP4Ch / kTile;  // tiles per range
      const int t0 = r * TPR, t1 = min(a.ntile, t0 + TPR) - 1;
      wave_wait_flags(&a.tflag[min(t0 + lane, t1) * kSyncStride + hw], &a.sync[kSyncErr], a.wlim);
    }
  } else if (tid == 0) {
    wait_geq(&a.sync[kSyncBin + hw], 1u, &a.sync[kSyncErr], a.wlim);
    sm.bstar = xload_u(&a.sync[kSyncBin + hw]) - 1u;
  }
  __syncthreads();
  {
    const int ch = r * kP4Ch + tid;
    const unsigned key = __float_as_uint(xload(&a.sabs[min(ch, n - 1)]));
    const bool cand = ch < n && (a.ts_mode ? __uint_as_float(key) >= a.tau_s
                                           : (key >> 20) >= sm.bstar);
    const uint64_t bw = __ballot(cand);
    if (lane == 0) sm.wcnt[wv] = (unsigned)__popcll(bw);
    __syncthreads();
    unsigned off = 0;
#pragma unroll
    for (int i = 0; i < kFW; ++i) off += i < wv ? sm.wcnt[i] : 0u;
    if (cand) {
      const unsigned pos = off + __builtin_amdgcn_mbcnt_hi((unsigned)(bw >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((unsigned)bw, 0u));
      sm.rs[pos] = ch;
      sm.rk[pos] = key;
    }
  }
  __syncthreads();
  int nr = 0;
#pragma unroll
  for (int i = 0; i < kFW; ++i) nr += (int)sm.wcnt[i];
  const size_t chunk_bytes = (size_t)a.d_ff * kDownCols * ESZ;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc((const char *)a.wd + cc * chunk_bytes, (uint32_t)chunk_bytes);
  const uint32_t voff = (uint32_t)lane * 4u * ESZ;
  using WT = typename std::conditional<BF16, u2, u4>::type;
  WT wr[U];
  auto load_batch = [&](int b0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = min(b0 + wv + kFW * u, nr - 1);
      const uint32_t rowoff =
          (uint32_t)__builtin_amdgcn_readfirstlane(sm.rs[rr]) * (uint32_t)(kDownCols * ESZ);
      if constexpr (BF16)
        wr[u] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, rowoff, kNT);
      else
        wr[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, rowoff, kNT);
    }
  };
  // 2. the first rows stream in while the range's P3 items and the select
  // finish: one batch into registers, the next ND rows straight into LDS.
  constexpr int ND = BF16 ? kP4LdsRows<SEL> : 0;  // multiple of kFW (or 0)
  constexpr int NB0 = kFW * U;  // rows of a register batch
  static_assert(ND % kFW == 0, "LDS rows per wave");
  if (nr > 0) load_batch(0);
  if constexpr (ND > 0) {
    const int dend = min(nr, NB0 + ND);
    for (int rr = NB0 + wv; rr < dend; rr += kFW) {
      const uint32_t rowoff =
          (uint32_t)__builtin_amdgcn_readfirstlane(sm.rs[rr]) * (uint32_t)(kDownCols * ESZ);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void *)&sm.rows[rr - NB0][h * 32], 4,
            (uint32_t)lane * 4u, rowoff + (uint32_t)h * 256u, 0, kNT);
    }
  }
  // 3. s of each listed channel, polled until its up/gate item has stored it
  // (the bin-b* ones included), while the select may still run; then 0 for a
  // bin-b* channel below the cut.
  {
    // T and J first, by the last thread: they are usually out long before the
    // last listed s, so their round trip hides behind the polls
    if (!a.ts_mode && tid == kFT - 1)
      wait_tj(&a.sync[kSyncSelect + hw], &a.sync[kSyncErr], &sm.tj[0], &sm.tj[1], a.wlim);
    float sj = 0.0f;
    if (tid < nr) {
      const unsigned *sp = (const unsigned *)&a.sdense[sm.rs[tid]];
      unsigned v, spins = 0;
      while ((v = xload_u(sp)) == kSNone) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > a.wlim) {
          atomicOr(&a.sync[kSyncErr], 1u);
          break;
        }
      }
      sj = __uint_as_float(v);
    }
    if (tid == 0) stamp_wait<SEL>(a);
    __syncthreads();
    const unsigned T = a.ts_mode ? 0u : sm.tj[0];
    const int J = a.ts_mode ? n : (int)sm.tj[1];
    if (tid < nr) {
      const int ch = sm.rs[tid];
      const unsigned key = sm.rk[tid];
      sm.sv[tid] = (key > T || (key == T && ch <= J)) ? sj : 0.0f;
    }
  }
  __syncthreads();
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // each wave adds its rows (wv, wv + 8, ...) in ascending order: the first
  // register batch, the LDS rows, then further register batches
  for (int b0 = 0; b0 < nr; b0 += (b0 == 0 ? NB0 + ND : NB0)) {
    if (b0 > 0) load_batch(b0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = b0 + wv + kFW * u;
      const float sv = rr < nr ? sm.sv[rr] : 0.0f;
      float wf[4];
      if constexpr (BF16) {
        wf[0] = bf16_to_f32(wr[u].x & 0xffffu);
        wf[1] = bf16_to_f32(wr[u].x >> 16);
        wf[2] = bf16_to_f32(wr[u].y & 0xffffu);
        wf[3] = bf16_to_f32(wr[u].y >> 16);
      } else {
        wf[0] = __uint_as_float(wr[u].x);
        wf[1] = __uint_as_float(wr[u].y);
        wf[2] = __uint_as_float(wr[u].z);
        wf[3] = __uint_as_float(wr[u].w);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = fmaf(sv, wf[c], acc[c]);
    }
    if constexpr (ND > 0) {
      if (b0 == 0 && nr > NB0) {
        wait_vmem();  // the LDS rows have landed
#pragma unroll 4
        for (int rr = NB0 + wv; rr < min(nr, NB0 + ND); rr += kFW) {
          const u2 w = sm.rows[rr - NB0][lane];
          const float sv = sm.sv[rr];
          acc[0] = fmaf(sv, bf16_to_f32(w.x & 0xffffu), acc[0]);
          acc[1] = fmaf(sv, bf16_to_f32(w.x >> 16), acc[1]);
          acc[2] = fmaf(sv, bf16_to_f32(w.y & 0xffffu), acc[2]);
          acc[3] = fmaf(sv, bf16_to_f32(w.y >> 16), acc[3]);
        }
      }
    }
  }
  *(float4 *)&sm.red[wv][lane * 4] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (tid < kDownCols) {
    const int c = tid;
    float v = sm.red[0][c];
#pragma unroll
    for (int q = 1; q < kFW; ++q) v += sm.red[q][c];
    xstore(&a.ypart[(size_t)r * a.d_model + cc * kDownCols + c], v);
  }
  // The last of the chunk's items to arrive adds the partials; it polls each
  // one until it has landed, so no item waits for its own stores first.
  __syncthreads();
  if (tid == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(&a.col_cnt[cc], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == (unsigned)a.nrange - 1u;
    if (last) __hip_atomic_store(&a.col_cnt[cc], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  if (!*s_flag) return;
  // Sum of the range partials of the chunk: wave q adds ranges q, q + 8, ...
  // of 4 columns per lane (agent-coherent 16-byte loads), then the 8 wave
  // sums are added in wave order.
  {
    const __amdgpu_buffer_rsrc_t yr =
        make_rsrc(a.ypart, (uint32_t)((size_t)a.nrange * a.d_model * sizeof(float)));
    const uint32_t coff = (uint32_t)(cc * kDownCols + lane * 4) * 4u;
    float4 s4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int r0 = wv; r0 < a.nrange; r0 += kFW * 8) {
      u4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int rr = min(r0 + kFW * u, a.nrange - 1);
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(yr, coff, (uint32_t)rr * a.d_model * 4u, kSelBits);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (r0 + kFW * u < a.nrange) {
          unsigned spins = 0;
          while (v[u].x == kSNone || v[u].y == kSNone || v[u].z == kSNone || v[u].w == kSNone) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > a.wlim) {
              atomicOr(&a.sync[kSyncErr], 1u);
              break;
            }
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(yr, coff, (uint32_t)(r0 + kFW * u) * a.d_model * 4u,
                                                         kSelBits);
          }
          s4.x += __uint_as_float(v[u].x);
          s4.y += __uint_as_float(v[u].y);
          s4.z += __uint_as_float(v[u].z);
          s4.w += __uint_as_float(v[u].w);
        }
      }
    }
    __syncthreads();  // every wave is done with red
    *(float4 *)&sm.red[wv][lane * 4] = s4;
  }
  __syncthreads();
  if (tid < kDownCols) {
    const int c = tid;
    float v = sm.red[0][c];
#pragma unroll
    for (int q = 1; q < kFW; ++q) v += sm.red[q][c];
    const int col = cc * kDownCols + c;
    st_elem<BF16>(a.y, col, v);
    if (a.resid) a.resid[col] += round_elem<BF16>(v);
  }
}

// ---------------------------------------------------------------------------
// The persistent kernel.
// ---------------------------------------------------------------------------
// NORM: x = RMSNorm(a.rnorm) is formed inside (a separate instance, so the
// plain forward keeps its register budget).  SEL: top-k (with the select
// item) rather than the threshold mask.
__device__ __forceinline__ unsigned draw_ticket(unsigned *ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


template <bool BF16, bool NORM, bool SEL>
__global__ __launch_bounds__(kFT) __attribute__((amdgpu_waves_per_eu(4, 8))) void ffn_fused_kernel(
    FusedArgs a) {
  auto &sm = g_fs<SEL>.u;
  int &s_ticket = g_fs<SEL>.ticket;
  int &s_flag = g_fs<SEL>.flag;
  const int total = a.n_p1 + a.n_p2 + a.n_p3 + a.n_p4;
  // The first min(grid, n_p1) tickets are the work-groups' own indices (all
  // work-groups of the grid are resident at once, see the launcher), which
  // spares the launch burst on the ticket counter; the rest are drawn.  Every
  // work-group stops at its first draw past the end, so a launch makes
  // exactly total - nfirst + grid draws, and the last of them resets the
  // count with the parity bit flipped for the next launch.
  const int nfirst = min((int)gridDim.x, a.n_p1);
  const unsigned last_draw = (unsigned)(total - nfirst) + gridDim.x - 1u;
  bool first = (int)blockIdx.x < nfirst;
  // On a work-group's first item thread 0 loads the parity word (used at the
  // item's partial-sum barrier); later items learn the parity from their draw.
  unsigned pw = 0u;
  for (;;) {
    __syncthreads();  // the previous item is done with the LDS
    if (threadIdx.x == 0) {
      int t;
      if (first) {
        t = (int)blockIdx.x;
        pw = xload_u(&a.sync[kSyncPar]);
      } else {
        const unsigned raw = draw_ticket(&a.sync[kSyncTicket]);
        const unsigned c = raw & 0x7fffffffu;
        g_fs<SEL>.hw = (raw >> 31) * 2u;
        if (c == last_draw) {
          const unsigned next = ~raw & 0x80000000u;
          xstore_u(&a.sync[kSyncPar], next);
          xstore_u(&a.sync[kSyncTicket], next);
        }
        t = nfirst + (int)c;
      }
      s_ticket = t;
    }
    const bool resolve = first;  // the half arrives with the parity word
    first = false;
    __syncthreads();
    const int t = s_ticket;
    if (t >= total) break;
    unsigned long long t0 = 0;
    if (a.trace && threadIdx.x == 0) {
      t0 = __builtin_amdgcn_s_memrealtime();
      g_fs<SEL>.twait = t0;
    }
    int phase;
    int r = t;
    if (r < a.n_p1) {
      phase = 1;
      p1_item<BF16, NORM, SEL>(a, r, sm.p1, &s_flag, pw, resolve);
    } else if ((r -= a.n_p1) < a.n_p2) {
      phase = 2;
      if constexpr (SEL) p2_select<SEL>(a, sm.p2);
    } else if ((r -= a.n_p2) < a.n_p3) {
      phase = 3;
      p3_item<BF16, NORM, SEL>(a, r, sm.p3);
    } else {
      phase = 4;
      p4_item<BF16, SEL>(a, r - a.n_p3, sm.p4, &s_flag);
    }
    if (a.trace && threadIdx.x == 0) {
      unsigned long long *e = a.trace + 4 * (size_t)t;
      e[0] = t0;
      e[1] = g_fs<SEL>.twait;
      e[2] = __builtin_amdgcn_s_memrealtime();
      e[3] = (unsigned long long)blockIdx.x | ((unsigned long long)phase << 32);
    }
  }
}

// The ascending list of kept channels and their s, from the P3 masks, the
// keys and T, J (for inspection only; the forward itself never builds it).
// One work-group.
__global__ __launch_bounds__(kFT) void fused_list_kernel(const unsigned *gmask, const unsigned *tj,
                                                         const float *sabs, const float *sdense,
                                                         int n_p3, int d_ff, int k, int *sel,
                                                         float *ssel, int *count) {
  __shared__ unsigned wsum[kFW];
  __shared__ unsigned base;
  if (threadIdx.x == 0) base = 0u;
  __syncthreads();
  const unsigned T = tj[0];
  const int J = (int)tj[1];
  for (int q0 = 0; q0 < n_p3; q0 += kFT) {
    const int q = q0 + (int)threadIdx.x;
    uint64_t m = 0ull;
    if (q < n_p3) {
      m = (uint64_t)gmask[4 * q] | ((uint64_t)gmask[4 * q + 1] << 32);
      uint64_t bm = (uint64_t)gmask[4 * q + 2] | ((uint64_t)gmask[4 * q + 3] << 32);
      while (bm) {
        const int b = __builtin_ctzll(bm);
        bm &= bm - 1ull;
        const int ch = q * kP3Ch + b;
        const unsigned key = __float_as_uint(sabs[ch]);
        if (key > T || (key == T && ch <= J)) m |= 1ull << b;
      }
    }
    unsigned tot;
    unsigned pos = base + block_excl_scan<kFW>((unsigned)__popcll(m), wsum, tot);
    while (m) {
      const int b = __builtin_ctzll(m);
      m &= m - 1ull;
      const int ch = q * kP3Ch + b;
      if (pos < (unsigned)k && ch < d_ff) {
        sel[pos] = ch;
        if (ssel) ssel[pos] = sdense[ch];
      }
      ++pos;
    }
    __syncthreads();
    if (threadIdx.x == 0) base += tot;
    __syncthreads();
  }
  if (count && threadIdx.x == 0) *count = (int)base;
}

// ---------------------------------------------------------------------------
// Launcher
// ---------------------------------------------------------------------------
template <bool BF16, bool NORM, bool SEL>
static hipError_t fused_go(FusedArgs &a, hipStream_t s) {
  auto fn = ffn_fused_kernel<BF16, NORM, SEL>;
  // Work-groups the current device holds at once for this instance, queried
  // once per device (per instance) and kept; threads that race on the first
  // query store the same value.
  constexpr int kDevCache = 64;
  static std::atomic<int> caps[kDevCache];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int cap = dev < kDevCache ? caps[dev].load(std::memory_order_relaxed) : 0;
  if (!cap) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)fn, kFT, 0) !=
            hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    cap = per_cu * cus;
    if (dev < kDevCache) caps[dev].store(cap, std::memory_order_relaxed);
  }
  const int total = a.n_p1 + a.n_p2 + a.n_p3 + a.n_p4;
  const int grid = total < cap ? total : cap;
  fn<<<grid, kFT, 0, s>>>(a);
  return hipGetLastError();
}

bool fused_supported(const Plan &p) {
  return (p.d_ff + kFT - 1) / kFT <= kMaxPer && ((size_t)p.d_model * p.esz) % 1024 == 0;
}

static int fused_n_p3(const Plan &p) { return (p.d_ff + kP3Ch - 1) / kP3Ch; }

// Sync block: control words, tile flags (one line each), the digit-1
// histogram, the P3 masks, each at a fixed word index sized for the
// largest supported d_ff (so layers of any shapes can share one block).
constexpr size_t kMaxP3 = kMaxDff / kP3Ch;
constexpr size_t kTflagWord = (size_t)kSyncCtl;
constexpr size_t kHistWord = kTflagWord + (size_t)(kMaxDff / kTile) * kSyncStride;
constexpr size_t kGmaskWord = kHistWord + 2048;

size_t fused_sync_words() { return kGmaskWord + 4 * kMaxP3; }

int fused_ypart_rows(const Plan &p) { return (p.d_ff + kP4Ch - 1) / kP4Ch; }

int fused_items(const Plan &p, bool ts_mode) {
  return p.ntile * p.nchunk + (ts_mode ? 0 : 1) + fused_n_p3(p) + p.ncol * fused_ypart_rows(p);
}

int fused_p3_items(const Plan &p) { return fused_n_p3(p); }

bool fused_norm_supported(const Plan &p) {
  return (size_t)p.d_model * p.esz <= sizeof(P3Smem::x);
}

hipError_t launch_fused(const Plan &p, const Bufs &b, const void *x, float tau, int k, void *y,
                        float *resid, hipStream_t s, const FusedOpts &o) {
  if (o.norm_r && !fused_norm_supported(p)) return hipErrorInvalidValue;
  const bool ts_mode = o.ts_mode;
  FusedArgs a{};
  a.rnorm = o.norm_r;
  a.eps = o.eps;
  a.xout = o.xout;
  a.trace = o.trace;
  a.ts_mode = ts_mode ? 1 : 0;
  a.act = p.act;
  a.tau_s = o.tau_s;
  a.wlim = p.wait_limit;
  a.drows = o.dbg ? b.drows : nullptr;
  a.dcnt = o.dbg ? b.dcnt : nullptr;
  a.pq = b.pq;
  a.psc = b.psc;
  a.wug = b.wug;
  a.wug_bytes = (uint32_t)((size_t)p.d_ff * 2 * p.d_model * p.esz);
  a.wd = b.wd;
  a.d_model = p.d_model;
  a.d_ff = p.d_ff;
  a.G = p.G;
  a.ngroups = p.ngroups;
  a.ntile = p.ntile;
  a.nchunk = p.nchunk;
  a.ncol = p.ncol;
  a.nrange = fused_ypart_rows(p);
  a.x = x;
  a.tau = tau;
  a.k = k;
  a.y = y;
  a.resid = resid;
  a.part = b.part;
  a.sabs = b.sabs;
  a.sdense = b.ssp;
  a.ypart = b.ypart;
  a.col_cnt = b.col_cnt;
  a.sync = b.sync;
  a.tflag = b.sync + kTflagWord;
  a.ghist = b.sync + kHistWord;
  a.gmask = b.sync + kGmaskWord;
  a.pred = b.pred;
  a.n_p1 = p.ntile * p.nchunk;
  a.n_p2 = ts_mode ? 0 : 1;
  a.n_p3 = fused_n_p3(p);
  a.n_p4 = p.ncol * a.nrange;
  if (!ts_mode) {
    if (o.norm_r) return p.bf16 ? fused_go<true, true, true>(a, s) : fused_go<false, true, true>(a, s);
    return p.bf16 ? fused_go<true, false, true>(a, s) : fused_go<false, false, true>(a, s);
  }
  if (o.norm_r) return p.bf16 ? fused_go<true, true, false>(a, s) : fused_go<false, true, false>(a, s);
  return p.bf16 ? fused_go<true, false, false>(a, s) : fused_go<false, false, false>(a, s);
}

hipError_t launch_fused_list(const Plan &p, const Bufs &b, int k, int *sel, float *ssel,
                             int *count, hipStream_t s) {
  const unsigned *gmask = b.sync + kGmaskWord;
  fused_list_kernel<<<1, kFT, 0, s>>>(gmask, b.sync + kSyncSelect + 4, b.sabs, b.ssp, fused_n_p3(p),
                                      p.d_ff, k, sel, ssel, count);
  return hipGetLastError();
}

}  // namespace prox
