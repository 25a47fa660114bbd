// HIP kernels of libprox for CDNA4 (gfx950): the Prox two-stage sparse
// SwiGLU FFN decode step.
//
// Method: "Prox: Training-Free FFN Activation Sparsity via Approximate
// Intermediate-Channel Salience in LLMs" (arXiv 2607.27591), Sec. 4.1
// (two-stage inference), Sec. 4.3 (INT4 proxy, fused kernels), App. A.6
// (top-k mask).
//
// Batch-1 decode is a chain of matrix-vector products, so every kernel here
// is bound by HBM bandwidth, not by arithmetic: no MFMA at batch 1.  For 2..8
// tokens the exact up/gate step has an MFMA form (a 16-channel x 16-token
// tile per instruction) beside the VALU one.  The weight layouts
// make each read a long contiguous run (see prox_internal.h), reads go
// through buffer loads with scalar row offsets, and every reduction across
// work-groups is deterministic (partials + last-arriving work-group, fixed
// summation order).
#include "prox_device.h"
#include <algorithm>
#include <type_traits>
#include <utility>

namespace prox {

// ---------------------------------------------------------------------------
// Prepare: relayout and INT4 quantization (Sec. 4.3)
// ---------------------------------------------------------------------------

// W [d_model][d_ff] (paper layout) -> wug[j][m][i], m = 0 up, 1 gate.
template <bool BF16>
__global__ __launch_bounds__(256) void transpose_kernel(const void *w_up,
                                                        const void *w_gate,
                                                        void *wug, int d_model,
                                                        int d_ff) {
  typedef typename std::conditional<BF16, uint16_t, float>::type E;
  __shared__ E tile[64][65];
  const int m = blockIdx.z;
  const E *src = (const E *)(m ? w_gate : w_up);
  E *dst = (E *)wug;
  const int j0 = blockIdx.x * 64, i0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int i = i0 + r, j = j0 + tx;
    if (i < d_model && j < d_ff) tile[r][tx] = src[(size_t)i * d_ff + j];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int j = j0 + r, i = i0 + tx;
    if (i < d_model && j < d_ff)
      dst[((size_t)j * 2 + m) * d_model + i] = tile[tx][r];
  }
}

// W_down [d_ff][d_model] -> wd[c][j][0..256): output-column chunks of 256
// stored one after another, so the rows a down-projection work-group reads
// for one chunk are contiguous 256-column runs.
template <bool BF16>
__global__ __launch_bounds__(256) void retile_down_kernel(const void *w_down, void *wd,
                                                          int d_model, int d_ff) {
  typedef typename std::conditional<BF16, uint16_t, float>::type E;
  const int j = blockIdx.x, cc = blockIdx.y, c = threadIdx.x;
  ((E *)wd)[((size_t)cc * d_ff + j) * kDownCols + c] =
      ((const E *)w_down)[(size_t)j * d_model + cc * kDownCols + c];
}

// One thread per proxy column of a tile, one work-group per (group, tile,
// matrix).  scale = absmax / 7, code = clamp(rint(w / scale), -7, 7), both
// divisions correctly rounded float32; stored as (code + 8) nibbles, two
// columns per byte (low nibble = even column).
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_kernel(const void *w_up,
                                                       const void *w_gate,
                                                       uint8_t *pq, float *psc,
                                                       int d_model, int d_ff,
                                                       int G, int ngroups) {
  const int g = blockIdx.x, t = blockIdx.y, m = blockIdx.z;
  const int c = threadIdx.x;
  const int j = t * kTile + c;
  const void *W = m ? w_gate : w_up;
  const bool live = j < d_ff;
  float a = 0.0f;
  if (live)
    for (int i = g * G; i < (g + 1) * G; ++i)
      a = fmaxf(a, fabsf(ld_elem<BF16>(W, (size_t)i * d_ff + j)));
  const float sc = live ? __fdiv_rn(a, 7.0f) : 0.0f;
  psc[((size_t)t * ngroups + g) * 512 + m * 256 + c] = sc;
  for (int i = g * G; i < (g + 1) * G; ++i) {
    int code = 0;
    if (live && a > 0.0f) {
      float r = rintf(__fdiv_rn(ld_elem<BF16>(W, (size_t)i * d_ff + j), sc));
      r = fminf(fmaxf(r, -7.0f), 7.0f);
      code = (int)r;
    }
    const unsigned nib = (unsigned)(code + 8);
    const unsigned odd = __shfl_xor(nib, 1, 64);
    if ((c & 1) == 0)
      pq[((size_t)t * d_model + i) * kTileBytes + m * 128 + (c >> 1)] =
          (uint8_t)(nib | (odd << 4));
  }
}

// Unpack a prepared proxy back to int8 codes [d_model][d_ff] and scales
// [ngroups][d_ff] (paper layout), for inspection.
__global__ __launch_bounds__(256) void export_proxy_kernel(
    const uint8_t *pq, const float *psc, int matrix, int d_model, int d_ff,
    int G, int ngroups, int8_t *codes, float *scales) {
  const int i = blockIdx.x, t = blockIdx.y, c = threadIdx.x;
  const int j = t * kTile + c;
  if (j >= d_ff) return;
  const uint8_t byte =
      pq[((size_t)t * d_model + i) * kTileBytes + matrix * 128 + (c >> 1)];
  const int nib = (c & 1) ? (byte >> 4) : (byte & 15);
  codes[(size_t)i * d_ff + j] = (int8_t)(nib - 8);
  if (i % G == 0)
    scales[(size_t)(i / G) * d_ff + j] =
        psc[((size_t)t * ngroups + i / G) * 512 + matrix * 256 + c];
}

// ---------------------------------------------------------------------------
// K-c  Stage 1: threshold + compact + INT4 proxy up/gate GEMV + SwiGLU
//      (Sec. 4.1, m_x and u~/h~ equations; Sec. 4.3, fused Stage 1 kernel)
// ---------------------------------------------------------------------------
// Grid (nchunk, ntile), 8 waves.  Wave w of chunk c handles the 64-row slice
// 8c + w of column tile t.  It finds the slice's surviving rows with one
// ballot (the compaction never leaves registers and LDS), parks their row
// numbers and masked x values in LDS, then streams only those rows' 256-byte
// code runs, 16 rows in flight while the previous 16 are consumed.  Lane l
// covers 8 consecutive columns: lanes 0-31 the up proxy, lanes 32-63 the
// gate proxy of the same columns.  A code is stored as nib = q + 8, and
//   sum_i x_i q_i = sum_i x_i nib_i - 8 sum_i x_i,
// so the offset and the group scale are applied once per slice.
//   bf16 layers: two surviving rows a, b are taken together; for each column
//   the pair (128 + nib_a, 128 + nib_b) is formed as two bf16 values by
//   placing the nibbles under the exponent byte 0x43 (128 + n is exact in
//   bf16 for n < 128), and one v_dot2_f32_bf16 with (x_a, x_b) adds
//   x_a nib_a + x_b nib_b + 128 (x_a + x_b); the slice then removes
//   136 sum x instead of 8 sum x.
//   float32 layers: byte -> float conversion and one FMA per code.
// The last work-group to finish a tile adds the partials of all chunks in a
// fixed order and writes |s~| = |u~ * SiLU(g~)| for the tile's columns.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct ProxyArgs {
  const uint8_t *pq;
  const unsigned *pq2;  // codes in 8-row words (matrix-core form), or null
  const float *psc;
  const void *x;
  float tau;
  int d_model, d_ff, G, ngroups, nchunk;
  float *part;
  unsigned *tile_cnt;
  float *sabs;
  int act;  // gate activation (gate_act)
  int *drows, *dcnt;  // debug: per-token survivors per 64-row slice (nullptr: off)
};

// 5..8 tokens: 8 rows per stage, so that the accumulators of all tokens and
// two stages of codes fit 128 VGPRs and two work-groups share a CU.
template <int NB, bool BF16>
__global__ __launch_bounds__(512, NB > 4 ? 2 : 1) void proxy_kernel(ProxyArgs a) {
  constexpr int NW = 8;             // waves (64-row slices) per work-group
  constexpr int U = NB > 4 ? 8 : 16;  // rows per pipeline stage
  constexpr int LL = 64 + 3 * U;    // list length incl. padding for prefetch
  __shared__ float red[NW][512];
  __shared__ __attribute__((aligned(16))) int rl[NW][LL];       // surviving rows
  __shared__ __attribute__((aligned(16))) float xc[NW][NB][LL]; // their x (0 if a token drops them)
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunk = blockIdx.x, t = blockIdx.y;
  const int sl = chunk * NW + wv;    // 64-row slice
  const int nsl = a.d_model >> 6;

  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[b][c] = 0.0f;

  if (sl < nsl) {
    // the slice's group scales first, so that their latency hides behind
    // the mask and the code stream instead of following it
    const int g = (sl * 64) / a.G;
    const float4 *sp = (const float4 *)(a.psc + ((size_t)t * a.ngroups + g) * 512 + (size_t)lane * 8);
    const float4 s0 = sp[0], s1 = sp[1];
    // Input mask of the slice's rows (Sec. 4.1, m_x), compacted in LDS: the
    // union over tokens decides which rows are read; each token keeps its
    // own x or 0.
    float xsum[NB];
    float xm[NB];
    uint64_t un = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float xl;
      const uint64_t mk = slice_mask<BF16>(a.x, (size_t)b * a.d_model + sl * 64, a.tau, xl);
      if (a.drows && t == 0)
        export_slice(a.drows + (size_t)b * a.d_model, a.dcnt + (size_t)b * nsl, sl, mk);
      xm[b] = ((mk >> lane) & 1ull) ? xl : 0.0f;
      xsum[b] = wave_sum(xm[b]);
      un |= mk;
    }
    const int cnt = (int)__popcll(un);
    if ((un >> lane) & 1ull) {
      const int pos = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(un >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((unsigned)un, 0u));
      rl[wv][pos] = lane;
#pragma unroll
      for (int b = 0; b < NB; ++b) xc[wv][b][pos] = xm[b];
    }
    // Padding: row 0 of the slice (a valid address) with x = 0.
    if (lane < 3 * U) {
      rl[wv][cnt + lane] = 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) xc[wv][b][cnt + lane] = 0.0f;
    }
    __builtin_amdgcn_wave_barrier();

    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(a.pq + (size_t)t * a.d_model * kTileBytes, (uint32_t)a.d_model * kTileBytes);
    const uint32_t voff = (uint32_t)lane * 4u;
    const uint32_t sbase = (uint32_t)sl * 64u * kTileBytes;

    // Stage `base`: 16 row numbers (uniform) and their code words.
    auto fetch = [&](int base, uint32_t (&w)[U]) {
#pragma unroll
      for (int q = 0; q < U / 4; ++q) {
        const int4 r4 = *(const int4 *)&rl[wv][base + 4 * q];
        const int rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane(rr[e]);
          w[4 * q + e] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, sbase + row * kTileBytes, kNT);
        }
      }
    };
    // 0x0f0f0f0f kept opaque to the optimizer: with a visible constant it
    // fuses mask + shift into one bit-field extract per nibble, while this
    // way one AND serves four nibbles.
    uint32_t nib_mask;
    asm volatile("s_mov_b32 %0, 0x0f0f0f0f" : "=s"(nib_mask));
    auto consume = [&](int base, const uint32_t (&w)[U]) {
      if constexpr (BF16) {
#pragma unroll
        for (int q = 0; q < U / 4; ++q) {
          // x of rows base+4q .. base+4q+3 as two bf16 pairs per token.
          uint32_t xp[NB][2];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const float4 x4 = *(const float4 *)&xc[wv][b][base + 4 * q];
            xp[b][0] = (__float_as_uint(x4.x) >> 16) | (__float_as_uint(x4.y) & 0xffff0000u);
            xp[b][1] = (__float_as_uint(x4.z) >> 16) | (__float_as_uint(x4.w) & 0xffff0000u);
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t wa = w[4 * q + 2 * h], wb = w[4 * q + 2 * h + 1];
            const uint32_t la = wa & nib_mask, ha = (wa >> 4) & nib_mask;
            const uint32_t lb = wb & nib_mask, hb = (wb >> 4) & nib_mask;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // bytes: [nib_a, 0, nib_b, 0] | 0x43004300 = bf16 (128+nib_a, 128+nib_b)
              const uint32_t sel = (uint32_t)i | 0x0c00u | ((uint32_t)(4 + i) << 16) | 0x0c000000u;
              const uint32_t pl = __builtin_amdgcn_perm(lb, la, sel) | 0x43004300u;
              const uint32_t ph = __builtin_amdgcn_perm(hb, ha, sel) | 0x43004300u;
#pragma unroll
              for (int b = 0; b < NB; ++b) {
                acc[b][2 * i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pl), as_bf16x2(xp[b][h]),
                                                                acc[b][2 * i], false);
                acc[b][2 * i + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                    as_bf16x2(ph), as_bf16x2(xp[b][h]), acc[b][2 * i + 1], false);
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < U / 4; ++q) {
          float4 x4[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) x4[b] = *(const float4 *)&xc[wv][b][base + 4 * q];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wcur = w[4 * q + e];
            const uint32_t lo = wcur & nib_mask;
            const uint32_t hi = (wcur >> 4) & nib_mask;
            float n[8];
            n[0] = (float)(lo & 0xffu);
            n[1] = (float)(hi & 0xffu);
            n[2] = (float)((lo >> 8) & 0xffu);
            n[3] = (float)((hi >> 8) & 0xffu);
            n[4] = (float)((lo >> 16) & 0xffu);
            n[5] = (float)((hi >> 16) & 0xffu);
            n[6] = (float)(lo >> 24);
            n[7] = (float)(hi >> 24);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const float xv = e == 0 ? x4[b].x : e == 1 ? x4[b].y : e == 2 ? x4[b].z : x4[b].w;
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[b][c] = fmaf(xv, n[c], acc[b][c]);
            }
          }
        }
      }
    };
    // Two buffers in turn: while one stage is consumed the next is in flight.
    uint32_t wa[U], wb[U];
    fetch(0, wa);
    for (int base = 0; base < cnt; base += 2 * U) {
      fetch(base + U, wb);
      consume(base, wa);
      fetch(base + 2 * U, wa);
      if (base + U < cnt) consume(base + U, wb);
    }
    // Group scale and code offset: contribution = scale * (acc - off * sum x).
    const float off = BF16 ? 136.0f : 8.0f;
    const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[b][c] = sc[c] * (acc[b][c] - off * xsum[b]);
  }

  // Sum the waves (fixed order) and publish this chunk's partials.
  float *part = a.part + ((size_t)t * a.nchunk + chunk) * NB * 512;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float4 *rp = (float4 *)&red[wv][lane * 8];
    rp[0] = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    rp[1] = make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
    __syncthreads();
    {
      const int e = threadIdx.x;  // 512 threads, 512 partials
      float v = red[0][e];
#pragma unroll
      for (int q = 1; q < NW; ++q) v += red[q][e];
      xstore(&part[b * 512 + e], v);
    }
    __syncthreads();
  }

  if (!arrive_last(&a.tile_cnt[t], (unsigned)a.nchunk, &s_last)) return;

  // Tile epilogue: u~, g~ per token, then |s~|, the chunk partials added in
  // chunk order, every partial of this thread's (token, column) pairs
  // requested at once, 8 chunks per round.
  const float *tp = a.part + (size_t)t * a.nchunk * NB * 512;
  constexpr int PP = (NB * 256 + 511) / 512;  // pairs per thread
  float su[PP], sg[PP];
#pragma unroll
  for (int p = 0; p < PP; ++p) su[p] = sg[p] = 0.0f;
  for (int cb = 0; cb < a.nchunk; cb += 8) {
    float vu[PP][8], vg[PP][8];
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      const int e = min((int)threadIdx.x + 512 * p, NB * 256 - 1);
      const int b = e >> 8, col = e & 255;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float *q = tp + ((size_t)min(cb + c, a.nchunk - 1) * NB + b) * 512 + col;
        vu[p][c] = xload(q);
        vg[p][c] = xload(q + 256);
      }
    }
#pragma unroll
    for (int p = 0; p < PP; ++p)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (cb + c < a.nchunk) {
          su[p] += vu[p][c];
          sg[p] += vg[p][c];
        }
  }
#pragma unroll
  for (int p = 0; p < PP; ++p) {
    const int e = (int)threadIdx.x + 512 * p;
    const int b = e >> 8, col = e & 255;
    const int j = t * kTile + col;
    if (e < NB * 256 && j < a.d_ff) a.sabs[(size_t)b * a.d_ff + j] = fabsf(su[p] * gate_act(sg[p], a.act));
  }
}

// Stage 1 on the matrix cores for 3..8 tokens (bf16 layers, G a multiple of
// 64, d_model of 32), the partials and tile epilogue of proxy_kernel: one
// work-group per (chunk of kMfmaRows rows, tile), wave w on proxy columns
// 64 w .. 64 w + 63 of the tile (up 0..255, gate 256..511), with 16 steps
// of codes in flight throughout.  The codes come from
// pq2, where one word holds 8 consecutive rows of one proxy column (byte q:
// row 2q low nibble, row 2q + 1 high nibble), so a lane's 16-byte load is
// the K-run of 8 rows for 4 columns: the A operand of 4 MFMAs at once.
// v_mfma_f32_16x16x32_bf16, per 32-row step s and r = 0..3:
//   A: lane l holds column c0 + 4 (l%16) + r, rows 32 s + 8 (l/16) .. +7, as
//      bf16 128 + nib (the nibble under the exponent byte 0x43, exact);
//   B: lane l holds token l%16 (tokens past NB repeat the last one; their
//      results are dropped), the same rows of x masked by its own
//      threshold, from LDS;
//   D: element i of lane l = column c0 + 16 (l/16) + 4 i + r, token l%16.
// sum_i x_i (128 + nib_i) = sum_i x_i q_i + 136 sum_i x_i, so at the end of
// each G-row group the step sums of x take out the offset and the column's
// group scale is applied: acc += S (D - 136 sum x).  The whole matrix is
// read whatever the input mask: at 2 or more tokens the union of the masks
// leaves few 8-row blocks empty.
__global__ __launch_bounds__(512) void retile_pq2_kernel(const uint8_t *pq, unsigned *pq2,
                                                         int d_model) {
  const int rb = blockIdx.x, t = blockIdx.y, pc = threadIdx.x;
  const uint8_t *src = pq + ((size_t)t * d_model + (size_t)rb * 8) * kTileBytes + (pc >> 1);
  const int sh = (pc & 1) * 4;
  unsigned w = 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) w |= (unsigned)((src[(size_t)e * kTileBytes] >> sh) & 0xfu) << (4 * e);
  pq2[((size_t)t * (d_model / 8) + rb) * 512 + pc] = w;
}

// Rows per work-group of the matrix-core Stage 1 (its own chunking; partials
// and the tile counter use kMfmaRows-row chunks).
constexpr int kMfmaRows = 1024;

// CH: rows per chunk, kMfmaRows or 2 * kMfmaRows (the latter for G a
// multiple of 128, so that its groups' scales fit the same LDS).  GS: G / 32
// when G is known at compile time (4: G = 128), else 0; then the group ends
// are fixed steps, and the first step of a group starts its MFMA sums from
// zero instead of clearing them at the previous group's end.
template <int NB, int CH, int GS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 8))) void proxy_mfma_kernel(
    ProxyArgs a) {
  constexpr int KS = CH / 32;  // 32-row steps per chunk
  constexpr int WIN = 12;  // steps of codes in flight per wave (16 measured no faster)
  constexpr int GMIN = CH == kMfmaRows ? 64 : 128;  // smallest group size served
  constexpr int NGC = CH / GMIN;                     // groups a chunk can touch
  __shared__ __attribute__((aligned(16))) uint16_t xs[NB][CH];  // masked x (bf16 bits)
  __shared__ float xk[NB][KS];                                  // its sum over each step
  __shared__ float ss[NGC][512];  // group scales of the chunk's groups
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int chunk = blockIdx.x, t = blockIdx.y;
  const int r0 = chunk * CH;
  const int nks = min(KS, (a.d_model - r0) / 32);
  const int c0 = wv * 64;
  const int grp0 = r0 / a.G;
  const int ngc = (r0 + 32 * nks - 1) / a.G - grp0 + 1;  // groups the chunk touches

  // Masked x of the chunk's first 1024 rows per token and the group scales
  // go out first; the first WIN steps of codes (16 bytes per lane per step)
  // right behind them, so that the staging below waits only for its own
  // loads.  Each later step's codes are requested as a step is consumed.
  const int i0 = threadIdx.x;
  float xv[2][NB];
  auto load_x = [&](int half0) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // clamped loads, no branch: every load in flight at once
        const int row = r0 + i0 + 512 * (half0 + h);
        const float v = ld_elem<true>(a.x, (size_t)b * a.d_model + min(row, a.d_model - 1));
        xv[h][b] = row < a.d_model ? v : 0.0f;
      }
  };
  load_x(0);
  float sv[NGC];
#pragma unroll
  for (int q = 0; q < NGC; ++q)
    sv[q] = a.psc[((size_t)t * a.ngroups + grp0 + min(q, ngc - 1)) * 512 + i0];
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(a.pq2 + (size_t)t * (a.d_model / 8) * 512, (uint32_t)a.d_model * kTileBytes);
  auto code_off = [&](int s) {
    return ((uint32_t)(r0 / 8 + 4 * s + g) * 512u + (uint32_t)(c0 + 4 * m)) * 4u;
  };
  u4 w[WIN];
#pragma unroll
  for (int s = 0; s < WIN; ++s)  // past d_model: 0, unused
    w[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, code_off(s), 0, kNT);
  // (kept ahead of the staging: the scheduler would sink them below it)
  __builtin_amdgcn_sched_barrier(0);
  // Staging, 1024 rows at a time (the next rows' x loads go out once these
  // are in LDS).
#pragma unroll
  for (int half0 = 0; half0 < CH / 512; half0 += 2) {
    if (half0 > 0) load_x(half0);
    if (a.drows && t == 0) {
      // the input mask this kernel applies, per token and 64-row slice
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row0 = r0 + 512 * (half0 + h) + 64 * wv;  // the wave's 64 rows
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const uint64_t mk = __ballot(fabsf(xv[h][b]) >= a.tau);
          if (row0 < a.d_model)
            export_slice(a.drows + (size_t)b * a.d_model, a.dcnt + (size_t)b * (a.d_model / 64),
                         row0 / 64, mk);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = i0 + 512 * (half0 + h);
        float v = fabsf(xv[h][b]) >= a.tau ? xv[h][b] : 0.0f;
        // K order of each 8-row block as the A operand holds it (rows 0, 2,
        // 4, 6, 1, 3, 5, 7; see the decode below)
        xs[b][(i & ~7) | ((i & 1) << 2) | ((i >> 1) & 3)] = (uint16_t)(__float_as_uint(v) >> 16);
        // sum over the 32 rows of this half-wave
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
        if ((lane & 31) == 0) xk[b][i >> 5] = v;
      }
  }
#pragma unroll
  for (int q = 0; q < NGC; ++q)
    if (q < ngc) ss[q][i0] = sv[q];
  // LDS written; the codes may still be in flight (a plain barrier, no wait
  // on memory loads)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  const int tok = min(m, NB - 1);
  f32x4_t acc[4], d[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    d[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  uint32_t nib_mask, c43;
  asm volatile("s_mov_b32 %0, 0x0f0f0f0f" : "=s"(nib_mask));
  asm volatile("s_mov_b32 %0, 0x43434343" : "=s"(c43));
  float xg = 0.0f;  // sum of this lane's token's masked x over the current group
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint32_t wd[4] = {w[s % WIN].x, w[s % WIN].y, w[s % WIN].z, w[s % WIN].w};
    if (s + WIN < KS) w[s % WIN] = __builtin_amdgcn_raw_buffer_load_b128(rs, code_off(s + WIN), 0, kNT);
    // (the bound also keeps the compiler from hoisting every group's scale
    // reads to the top, which spilled registers)
    if (s < nks) {
      bf16x8_t B;
      __builtin_memcpy(&B, &xs[tok][32 * s + 8 * g], 16);
      // a chunk starts on a group boundary (CH and r0 are multiples of G)
      constexpr bool kNone = false;
      const bool gbeg = GS ? (s % (GS ? GS : 1) == 0) : kNone;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // lo holds the codes of rows 0, 2, 4, 6 of the 8-row word (one per
        // byte), hi those of rows 1, 3, 5, 7; each bf16 is 128 + code, the
        // code byte under the exponent byte 0x43, so one v_perm from
        // (0x43434343, lo or hi) makes two of them.  The A operand's K order
        // is therefore rows 0, 2, 4, 6, 1, 3, 5, 7, and x is staged in LDS in
        // the same order.
        const uint32_t lo = wd[r] & nib_mask, hi = (wd[r] >> 4) & nib_mask;
        const uint32_t q[4] = {__builtin_amdgcn_perm(c43, lo, 0x04010400u),
                               __builtin_amdgcn_perm(c43, lo, 0x04030402u),
                               __builtin_amdgcn_perm(c43, hi, 0x04010400u),
                               __builtin_amdgcn_perm(c43, hi, 0x04030402u)};
        bf16x8_t A;
        __builtin_memcpy(&A, q, 16);
        d[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            A, B, gbeg ? f32x4_t{0.0f, 0.0f, 0.0f, 0.0f} : d[r], 0, 0, 0);
      }
      xg += xk[tok][s];
      const int row_end = r0 + 32 * (s + 1);
      const bool gend = GS ? ((s + 1) % (GS ? GS : 1) == 0) : (s == nks - 1 || row_end % a.G == 0);
      if (gend) {
        const int gi = GS ? s / (GS ? GS : 1) : (row_end - 1) / a.G - grp0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[r][i] += ss[gi][c0 + 16 * g + 4 * i + r] * (d[r][i] - 136.0f * xg);
            if (!GS) d[r][i] = 0.0f;
          }
        xg = 0.0f;
      }
    }
  }
  // This chunk's partials: lane l holds columns c0 + 16 (l/16) .. +15 of
  // token l%16; through LDS (the scales' space) so that the stores are whole
  // rows.
  __syncthreads();  // every wave is done with the scales
  float (*red)[512] = ss;
  static_assert(NB <= NGC, "partials fit the scale array");
  if (m < NB) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(float4 *)&red[m][c0 + 16 * g + 4 * i] = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
  }
  __syncthreads();
  {
    float *part = a.part + ((size_t)t * a.nchunk + chunk) * NB * 512;
#pragma unroll
    for (int b = 0; b < NB; ++b) xstore(&part[b * 512 + i0], red[b][i0]);
  }
  if (!arrive_last(&a.tile_cnt[t], (unsigned)a.nchunk, &s_last)) return;

  // Tile epilogue: u~, g~ per token, then |s~|, the chunk partials added in
  // chunk order (as proxy_kernel does), every partial of this thread's
  // (token, column) pairs requested at once, 8 chunks per round.
  const float *tp = a.part + (size_t)t * a.nchunk * NB * 512;
  constexpr int PP = (NB * 256 + 511) / 512;  // pairs per thread
  float su[PP], sg[PP];
#pragma unroll
  for (int p = 0; p < PP; ++p) su[p] = sg[p] = 0.0f;
  for (int cb = 0; cb < a.nchunk; cb += 8) {
    float vu[PP][8], vg[PP][8];
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      const int e = min((int)threadIdx.x + 512 * p, NB * 256 - 1);
      const int b = e >> 8, col = e & 255;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float *q = tp + ((size_t)min(cb + c, a.nchunk - 1) * NB + b) * 512 + col;
        vu[p][c] = xload(q);
        vg[p][c] = xload(q + 256);
      }
    }
#pragma unroll
    for (int p = 0; p < PP; ++p)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (cb + c < a.nchunk) {
          su[p] += vu[p][c];
          sg[p] += vg[p][c];
        }
  }
#pragma unroll
  for (int p = 0; p < PP; ++p) {
    const int e = (int)threadIdx.x + 512 * p;
    const int b = e >> 8, col = e & 255;
    const int j = t * kTile + col;
    if (e < NB * 256 && j < a.d_ff) a.sabs[(size_t)b * a.d_ff + j] = fabsf(su[p] * gate_act(sg[p], a.act));
  }
}

// ---------------------------------------------------------------------------
// K-d  Top-k channel mask (App. A.6, top-k equation), ties to the lower index
// ---------------------------------------------------------------------------
// One 1024-thread work-group per token.  |s~| >= 0, so its float32 bit
// pattern orders like the value: a most-significant-digit radix select on the
// bits (digits of 11, 11 and 9 bits below the always-zero sign bit) finds the
// k-th largest key T and how many keys equal to T are taken (kk).
// Channel j is held by thread j % 1024 in register slot j / 1024, so loads
// are coalesced and each slot is one run of 1024 consecutive channels: the
// output position of a kept channel is (kept in earlier slots) + (kept in
// earlier waves of its slot) + (kept in lower lanes), from ballots and one
// scan of the per-(slot, wave) counts, so the list comes out ascending.
// Each digit's bin is picked by the whole work-group (pick_bin).

// All 1024 threads find the bin holding the kk-th largest key: thread t
// owns bins [NBINS - (t + 1) * BPT, NBINS - t * BPT) (from the top; threads
// past the bins own none), reads them from consecutive LDS words and a block
// scan gives the keys above its bins.  hist(b) returns the count of bin b.
// Writes the bin and the remaining rank to *s_bin / *s_kk (2 barriers
// inside; the caller's barrier publishes them).
template <int NBINS, typename H>
__device__ __forceinline__ void pick_bin(H hist, unsigned kk, unsigned *wsum, unsigned *s_bin,
                                         unsigned *s_kk) {
  constexpr int BPT = NBINS >= 1024 ? NBINS / 1024 : 1;
  const int t = threadIdx.x;
  unsigned c[BPT];
  unsigned sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int r = t * BPT + i;  // rank of the bin from the top
    c[i] = r < NBINS ? hist(NBINS - 1 - r) : 0u;
    sum += c[i];
  }
  unsigned tot;
  unsigned above = block_excl_scan<16>(sum, wsum, tot);
  if (above < kk && above + sum >= kk) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (above < kk && above + c[i] >= kk) {
        *s_bin = (unsigned)(NBINS - 1 - (t * BPT + i));
        *s_kk = kk - above;
      }
      above += c[i];
    }
  }
}

// Union of the per-token mask words (several tokens): U ascending, plus for
// each entry the bit set of tokens whose mask holds it.  All 1024 threads of
// one work-group; thread w owns mask word w (channels 32 w .. 32 w + 31, d_ff
// <= 32768), reads that word of every token and places its union entries at
// its exclusive prefix of the word popcounts, in LDS; the work-group then
// writes the list out in order, consecutive threads on consecutive entries.
__device__ __forceinline__ void mask_union(const unsigned *selw, int d_ff, int nb, int *uni,
                                           int *nuni, uint8_t *umask, unsigned *wsum,
                                           uint16_t *su, uint8_t *sb) {
  const int w = threadIdx.x;
  const int words = (d_ff + 31) >> 5;
  unsigned tw[kMaxBatch], u = 0u;
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) {
    tw[b] = (b < nb && w < words) ? xload_u(&selw[(size_t)b * words + w]) : 0u;
    u |= tw[b];
  }
  unsigned total;
  unsigned pos = block_excl_scan<16>((unsigned)__popc(u), wsum, total);
  while (u) {
    const int bit = __builtin_ctz(u);
    u &= u - 1u;
    unsigned m = 0u;
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) m |= ((tw[b] >> bit) & 1u) << b;
    su[pos] = (uint16_t)(w * 32 + bit);
    sb[pos] = (uint8_t)m;
    ++pos;
  }
  __syncthreads();
  for (int p = w; p < (int)total; p += 1024) {
    uni[p] = (int)su[p];
    umask[p] = sb[p];
  }
  if (w == 0) *nuni = (int)total;
}

// f(std::integral_constant<int, 0>{}), ..., f(<N - 1>): a loop whose index
// is a compile-time constant in the body.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// With several tokens (ucnt set) the last work-group to finish also builds
// the union of the masks, so top-k and union are one launch.
template <int PER>
__global__ __launch_bounds__(1024) void topk_kernel(const float *sabs, int d_ff, int k,
                                                    int *sel, unsigned *selw, unsigned *ucnt,
                                                    int *uni, int *nuni, uint8_t *umask) {
  // digit 1 in 4 copies, picked by lane % 4 and interleaved (a bin's copies
  // are 4 consecutive words, in 4 banks): the lanes of one wave whose keys
  // fall in the same crowded bin then queue on 4 addresses instead of 1
  __shared__ __attribute__((aligned(16))) unsigned h1[2048][4];
  __shared__ unsigned h2[2048];
  __shared__ unsigned h3[512];
  __shared__ unsigned cnt[PER * 16];
  __shared__ unsigned s_bin, s_kk;
  __shared__ unsigned wsum[16];
  __shared__ int s_last;
  // the union list before it goes out (last work-group, several tokens)
  __shared__ uint16_t su[kMaxDff];
  __shared__ uint8_t sb[kMaxDff];
  const int b = blockIdx.x;
  if (k <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float *z = sabs + (size_t)b * d_ff;
  int *out = sel ? sel + (size_t)b * d_ff : nullptr;
  const int words = (d_ff + 31) >> 5;
  unsigned *outw = selw ? selw + (size_t)b * words : nullptr;
  unsigned key[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = e * 1024 + tid;
    key[e] = (j < d_ff) ? __float_as_uint(z[j]) : 0u;
  }
  *(uint4 *)h1[tid] = make_uint4(0u, 0u, 0u, 0u);
  *(uint4 *)h1[tid + 1024] = make_uint4(0u, 0u, 0u, 0u);
  h2[tid] = 0u; h2[tid + 1024] = 0u;
  if (tid < 512) h3[tid] = 0u;
  __syncthreads();

  // Digit 1: bits 30..20.
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (e * 1024 + tid < d_ff) atomicAdd(&h1[key[e] >> 20][lane & 3], 1u);
  __syncthreads();
  pick_bin<2048>([&](int i) { return h1[i][0] + h1[i][1] + h1[i][2] + h1[i][3]; }, (unsigned)k,
                 wsum, &s_bin, &s_kk);
  __syncthreads();
  const unsigned b1 = s_bin;
  unsigned kk = s_kk;

  // Digit 2: bits 19..9 of the keys with digit 1 = b1.
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (e * 1024 + tid < d_ff && (key[e] >> 20) == b1) atomicAdd(&h2[(key[e] >> 9) & 2047u], 1u);
  __syncthreads();
  pick_bin<2048>([&](int i) { return h2[i]; }, kk, wsum, &s_bin, &s_kk);
  __syncthreads();
  const unsigned p2 = (b1 << 11) | s_bin;
  kk = s_kk;

  // Digit 3: bits 8..0 of the keys with digits 1-2 = p2.
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (e * 1024 + tid < d_ff && (key[e] >> 9) == p2) atomicAdd(&h3[key[e] & 511u], 1u);
  __syncthreads();
  pick_bin<512>([&](int i) { return h3[i]; }, kk, wsum, &s_bin, &s_kk);
  __syncthreads();
  const unsigned T = (p2 << 9) | s_bin;
  kk = s_kk;  // keys equal to T that are kept (the lowest-index ones)

  // No list wanted and every key equal to T kept (h3 counts the keys equal
  // to T): the mask is key >= T, written as bit words only.
  // The mask words of this wave's channels: slot e's 64 channels are words
  // 32 e + 2 w and 32 e + 2 w + 1, gathered into lanes 2 e and 2 e + 1 and
  // written by one store (a store per word cost 4 us of issue on this CU).
  unsigned mw = 0u;
  auto put_words = [&](auto e, uint64_t km) {
    constexpr int l0 = 2 * decltype(e)::value;
    mw = lane == l0 ? (unsigned)km : mw;
    mw = lane == l0 + 1 ? (unsigned)(km >> 32) : mw;
  };
  auto store_words = [&]() {
    const int wi = (lane >> 1) * 32 + w * 2 + (lane & 1);
    if (lane < 2 * PER && wi < words) xstore_u(&outw[wi], mw);
  };
  if (!sel && outw && kk == h3[s_bin]) {
    static_for<PER>([&](auto e) {
      const int j = decltype(e)::value * 1024 + tid;
      put_words(e, __ballot(j < d_ff && key[decltype(e)::value] >= T));
    });
    store_words();
  } else {

    // Compaction.  Pass A: per (slot, wave) counts of keys > T and == T.
    uint64_t mgt[PER], meq[PER];
  #pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool ok = e * 1024 + tid < d_ff;
      mgt[e] = __ballot(ok && key[e] > T);
      meq[e] = __ballot(ok && key[e] == T);
      if (lane == 0) cnt[e * 16 + w] = ((unsigned)__popcll(meq[e]) << 16) | (unsigned)__popcll(mgt[e]);
    }
    __syncthreads();
    // Wave 0: exclusive scan of the PER*16 counts in (slot, wave) order.
    if (w == 0) {
      constexpr int CPL = (PER * 16 + 63) / 64;
      unsigned c[CPL], sum = 0;
  #pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int q = lane * CPL + i;
        c[i] = q < PER * 16 ? cnt[q] : 0u;
        sum += c[i];
      }
      unsigned run = wave_incl_scan(sum) - sum;
  #pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int q = lane * CPL + i;
        if (q < PER * 16) cnt[q] = run;
        run += c[i];
      }
    }
    __syncthreads();
    // Pass B: positions.  Before this key: gt_b keys > T and eq_b keys == T;
    // it is kept if > T, or == T with eq_b < kk; its position is gt_b + min(eq_b, kk).
    const uint64_t below = (1ull << lane) - 1ull;
    static_for<PER>([&](auto ec) {
      constexpr int e = decltype(ec)::value;
      const int j = e * 1024 + tid;
      const unsigned base = cnt[e * 16 + w];
      const unsigned gt_b = (base & 0xffffu) + (unsigned)__popcll(mgt[e] & below);
      const unsigned eq_b = (base >> 16) + (unsigned)__popcll(meq[e] & below);
      const bool kept = j < d_ff && (key[e] > T || (key[e] == T && eq_b < kk));
      if (kept && out) out[key[e] > T ? gt_b + min(eq_b, kk) : gt_b + eq_b] = j;
      // the same mask as bit words
      if (outw) put_words(ec, __ballot(kept));
    });
    if (outw) store_words();
  }
  if (ucnt) {
    if (!arrive_last(ucnt, gridDim.x, &s_last)) return;
    mask_union(selw, d_ff, (int)gridDim.x, uni, nuni, umask, wsum, su, sb);
  }
}
// ---------------------------------------------------------------------------
// K-e  Stage 2a: exact gathered up/gate GEMV fused with SiLU and the product
//      (Sec. 4.1, Stage 2 equations: u_sp, h_sp, s_sp over the full x)
// ---------------------------------------------------------------------------
// One wave per selected channel j (grid-stride over list positions).  The
// channel's up row and gate row are one contiguous run of 2*d_model elements
// (channel-major layout), read 16 bytes per lane per step; x sits in LDS.
// mode 0: position p -> channel sel[p] (one token); mode 1: channel uni[p],
// s zeroed for tokens whose own mask lacks it; mode 2: dense, channel p;
// mode 3 (several tokens): channel p if the union of the tokens' mask words
// holds it (else skipped), s zeroed for tokens whose own mask lacks it and
// stored by channel, so no union list is built.
// Exact s of the selected channels: one token, ssp[p] for list position p;
// NB >= 2 tokens, ssp[p * sstride(NB) + b], the tokens of a position side by
// side (stride rounded up to 4 floats, so a row's values are whole 16-byte
// loads for the down projection).
__host__ __device__ constexpr int sstride(int nb) { return nb == 1 ? 1 : (nb + 3) & ~3; }

// Channels per wave block of the mode-3 up/gate kernel: one at 2 tokens,
// 4 at 3 and 4 tokens, 8 from 5 (measured 70B-shaped steps: 2 tokens 189 us
// with one channel per block against 202 with 8; 4 tokens 246.4 us with 4
// against 249.5 with 8 and 248.1 with 2; 8 tokens 310 with 8 against 314
// with 4).  A power of two up to 32, so a block lies in one mask word.
__host__ __device__ constexpr int upgate_block(int nb) { return nb <= 2 ? 1 : nb <= 4 ? 4 : 8; }

struct UpGateArgs {
  const void *wug;
  uint32_t wug_bytes;
  const void *x;
  int d_model, d_ff, n;
  const int *n_ptr;
  const int *list;
  const uint8_t *umask;
  float *ssp;
  int act;  // gate activation (gate_act)
  const unsigned *selw;  // mode 3: [NB][ceil(d_ff / 32)] per-token mask words
};


template <int NB, bool BF16, int MODE, int NWV>
__global__ __launch_bounds__(NWV * 64) void upgate_kernel(UpGateArgs a) {
  extern __shared__ u4 xs[];
  constexpr int EPL = BF16 ? 8 : 4;   // elements per 16-byte load
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int MU = 8;               // 16-byte steps in flight per matrix
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row16 = a.d_model / EPL;  // 16-byte units per row
  for (int i = threadIdx.x; i < NB * row16; i += NWV * 64) xs[i] = ((const u4 *)a.x)[i];
  __syncthreads();

  const int n = a.n_ptr ? *a.n_ptr : a.n;
  const int nsteps = row16 / 64;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.wug, a.wug_bytes);
  const int W = gridDim.x * NWV;
  // One channel: its up and gate rows against every token's x; s stored at
  // slot p (list position, or the channel in mode 3), zero for tokens not in
  // tok.
  auto channel = [&](int p, int j, unsigned tok) {
    const uint32_t ubase = (uint32_t)j * 2u * (uint32_t)a.d_model * ESZ;
    const uint32_t gbase = ubase + (uint32_t)a.d_model * ESZ;
    float au[NB], ag[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) au[b] = ag[b] = 0.0f;
    for (int m0 = 0; m0 < nsteps; m0 += MU) {
      u4 wu[MU], wg[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const uint32_t off = (uint32_t)((m0 + u) * 64 + lane) * 16u;
        if (m0 + u < nsteps) {
          wu[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, ubase, kNT);
          wg[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, gbase, kNT);
        }
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        if (m0 + u < nsteps) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const u4 xv = xs[b * row16 + (m0 + u) * 64 + lane];
            au[b] = dot16<BF16>(wu[u], xv, au[b]);
            ag[b] = dot16<BF16>(wg[u], xv, ag[b]);
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float u = wave_sum(au[b]);
      const float g = wave_sum(ag[b]);
      if (lane == 0)
        a.ssp[(size_t)p * sstride(NB) + b] = ((tok >> b) & 1u) ? u * gate_act(g, a.act) : 0.0f;
    }
  };
  if constexpr (MODE == 3) {
    // Blocks of upgate_block(NB) consecutive channels per wave: the tokens'
    // mask bits of a block come in once, and only the channels of their
    // union are visited.
    constexpr int BLK = upgate_block(NB);
    const int words = (a.d_ff + 31) >> 5;
    const int nblk = (a.d_ff + BLK - 1) / BLK;
    for (int q = blockIdx.x * NWV + wv; q < nblk; q += W) {
      const int c0 = q * BLK;
      unsigned tb[NB], um = 0u;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        tb[b] = (a.selw[(size_t)b * words + (c0 >> 5)] >> (c0 & 31)) & ((1u << BLK) - 1u);
        um |= tb[b];
      }
      while (um) {  // wave-uniform
        const int i = __builtin_ctz(um);
        um &= um - 1u;
        unsigned tok = 0u;
#pragma unroll
        for (int b = 0; b < NB; ++b) tok |= ((tb[b] >> i) & 1u) << b;
        channel(c0 + i, c0 + i, tok);
      }
    }
  } else {
    for (int p = blockIdx.x * NWV + wv; p < n; p += W)
      channel(p, MODE == 2 ? p : a.list[p], MODE == 1 ? (unsigned)a.umask[p] : 0xffu);
  }
}

// Batch-1 form of K-e: x (d_model elements, 16 bytes per lane per step) is
// held in registers, so a wave starts streaming weights at once, with no LDS
// prologue or barrier.  Wave w takes the contiguous list positions
// [w*per, (w+1)*per), per chosen by the host so that all waves are resident
// and carry equal work.  NSTEP = d_model / (64 lanes * 16 bytes / element).
template <bool BF16, int MODE, int NSTEP>
__global__ __launch_bounds__(256) void upgate1_kernel(UpGateArgs a, int per) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p0 = gw * per;
  const int p1 = min(a.n, p0 + per);
  if (p0 >= a.n) return;
  constexpr int ESZ = BF16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.wug, a.wug_bytes);
  const uint32_t rowb = (uint32_t)a.d_model * ESZ;  // bytes of one up (or gate) row
  u4 xr[NSTEP];
#pragma unroll
  for (int m = 0; m < NSTEP; ++m) xr[m] = ((const u4 *)a.x)[m * 64 + lane];
  for (int p = p0; p < p1; ++p) {
    const int j = (MODE == 2) ? p : a.list[p];
    const uint32_t ubase = (uint32_t)j * 2u * rowb;
    u4 wu[NSTEP], wg[NSTEP];
#pragma unroll
    for (int m = 0; m < NSTEP; ++m) {
      const uint32_t off = (uint32_t)(m * 64 + lane) * 16u;
      wu[m] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, ubase, kNT);
      wg[m] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, ubase + rowb, kNT);
    }
    // Keep every load of the channel in flight before the first use.
    __builtin_amdgcn_sched_barrier(0);
    float au = 0.0f, ag = 0.0f;
#pragma unroll
    for (int m = 0; m < NSTEP; ++m) {
      au = dot16<BF16>(wu[m], xr[m], au);
      ag = dot16<BF16>(wg[m], xr[m], ag);
    }
    const float u = wave_sum(au);
    const float g = wave_sum(ag);
    if (lane == 0) a.ssp[p] = u * gate_act(g, a.act);
  }
}

// ---------------------------------------------------------------------------
// K-f  Stage 2b: input-sparse down projection y = s_sp W_down[sel, :]
//      (Sec. 4.1, Stage 2 equations; Sec. 3.1, weighted-sum view)
// ---------------------------------------------------------------------------
// Grid (ncol, nrc), NW waves.  Work-group (c, r) covers output columns
// [256c, 256c + 256) and list positions [rR, rR + R).  float32: lane l owns 4
// columns of the wave's row (16 bytes), row index and s uniform across the
// wave.  bfloat16: a 512-byte row is half a wave, so one load covers two
// rows, lane l owning 8 columns of row l / 32; the halves are folded at the
// end.  Waves split the rows and add up in LDS.  W_down is stored in
// 256-column chunks (see retile_down_kernel), so a chunk's rows are
// contiguous and a dense pass streams each chunk sequentially.  The last work-group of a
// column chunk adds the nrc partials in order, casts y to the layer dtype
// and, for the stack, adds it to the float32 residual.
struct DownArgs {
  const void *wd;
  uint32_t wd_bytes;
  int d_model, d_ff, n, nrc;
  const int *n_ptr;
  const int *list;
  const float *ssp;
  float *ypart;
  unsigned *col_cnt;
  void *y;
  float *resid;
  const unsigned *selw;  // mode 3: [NB][ceil(d_ff / 32)] per-token mask words
};
// Mode 3 of the down kernel: work-group row ranges of whole mask words, each
// holding at most this many channels (its union list sits in LDS).
constexpr int kDownLocal = 4096;

// s of list position pc for NB tokens (zeros unless ok): one float for one
// token, else whole 16-byte loads of the position's row of ssp.
template <int NB>
__device__ __forceinline__ void load_s(const float *ssp, int pc, bool ok, float (&sv)[NB]) {
  if constexpr (NB == 1) {
    const float v = ssp[pc];
    sv[0] = ok ? v : 0.0f;
  } else {
    const float4 *r = (const float4 *)(ssp + (size_t)pc * sstride(NB));
#pragma unroll
    for (int q = 0; q < (NB + 3) / 4; ++q) {
      const float4 v = r[q];
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < NB) sv[4 * q + i] = ok ? e[i] : 0.0f;
    }
  }
}

template <int NB, bool BF16, int MODE, int NW>
__global__ __launch_bounds__(NW * 64, NW == 16 ? 8 : 4) void down_kernel(DownArgs a) {
  // rows in flight per wave: float32 one row per load (16 bytes a lane);
  // bfloat16 two rows per load (lanes 0-31 and 32-63, 16 bytes a lane).
  // 3 and 4 tokens take 8 loads in the dense and mask-word modes (70B-shaped
  // 4-token step 263 us against 272 with 6; 10 spills), 6 in the list modes,
  // where 8 would spill.
  constexpr int U = BF16 ? (NB > 6 ? 3 : NB > 4 ? 4 : NB == 2 ? 8 : NB == 1 ? 6 : MODE >= 2 ? 8 : 6)
                         : 8;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int CPL = BF16 ? 8 : 4;      // columns per lane
  __shared__ float red[NW][NB][kDownCols];
  __shared__ int s_last;
  // mode 3: this work-group's union channels, ascending
  __shared__ uint16_t s_list[MODE == 3 ? kDownLocal : 1];
  __shared__ unsigned wsum[NW];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cc = blockIdx.x, rc = blockIdx.y;
  int p0, p1;  // list positions of this work-group
  if constexpr (MODE == 3) {
    // Channels [c0, c1), whole mask words: the union of the tokens' words,
    // one word per thread, placed by a block scan of the popcounts.
    // (c0 stays a multiple of 32; past d_ff the range is empty: c1 <= c0)
    const int R = (((a.d_ff + a.nrc - 1) / a.nrc) + 31) & ~31;
    const int c0 = rc * R, c1 = min(a.d_ff, c0 + R);
    const int w = (c0 >> 5) + (int)threadIdx.x;
    unsigned u = 0u;
    if (w * 32 < c1) {
      const int words = (a.d_ff + 31) >> 5;
#pragma unroll
      for (int b = 0; b < NB; ++b) u |= a.selw[(size_t)b * words + w];
      if (c1 - w * 32 < 32) u &= (1u << (c1 - w * 32)) - 1u;
    }
    unsigned tot;
    unsigned pos = block_excl_scan<NW>((unsigned)__popc(u), wsum, tot);
    while (u) {
      const int bit = __builtin_ctz(u);
      u &= u - 1u;
      s_list[pos++] = (uint16_t)(w * 32 + bit);
    }
    __syncthreads();
    p0 = 0;
    p1 = (int)tot;
  } else {
    const int n = a.n_ptr ? *a.n_ptr : a.n;
    const int R = (n + a.nrc - 1) / a.nrc;
    p0 = rc * R;
    p1 = min(n, p0 + R);
  }
  // channel of list position pp, and where its s is kept (by position, or by
  // channel in mode 3)
  auto row_of = [&](int pp) -> int {
    if constexpr (MODE == 2) return pp;
    else if constexpr (MODE == 3) return (int)s_list[pp];
    else return a.list[pp];
  };
  // this chunk's rows: [d_ff][256] elements starting at chunk cc
  const size_t chunk_bytes = (size_t)a.d_ff * kDownCols * ESZ;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc((const char *)a.wd + cc * chunk_bytes, (uint32_t)chunk_bytes);

  float acc[NB][CPL];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[b][c] = 0.0f;

  if constexpr (BF16) {
    // Wave wv takes row pairs wv, wv+NW, ...; half h = lane / 32 of the wave
    // takes the pair's row h, lane % 32 its columns 8 (lane % 32) .. +7.  An
    // out-of-range slot re-reads row p0 and gets s = 0 (no branches).
    const int h = lane >> 5;
    const uint32_t voff = (uint32_t)(lane & 31) * 16u;
    constexpr int STEP = 2 * NW * U;
    // Channel numbers of the next step are fetched while this step's rows
    // are in flight, so a step waits for one memory round trip, not two
    // (list entry, then row).
    int jn[U];
    auto fetch_j = [&](int pb) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pp = pb + 2 * NW * u + h;
        const int ppc = pp < p1 ? pp : p0;
        jn[u] = row_of(ppc);
      }
    };
    const int pstart = p0 + 2 * wv;
    if (pstart < p1) fetch_j(pstart);
    for (int p = pstart; p < p1; p += STEP) {
      u4 w[U];
      float sv[U][NB];
#pragma unroll
      for (int u = 0; u < U; ++u)
        w[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + (uint32_t)jn[u] * (kDownCols * 2u), 0, kNT);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pp = p + 2 * NW * u + h;
        const bool ok = pp < p1;
        // unconditional loads of a valid slot, then select: no branch
        load_s<NB>(a.ssp, MODE == 3 ? jn[u] : (ok ? pp : p0), ok, sv[u]);
      }
      fetch_j(p + STEP);  // past the end: clamped, valid, unused
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(ww[q] << 16), hi = __uint_as_float(ww[q] & 0xffff0000u);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            acc[b][2 * q] = fmaf(sv[u][b], lo, acc[b][2 * q]);
            acc[b][2 * q + 1] = fmaf(sv[u][b], hi, acc[b][2 * q + 1]);
          }
        }
      }
    }
    // The two halves hold the same columns: fold the upper into the lower.
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[b][c] += __shfl_xor(acc[b][c], 32);
    if (lane < 32) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        *(float4 *)&red[wv][b][lane * 8] = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
        *(float4 *)&red[wv][b][lane * 8 + 4] = make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
      }
    }
  } else {
    const uint32_t voff = (uint32_t)lane * 16u;
    // Rows p0+wv, p0+wv+NW, ... of this chunk; an out-of-range slot re-reads a
    // valid row and gets s = 0, so the loop body has no branches.
    for (int p = p0 + wv; p < p1; p += NW * U) {
      float wf[U][4];
      float sv[U][NB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pp = p + NW * u;
        const bool ok = pp < p1;
        const int ppc = ok ? pp : p;
        const int j = row_of(ppc);
        load_s<NB>(a.ssp, MODE == 3 ? j : ppc, ok, sv[u]);
        const uint32_t rowoff = (uint32_t)j * (uint32_t)(kDownCols * ESZ);
        const u4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, rowoff, kNT);
        wf[u][0] = __uint_as_float(w.x);
        wf[u][1] = __uint_as_float(w.y);
        wf[u][2] = __uint_as_float(w.z);
        wf[u][3] = __uint_as_float(w.w);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[b][c] = fmaf(sv[u][b], wf[u][c], acc[b][c]);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      *(float4 *)&red[wv][b][lane * 4] = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
  }
  __syncthreads();
  float *yp = a.ypart + (size_t)rc * NB * a.d_model;
  for (int e = threadIdx.x; e < NB * kDownCols; e += NW * 64) {
    const int b = e / kDownCols, c = e % kDownCols;
    float v = red[0][b][c];
#pragma unroll
    for (int q = 1; q < NW; ++q) v += red[q][b][c];
    xstore(&yp[(size_t)b * a.d_model + cc * kDownCols + c], v);
  }
  if (!arrive_last(&a.col_cnt[cc], (unsigned)a.nrc, &s_last)) return;
  for (int e = threadIdx.x; e < NB * kDownCols; e += NW * 64) {
    const int b = e / kDownCols, c = cc * kDownCols + e % kDownCols;
    const float v = xsum_strided(&a.ypart[(size_t)b * a.d_model + c], a.nrc,
                                 (size_t)NB * a.d_model);
    const size_t o = (size_t)b * a.d_model + c;
    st_elem<BF16>(a.y, o, v);
    if (a.resid) a.resid[o] += round_elem<BF16>(v);
  }
}

// ---------------------------------------------------------------------------
// Verification helpers (debug entries only).
// ---------------------------------------------------------------------------
// The per-slice survivor lists a Stage 1 kernel exported (export_slice)
// concatenated in slice order: n1[b] and the ascending idx[b][0..n1).  One
// work-group per token.
__global__ __launch_bounds__(256) void survivors_kernel(const int *rows, const int *cnt,
                                                        int d_model, int *n1, int *idx) {
  __shared__ int off[kMaxDmodel / 64 + 1];
  const int b = blockIdx.x, nsl = d_model / 64;
  const int *rb = rows + (size_t)b * d_model;
  const int *cb = cnt + (size_t)b * nsl;
  if (threadIdx.x == 0) {
    int o = 0;
    for (int q = 0; q < nsl; ++q) {
      off[q] = o;
      o += cb[q];
    }
    off[nsl] = o;
    n1[b] = o;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < nsl; q += blockDim.x)
    for (int i = 0; i < cb[q]; ++i) idx[(size_t)b * d_model + off[q] + i] = rb[q * 64 + i];
}

// The workspace status word: copied out and cleared; after a timed-out wait
// (bit 0) the whole synchronisation block and the layer's cut guess are
// reset as well, so the next launch starts from the state it expects.
__global__ __launch_bounds__(1024) void read_status_kernel(unsigned *hdr, size_t nwords,
                                                           int err_word, unsigned *pred,
                                                           int *out) {
  const unsigned e = xload_u(&hdr[err_word]);
  __syncthreads();  // every thread has read the word before anyone clears it
  if (threadIdx.x == 0) *out = (int)e;
  if (e & 1u) {
    for (size_t i = threadIdx.x; i < nwords; i += blockDim.x) xstore_u(&hdr[i], 0u);
    if (threadIdx.x == 0) xstore_u(pred, 0u);
  } else if (threadIdx.x == 0) {
    xstore_u(&hdr[err_word], 0u);
  }
}

// ---------------------------------------------------------------------------
// Stack glue: x = cast(r / sqrt(mean(r^2) + eps)), unit gain.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kRmsThreads) void rmsnorm_kernel(const float *resid, int d_model,
                                                             float eps, void *x) {
  __shared__ float part[kRmsThreads / 64];
  const int b = blockIdx.x;
  const float *r = resid + (size_t)b * d_model;
  const float inv = block_inv_rms<kRmsThreads>(r, d_model, eps, part);
  for (int i = threadIdx.x; i < d_model; i += kRmsThreads)
    st_elem<BF16>(x, (size_t)b * d_model + i, r[i] * inv);
}

template <bool BF16>
__global__ void zero_kernel(void *y, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) st_elem<BF16>(y, i, 0.0f);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
#define PROX_DISPATCH_NB(NBVAR, BODY)                  \
  switch (NBVAR) {                                     \
    case 1: { constexpr int NB = 1; BODY; } break;     \
    case 2: { constexpr int NB = 2; BODY; } break;     \
    case 3: { constexpr int NB = 3; BODY; } break;     \
    case 4: { constexpr int NB = 4; BODY; } break;     \
    case 5: { constexpr int NB = 5; BODY; } break;     \
    case 6: { constexpr int NB = 6; BODY; } break;     \
    case 7: { constexpr int NB = 7; BODY; } break;     \
    case 8: { constexpr int NB = 8; BODY; } break;     \
    default: return hipErrorInvalidValue;              \
  }

hipError_t launch_prepare(const Plan &p, const Bufs &b, const void *w_up,
                          const void *w_gate, const void *w_down,
                          hipStream_t s) {
  dim3 tg((p.d_ff + 63) / 64, (p.d_model + 63) / 64, 2);
  if (p.bf16)
    transpose_kernel<true><<<tg, 256, 0, s>>>(w_up, w_gate, b.wug, p.d_model, p.d_ff);
  else
    transpose_kernel<false><<<tg, 256, 0, s>>>(w_up, w_gate, b.wug, p.d_model, p.d_ff);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 rg(p.d_ff, p.ncol);
  if (p.bf16)
    retile_down_kernel<true><<<rg, kDownCols, 0, s>>>(w_down, b.wd, p.d_model, p.d_ff);
  else
    retile_down_kernel<false><<<rg, kDownCols, 0, s>>>(w_down, b.wd, p.d_model, p.d_ff);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Padding columns of the last tile keep code 0 (nibble 8) and scale 0.
  e = hipMemsetAsync(b.pq, 0x88, (size_t)p.ntile * p.d_model * kTileBytes, s);
  if (e != hipSuccess) return e;
  dim3 qg(p.ngroups, p.ntile, 2);
  if (p.bf16)
    quantize_kernel<true><<<qg, 256, 0, s>>>(w_up, w_gate, b.pq, b.psc, p.d_model,
                                             p.d_ff, p.G, p.ngroups);
  else
    quantize_kernel<false><<<qg, 256, 0, s>>>(w_up, w_gate, b.pq, b.psc, p.d_model,
                                              p.d_ff, p.G, p.ngroups);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.proxy_mfma && b.pq2) {
    retile_pq2_kernel<<<dim3(p.d_model / 8, p.ntile), 512, 0, s>>>(b.pq, b.pq2, p.d_model);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;  // the caller zeroes the workspace's synchronisation block
}

hipError_t launch_export_proxy(const Plan &p, const Bufs &b, int matrix,
                               int8_t *codes, float *scales, hipStream_t s) {
  dim3 g(p.d_model, p.ntile);
  export_proxy_kernel<<<g, 256, 0, s>>>(b.pq, b.psc, matrix, p.d_model, p.d_ff,
                                        p.G, p.ngroups, codes, scales);
  return hipGetLastError();
}

hipError_t launch_proxy(const Plan &p, const Bufs &b, const void *x, int batch,
                        float tau, hipStream_t s, bool dbg) {
  ProxyArgs a{b.pq, b.pq2, b.psc, x, tau, p.d_model, p.d_ff, p.G, p.ngroups,
              p.nchunk, b.part, b.tile_cnt, b.sabs, p.act,
              dbg ? b.drows : nullptr, dbg ? b.dcnt : nullptr};
  dim3 g(p.nchunk, p.ntile);
  // On the matrix cores from p.proxy_mfma (2) tokens unless the layer asks
  // for the vector form, which reads only the rows the union of the input
  // masks keeps (about 3/4 of them at 2 tokens) but decodes and multiplies
  // on the VALU.  Its own grid: ceil(d_model / CH) work-groups
  // per tile, CH = 2 * kMfmaRows rows when the 1024-row grid would take more
  // than one round of the resident work-groups (two per CU) and the
  // 2048-row grid still fills three quarters of one (70B shape: 448
  // work-groups instead of 896), else kMfmaRows.
  if (p.proxy_mfma && b.pq2 && batch >= p.proxy_mfma) {
    static int cus = 0;
    if (!cus) {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    }
    const int g1 = (p.d_model + kMfmaRows - 1) / kMfmaRows * p.ntile;
    const int g2 = (p.d_model + 2 * kMfmaRows - 1) / (2 * kMfmaRows) * p.ntile;
    const bool big = p.G % 128 == 0 && (2 * kMfmaRows) % p.G == 0 && g1 > 2 * cus &&
                     4 * g2 >= 3 * 2 * cus;
    const int ch = big ? 2 * kMfmaRows : kMfmaRows;
    a.nchunk = (p.d_model + ch - 1) / ch;
    const dim3 gm(a.nchunk, p.ntile);
    const bool g128 = p.G == 128;
    if (big && g128) {
      PROX_DISPATCH_NB(batch, (proxy_mfma_kernel<NB, 2 * kMfmaRows, 4><<<gm, 512, 0, s>>>(a)));
    } else if (big) {
      PROX_DISPATCH_NB(batch, (proxy_mfma_kernel<NB, 2 * kMfmaRows, 0><<<gm, 512, 0, s>>>(a)));
    } else if (g128) {
      PROX_DISPATCH_NB(batch, (proxy_mfma_kernel<NB, kMfmaRows, 4><<<gm, 512, 0, s>>>(a)));
    } else {
      PROX_DISPATCH_NB(batch, (proxy_mfma_kernel<NB, kMfmaRows, 0><<<gm, 512, 0, s>>>(a)));
    }
  } else if (p.bf16) {
    PROX_DISPATCH_NB(batch, (proxy_kernel<NB, true><<<g, 512, 0, s>>>(a)));
  } else {
    PROX_DISPATCH_NB(batch, (proxy_kernel<NB, false><<<g, 512, 0, s>>>(a)));
  }
  return hipGetLastError();
}

template <int PER>
static void topk_launch(const Plan &p, const Bufs &b, int batch, int k, bool lists,
                        bool union_list, hipStream_t s) {
  // one token: the list only (it drives Stage 2); several: the mask words,
  // their union list (built by the last work-group) only when asked for, and
  // the per-token lists only when asked for
  const bool several = batch > 1;
  topk_kernel<PER><<<batch, 1024, 0, s>>>(b.sabs, p.d_ff, k, lists ? b.sel : nullptr,
                                          several ? b.selw : nullptr,
                                          several && union_list ? b.ucnt : nullptr,
                                          b.uni, b.nuni, b.umask);
}

hipError_t launch_topk(const Plan &p, const Bufs &b, int batch, int k, bool lists,
                       bool union_list, hipStream_t s) {
  // Key slots per thread: instances sized for the 8B (14) and 70B (28)
  // widths, whose passes then walk no empty slot (70B 8-token top-k
  // 16.8 -> 15.8 us against the 32-slot instance).
  const int per = (p.d_ff + 1023) / 1024;
  if (per <= 1) topk_launch<1>(p, b, batch, k, lists, union_list, s);
  else if (per <= 4) topk_launch<4>(p, b, batch, k, lists, union_list, s);
  else if (per <= 8) topk_launch<8>(p, b, batch, k, lists, union_list, s);
  else if (per <= 14) topk_launch<14>(p, b, batch, k, lists, union_list, s);
  else if (per <= 16) topk_launch<16>(p, b, batch, k, lists, union_list, s);
  else if (per <= 28) topk_launch<28>(p, b, batch, k, lists, union_list, s);
  else if (per <= 32) topk_launch<32>(p, b, batch, k, lists, union_list, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}


// MFMA form of the batched up/gate step (bf16, 2 <= NB <= 8 tokens): one
// wave per tile of 16 list positions.  v_mfma_f32_16x16x32_bf16 computes
// D[m][n] = sum_k A[m][k] B[k][n] with A = 16 channel rows (lane l holds row
// l%16, k = 8 (l/16) .. +7: 16 contiguous bytes of that row) and B = x of the
// tokens (lane l holds token l%16, same k), so D holds u (or g) of channel
// 4 (l/16) + i for token l%16 in element i of lane l.  Column n of D depends
// on column n of B alone, so lanes of tokens >= NB load token NB-1 and their
// results are dropped.  UK = 8 steps of K = 32 keep 16 KB of weights per wave
// in flight; x comes from L2.  Each load instruction reads 64 bytes from each
// of 16 rows, against 1 KB of one row in the VALU form, and measured slower
// than the VALU form at 2, 4 and 8 tokens, so it runs only on request.

template <int NB, int MODE>
__global__ __launch_bounds__(256) void upgate_mfma_kernel(UpGateArgs a) {
  constexpr int UK = 8;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int n = a.n_ptr ? *a.n_ptr : a.n;
  const int ntiles = (n + 15) >> 4;
  const uint32_t rowb = (uint32_t)a.d_model * 2u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.wug, a.wug_bytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)NB * rowb);
  const uint32_t xbase = (uint32_t)min(m, NB - 1) * rowb;
  for (int tile = blockIdx.x * 4 + wv; tile < ntiles; tile += gridDim.x * 4) {
    const int pc = min(tile * 16 + m, n - 1);
    const int j = (MODE == 2) ? pc : a.list[pc];
    const uint32_t ubase = (uint32_t)j * 2u * rowb;
    const uint32_t gbase = ubase + rowb;
    f32x4_t au = {0.0f, 0.0f, 0.0f, 0.0f}, ag = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < a.d_model; k0 += 32 * UK) {
      u4 wu[UK], wg[UK], xv[UK];
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        const uint32_t off = (uint32_t)(k0 + 32 * u + 8 * g) * 2u;
        wu[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, ubase + off, 0, kNT);
        wg[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, gbase + off, 0, kNT);
        xv[u] = __builtin_amdgcn_raw_buffer_load_b128(xr, xbase + off, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UK; ++u) {
        bf16x8_t A, B, G;
        __builtin_memcpy(&A, &wu[u], 16);
        __builtin_memcpy(&G, &wg[u], 16);
        __builtin_memcpy(&B, &xv[u], 16);
        au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, au, 0, 0, 0);
        ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(G, B, ag, 0, 0, 0);
      }
    }
    if (m < NB) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tile * 16 + 4 * g + i;
        if (p < n) {
          const unsigned tok = (MODE == 1) ? a.umask[p] : 0xffu;
          a.ssp[(size_t)p * sstride(NB) + m] = ((tok >> m) & 1u) ? au[i] * gate_act(ag[i], a.act) : 0.0f;
        }
      }
    }
  }
}

template <int NB, int MODE>
static hipError_t upgate_mfma_go(const UpGateArgs &a, int maxn, int cap, hipStream_t s) {
  int grid = ((maxn + 15) / 16 + 3) / 4;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  upgate_mfma_kernel<NB, MODE><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// x of all tokens sits in LDS, so once it takes more than a quarter of a
// CU's LDS the kernel runs 16-wave work-groups to keep the CU's waves up.
template <int NWV, int NB, bool BF16, int MODE>
static hipError_t upgate_go_w(const UpGateArgs &a, int maxn, int cap, size_t lds, hipStream_t s) {
  auto fn = upgate_kernel<NB, BF16, MODE, NWV>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void *)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  int grid = (maxn + NWV - 1) / NWV;
  if (grid > cap * 4 / NWV) grid = cap * 4 / NWV;
  fn<<<grid, NWV * 64, lds, s>>>(a);
  return hipGetLastError();
}

template <int NB, bool BF16, int MODE>
static hipError_t upgate_go(const UpGateArgs &a, int maxn, int cap, size_t lds, hipStream_t s) {
  if (lds > kMaxLds / 4) return upgate_go_w<16, NB, BF16, MODE>(a, maxn, cap, lds, s);
  return upgate_go_w<4, NB, BF16, MODE>(a, maxn, cap, lds, s);
}

// Waves of a kernel that fit on the device at once (occupancy x CUs).
static int resident_waves(const void *fn, int block) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return per_cu * cus * (block / 64);
}

template <bool BF16, int MODE, int NSTEP>
static hipError_t upgate1_go(const UpGateArgs &a, hipStream_t s) {
  auto fn = upgate1_kernel<BF16, MODE, NSTEP>;
  static int cap = 0;
  if (!cap) cap = resident_waves((const void *)fn, 256);
  const int per = (a.n + cap - 1) / cap;    // equal share per wave
  const int waves = (a.n + per - 1) / per;
  fn<<<(waves + 3) / 4, 256, 0, s>>>(a, per);
  return hipGetLastError();
}

template <bool BF16, int MODE>
static bool upgate1_dispatch(const Plan &p, const UpGateArgs &a, hipStream_t s, hipError_t &e) {
  const int nstep = p.d_model / (64 * (BF16 ? 8 : 4));
  switch (nstep) {
    case 1: e = upgate1_go<BF16, MODE, 1>(a, s); return true;
    case 2: e = upgate1_go<BF16, MODE, 2>(a, s); return true;
    case 4: e = upgate1_go<BF16, MODE, 4>(a, s); return true;
    case 8: e = upgate1_go<BF16, MODE, 8>(a, s); return true;
    case 10: e = upgate1_go<BF16, MODE, 10>(a, s); return true;
    case 16: e = upgate1_go<BF16, MODE, 16>(a, s); return true;
    default: return false;
  }
}

hipError_t launch_upgate(const Plan &p, const Bufs &b, const void *x, int batch,
                         int mode, int n, hipStream_t s) {
  UpGateArgs a{b.wug, (uint32_t)((size_t)p.d_ff * 2 * p.d_model * p.esz), x,
               p.d_model, p.d_ff, n, nullptr,
               mode == 0 ? b.sel : b.uni, b.umask, b.ssp, p.act, b.selw};
  if (mode == 1) a.n_ptr = b.nuni;
  if (mode == 3) a.n = p.d_ff;
  // mode 3: one wave per block of channels (grid sized by the blocks)
  const int maxn = mode == 3 ? (p.d_ff + upgate_block(batch) - 1) / upgate_block(batch)
                             : (mode == 1 ? p.d_ff : a.n);
  if (mode == 3 && (batch < 2 || (p.bf16 && p.batch_mfma))) return hipErrorInvalidValue;
  if (maxn <= 0) return hipSuccess;
  if (batch == 1 && mode != 1) {
    hipError_t e1 = hipSuccess;
    bool done;
    if (p.bf16)
      done = mode == 0 ? upgate1_dispatch<true, 0>(p, a, s, e1) : upgate1_dispatch<true, 2>(p, a, s, e1);
    else
      done = mode == 0 ? upgate1_dispatch<false, 0>(p, a, s, e1) : upgate1_dispatch<false, 2>(p, a, s, e1);
    if (done) return e1;
  }
  hipError_t e = hipErrorInvalidValue;
  if (p.bf16 && batch >= 2 && mode != 0 && p.batch_mfma) {
#define PROX_MFMA_NB(MD)                                                     \
  switch (batch) {                                                           \
    case 2: return upgate_mfma_go<2, MD>(a, maxn, p.upgate_cap, s);          \
    case 3: return upgate_mfma_go<3, MD>(a, maxn, p.upgate_cap, s);          \
    case 4: return upgate_mfma_go<4, MD>(a, maxn, p.upgate_cap, s);          \
    case 5: return upgate_mfma_go<5, MD>(a, maxn, p.upgate_cap, s);          \
    case 6: return upgate_mfma_go<6, MD>(a, maxn, p.upgate_cap, s);          \
    case 7: return upgate_mfma_go<7, MD>(a, maxn, p.upgate_cap, s);          \
    case 8: return upgate_mfma_go<8, MD>(a, maxn, p.upgate_cap, s);          \
    default: return hipErrorInvalidValue;                                    \
  }
    if (mode == 1) { PROX_MFMA_NB(1) } else { PROX_MFMA_NB(2) }
#undef PROX_MFMA_NB
  }
  const int cap = p.upgate_cap;
  const size_t lds = (size_t)batch * p.d_model * p.esz;
  if (p.bf16) {
    if (mode == 0) { PROX_DISPATCH_NB(batch, (e = upgate_go<NB, true, 0>(a, maxn, cap, lds, s))); }
    else if (mode == 1) { PROX_DISPATCH_NB(batch, (e = upgate_go<NB, true, 1>(a, maxn, cap, lds, s))); }
    else if (mode == 3) { PROX_DISPATCH_NB(batch, (e = upgate_go<NB, true, 3>(a, maxn, cap, lds, s))); }
    else { PROX_DISPATCH_NB(batch, (e = upgate_go<NB, true, 2>(a, maxn, cap, lds, s))); }
  } else {
    if (mode == 0) { PROX_DISPATCH_NB(batch, (e = upgate_go<NB, false, 0>(a, maxn, cap, lds, s))); }
    else if (mode == 1) { PROX_DISPATCH_NB(batch, (e = upgate_go<NB, false, 1>(a, maxn, cap, lds, s))); }
    else if (mode == 3) { PROX_DISPATCH_NB(batch, (e = upgate_go<NB, false, 3>(a, maxn, cap, lds, s))); }
    else { PROX_DISPATCH_NB(batch, (e = upgate_go<NB, false, 2>(a, maxn, cap, lds, s))); }
  }
  return e;
}

template <int NB, bool BF, int MD>
static void down_go(const DownArgs &a, dim3 g, hipStream_t s) {
  if constexpr (NB == 1 || (NB == 2 && !BF)) down_kernel<NB, BF, MD, 16><<<g, 1024, 0, s>>>(a);
  else if constexpr (NB <= 4 || BF) down_kernel<NB, BF, MD, 8><<<g, 512, 0, s>>>(a);
  else down_kernel<NB, BF, MD, 4><<<g, 256, 0, s>>>(a);
}

hipError_t launch_down(const Plan &p, const Bufs &b, int batch, int mode, int n,
                       void *y, float *resid, hipStream_t s) {
  // Row chunks: the dense batch-1 pass streams every row, so half as many
  // chunks (one 16-wave work-group per CU at the 8B shape) keep it streaming
  // with half the partial sums to add (measured at 8B: 21.6 us against 23.0
  // with 32 chunks); the sparse and batch passes keep p.nrc.
  const int nrc = (mode == 2 && batch == 1) ? std::max(1, std::min(p.nrc, 256 / p.ncol)) : p.nrc;
  DownArgs a{b.wd, (uint32_t)((size_t)p.d_ff * p.d_model * p.esz), p.d_model,
             p.d_ff, n, nrc, nullptr, mode == 0 ? b.sel : b.uni, b.ssp,
             b.ypart, b.col_cnt, y, resid, b.selw};
  if (mode == 1) a.n_ptr = b.nuni;
  if (mode == 3 && (batch < 2 || (((p.d_ff + nrc - 1) / nrc + 31) & ~31) > kDownLocal))
    return hipErrorInvalidValue;
  dim3 g(p.ncol, nrc);
  // Waves per work-group: 16 for one token (two for float32), else 8, so
  // that two work-groups fit a CU; float32 layers of 5..8 tokens take 4
  // waves to bound the LDS reduction buffer (32 KiB).
#define PROX_DOWN(BF, MD)                                                       \
  PROX_DISPATCH_NB(batch, (down_go<NB, BF, MD>(a, g, s)))
  if (p.bf16) {
    if (mode == 0) { PROX_DOWN(true, 0); }
    else if (mode == 1) { PROX_DOWN(true, 1); }
    else if (mode == 3) { PROX_DOWN(true, 3); }
    else { PROX_DOWN(true, 2); }
  } else {
    if (mode == 0) { PROX_DOWN(false, 0); }
    else if (mode == 1) { PROX_DOWN(false, 1); }
    else if (mode == 3) { PROX_DOWN(false, 3); }
    else { PROX_DOWN(false, 2); }
  }
#undef PROX_DOWN
  return hipGetLastError();
}

// Debug: s of the union list by position, token-major (out[t][p] = s of
// token t at union entry p), from s kept by channel (mode 3) or by position.
__global__ __launch_bounds__(256) void union_s_kernel(const float *ssp, int nbp, const int *uni,
                                                      const int *nuni, int d_ff, int batch,
                                                      int by_channel, float *out) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  const int t = blockIdx.y;
  if (p >= d_ff || t >= batch) return;
  const int nu = *nuni;
  const int row = p < nu ? (by_channel ? uni[p] : p) : 0;
  out[(size_t)t * d_ff + p] = p < nu ? ssp[(size_t)row * nbp + t] : 0.0f;
}

hipError_t launch_union_s(const Plan &p, const Bufs &b, int batch, bool by_channel, float *out,
                          hipStream_t s) {
  const dim3 g((p.d_ff + 255) / 256, batch);
  union_s_kernel<<<g, 256, 0, s>>>(b.ssp, (batch + 3) & ~3, b.uni, b.nuni, p.d_ff, batch,
                                   by_channel ? 1 : 0, out);
  return hipGetLastError();
}

hipError_t launch_survivors(const Plan &p, const Bufs &b, int batch, int *n1, int *idx,
                            hipStream_t s) {
  survivors_kernel<<<batch, 256, 0, s>>>(b.drows, b.dcnt, p.d_model, n1, idx);
  return hipGetLastError();
}

hipError_t launch_read_status(const Plan &p, const Bufs &b, int *out, hipStream_t s) {
  (void)p;
  read_status_kernel<<<1, 1024, 0, s>>>(b.sync, sync_block_bytes() / sizeof(unsigned),
                                        kFusedErrWord, b.pred, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const Plan &p, const float *resid, int batch,
                          float eps, void *x, hipStream_t s) {
  if (p.bf16)
    rmsnorm_kernel<true><<<batch, kRmsThreads, 0, s>>>(resid, p.d_model, eps, x);
  else
    rmsnorm_kernel<false><<<batch, kRmsThreads, 0, s>>>(resid, p.d_model, eps, x);
  return hipGetLastError();
}

__global__ void zero_words_kernel(unsigned *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero_bytes(void *p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
  zero_words_kernel<<<blocks, 256, 0, s>>>((unsigned *)p, n);
  return hipGetLastError();
}

hipError_t launch_zero_y(const Plan &p, void *y, int batch, hipStream_t s) {
  const size_t n = (size_t)batch * p.d_model;
  const int blocks = (int)((n + 255) / 256);
  if (p.bf16)
    zero_kernel<true><<<blocks, 256, 0, s>>>(y, n);
  else
    zero_kernel<false><<<blocks, 256, 0, s>>>(y, n);
  return hipGetLastError();
}

}  // namespace prox
