// Input-sparse bf16 GEMV of the up and gate projections: the full-precision
// counterpart of the Stage 1 INT4 proxy, used to measure the cost ratio alpha
// of the pages' allocation model.
//
// Method: "Prox: Training-Free FFN Activation Sparsity via Approximate
// Intermediate-Channel Salience in LLMs" (arXiv 2607.27591), Sec. 4.2 (alpha:
// the cost of one INT4 proxy GEMV relative to an FP16 GEMV at the same input
// sparsity) and App. A.3 (its measurement).  Here the reference GEMV is
// bf16: u_j = sum_{i : |x_i| >= tau} x_i W_up[i][j] and likewise g_j, with
// float32 accumulation.
//
// Weights are the caller's row-major [d_model][d_ff] tensors (x.W layout): a
// surviving input row i is read as contiguous 512-byte runs, one per
// 256-column tile, and a pruned row is skipped whole.  Work-group = (tile,
// 512-row chunk), one wave per 64-row slice: lanes 0..31 read the up run,
// lanes 32..63 the gate run, 16 bytes (8 columns) each.  Chunk partials go
// through agent-coherent stores; the last chunk of a tile adds them in chunk
// order.
#include "prox_device.h"

namespace prox {

struct SgemvArgs {
  const uint16_t *w_up, *w_gate;
  const void *x;
  float tau;
  int d_model, d_ff, nchunk;
  float *part;
  unsigned *tile_cnt;
  float *u, *g;
};

__global__ __launch_bounds__(512) void sgemv_kernel(SgemvArgs a) {
  constexpr int NW = 8, U = 8;
  __shared__ float red[NW][512];
  __shared__ int rl[NW][64 + U];
  __shared__ float xc[NW][64 + U];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunk = blockIdx.x, t = blockIdx.y;
  const int sl = chunk * NW + wv;
  const int half = lane >> 5;                   // 0: up, 1: gate
  const int col = t * 256 + (lane & 31) * 8;    // first of this lane's 8 columns
  const bool colok = col < a.d_ff;              // d_ff is a multiple of 8
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  if (sl * 64 < a.d_model) {
    float xl;
    const uint64_t un = slice_mask<true>(a.x, (size_t)sl * 64, a.tau, xl);
    const int cnt = (int)__popcll(un);
    if ((un >> lane) & 1ull) {
      const int pos = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(un >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((unsigned)un, 0u));
      rl[wv][pos] = sl * 64 + lane;
      xc[wv][pos] = xl;
    }
    if (lane < U) {
      rl[wv][cnt + lane] = sl * 64;
      xc[wv][cnt + lane] = 0.0f;
    }
    __builtin_amdgcn_wave_barrier();
    const uint16_t *base = half ? a.w_gate : a.w_up;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base, (uint32_t)((size_t)a.d_model * a.d_ff * 2));
    const uint32_t voff = (uint32_t)col * 2u;
    for (int r0 = 0; r0 < cnt; r0 += U) {
      u4 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t row = (uint32_t)__builtin_amdgcn_readfirstlane(rl[wv][r0 + u]);
        // past the survivors (uniform) or past d_ff (this lane): no load
        w[u] = (colok && r0 + u < cnt)
                   ? __builtin_amdgcn_raw_buffer_load_b128(rs, voff, row * (uint32_t)a.d_ff * 2u, kNT)
                   : u4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float xv = xc[wv][r0 + u];
        const unsigned ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(xv, bf16_to_f32(ww[q] & 0xffffu), acc[2 * q]);
          acc[2 * q + 1] = fmaf(xv, bf16_to_f32(ww[q] >> 16), acc[2 * q + 1]);
        }
      }
    }
  }
  // red[w][e]: e < 256 up columns, e >= 256 gate columns of the tile
  float4 *rp = (float4 *)&red[wv][half * 256 + (lane & 31) * 8];
  rp[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  rp[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  float *part = a.part + ((size_t)t * a.nchunk + chunk) * 512;
  {
    const int e = threadIdx.x;
    float v = red[0][e];
#pragma unroll
    for (int q = 1; q < NW; ++q) v += red[q][e];
    xstore(&part[e], v);
  }
  if (!arrive_last(&a.tile_cnt[t], (unsigned)a.nchunk, &s_last)) return;
  const float *tp = a.part + (size_t)t * a.nchunk * 512;
  const int e = threadIdx.x;
  const float v = xsum_strided(&tp[e], a.nchunk, 512);
  const int j = t * 256 + (e & 255);
  if (j < a.d_ff) (e < 256 ? a.u : a.g)[j] = v;
}

size_t sgemv_workspace_bytes(int d_model, int d_ff) {
  const int ntile = (d_ff + 255) / 256, nchunk = (d_model / 64 + 7) / 8;
  return (size_t)ntile * nchunk * 512 * 4 + (size_t)ntile * 4 + 256;
}

hipError_t launch_sgemv(const void *w_up, const void *w_gate, int d_model, int d_ff, const void *x,
                        float tau, float *u, float *g, void *workspace, hipStream_t s) {
  const int ntile = (d_ff + 255) / 256, nchunk = (d_model / 64 + 7) / 8;
  SgemvArgs a{};
  a.w_up = (const uint16_t *)w_up;
  a.w_gate = (const uint16_t *)w_gate;
  a.x = x;
  a.tau = tau;
  a.d_model = d_model;
  a.d_ff = d_ff;
  a.nchunk = nchunk;
  a.part = (float *)workspace;
  a.tile_cnt = (unsigned *)((char *)workspace + (size_t)ntile * nchunk * 512 * 4);
  a.u = u;
  a.g = g;
  sgemv_kernel<<<dim3(nchunk, ntile), 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace prox
