// Device helpers shared by the kernels of libprox (prox_kernels.hip and
// prox_fused.hip).  Internal; not part of the public interface.
#pragma once

#include "prox_internal.h"

#include <math.h>

namespace prox {

typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// float32 -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float ld_elem(const void *p, size_t i) {
  if constexpr (BF16)
    return bf16_to_f32(((const uint16_t *)p)[i]);
  else
    return ((const float *)p)[i];
}

template <bool BF16>
__device__ __forceinline__ void st_elem(void *p, size_t i, float v) {
  if constexpr (BF16)
    ((uint16_t *)p)[i] = f32_to_bf16(v);
  else
    ((float *)p)[i] = v;
}

// Value as stored in the layer dtype (what a caller reads back).
template <bool BF16>
__device__ __forceinline__ float round_elem(float v) {
  if constexpr (BF16)
    return bf16_to_f32(f32_to_bf16(v));
  else
    return v;
}

// Cache policy of weight-stream loads: non-temporal (each weight byte is read
// once per call; keeping it out of the caches lifts streaming bandwidth).
constexpr int kNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base,
                                                            uint32_t bytes) {
  // raw buffer: stride 0, num_records = bytes; out-of-range reads return 0.
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes,
                                           0x00020000);
}

// Cross-work-group exchange of partial sums.  Partials are written and read
// with agent-scope atomic accesses, which are coherent across the XCDs' L2
// caches on their own (write-through / read-through), so no L2-wide
// writeback or invalidate is needed.  A work-group publishes its partials,
// waits until its own stores have completed, and only then counts its
// arrival; the last arrival reads every partial.
__device__ __forceinline__ void xstore(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float xload(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// sum_{c < n} p[c * stride], loads issued 16 at a time before any is used,
// added in index order (deterministic).
__device__ __forceinline__ float xsum_strided(const float *p, int n, size_t stride) {
  float acc = 0.0f;
  for (int c0 = 0; c0 < n; c0 += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = xload(p + (size_t)min(c0 + u, n - 1) * stride);
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += (c0 + u < n) ? v[u] : 0.0f;
  }
  return acc;
}

// Wait until this wave's vector memory operations are complete (loads
// returned, stores acknowledged, direct-to-LDS loads landed).  It is the
// compiler's own instruction, so the compiler's wait bookkeeping learns that
// the direct-to-LDS loads have landed; after an opaque asm wait it would
// still count them as pending and make later barriers wait for every
// outstanding store again.  The empty asm statements keep memory accesses
// from moving across it.
__device__ __forceinline__ void wait_vmem() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt not waited for
  asm volatile("" ::: "memory");
}

// Counts this work-group's arrival at *cnt (after its own stores have
// completed) and returns true in every thread of the last of `total` to
// arrive.  The counter is left at `total` (for waiters that poll it); the
// caller resets it later.
__device__ __forceinline__ bool arrive_count(unsigned *cnt, unsigned total, int *s_flag) {
  wait_vmem();      // own partial stores done
  __syncthreads();  // ... in every wave
  if (threadIdx.x == 0)
    *s_flag = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              total - 1u;
  __syncthreads();
  return *s_flag != 0;
}

// Returns true in every thread of the last work-group to arrive at *cnt
// (of `total`), which also resets the counter for the next launch.
__device__ __forceinline__ bool arrive_last(unsigned *cnt, unsigned total, int *s_flag) {
  wait_vmem();  // own partial stores done
  __syncthreads();                                   // ... in every wave
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == total - 1u;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Sum over the 64 lanes of a wave, returned uniform: DPP within each row of
// 16 lanes (quad swaps, then row rotations by 4 and 8), then the four row
// sums in a fixed order.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int r;
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, true); break;
    case 1: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, true); break;
    case 2: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xf, 0xf, true); break;
    default: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, true); break;
  }
  return v + __int_as_float(r);
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add(v, 0);  // quad_perm [1,0,3,2]
  v = dpp_add(v, 1);  // quad_perm [2,3,0,1]
  v = dpp_add(v, 2);  // row_ror:4
  v = dpp_add(v, 3);  // row_ror:8
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// 1 / sqrt(mean(r^2) + eps) over d_model elements, computed by all NT threads
// of a work-group in one fixed order (thread t adds r[t]^2, r[t + NT]^2, ...
// with fmaf, a fixed wave reduction, then the NT / 64 wave sums in order), so
// every kernel that normalizes the same r with the same NT gets the same bits.
// part: NT / 64 floats of LDS.
template <int NT>
__device__ __forceinline__ float block_inv_rms(const float *r, int d_model, float eps,
                                               float *part) {
  float ss = 0.0f;
  for (int i = threadIdx.x; i < d_model; i += NT) ss = fmaf(r[i], r[i], ss);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int q = 0; q < NT / 64; ++q) tot += part[q];
  __syncthreads();  // part is free again
  return 1.0f / sqrtf(tot / (float)d_model + eps);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Gate activation: SiLU (act 0, SwiGLU) or the tanh form of GELU (act 1,
// GeGLU), 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float u = 0.7978845608028654f * (z + 0.044715f * z * z * z);
  return 0.5f * z * (1.0f + tanhf(u));
}
__device__ __forceinline__ float gate_act(float z, int act) { return act ? gelu_tanh(z) : silu(z); }

// Reinterpret 32 bits as two bf16 lanes.  (Written with memcpy: a
// __builtin_bit_cast of a single element of a 4 x u32 vector was folded back
// to element 0 by the optimizer in this toolchain.)
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned v) {
  bf16x2 r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}

// Dot product of 16 bytes of weights with 16 bytes of activations.
template <bool BF16>
__device__ __forceinline__ float dot16(u4 w, u4 x, float acc) {
  if constexpr (BF16) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.w), acc, false);
    return acc;
  } else {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
    return acc;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    unsigned t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over a work-group of NWAVES waves; also returns the
// total.  wsum: NWAVES words of LDS.  Contains two barriers.
template <int NWAVES>
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned *wsum,
                                                    unsigned &total) {
  const unsigned inc = wave_incl_scan(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) wsum[w] = inc;
  __syncthreads();
  unsigned off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    const unsigned s = wsum[i];
    off += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + inc - v;
}

// Debug export of the survivors a Stage 1 kernel found in one 64-row slice
// (its m_x decision, Sec. 4.1): rows[sl * 64 + i] = the i-th surviving row,
// cnt[sl] = their number.  Called by every lane of the wave with the slice's
// ballot m.
__device__ __forceinline__ void export_slice(int *rows, int *cnt, int sl, uint64_t m) {
  const int lane = threadIdx.x & 63;
  if ((m >> lane) & 1ull)
    rows[sl * 64 + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u))] =
        sl * 64 + lane;
  if (lane == 0) cnt[sl] = (int)__popcll(m);
}

// Stage 1 input mask for one 64-row slice (Sec. 4.1, m_x equation): each lane
// tests its own row, |x_i| >= tau keeps it; the wave gets the 64-bit mask.
// Shared by the proxy kernel and the compaction debug kernel, so the
// survivors checked by the tests are the ones the proxy uses.
template <bool BF16>
__device__ __forceinline__ uint64_t slice_mask(const void *x, size_t row0,
                                               float tau, float &xl) {
  xl = ld_elem<BF16>(x, row0 + (threadIdx.x & 63));
  return __ballot(fabsf(xl) >= tau);
}

// Inclusive prefix sum over a wave with DPP: row_shr 1, 2, 4, 8 inside each
// row of 16 lanes, then row_bcast:15 and row_bcast:31 across rows.
__device__ __forceinline__ unsigned wave_incl_scan_dpp(unsigned v) {
  const int lane = threadIdx.x & 63, rl = lane & 15;
  unsigned t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);
  if (rl >= 1) v += t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);
  if (rl >= 2) v += t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);
  if (rl >= 4) v += t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);
  if (rl >= 8) v += t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);
  if ((lane & 31) >= 16) v += t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);
  if (lane >= 32) v += t;
  return v;
}

// Agent-coherent integer accesses (see xstore / xload).
__device__ __forceinline__ void xstore_u(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned xload_u(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *p >= target, polling with short sleeps.  Bounded: after
// `limit` polls (the default, 2^22, is seconds) it sets bit 0 of *err and
// returns, so a kernel always terminates even if a producer never signals.
__device__ __forceinline__ void wait_geq(const unsigned *p, unsigned target, unsigned *err,
                                         unsigned limit) {
  unsigned n = 0;
  while (xload_u(p) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (++n > limit) {
      atomicOr(err, 1u);
      return;
    }
  }
}

}  // namespace prox
