// Device helpers shared by the HIP kernel sources of this library (gfx950):
// element loads, order keys of fp32 values, DPP wave scans and block scans,
// and the event-stamped launch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pariskv_internal.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Element loads: 8 consecutive elements of a bf16 or fp32 row as fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Streaming loads (the `nt` bit: no retention in L2 or the Infinity Cache),
// for data a decode step reads once: the id plane in the scans, the score
// bytes in the compaction and the gathered K/V rows in the attention.  On the million-token layer (its ids
// do not fit the Infinity Cache) they keep the scores, records and partials
// that the next kernels read in the caches.
typedef uint32_t stream_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const stream_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const stream_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
typedef uint32_t stream_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const stream_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const stream_u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void load8_stream(const uint16_t* p, float (&x)[8]) {
  const uint4 v = load_stream(reinterpret_cast<const uint4*>(p));
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void load8_stream(const float* p, float (&x)[8]) {
  const uint4 a = load_stream(reinterpret_cast<const uint4*>(p));
  const uint4 b = load_stream(reinterpret_cast<const uint4*>(p) + 1);
  x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
  x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
  x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
  x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
}

// Order key of an estimate: unsigned order == (est desc) order, -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Inverse of order_key (a -0 input comes back as +0).
__device__ __forceinline__ float key_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4 and 8 within each row of 16 lanes, then the last lane of row 0 (2) added
// to row 1 (3) and the last lane of row 1 added to rows 2 and 3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of a pair of uint32 values (NT threads): DPP
// scans within each wave, wave totals through LDS.  SYNC_AFTER: a closing
// barrier, so the caller may write s_warp again at once; callers that do not
// touch s_warp before another barrier leave it out.
// ---------------------------------------------------------------------------
template <int NT, bool SYNC_AFTER = true>
__device__ __forceinline__ uint2 block_exscan2(uint2 v, uint2* s_warp, uint2& total) {
  constexpr int NW = NT / 64;
  // the wave index as a scalar, so the per-wave tests below are scalar
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ix = wave_incl_scan(v.x), iy = wave_incl_scan(v.y);
  if (lane == 63) s_warp[wv] = make_uint2(ix, iy);
  __syncthreads();
  uint2 base = make_uint2(0, 0), tot = make_uint2(0, 0);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint2 t = s_warp[w];
    if (w < wv) { base.x += t.x; base.y += t.y; }
    tot.x += t.x; tot.y += t.y;
  }
  if constexpr (SYNC_AFTER) __syncthreads();  // s_warp may be reused by the caller
  total = tot;
  return make_uint2(base.x + ix - v.x, base.y + iy - v.y);
}

// Block-wide exclusive scan of two uint32 values per thread (NT threads),
// each the packed pair (lo 16 bits, hi 16 bits) of counts whose block total
// stays below 65536.
template <int NT>
__device__ __forceinline__ uint2 block_exscan_packed(uint2 v, uint2* s_warp, uint2& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ix = wave_incl_scan(v.x), iy = wave_incl_scan(v.y);
  if (lane == 63) s_warp[wv] = make_uint2(ix, iy);
  __syncthreads();
  uint2 base = make_uint2(0, 0), tot = make_uint2(0, 0);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint2 t = s_warp[w];
    if (w < wv) { base.x += t.x; base.y += t.y; }
    tot.x += t.x; tot.y += t.y;
  }
  total = tot;
  return make_uint2(base.x + ix - v.x, base.y + iy - v.y);
}

// the lowest r set bits of m
__device__ __forceinline__ uint32_t lowest_bits(uint32_t m, uint32_t r) {
  uint32_t out = 0;
  for (uint32_t i = 0; i < r && m; ++i) {
    const uint32_t low = m & (0u - m);
    out |= low;
    m ^= low;
  }
  return out;
}

// KPT consecutive score bytes (16, 8 and 4 in one load)
template <int KPT>
__device__ __forceinline__ void load_scores(const uint8_t* sp, uint8_t (&sc)[KPT]) {
  if constexpr (KPT == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(sp);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 16; ++t) sc[t] = (uint8_t)(w4[t >> 2] >> ((t & 3) * 8));
  } else if constexpr (KPT == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(sp);
#pragma unroll
    for (int t = 0; t < 8; ++t) sc[t] = (uint8_t)(((t < 4) ? v.x : v.y) >> ((t & 3) * 8));
  } else if constexpr (KPT == 4) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(sp);
#pragma unroll
    for (int t = 0; t < 4; ++t) sc[t] = (uint8_t)(v >> (t * 8));
  } else {
#pragma unroll
    for (int t = 0; t < KPT; ++t) sc[t] = sp[t];
  }
}

// one element of a bf16 (raw bits) or fp32 row as fp32
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// launch with start/stop events stamped by the dispatch itself (null: none)
template <typename F, typename... Args>
static hipError_t launch(F kernel, dim3 grid, dim3 block, hipStream_t st, const EvPair& ev,
                         Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  return hipGetLastError();
}

}  // namespace pkv
