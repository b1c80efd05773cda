// HIP kernels (gfx950 / CDNA4) for the ParisKV decode-step retrieval path.
//
// Method: "Technical Summary: ParisKV" (gist.science/paper/2602.07721),
// cited as [TS] with section names.  Data-parallel structure: every
// (batch, KV head) pair owns its own index, scan, selection and attention,
// so grids are (work tile, b*H_kv + h).
//
// Bit-exactness: bucket ids, RSQ-IP codes, fp16 calibration factors, vote
// scores, candidate lists, estimates and top-k lists are produced with the
// exact fp32 operation sequence stated at each kernel (no contraction: this
// file is built with -ffp-contract=off; division and square root are the
// correctly rounded HIP defaults).  Attention is tolerance-checked and uses
// explicit fused multiply-adds.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codebook_tables.h"
#include "pariskv_internal.h"

#pragma clang fp contract(off)

namespace pkv {

__constant__ float c_levels[8] = {
    kLevels_m8[0], kLevels_m8[1], kLevels_m8[2], kLevels_m8[3],
    kLevels_m8[4], kLevels_m8[5], kLevels_m8[6], kLevels_m8[7]};
__constant__ float c_thresh[7] = {
    kThresh_m8[0], kThresh_m8[1], kThresh_m8[2], kThresh_m8[3],
    kThresh_m8[4], kThresh_m8[5], kThresh_m8[6]};

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

// ---------------------------------------------------------------------------
// Shared SRHT rotation, [TS] Core Algorithmic Innovations 1 ("Normalization
// and Rotation"): y = c * H * (D .* x), H Sylvester-ordered, d = 128.
// A 16-lane group holds one vector, lane `sub` owning coordinates
// [8 sub, 8 sub + 8) -- exactly subspace `sub` (m = 8).  Butterfly stages
// h = 1, 2, 4 are lane-local; h = 8, 16, 32, 64 pair lane `sub` with lane
// sub ^ (h / 8).  For the pair (j, j + h) the lower element becomes a + b and
// the upper a - b, stage by stage in ascending h, then every element is
// multiplied by c -- the same fp32 operations in the same order as the
// definition, so the result is bit-identical to a sequential evaluation.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void srht16(float (&x)[8], uint32_t sign_byte, int sub, float c) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if ((sign_byte >> j) & 1u) x[j] = -x[j];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int blk = 0; blk < 8; blk += 2 * h)
#pragma unroll
      for (int j = blk; j < blk + h; ++j) {
        float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) {
    const bool upper = (sub & s) != 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float o = __shfl_xor(x[j], s, 16);
      x[j] = upper ? (o - x[j]) : (x[j] + o);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = x[j] * c;
}

__device__ __forceinline__ uint32_t sign_byte_of(const SignMask& sg, int sub) {
  return (sg.w[sub >> 2] >> ((sub & 3) * 8)) & 0xFFu;
}

// ---------------------------------------------------------------------------
// K1 encode: [TS] Coarse Candidate Generation (bucket = nearest analytic
// sign centroid of each subspace direction) and Candidate Reranking (RSQ-IP)
// Quantization + Calibration.  One key per 16-lane group; lane `sub` encodes
// subspace `sub` of its key:
//   id   = sum_j [z_j < 0] 2^j
//   n    = sqrt(((z_0 z_0 + z_1 z_1) + ...) + z_7 z_7)
//   u_j  = z_j / n; mag_j = #{l : |u_j| >= tau_l}; code_j = sign_j << 3 | mag_j
//   a    = ((v_0 u_0 + v_1 u_1) + ...), v_j = +-L[mag_j]
//   w    = fp16_rne(n / a)           (n == 0: magnitudes 0, w = 0)
// Index layout per (b,h): ids [cap][16] bytes, codes [cap][16] dwords
// (nibble j of dword s = coordinate 8 s + j), w [cap][16] fp16.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_encode(const T* __restrict__ K, int64_t rows_per_head,
                                                int64_t lo, int64_t n, int64_t total, int64_t cap,
                                                uint8_t* __restrict__ ids, uint32_t* __restrict__ nib,
                                                uint16_t* __restrict__ wq, SignMask sg, float c) {
  const int sub = threadIdx.x & 15;
  const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (g >= total) return;  // whole 16-lane groups leave together
  const int64_t bh = g / n;
  const int64_t r = g - bh * n;
  float x[8];
  load8(K + ((bh * rows_per_head + r) << 7) + sub * 8, x);
  srht16(x, sign_byte_of(sg, sub), sub, c);

  uint32_t id = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) id |= (x[j] < 0.0f ? 1u : 0u) << j;
  float n2 = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) n2 = n2 + x[j] * x[j];
  const float nrm = sqrtf(n2);
  uint32_t code = 0;
  uint16_t wbits = 0;
  if (nrm != 0.0f) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = x[j] / nrm;
      const float au = fabsf(u);
      uint32_t mag = 0;
      float lv = c_levels[0];
#pragma unroll
      for (int l = 0; l < 7; ++l)
        if (au >= c_thresh[l]) { mag = l + 1; lv = c_levels[l + 1]; }
      const uint32_t sgn = (id >> j) & 1u;
      const float v = sgn ? -lv : lv;
      a = a + v * u;
      code |= ((sgn << 3) | mag) << (4 * j);
    }
    const _Float16 hw = (_Float16)(nrm / a);
    wbits = __builtin_bit_cast(uint16_t, hw);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) code |= ((id >> j) & 1u) << (4 * j + 3);
  }
  const int64_t key = bh * cap + lo + r;
  ids[key * 16 + sub] = (uint8_t)id;
  nib[key * 16 + sub] = code;
  wq[key * 16 + sub] = wbits;
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of a pair of uint32 values (NT threads).
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ uint2 block_exscan2(uint2 v, uint2* s_warp, uint2& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint2 inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t a = __shfl_up(inc.x, off), b = __shfl_up(inc.y, off);
    if (lane >= off) { inc.x += a; inc.y += b; }
  }
  if (lane == 63) s_warp[wv] = inc;
  __syncthreads();
  uint2 base = make_uint2(0, 0), tot = make_uint2(0, 0);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint2 t = s_warp[w];
    if (w < wv) { base.x += t.x; base.y += t.y; }
    tot.x += t.x; tot.y += t.y;
  }
  __syncthreads();  // s_warp may be reused by the caller
  total = tot;
  return make_uint2(base.x + inc.x - v.x, base.y + inc.y - v.y);
}

// ---------------------------------------------------------------------------
// K2 query prep: [TS] Coarse Candidate Generation, query side.  Group query
// q = (q_0 + q_1 + ... + q_{G-1}) * fp32(1/G) in head order, yq = SRHT(q).
// Per subspace s, the 256 centroid scores sc_p = sum_j (bit j of p ? -yq : +yq)
// (sequential in j from the j = 0 term); the rho best by (sc desc, p asc)
// get tier weights in the vote LUT, all other centroids 0.
// One block (256 threads) per (b, h).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_qprep(const T* __restrict__ Q, int n_kv_heads, int G,
                                               float invG, SignMask sg, float c, int rho, Tiers tw,
                                               uint8_t* __restrict__ lut_out, float* __restrict__ yq_out) {
  const int bh = blockIdx.x;
  const int b = bh / n_kv_heads, h = bh - b * n_kv_heads;
  const int Hq = n_kv_heads * G;
  const int tid = threadIdx.x;
  __shared__ float s_yq[128];
  __shared__ float s_sc[16][256];
  if (tid < 16) {
    const int sub = tid;
    float x[8];
    const T* q0 = Q + ((int64_t)(b * Hq + h * G) << 7) + sub * 8;
    load8(q0, x);
    for (int g = 1; g < G; ++g) {
      float t[8];
      load8(q0 + ((int64_t)g << 7), t);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = x[j] + t[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = x[j] * invG;
    srht16(x, sign_byte_of(sg, sub), sub, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s_yq[sub * 8 + j] = x[j];
      yq_out[(int64_t)bh * 128 + sub * 8 + j] = x[j];
    }
  }
  __syncthreads();
  {
    const int p = tid;
#pragma unroll 4
    for (int s = 0; s < 16; ++s) {
      const float* z = s_yq + s * 8;
      float acc = (p & 1) ? -z[0] : z[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) acc = acc + (((p >> j) & 1) ? -z[j] : z[j]);
      s_sc[s][p] = acc;
    }
  }
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6;
  for (int s = wv; s < 16; s += 4) {
    float v[4];
    int pi[4];
    bool taken[4] = {false, false, false, false};
    uint32_t lv[4] = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) { pi[t] = lane + 64 * t; v[t] = s_sc[s][pi[t]]; }
    for (int r = 0; r < rho; ++r) {
      float bv = -INFINITY;
      int bp = 0x7FFFFFFF;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (!taken[t] && (v[t] > bv || (v[t] == bv && pi[t] < bp))) { bv = v[t]; bp = pi[t]; }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int op = __shfl_xor(bp, off);
        if (ov > bv || (ov == bv && op < bp)) { bv = ov; bp = op; }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (pi[t] == bp) { taken[t] = true; lv[t] = (uint32_t)tw.w[r]; }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) lut_out[((int64_t)bh * 16 + s) * 256 + pi[t]] = (uint8_t)lv[t];
  }
}

// ---------------------------------------------------------------------------
// K3 vote scan: [TS] Coarse Candidate Generation: score_i = sum_b lut_b[id_{i,b}]
// for i in [S, N).  The dominant HBM stream: 16 bytes of bucket ids per key,
// read once, coalesced (256 threads x 16 B per step).  The 4 KB vote LUT
// sits in LDS; one ds_read_u8 per subspace (each subspace's 256-byte row
// spans 64 dwords, so a wave's lookups for one subspace conflict at most
// 2-way).  Writes one score byte per key and a per-chunk histogram of the
// scores (zeros counted by wave ballot, the rest by LDS atomics).
// Grid: (chunks, b*H_kv); chunk = KPT * 256 keys.
// ---------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(256) void k_scan(const uint4* __restrict__ ids, int64_t cap, int64_t S,
                                              int64_t E, const uint8_t* __restrict__ lut,
                                              uint8_t* __restrict__ scores, int64_t Epad,
                                              uint32_t* __restrict__ chist, int chunk_stride, int nbins) {
  const int bh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  __shared__ uint8_t s_lut[16 * 256];
  __shared__ uint32_t s_hist[4][256];
  reinterpret_cast<uint4*>(s_lut)[tid] = reinterpret_cast<const uint4*>(lut + (int64_t)bh * 4096)[tid];
  for (int i = tid; i < 4 * 256; i += 256) (&s_hist[0][0])[i] = 0;
  __syncthreads();

  const int64_t p0 = (int64_t)chunk * (KPT * 256) + tid;
  const uint4* src = ids + bh * cap + S;
  uint8_t* dst = scores + bh * Epad;
  uint4 x[KPT];
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int64_t p = p0 + t * 256;
    x[t] = (p < E) ? src[p] : make_uint4(0, 0, 0, 0);
  }
  uint32_t zeros = 0;
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int64_t p = p0 + t * 256;
    const bool valid = p < E;
    const uint32_t w4[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
    uint32_t s = 0;
#pragma unroll
    for (int b = 0; b < 16; ++b) s += s_lut[b * 256 + ((w4[b >> 2] >> ((b & 3) * 8)) & 0xFFu)];
    const uint64_t zm = __ballot(valid && s == 0);
    zeros += (uint32_t)__popcll(zm);
    if (valid) {
      dst[p] = (uint8_t)s;
      if (s != 0) atomicAdd(&s_hist[wv][s], 1u);
    }
  }
  if (lane == 0) s_hist[wv][0] = zeros;
  __syncthreads();
  for (int v = tid; v < nbins; v += 256)
    chist[((int64_t)bh * chunk_stride + chunk) * nbins + v] =
        s_hist[0][v] + s_hist[1][v] + s_hist[2][v] + s_hist[3][v];
}

// ---------------------------------------------------------------------------
// K4a threshold: [TS] Coarse Candidate Generation keeps the top fraction.
// Candidates = the first C eligible keys in (score desc, index asc) order:
// T = largest v with #(score >= v) >= C; every key with score > T, plus the
// first Q = C - #(score > T) keys with score == T in index order.  From the
// per-chunk histograms: per chunk, the ties before it and the output offset
// of its first candidate (exclusive scans over chunks).
// One block per (b, h).  meta[bh] = (T, #gt, Q, C).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_thresh(const uint32_t* __restrict__ chist, int chunk_stride,
                                                int nchunks, int nbins, int64_t C,
                                                int32_t* __restrict__ meta, uint32_t* __restrict__ coff) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  __shared__ uint32_t s_tot[256];
  __shared__ int s_T;
  __shared__ uint32_t s_gt;
  __shared__ uint2 s_w[4];
  const uint32_t* hb = chist + (int64_t)bh * chunk_stride * nbins;
  for (int v = tid; v < nbins; v += 256) {
    uint32_t acc = 0;
    for (int c = 0; c < nchunks; ++c) acc += hb[(int64_t)c * nbins + v];
    s_tot[v] = acc;
  }
  __syncthreads();
  if (tid == 0) {
    uint64_t cum = 0;
    int T = 0;
    for (int v = nbins - 1; v >= 0; --v) {
      if (cum + s_tot[v] >= (uint64_t)C) { T = v; break; }
      cum += s_tot[v];
    }
    s_T = T;
    s_gt = (uint32_t)cum;
    meta[bh * 4 + 0] = T;
    meta[bh * 4 + 1] = (int32_t)cum;
    meta[bh * 4 + 2] = (int32_t)(C - (int64_t)cum);
    meta[bh * 4 + 3] = (int32_t)C;
  }
  __syncthreads();
  const int T = s_T;
  const int64_t Q = C - (int64_t)s_gt;
  uint32_t carry_tie = 0, carry_off = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 256) {
    const int c = c0 + tid;
    uint32_t gt = 0, eq = 0;
    if (c < nchunks) {
      const uint32_t* hc = hb + (int64_t)c * nbins;
      for (int v = T + 1; v < nbins; ++v) gt += hc[v];
      eq = hc[T];
    }
    uint2 tot;
    const uint2 ex = block_exscan2<256>(make_uint2(eq, 0), s_w, tot);
    const uint32_t tie_before = carry_tie + ex.x;
    int64_t quota = Q - (int64_t)tie_before;
    if (quota < 0) quota = 0;
    const uint32_t sel = gt + (uint32_t)((int64_t)eq < quota ? eq : quota);
    uint2 tot2;
    const uint2 ex2 = block_exscan2<256>(make_uint2(sel, 0), s_w, tot2);
    if (c < nchunks) {
      coff[((int64_t)bh * chunk_stride + c) * 2 + 0] = carry_off + ex2.x;
      coff[((int64_t)bh * chunk_stride + c) * 2 + 1] = tie_before;
    }
    carry_tie += tot.x;
    carry_off += tot2.x;
  }
}

// ---------------------------------------------------------------------------
// K4b + K5 compact and rerank.  Ordered compaction of this chunk's
// candidates (see K4a), then [TS] Candidate Reranking (RSQ-IP) "Estimation"
// for each: est = sum_b w_b <v_b, yq_b>, evaluated in fp32 as
//   est = 0; for b: { p = 0; for j: p = p + fl(v_{b,j} yq_{b,j}); est = est + fl(w_b p) }
// The products fl(v yq) for all 16 codes of each coordinate are tabulated in
// LDS (fl(-L yq) = -fl(L yq) exactly), so each coordinate costs one LDS read
// and one add in the stated order.  Reads 64 B of codes + 32 B of w per
// candidate; writes (position, estimate) at the candidate's rank in
// ascending-position order.  Grid (chunks, b*H_kv), same chunking as K3.
// ---------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(256) void k_compact_rerank(
    const uint8_t* __restrict__ scores, int64_t Epad, int64_t S, int64_t E,
    const int32_t* __restrict__ meta, const uint32_t* __restrict__ coff, int chunk_stride,
    const float* __restrict__ yq, const uint4* __restrict__ nib, const uint4* __restrict__ wq,
    int64_t cap, int32_t* __restrict__ cand, float* __restrict__ est, int64_t cstride,
    int64_t C) {
  constexpr int CH = KPT * 256;
  const int bh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  __shared__ float s_P[128 * 16];
  __shared__ uint16_t s_list[CH];
  __shared__ uint2 s_w[4];
  for (int e = tid; e < 2048; e += 256) {
    const int j = e >> 4, code = e & 15;
    const float pr = c_levels[code & 7] * yq[(int64_t)bh * 128 + j];
    s_P[e] = (code & 8) ? -pr : pr;
  }
  const int T = meta[bh * 4 + 0];
  const int64_t Q = meta[bh * 4 + 2];
  const uint32_t off_c = coff[((int64_t)bh * chunk_stride + chunk) * 2 + 0];
  const uint32_t tieb_c = coff[((int64_t)bh * chunk_stride + chunk) * 2 + 1];
  int64_t quota = Q - (int64_t)tieb_c;
  if (quota < 0) quota = 0;

  const int64_t pbase = (int64_t)chunk * CH + tid * KPT;
  const uint8_t* sp = scores + bh * Epad + pbase;
  uint8_t sc[KPT];
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
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const bool valid = pbase + t < E;
    ngt += (valid && sc[t] > T) ? 1u : 0u;
    neq += (valid && sc[t] == T) ? 1u : 0u;
  }
  uint2 tot;
  const uint2 ex = block_exscan2<256>(make_uint2(ngt, neq), s_w, tot);
  uint32_t pos = ex.x + (uint32_t)((int64_t)ex.y < quota ? ex.y : quota);
  uint32_t tie_seen = ex.y;
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const bool valid = pbase + t < E;
    bool sel = false;
    if (valid) {
      if (sc[t] > T) sel = true;
      else if (sc[t] == T) { sel = (int64_t)tie_seen < quota; ++tie_seen; }
    }
    if (sel) s_list[pos++] = (uint16_t)(tid * KPT + t);
  }
  const uint32_t nsel = tot.x + (uint32_t)((int64_t)tot.y < quota ? tot.y : quota);
  __syncthreads();

  for (uint32_t j = tid; j < nsel; j += 256) {
    const int64_t i = S + (int64_t)chunk * CH + s_list[j];
    const uint4* np = nib + (bh * cap + i) * 4;
    const uint4* wp = wq + (bh * cap + i) * 2;
    const uint4 n0 = np[0], n1 = np[1], n2 = np[2], n3 = np[3];
    const uint4 w0 = wp[0], w1 = wp[1];
    const uint32_t cw[16] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w,
                             n2.x, n2.y, n2.z, n2.w, n3.x, n3.y, n3.z, n3.w};
    const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float e = 0.0f;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      float p = 0.0f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) p = p + s_P[(b * 8 + jj) * 16 + ((cw[b] >> (4 * jj)) & 15u)];
      const uint16_t hb = (uint16_t)(ww[b >> 1] >> ((b & 1) * 16));
      const float wf = (float)__builtin_bit_cast(_Float16, hb);
      e = e + wf * p;
    }
    if ((int64_t)off_c + j < C) {  // always true when K4a and this kernel agree
      cand[bh * cstride + off_c + j] = (int32_t)i;
      est[bh * cstride + off_c + j] = e;
    }
  }
}

// ---------------------------------------------------------------------------
// K6 exact top-k over the reranked candidates ([TS] Key Contributions 2:
// Top-k selection on the compressed codes).  Order: (est desc, position asc),
// -0 == +0.  Radix select of the k'-th largest order key (11 + 11 + 10 bits,
// LDS histograms), then an ordered compaction: keys above the threshold plus
// the first `remaining` ties in position order, written after the S sinks
// in ascending position order.  One 1024-thread block per (b, h).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(1024) void k_topk(const float* __restrict__ est,
                                               const int32_t* __restrict__ cand, int64_t cstride,
                                               int C, int kprime, int S, int k,
                                               int32_t* __restrict__ out_idx,
                                               float* __restrict__ out_est) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* e = est + bh * cstride;
  const int32_t* cd = cand + bh * cstride;
  int32_t* oi = out_idx + (int64_t)bh * k;
  __shared__ uint32_t s_hist[2048];
  __shared__ uint2 s_w[16];
  __shared__ uint32_t s_digit, s_rem;
  for (int t = tid; t < S; t += 1024) oi[t] = t;

  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)kprime;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass], nb = 1 << widths[pass];
    for (int i = tid; i < nb; i += 1024) s_hist[i] = 0;
    __syncthreads();
    for (int c = tid; c < C; c += 1024) {
      const uint32_t o = order_key(e[c]);
      if ((o & pmask) == prefix) atomicAdd(&s_hist[(o >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    // bins in descending order; thread t owns bins nb-1-bpt*t ... (bpt bins)
    const int bpt = nb / 1024;
    uint32_t mine = 0;
    for (int q = 0; q < bpt; ++q) mine += s_hist[nb - 1 - (tid * bpt + q)];
    uint2 tot;
    const uint2 ex = block_exscan2<1024>(make_uint2(mine, 0), s_w, tot);
    uint32_t above = ex.x;
    for (int q = 0; q < bpt; ++q) {
      const int bin = nb - 1 - (tid * bpt + q);
      const uint32_t cnt = s_hist[bin];
      if (above < remaining && remaining <= above + cnt) {
        s_digit = (uint32_t)bin;
        s_rem = remaining - above;
      }
      above += cnt;
    }
    __syncthreads();
    prefix |= s_digit << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    remaining = s_rem;
    __syncthreads();
  }
  const uint32_t thr = prefix;
  // ordered compaction over contiguous per-thread ranges
  const int per = (C + 1023) / 1024;
  const int c0 = tid * per;
  const int c1 = (c0 + per < C) ? c0 + per : C;
  uint32_t ngt = 0, neq = 0;
  for (int c = c0; c < c1; ++c) {
    const uint32_t o = order_key(e[c]);
    ngt += o > thr;
    neq += o == thr;
  }
  uint2 tot;
  const uint2 ex = block_exscan2<1024>(make_uint2(ngt, neq), s_w, tot);
  uint32_t pos = ex.x + (ex.y < remaining ? ex.y : remaining);
  uint32_t tie_seen = ex.y;
  for (int c = c0; c < c1; ++c) {
    const float ev = e[c];
    const uint32_t o = order_key(ev);
    bool sel = o > thr;
    if (o == thr) { sel = tie_seen < remaining; ++tie_seen; }
    if (sel && pos < (uint32_t)kprime) {  // bound holds by construction
      oi[S + pos] = cd[c];
      if (out_est) out_est[(int64_t)bh * kprime + pos] = ev;
      ++pos;
    }
  }
}

// ---------------------------------------------------------------------------
// K7 split-K sparse attention ([TS] Problem Statement; System-Level
// Innovations 1: only the selected rows are fetched).  Block = 64 selected
// rows of one (b, h); 16 lanes per row (16 B of K and of V per lane), 16 row
// slots x 4 rows.  The G query heads of the KV head are held in registers
// (pre-multiplied by scale * log2 e), logits reduced across the 16 lanes,
// softmax statistics combined across slots in LDS; writes per query head a
// partial (o[128], m, l) in the log2 domain.
// ---------------------------------------------------------------------------
template <typename T, int G>
__global__ __launch_bounds__(256) void k_attn_split(const T* __restrict__ Q, const T* __restrict__ K,
                                                    const T* __restrict__ V, int64_t rows_per_head,
                                                    const int32_t* __restrict__ idx, int k,
                                                    int n_kv_heads, float qscale,
                                                    float* __restrict__ part, int nch) {
  const int bh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int b = bh / n_kv_heads, h = bh - b * n_kv_heads;
  const int Hq = n_kv_heads * G;
  const int slot = tid >> 4, sub = tid & 15;
  __shared__ float s_m[16][G], s_l[16][G];
  __shared__ float s_o[16][G][128];

  float q[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    load8(Q + ((int64_t)(b * Hq + h * G + g) << 7) + sub * 8, q[g]);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[g][j] *= qscale;
  }
  const int32_t* ib = idx + (int64_t)bh * k;
  const T* Kb = K + ((int64_t)bh * rows_per_head << 7) + sub * 8;
  const T* Vb = V + ((int64_t)bh * rows_per_head << 7) + sub * 8;
  float kx[4][8], vx[4][8];
  bool valid[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = chunk * 64 + slot + 16 * it;
    valid[it] = r < k;
    const int64_t row = valid[it] ? (int64_t)ib[r] : 0;
    load8(Kb + (row << 7), kx[it]);
    load8(Vb + (row << 7), vx[it]);
  }
  float lg[4][G];
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) s = __builtin_fmaf(q[g][j], kx[it][j], s);
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off, 16);
      lg[it][g] = valid[it] ? s : -INFINITY;
    }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = lg[0][g];
#pragma unroll
    for (int it = 1; it < 4; ++it) m = fmaxf(m, lg[it][g]);
    float l = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (m != -INFINITY) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float p = exp2f(lg[it][g] - m);
        l += p;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = __builtin_fmaf(p, vx[it][j], o[j]);
      }
    }
    if (sub == 0) { s_m[slot][g] = m; s_l[slot][g] = l; }
#pragma unroll
    for (int j = 0; j < 8; ++j) s_o[slot][g][sub * 8 + j] = o[j];
  }
  __syncthreads();
  for (int e = tid; e < G * 128; e += 256) {
    const int g = e >> 7, j = e & 127;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < 16; ++s) M = fmaxf(M, s_m[s][g]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const float ms = s_m[s][g];
      const float f = (ms == -INFINITY) ? 0.0f : exp2f(ms - M);
      o = __builtin_fmaf(f, s_o[s][g][j], o);
      l = __builtin_fmaf(f, s_l[s][g], l);
    }
    float* pp = part + (((int64_t)(b * Hq + h * G + g)) * nch + chunk) * 130;
    pp[j] = o;
    if (j == 0) { pp[128] = M; pp[129] = l; }
  }
}

// K8 log-sum-exp merge of the split-K partials -> output row per query head.
template <typename T>
__global__ __launch_bounds__(128) void k_attn_merge(const float* __restrict__ part, int nch,
                                                    T* __restrict__ out) {
  const int bq = blockIdx.x, j = threadIdx.x;
  const float* pp = part + (int64_t)bq * nch * 130;
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, pp[c * 130 + 128]);
  float o = 0.0f, l = 0.0f;
  for (int c = 0; c < nch; ++c) {
    const float f = exp2f(pp[c * 130 + 128] - M);
    o = __builtin_fmaf(f, pp[c * 130 + j], o);
    l = __builtin_fmaf(f, pp[c * 130 + 129], l);
  }
  const float r = o / l;
  if constexpr (sizeof(T) == 2) {
    // fp32 -> bf16, round to nearest even
    uint32_t u = __float_as_uint(r);
    u += 0x7FFFu + ((u >> 16) & 1u);
    out[(int64_t)bq * 128 + j] = (T)(u >> 16);
  } else {
    out[(int64_t)bq * 128 + j] = r;
  }
}

// ---------------------------------------------------------------------------
// Launchers (host side, called from the C ABI).  Every launch goes through
// hipExtLaunchKernelGGL: with a non-null start/stop event pair the dispatch
// itself timestamps the kernel's execution (exact per-kernel durations even
// when launches are host-bound); with null events it is a plain launch.
// ---------------------------------------------------------------------------
template <typename F, typename... Args>
static hipError_t launch(F kernel, dim3 grid, dim3 block, hipStream_t st, const EvPair& ev,
                         Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  return hipGetLastError();
}

hipError_t launch_encode(int dtype, const void* K, int64_t rows_per_head, int64_t lo, int64_t n,
                         int BH, int64_t cap, uint8_t* ids, uint32_t* nib, uint16_t* wq,
                         const SignMask& sg, float c, hipStream_t st, const EvPair& ev) {
  const int64_t total = (int64_t)BH * n;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 15) / 16));
  if (dtype == 0)
    return launch(k_encode<uint16_t>, grid, dim3(256), st, ev, (const uint16_t*)K,
                  rows_per_head, lo, n, total, cap, ids, nib, wq, sg, c);
  return launch(k_encode<float>, grid, dim3(256), st, ev, (const float*)K, rows_per_head, lo, n,
                total, cap, ids, nib, wq, sg, c);
}

hipError_t launch_qprep(int dtype, const void* Q, int BH, int n_kv_heads, int G,
                        const SignMask& sg, float c, int rho, const Tiers& tw, uint8_t* lut,
                        float* yq, hipStream_t st, const EvPair& ev) {
  const float invG = 1.0f / (float)G;
  if (dtype == 0)
    return launch(k_qprep<uint16_t>, dim3(BH), dim3(256), st, ev, (const uint16_t*)Q,
                  n_kv_heads, G, invG, sg, c, rho, tw, lut, yq);
  return launch(k_qprep<float>, dim3(BH), dim3(256), st, ev, (const float*)Q, n_kv_heads, G,
                invG, sg, c, rho, tw, lut, yq);
}

hipError_t launch_scan(int kpt, int nchunks, int BH, const uint8_t* ids, int64_t cap, int64_t S,
                       int64_t E, const uint8_t* lut, uint8_t* scores, int64_t Epad,
                       uint32_t* chist, int chunk_stride, int nbins, hipStream_t st,
                       const EvPair& ev) {
  const dim3 grid(nchunks, BH);
  const uint4* id4 = (const uint4*)ids;
  switch (kpt) {
#define PKV_SCAN(K)                                                                          \
  case K:                                                                                    \
    return launch(k_scan<K>, grid, dim3(256), st, ev, id4, cap, S, E, lut, scores, Epad,     \
                  chist, chunk_stride, nbins);
    PKV_SCAN(1) PKV_SCAN(2) PKV_SCAN(4) PKV_SCAN(8) PKV_SCAN(16)
#undef PKV_SCAN
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_thresh(int BH, const uint32_t* chist, int chunk_stride, int nchunks, int nbins,
                         int64_t C, int32_t* meta, uint32_t* coff, hipStream_t st,
                         const EvPair& ev) {
  return launch(k_thresh, dim3(BH), dim3(256), st, ev, chist, chunk_stride, nchunks, nbins, C,
                meta, coff);
}

hipError_t launch_compact_rerank(int kpt, int nchunks, int BH, const uint8_t* scores,
                                 int64_t Epad, int64_t S, int64_t E, const int32_t* meta,
                                 const uint32_t* coff, int chunk_stride, const float* yq,
                                 const uint32_t* nib, const uint16_t* wq, int64_t cap,
                                 int32_t* cand, float* est, int64_t cstride, int64_t C,
                                 hipStream_t st, const EvPair& ev) {
  const dim3 grid(nchunks, BH);
  const uint4* n4 = (const uint4*)nib;
  const uint4* w4 = (const uint4*)wq;
  switch (kpt) {
#define PKV_CR(K)                                                                            \
  case K:                                                                                    \
    return launch(k_compact_rerank<K>, grid, dim3(256), st, ev, scores, Epad, S, E, meta,    \
                  coff, chunk_stride, yq, n4, w4, cap, cand, est, cstride, C);
    PKV_CR(1) PKV_CR(2) PKV_CR(4) PKV_CR(8) PKV_CR(16)
#undef PKV_CR
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_topk(int BH, const float* est, const int32_t* cand, int64_t cstride, int C,
                       int kprime, int S, int k, int32_t* out_idx, float* out_est,
                       hipStream_t st, const EvPair& ev) {
  return launch(k_topk, dim3(BH), dim3(1024), st, ev, est, cand, cstride, C, kprime, S, k,
                out_idx, out_est);
}

hipError_t launch_attn_split(int dtype, int G, const void* Q, const void* K, const void* V,
                             int64_t rows_per_head, const int32_t* idx, int k, int batch,
                             int n_kv_heads, float qscale, float* part, int nch, hipStream_t st,
                             const EvPair& ev) {
  const dim3 grid(nch, batch * n_kv_heads);
#define PKV_AS(T, GG)                                                                         \
  return launch(k_attn_split<T, GG>, grid, dim3(256), st, ev, (const T*)Q, (const T*)K,     \
                (const T*)V, rows_per_head, idx, k, n_kv_heads, qscale, part, nch)
  if (dtype == 0) {
    switch (G) {
      case 1: PKV_AS(uint16_t, 1);
      case 2: PKV_AS(uint16_t, 2);
      case 4: PKV_AS(uint16_t, 4);
      case 8: PKV_AS(uint16_t, 8);
      default: return hipErrorInvalidValue;
    }
  }
  switch (G) {
    case 1: PKV_AS(float, 1);
    case 2: PKV_AS(float, 2);
    case 4: PKV_AS(float, 4);
    case 8: PKV_AS(float, 8);
    default: return hipErrorInvalidValue;
  }
#undef PKV_AS
}

hipError_t launch_attn_merge(int dtype, const float* part, int nch, int rows, void* out,
                             hipStream_t st, const EvPair& ev) {
  if (dtype == 0)
    return launch(k_attn_merge<uint16_t>, dim3(rows), dim3(128), st, ev, part, nch,
                  (uint16_t*)out);
  return launch(k_attn_merge<float>, dim3(rows), dim3(128), st, ev, part, nch, (float*)out);
}

void codebook_m8(float* L, float* tau) {
  for (int i = 0; i < 8; ++i) L[i] = kLevels_m8[i];
  for (int i = 0; i < 7; ++i) tau[i] = kThresh_m8[i];
}
void codebook_m4(float* L, float* tau) {
  for (int i = 0; i < 8; ++i) L[i] = kLevels_m4[i];
  for (int i = 0; i < 7; ++i) tau[i] = kThresh_m4[i];
}

}  // namespace pkv
