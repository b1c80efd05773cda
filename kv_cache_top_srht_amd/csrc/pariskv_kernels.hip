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
#include <algorithm>
#include <stdint.h>
#include <type_traits>

#include "codebook_tables.h"
#include "pariskv_device.h"
#include "pariskv_internal.h"

#pragma clang fp contract(off)

namespace pkv {

__constant__ float c_levels[8] = {
    kLevels_m8[0], kLevels_m8[1], kLevels_m8[2], kLevels_m8[3],
    kLevels_m8[4], kLevels_m8[5], kLevels_m8[6], kLevels_m8[7]};
__constant__ float c_thresh[7] = {
    kThresh_m8[0], kThresh_m8[1], kThresh_m8[2], kThresh_m8[3],
    kThresh_m8[4], kThresh_m8[5], kThresh_m8[6]};
__constant__ float c_levels4[8] = {
    kLevels_m4[0], kLevels_m4[1], kLevels_m4[2], kLevels_m4[3],
    kLevels_m4[4], kLevels_m4[5], kLevels_m4[6], kLevels_m4[7]};
__constant__ float c_thresh4[7] = {
    kThresh_m4[0], kThresh_m4[1], kThresh_m4[2], kThresh_m4[3],
    kThresh_m4[4], kThresh_m4[5], kThresh_m4[6]};

// codebook of subspace size M (8 or 4): level i and threshold i
template <int M>
__device__ __forceinline__ float cb_level(int i) {
  if constexpr (M == 8) return c_levels[i];
  else return c_levels4[i];
}
template <int M>
__device__ __forceinline__ float cb_thresh(int i) {
  if constexpr (M == 8) return c_thresh[i];
  else return c_thresh4[i];
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
// Quantization + Calibration.  One key per 16-lane group; lane `sub` owns
// coordinates [8 sub, 8 sub + 8): one subspace of M = 8, or the two
// subspaces 2 sub, 2 sub + 1 of M = 4.  Per subspace z (coordinates j):
//   id   = sum_j [z_j < 0] 2^j
//   n    = sqrt(((z_0 z_0 + z_1 z_1) + ...) + z_{M-1} z_{M-1})
//   u_j  = z_j / n; mag_j = #{l : |u_j| >= tau_l}; code_j = sign_j << 3 | mag_j
//   a    = ((v_0 u_0 + v_1 u_1) + ...), v_j = +-L[mag_j]
//   w    = fp16_rne(n / a)           (n == 0: magnitudes 0, w = 0)
// with the Lloyd-Max codebook (L, tau) of subspace size M.
// Index layout per (b,h): ids [cap][16] bytes and a 128-byte record per key
// (one L2 line): dwords 0..15 = codes (nibble j of dword s = coordinate
// 8 s + j), then w as fp16 per subspace from byte 64 (M = 8: 16 of them,
// bytes 96..127 unused; M = 4: 32 of them).  Byte s of the ids holds the
// sign bits of coordinates 8 s .. 8 s + 7: the id of subspace s (M = 8), or
// the ids of subspaces 2 s (low nibble) and 2 s + 1 (high nibble) (M = 4).
// ---------------------------------------------------------------------------
// Encodes key row r of (b, h) = bh (16 lanes, lane `sub` = coordinates
// 8 sub .. 8 sub + 7) into index position `pos`; returns the lane's id byte.
template <typename T, int M>
__device__ __forceinline__ uint32_t encode_key(const T* __restrict__ K, int64_t rows_per_head,
                                           int64_t bh, int64_t r, int64_t pos, int64_t cap,
                                           uint8_t* __restrict__ ids, uint32_t* __restrict__ rec,
                                           const SignMask& sg, float c, int sub) {
  static_assert(M == 8 || M == 4, "subspaces of 8 or 4 coordinates");
  float x[8];
  load8(K + ((bh * rows_per_head + r) << 7) + sub * 8, x);
  srht16(x, sign_byte_of(sg, sub), sub, c);

  uint32_t id = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) id |= (x[j] < 0.0f ? 1u : 0u) << j;
  uint32_t code = 0, wpack = 0;
#pragma unroll
  for (int sb = 0; sb < 8 / M; ++sb) {
    const int j0 = sb * M;
    float n2 = 0.0f;
#pragma unroll
    for (int j = j0; j < j0 + M; ++j) n2 = n2 + x[j] * x[j];
    const float nrm = sqrtf(n2);
    if (nrm != 0.0f) {
      float a = 0.0f;
#pragma unroll
      for (int j = j0; j < j0 + M; ++j) {
        const float u = x[j] / nrm;
        const float au = fabsf(u);
        uint32_t mag = 0;
        float lv = cb_level<M>(0);
#pragma unroll
        for (int l = 0; l < 7; ++l)
          if (au >= cb_thresh<M>(l)) { mag = l + 1; lv = cb_level<M>(l + 1); }
        const uint32_t sgn = (id >> j) & 1u;
        const float v = sgn ? -lv : lv;
        a = a + v * u;
        code |= ((sgn << 3) | mag) << (4 * j);
      }
      const _Float16 hw = (_Float16)(nrm / a);
      wpack |= (uint32_t)__builtin_bit_cast(uint16_t, hw) << (16 * sb);
    } else {
#pragma unroll
      for (int j = j0; j < j0 + M; ++j) code |= ((id >> j) & 1u) << (4 * j + 3);
    }
  }
  const int64_t key = bh * cap + pos;
  ids[key * 16 + sub] = (uint8_t)id;
  rec[key * 32 + sub] = code;
  if constexpr (M == 8)
    reinterpret_cast<uint16_t*>(rec)[key * 64 + 32 + sub] = (uint16_t)wpack;
  else
    rec[key * 32 + 16 + sub] = wpack;
  return id;
}

template <typename T, int M>
__global__ __launch_bounds__(256) void k_encode(const T* __restrict__ K, int64_t rows_per_head,
                                                int64_t lo, int64_t n, int64_t total, int64_t cap,
                                                uint8_t* __restrict__ ids, uint32_t* __restrict__ rec,
                                                SignMask sg, float c) {
  const int sub = threadIdx.x & 15;
  const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (g >= total) return;  // whole 16-lane groups leave together
  const int64_t bh = g / n;
  const int64_t r = g - bh * n;
  encode_key<T, M>(K, rows_per_head, bh, r, lo + r, cap, ids, rec, sg, c, sub);
}

// ---------------------------------------------------------------------------
// K2 query prep: [TS] Coarse Candidate Generation, query side.  Group query
// q = (q_0 + q_1 + ... + q_{G-1}) * fp32(1/G) in head order, yq = SRHT(q).
// Per subspace, the 2^M centroid scores sc_p = sum_j (bit j of p ? -yq : +yq)
// (sequential in j from the j = 0 term); the rho best by (sc desc, p asc)
// get tier weights, all other centroids 0.
// One 1024-thread block per (b, h); wave s builds row s of the vote table,
// indexed by byte s of a key's ids.  M = 8: row s is subspace s's LUT; lane
// l scores centroids 4 l .. 4 l + 3 and keeps them in order; rho rounds of a
// wave maximum over 64-bit (score, centroid) keys pick the winners.  M = 4:
// row s is the pair table of subspaces 2 s and 2 s + 1, entry v = lut_2s[v &
// 15] + lut_2s+1[v >> 4], so the scan's sum over 16 bytes equals the sum
// over the 32 subspaces; rows 0 and 1 of the wave (16 lanes each) score the
// 16 centroids of the two subspaces and pick their winners by row maxima.
// ---------------------------------------------------------------------------
// Centroid p of a subspace with score sc as one 64-bit key: larger key means
// earlier in (sc desc, p asc); -0 and +0 tie.
__device__ __forceinline__ uint64_t centroid_key(float sc, int p) {
  return ((uint64_t)order_key(sc) << 32) | (uint64_t)(255 - p);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over each row of 16 lanes, received by every lane of the row: DPP
// quad swaps (lane ^ 1, lane ^ 2), the half-row mirror and the row mirror.
__device__ __forceinline__ uint64_t row_max64(uint64_t k) {
  k = max64(k, dpp64<0xB1>(k));   // quad_perm [1, 0, 3, 2]
  k = max64(k, dpp64<0x4E>(k));   // quad_perm [2, 3, 0, 1]
  k = max64(k, dpp64<0x141>(k));  // row_half_mirror
  k = max64(k, dpp64<0x140>(k));  // row_mirror
  return k;
}

// lane l's value, wave-uniform
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
// Maximum over the 64 lanes, received by every lane: the row maxima, then
// the four rows' values read into scalar registers (lanes 0, 16, 32, 48).
__device__ __forceinline__ uint64_t wave_max64(uint64_t k) {
  k = row_max64(k);
  return max64(max64(readlane64(k, 0), readlane64(k, 16)), max64(readlane64(k, 32), readlane64(k, 48)));
}

// Word l (entries 4 l .. 4 l + 3) of row s of the vote table, computed by
// lane l of one wave from the rotated query yq (LDS).  M = 8: row s is
// subspace s, its 256 centroids scored 4 per lane, the rho best by wave
// maxima of 64-bit (score, centroid) keys get the tier weights.  M = 4: row s
// is the byte table of subspaces 2 s and 2 s + 1, each a row of 16 lanes
// taking its rho best of 16 centroids by row maxima.
template <int M>
__device__ __forceinline__ uint32_t vote_table_word(const float* s_yq, int s, int l, int rho,
                                                    const Tiers& tw) {
  if constexpr (M == 4) {
    // lane l scores centroid p = l & 15 of subspace 2 s + ((l >> 4) & 1)
    // (rows 2 and 3 repeat rows 0 and 1)
    const int half = (l >> 4) & 1, p = l & 15;
    float z4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) z4[j] = s_yq[s * 8 + half * 4 + j];
    float acc = (p & 1) ? -z4[0] : z4[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) acc = acc + (((p >> j) & 1) ? -z4[j] : z4[j]);
    uint64_t key = centroid_key(acc, p);
    // rho rounds: the row's best remaining centroid gets tier weight r and
    // drops out (key 0 is below every centroid)
    uint32_t wt = 0;
    for (int r = 0; r < rho; ++r) {
      const uint64_t W = row_max64(key);
      if (key == W) {
        wt = (uint32_t)tw.w[r];
        key = 0;
      }
    }
    // entries v = 4 l .. 4 l + 3: low nibble's weight from row 0, high
    // nibble's (v >> 4 = l >> 2) from row 1
    const uint32_t whi = (uint32_t)__shfl((int)wt, 16 + (l >> 2));
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wlo = (uint32_t)__shfl((int)wt, (4 * l + q) & 15);
      word |= (wlo + whi) << (8 * q);
    }
    return word;
  }
  float z[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = s_yq[s * 8 + j];
  uint64_t key[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = l * 4 + q;
    float acc = (p & 1) ? -z[0] : z[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) acc = acc + (((p >> j) & 1) ? -z[j] : z[j]);
    key[q] = centroid_key(acc, p);
  }
  // the lane's 4 in descending key order
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3 - i; ++j)
      if (key[j + 1] > key[j]) { const uint64_t t = key[j]; key[j] = key[j + 1]; key[j + 1] = t; }
  // rho rounds: the wave's best remaining centroid gets tier weight r; its
  // owner lane drops it (an exhausted lane offers key 0, below every centroid)
  uint32_t lv[4] = {0, 0, 0, 0};
  for (int r = 0; r < rho; ++r) {
    const uint64_t W = wave_max64(key[0]);
    const int wp = 255 - (int)(uint32_t)(W & 0xFFu);
    if ((wp >> 2) == l) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((wp & 3) == q) lv[q] = (uint32_t)tw.w[r];
    }
    if (key[0] == W) {
      key[0] = key[1];
      key[1] = key[2];
      key[2] = key[3];
      key[3] = 0;
    }
  }
  return lv[0] | (lv[1] << 8) | (lv[2] << 16) | (lv[3] << 24);
}

// One 64-thread block per (retrieval unit, vote-table row s): its 16 lanes
// 0..15 form the unit's mean query and rotate it (every block of the unit
// the same fp32 operations, so the same yq), then the block writes row s of
// the vote table, the product-table entries of coordinates 8 s .. 8 s + 7
// and (lanes s) those 8 coordinates of yq.  Short blocks that start at once
// on idle CUs, rather than a long one per unit.
template <typename T, int G, int M>
__global__ __launch_bounds__(64) void k_qprep(const T* __restrict__ Q, int n_kv_heads,
                                              float invG, SignMask sg, float c, int rho, Tiers tw,
                                              uint8_t* __restrict__ lut_out, float* __restrict__ yq_out,
                                              float* __restrict__ ptab_out, AppendJob app,
                                              int unit_div, int n_units) {
  // blocks 16 u + s: retrieval unit u, a (b, KV head), or a (b, query head)
  // with unit_div = G units per KV head (then G = 1 here and n_kv_heads
  // counts units per batch entry); blocks 16 n_units.. encode appended keys
  const int blk = blockIdx.x;
  const int tid = threadIdx.x;
  if (blk >= 16 * n_units) {
    // blocks past the units encode the keys appended since the last
    // retrieval (16 lanes per (KV head, key), 4 per block), so the vote scan
    // sees them
    const int pair = (blk - 16 * n_units) * 4 + (tid >> 4);
    const int kvh = pair / app.n, r = pair - kvh * app.n;
    if (kvh < n_units / unit_div)
      encode_key<T, M>((const T*)app.K, app.rows_per_head, kvh, r, app.lo + r, app.cap, app.ids,
                       app.rec, sg, c, tid & 15);
    return;
  }
  const int bh = blk >> 4, s = blk & 15;
  const int b = bh / n_kv_heads, h = bh - b * n_kv_heads;
  const int Hq = n_kv_heads * G;
  __shared__ float s_yq[128];
  if (tid < 16) {
    const int sub = tid;
    // all G query rows are loaded at once, then summed in head order
    float xg[G][8];
    const T* q0 = Q + ((int64_t)(b * Hq + h * G) << 7) + sub * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) load8(q0 + ((int64_t)g << 7), xg[g]);
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = xg[0][j];
#pragma unroll
    for (int g = 1; g < G; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = x[j] + xg[g][j];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = x[j] * invG;
    srht16(x, sign_byte_of(sg, sub), sub, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) s_yq[sub * 8 + j] = x[j];
    if (sub == s) {
      reinterpret_cast<float4*>(yq_out + (int64_t)bh * 128 + sub * 8)[0] =
          make_float4(x[0], x[1], x[2], x[3]);
      reinterpret_cast<float4*>(yq_out + (int64_t)bh * 128 + sub * 8)[1] =
          make_float4(x[4], x[5], x[6], x[7]);
    }
  }
  __syncthreads();
  // product table for the rerank: ptab[j][code] = fl(+-L[code & 7] yq_j), the
  // sign bit (code & 8) negating the product exactly; entries 128 s ..
  // 128 s + 127 are coordinates 8 s .. 8 s + 7
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 128 * s + tid + 64 * i;
    const float pr = cb_level<M>(e & 7) * s_yq[e >> 4];
    ptab_out[(int64_t)bh * 2048 + e] = (e & 8) ? -pr : pr;
  }
  reinterpret_cast<uint32_t*>(lut_out + ((int64_t)bh * 16 + s) * 256)[tid] =
      vote_table_word<M>(s_yq, s, tid, rho, tw);
}

// ---------------------------------------------------------------------------
// K3 vote scan: [TS] Coarse Candidate Generation: score_i = sum_b lut_b[id_{i,b}]
// for i in [S, N).  The dominant HBM stream: 16 bytes of bucket ids per key,
// read once, coalesced (256 threads x 16 B per step).  The 4 KB vote LUT
// sits in LDS; one ds_read_u8 per subspace.  Writes one score byte per key
// and a per-chunk histogram of the scores (zeros counted by wave ballot, the
// rest by per-wave LDS atomics), stored cumulatively: row[v] = #(score >= v)
// within the chunk.
// Grid (chunks, b*H_kv); chunk = KPT * 256 keys.
// ---------------------------------------------------------------------------
// The keys of one chunk: loads (clamped to E - 1 unless the chunk is full,
// i.e. FULL), the LUT into LDS, then per key the score byte and the wave
// histogram.  A full chunk has no per-key bounds tests.
template <int KPT, int NT, bool FULL>
__device__ __forceinline__ void scan_keys(const uint4* __restrict__ src, int chunk, int64_t E,
                                          const uint4 lutv, uint8_t* s_lut,
                                          uint32_t (*s_hist)[256], uint8_t* __restrict__ dst) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t p0 = (int64_t)chunk * (KPT * NT) + tid;
  uint4 x[KPT];
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int64_t p = p0 + t * NT;
    x[t] = load_stream(&src[(FULL || p < E) ? p : E - 1]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // the LUT store waits for the LUT load alone (issued before the keys)
  reinterpret_cast<uint4*>(s_lut)[tid & 255] = lutv;
  for (int i = tid; i < NW * 256; i += NT) (&s_hist[0][0])[i] = 0;
  __syncthreads();
  uint32_t zeros = 0;
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int64_t p = p0 + t * NT;
    const bool valid = FULL || p < E;
    const uint32_t w4[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
    uint32_t sc = 0;
#pragma unroll
    for (int b = 0; b < 16; ++b) sc += s_lut[b * 256 + ((w4[b >> 2] >> ((b & 3) * 8)) & 0xFFu)];
    const uint64_t zm = __ballot(valid && sc == 0);
    zeros += (uint32_t)__popcll(zm);
    if (valid) {
      dst[p] = (uint8_t)sc;
      if (sc != 0) atomicAdd(&s_hist[wv][sc], 1u);
    }
  }
  if (lane == 0) s_hist[wv][0] = zeros;
}

// The chunk's cumulative row from the wave histograms: wave 0 alone, lane l
// adding bins 4 l .. 4 l + 3 of every wave's histogram (16-byte LDS reads),
// while the other waves are done.
template <int NT>
__device__ __forceinline__ void scan_rows(uint32_t (*s_hist)[256], uint32_t* __restrict__ row,
                                          int nbins, int rstride) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __syncthreads();
  // chunk row = #(score >= v) for every v: suffix sums by wave 0, lane l
  // owning bins 4 l .. 4 l + 3 (rows rstride words apart; bins >= nbins are 0)
  if (wv == 0) {
    uint32_t hs[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint4 x = reinterpret_cast<const uint4*>(s_hist[w])[lane];
      hs[0] += x.x;
      hs[1] += x.y;
      hs[2] += x.z;
      hs[3] += x.w;
    }
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = (4 * lane + r < nbins) ? hs[r] : 0u;
    const uint32_t loc = h[0] + h[1] + h[2] + h[3];
    uint32_t inc = loc;  // sum over lanes >= this one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_down(inc, off);
      if (lane + off < 64) inc += t;
    }
    uint32_t ge[4];
    ge[3] = inc - loc + h[3];
    ge[2] = ge[3] + h[2];
    ge[1] = ge[2] + h[1];
    ge[0] = ge[1] + h[0];
    if (4 * lane < rstride) reinterpret_cast<uint4*>(row)[lane] = make_uint4(ge[0], ge[1], ge[2], ge[3]);
  }
}

// one chunk of KPT * NT keys per block
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void k_scan(const uint4* __restrict__ ids, int64_t cap, int64_t S,
                                             int64_t E, const uint8_t* __restrict__ lut,
                                             uint8_t* __restrict__ scores, int64_t Epad,
                                             uint32_t* __restrict__ chist, int chunk_stride, int nbins,
                                             int rstride, int unit_div) {
  const int bh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  __shared__ uint8_t s_lut[16 * 256];
  __shared__ __align__(16) uint32_t s_hist[NT / 64][256];
  // The LUT load goes out first, from every thread (a load under a branch
  // would make the compiler wait for it at the join, before the key loads
  // are issued; threads tid and tid + 256 store the same bytes).
  const uint4 lutv = reinterpret_cast<const uint4*>(lut + (int64_t)bh * 4096)[tid & 255];
  __builtin_amdgcn_sched_barrier(0);
  const int kvh = unit_div == 1 ? bh : bh / unit_div;  // the unit's KV head
  const uint4* src = ids + (int64_t)kvh * cap + S;
  uint8_t* dst = scores + bh * Epad;
  if ((int64_t)(chunk + 1) * (KPT * NT) <= E)
    scan_keys<KPT, NT, true>(src, chunk, E, lutv, s_lut, s_hist, dst);
  else
    scan_keys<KPT, NT, false>(src, chunk, E, lutv, s_lut, s_hist, dst);
  scan_rows<NT>(s_hist, chist + ((int64_t)bh * chunk_stride + chunk) * rstride, nbins, rstride);
}

// ---------------------------------------------------------------------------
// K3 for unshared retrieval: the GU query heads of one KV head scan its ids in
// one pass, so each key's 16 B are read once instead of GU times.  Their GU
// vote tables are interleaved in LDS, entry (s, v) holding head g's vote in
// byte g % 4 of word g / 4, so one 32-bit read per subspace returns four
// heads' votes and 32-bit adds sum them bytewise (a head's score is at most
// 255, so no byte carries into the next).  Per head the outputs are those of
// k_scan: score bytes and the cumulative chunk row, with per-wave histograms
// of two 16-bit bins per word (a wave counts at most 512 keys).
// Grid (chunks, b*H_kv); units kvh*GU .. kvh*GU + GU - 1 are the KV head's.
// ---------------------------------------------------------------------------
template <int KPT, int NT, int GU>
__global__ __launch_bounds__(NT) void k_scan_group(const uint4* __restrict__ ids, int64_t cap,
                                                   int64_t S, int64_t E,
                                                   const uint8_t* __restrict__ lut,
                                                   uint8_t* __restrict__ scores, int64_t Epad,
                                                   uint32_t* __restrict__ chist,
                                                   int chunk_stride, int nbins, int rstride) {
  constexpr int NW = NT / 64;
  constexpr int W = (GU + 3) / 4;  // words per table entry
  constexpr int NQ = 1024 / NT;    // entry quads per thread and head
  static_assert(NW >= GU, "one wave per head builds the chunk rows");
  static_assert(KPT * 64 <= 65535, "16-bit wave bins");
  const int kvh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  __shared__ uint32_t s_lut[W][16 * 256];
  __shared__ uint32_t s_hist[GU][NW][128];
  // table loads first, then the keys (unconditional, index clamped)
  uint32_t lv[NQ][GU];
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int g = 0; g < GU; ++g)
      lv[i][g] = reinterpret_cast<const uint32_t*>(lut + ((int64_t)kvh * GU + g) * 4096)[tid + i * NT];
  const uint4* src = ids + (int64_t)kvh * cap + S;
  const int64_t p0 = (int64_t)chunk * (KPT * NT) + tid;
  uint4 x[KPT];
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int64_t p = p0 + t * NT;
    x[t] = load_stream(&src[p < E ? p : E - 1]);
  }
  // interleave: entry 4 q + e gets byte e of head g's word in byte g % 4
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int q4 = tid + i * NT;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
      for (int g = 4 * w; g < 4 * w + 4 && g < GU; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] |= ((lv[i][g] >> (8 * e)) & 0xFFu) << (8 * (g & 3));
      reinterpret_cast<uint4*>(&s_lut[w][0])[q4] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  for (int i = tid; i < GU * NW * 128; i += NT) (&s_hist[0][0][0])[i] = 0;
  __syncthreads();

  uint32_t zeros[GU];
#pragma unroll
  for (int g = 0; g < GU; ++g) zeros[g] = 0;
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int64_t p = p0 + t * NT;
    const bool valid = p < E;
    const uint32_t w4[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
    uint32_t acc[W];
#pragma unroll
    for (int w = 0; w < W; ++w) acc[w] = 0;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const uint32_t v = (w4[b >> 2] >> ((b & 3) * 8)) & 0xFFu;
#pragma unroll
      for (int w = 0; w < W; ++w) acc[w] += s_lut[w][b * 256 + v];
    }
#pragma unroll
    for (int g = 0; g < GU; ++g) {
      const uint32_t sc = (acc[g >> 2] >> (8 * (g & 3))) & 0xFFu;
      zeros[g] += (uint32_t)__popcll(__ballot(valid && sc == 0));
      if (valid) {
        scores[((int64_t)kvh * GU + g) * Epad + p] = (uint8_t)sc;
        if (sc != 0) atomicAdd(&s_hist[g][wv][sc >> 1], 1u << (16 * (sc & 1)));
      }
    }
  }
  if (lane == 0)
#pragma unroll
    for (int g = 0; g < GU; ++g) atomicAdd(&s_hist[g][wv][0], zeros[g]);
  __syncthreads();
  // sum the wave histograms of every head into its row 0 (bins stay packed)
  for (int i = tid; i < GU * 128; i += NT) {
    const int g = i >> 7, wd = i & 127;
    uint32_t a = s_hist[g][0][wd];
#pragma unroll
    for (int w = 1; w < NW; ++w) a += s_hist[g][w][wd];
    s_hist[g][0][wd] = a;
  }
  __syncthreads();
  // wave g: head g's row = #(score >= v), lane l owning bins 4 l .. 4 l + 3
  if (wv < GU) {
    const int g = wv;
    const uint32_t wa = s_hist[g][0][2 * lane], wb = s_hist[g][0][2 * lane + 1];
    const uint32_t hv[4] = {wa & 0xFFFFu, wa >> 16, wb & 0xFFFFu, wb >> 16};
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = (4 * lane + r < nbins) ? hv[r] : 0u;
    const uint32_t loc = h[0] + h[1] + h[2] + h[3];
    uint32_t inc = loc;  // sum over lanes >= this one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_down(inc, off);
      if (lane + off < 64) inc += t;
    }
    uint32_t ge[4];
    ge[3] = inc - loc + h[3];
    ge[2] = ge[3] + h[2];
    ge[1] = ge[2] + h[1];
    ge[0] = ge[1] + h[0];
    uint32_t* row = chist + (((int64_t)kvh * GU + g) * chunk_stride + chunk) * rstride;
    if (4 * lane < rstride) reinterpret_cast<uint4*>(row)[lane] = make_uint4(ge[0], ge[1], ge[2], ge[3]);
  }
}

// ---------------------------------------------------------------------------
// K4a threshold: [TS] Coarse Candidate Generation keeps the top fraction.
// Candidates = the first C eligible keys in (score desc, index asc) order:
// T = largest v with #(score >= v) >= C; every key with score > T, plus the
// first Q = C - #(score > T) keys with score == T in index order.  From the
// cumulative per-chunk rows: totals (column sums over the rows read as one
// flat array), T, then per chunk the ties before it and the output offset of
// its first candidate (block scans over chunks, 1024 per pass).
// One 1024-thread block per (b, h).  meta[bh] = (T, #gt, Q, C).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_thresh(const uint32_t* __restrict__ chist, int chunk_stride,
                                                 int nchunks, int nbins, int rstride, int64_t C,
                                                 int all_ties, int32_t* __restrict__ meta,
                                                 uint32_t* __restrict__ coff) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  __shared__ uint32_t s_tot[260];
  __shared__ int s_T;
  __shared__ uint2 s_w[16];
  const uint32_t* hb = chist + (int64_t)bh * chunk_stride * rstride;
  for (int v = tid; v < 260; v += 1024) s_tot[v] = 0;
  // column sums over the chunk rows: thread = (row r0, group g of 4 bins),
  // 16-byte loads, 16 rows in flight per thread (a million-token unit's 512
  // rows of 65 bins in one round), summed in registers
  const int ng = rstride >> 2, rpp = 1024 / ng;
  const int g = tid % ng, r0 = tid / ng;
  uint32_t acc[4] = {0u, 0u, 0u, 0u};
  if (r0 < rpp) {
    const uint4* h4 = reinterpret_cast<const uint4*>(hb);
    for (int rb = r0; rb < nchunks; rb += 16 * rpp) {
      uint4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int row = rb + u * rpp;
        v[u] = (row < nchunks) ? h4[(int64_t)row * ng + g] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        acc[0] += v[u].x;
        acc[1] += v[u].y;
        acc[2] += v[u].z;
        acc[3] += v[u].w;
      }
    }
  }
  __syncthreads();
  if (r0 < rpp) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (acc[i] && 4 * g + i < nbins) atomicAdd(&s_tot[4 * g + i], acc[i]);
  }
  __syncthreads();
  if (tid < nbins && (int64_t)s_tot[tid] >= C && (int64_t)s_tot[tid + 1] < C) {
    // all_ties: every key of bin T is kept, so C grows to #(score >= T)
    const int64_t Ce = all_ties ? (int64_t)s_tot[tid] : C;
    s_T = tid;
    meta[bh * 4 + 0] = tid;
    meta[bh * 4 + 1] = (int32_t)s_tot[tid + 1];
    meta[bh * 4 + 2] = (int32_t)(Ce - (int64_t)s_tot[tid + 1]);
    meta[bh * 4 + 3] = (int32_t)Ce;
  }
  __syncthreads();
  const int T = s_T;
  const int64_t Q = (all_ties ? (int64_t)s_tot[T] : C) - (int64_t)s_tot[T + 1];
  // Ties are taken in position order until the quota Q is used up, so the
  // chunks before c hold min(#ties before c, Q) of them: one scan of (ties,
  // keys above T) gives a chunk both its ties before and its offset.
  uint32_t carry_tie = 0, carry_gt = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 1024) {
    const int c = c0 + tid;
    uint32_t gt = 0, eq = 0;
    if (c < nchunks) {
      const uint32_t* hc = hb + (int64_t)c * rstride;
      gt = (T + 1 < nbins) ? hc[T + 1] : 0u;
      eq = hc[T] - gt;
    }
    uint2 tot;
    const uint2 ex = block_exscan2<1024, false>(make_uint2(eq, gt), s_w, tot);
    const uint32_t tie_before = carry_tie + ex.x;
    const int64_t taken = (int64_t)tie_before < Q ? (int64_t)tie_before : Q;
    if (c < nchunks) {
      coff[((int64_t)bh * chunk_stride + c) * 2 + 0] = carry_gt + ex.y + (uint32_t)taken;
      coff[((int64_t)bh * chunk_stride + c) * 2 + 1] = tie_before;
    }
    carry_tie += tot.x;
    carry_gt += tot.y;
    if (c0 + 1024 < nchunks) __syncthreads();  // the next pass writes s_w again
  }
}

// ---------------------------------------------------------------------------
// K4b + K5 compact and rerank.  Ordered compaction of two consecutive
// chunks' candidates (see K4a), then [TS] Candidate Reranking (RSQ-IP)
// "Estimation" for each: est = sum_b w_b <v_b, yq_b>, evaluated in fp32 as
//   est = 0; for b: { p = 0; for j: p = p + fl(v_{b,j} yq_{b,j}); est = est + fl(w_b p) }
// The products fl(v yq_j) for all 16 codes of each coordinate come from the
// table K2 wrote (fl(-L yq) = -fl(L yq) exactly), staged in LDS, so each
// coordinate costs a nibble extract, one LDS read and one add in the stated
// order.  Reads the candidate's 128-byte record (96 B
// used); writes (position, estimate) at the candidate's rank in
// ascending-position order, and the block's estimate range (order keys).
// Grid (ceil(chunks / 2), b*H_kv), 256 threads.
// ---------------------------------------------------------------------------
// key masks of one chunk's KPT scores of this thread: bit t of gtm / eqm is
// set when key t (t < nval) has score > T / == T.  For 8 keys with every
// score below 128 the bytes are compared four at a time (SWAR: adding
// 0x7F - T (0x80 - T) to each byte sets its top bit exactly when the byte is
// > T (>= T), with no carry out of a byte).
template <int KPT>
__device__ __forceinline__ void score_masks(const uint8_t (&sc)[KPT], const uint2 raw, int T,
                                            int nval, bool swar, uint32_t& gtm, uint32_t& eqm) {
  gtm = 0;
  eqm = 0;
  if constexpr (KPT == 8) {
    if (swar) {
      const uint32_t ag = (uint32_t)(0x7F - T) * 0x01010101u, ae = (uint32_t)(0x80 - T) * 0x01010101u;
      const uint32_t g0 = (raw.x + ag) & 0x80808080u, g1 = (raw.y + ag) & 0x80808080u;
      const uint32_t e0 = ((raw.x + ae) & 0x80808080u) ^ g0, e1 = ((raw.y + ae) & 0x80808080u) ^ g1;
      // gather the top bits of the 4 bytes into a nibble (bit i from byte i)
      gtm = (((g0 >> 7) * 0x10204080u) >> 28) | ((((g1 >> 7) * 0x10204080u) >> 28) << 4);
      eqm = (((e0 >> 7) * 0x10204080u) >> 28) | ((((e1 >> 7) * 0x10204080u) >> 28) << 4);
      const uint32_t vm = (nval >= 8) ? 0xFFu : ((1u << nval) - 1u);
      gtm &= vm;
      eqm &= vm;
      return;
    }
  }
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    if (t < nval) {
      gtm |= (sc[t] > T) ? (1u << t) : 0u;
      eqm |= (sc[t] == T) ? (1u << t) : 0u;
    }
  }
}

// value of lane S of this lane's group of 4 (DPP quad permutation, no LDS)
template <int S>
__device__ __forceinline__ float quad_lane(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x55 * S, 0xF, 0xF, true));
}

// value of the pair lane (lane ^ 1), a DPP quad permutation [1, 0, 3, 2]
__device__ __forceinline__ float dppf_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// LDS product table: subspace b's 128 entries ([j][code]) start at b * 132
// floats, so the 4 lanes of a group (subspaces 4q + bb, q = 0..3) read
// disjoint 16-bank ranges.
constexpr int kPtabRow = 132;
constexpr int kPtabLds = 16 * kPtabRow;

// RSQ-IP estimate of one candidate by a group of 4 lanes (DPP quads): lane q
// holds the codes of coordinates 32 q .. 32 q + 31 (cw) and the fp16 w of
// their NB = 32 / M subspaces (ww), forms w_b p_b for them from the signed
// product table in LDS, and every lane of the group returns the sum of all
// B terms in b order.
template <int M>
__device__ __forceinline__ void rerank_terms(
    const uint4 cw, const typename std::conditional<M == 8, uint2, uint4>::type ww,
    const float* s_P, int q, float (&t)[32 / M]) {
  constexpr int NB = 32 / M;
  const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
  uint32_t wsw[NB / 2];
  wsw[0] = ww.x;
  wsw[1] = ww.y;
  if constexpr (M == 4) {
    wsw[2] = ww.z;
    wsw[3] = ww.w;
  }
  // every table value of the NB subspaces first: the 32 LDS reads are
  // independent and all go out before the first sum waits (left to itself the
  // compiler waits after each subspace's 8), then each subspace's sum in
  // coordinate order
  // byte offsets code * 4 of a dword's 8 nibbles, two masked shifts per
  // dword: the even nibbles in the bytes of ev, the odd ones in od; each read
  // address is then the row base plus one byte (a byte-select add)
  uint32_t ev[4], od[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    ev[c] = (cws[c] << 2) & 0x3C3C3C3Cu;
    od[c] = (cws[c] >> 2) & 0x3C3C3C3Cu;
    // opaque to the optimiser, which would otherwise fold the masks back
    // into one shift-and pair per nibble
    asm("" : "+v"(ev[c]));
    asm("" : "+v"(od[c]));
  }
  float v[NB][M];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    // subspace 4 q NB / 4 + i: coordinates from nibble j0 of code dword bb
    const int bb = (i * M) >> 3, j0 = (i * M) & 7;
    const char* pb = reinterpret_cast<const char*>(s_P + (4 * q + bb) * kPtabRow);
#pragma unroll
    for (int jj = 0; jj < M; ++jj) {
      const int n = j0 + jj;
      const uint32_t off = (((n & 1) ? od[bb] : ev[bb]) >> (8 * (n >> 1))) & 0xFFu;
      v[i][jj] = *reinterpret_cast<const float*>(pb + n * 64 + off);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float p = 0.0f;
#pragma unroll
    for (int jj = 0; jj < M; ++jj) p = p + v[i][jj];
    const uint16_t hb = (uint16_t)(wsw[i >> 1] >> ((i & 1) * 16));
    t[i] = (float)__builtin_bit_cast(_Float16, hb) * p;
  }
}

// the estimate by lanes 4 c + q of a quad (lane q of the quad holds
// quarter q's terms): every lane of the quad returns the sum of all B terms
// in b order
template <int M>
__device__ __forceinline__ float rerank_estimate(
    const uint4 cw, const typename std::conditional<M == 8, uint2, uint4>::type ww,
    const float* s_P, int q) {
  constexpr int NB = 32 / M;
  float t[NB];
  rerank_terms<M>(cw, ww, s_P, q, t);
  float e = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) e = e + quad_lane<0>(t[i]);
#pragma unroll
  for (int i = 0; i < NB; ++i) e = e + quad_lane<1>(t[i]);
#pragma unroll
  for (int i = 0; i < NB; ++i) e = e + quad_lane<2>(t[i]);
#pragma unroll
  for (int i = 0; i < NB; ++i) e = e + quad_lane<3>(t[i]);
  return e;
}

// The estimate with a candidate's quarters q = 2 h + b on lanes 32 h + 2 c + b
// of a wave (c = the candidate's slot, 0..15): a half-wave then holds two
// quarters of 16 candidates, whose product-table reads (rows 4 q + i, 132
// floats apart) fall in disjoint 16-bank ranges of 32.  Lane 2 c (quarter 0)
// gathers the other quarters' terms -- quarter 1 from its pair lane by a DPP
// move, quarters 2 and 3 from the upper half by a lane swap -- and adds all
// B terms in b order; the other lanes' results are not used.
template <int M>
__device__ __forceinline__ float rerank_estimate_halves(
    const uint4 cw, const typename std::conditional<M == 8, uint2, uint4>::type ww,
    const float* s_P, int q) {
  constexpr int NB = 32 / M;
  float t[NB], u[NB];
  rerank_terms<M>(cw, ww, s_P, q, t);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    // lanes 0..31 receive lane + 32's value
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[i]), __float_as_uint(t[i]),
                                                     false, false);
    u[i] = __uint_as_float(sw[1]);
  }
  float e = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) e = e + t[i];
#pragma unroll
  for (int i = 0; i < NB; ++i) e = e + dppf_xor1(t[i]);
#pragma unroll
  for (int i = 0; i < NB; ++i) e = e + u[i];
#pragma unroll
  for (int i = 0; i < NB; ++i) e = e + dppf_xor1(u[i]);
  return e;
}

// FT (at most kFusedThreshChunks chunks per unit): no separate threshold
// kernel.  Every block finds T and the tie quota from the column sums of the
// unit's chunk rows, and its chunks' offsets from block scans over the rows
// before them -- the K4a arithmetic, repeated per block (block 0 of each unit
// also writes meta); meta and coff are then not read.
template <int KPT, int CPB, int M, bool FT>
__device__ __forceinline__ void compact_rerank(
    const uint8_t* __restrict__ scores, int64_t Epad, int64_t S, int64_t E,
    const int32_t* __restrict__ meta, const uint32_t* __restrict__ coff, int chunk_stride,
    int nchunks, const float* __restrict__ ptab, const uint32_t* __restrict__ rec,
    int64_t cap, int32_t* __restrict__ cand,
    float* __restrict__ est, int64_t cstride, int64_t C, uint32_t* __restrict__ mm, int swar,
    int unit_div, const uint32_t* __restrict__ chist, int nbins, int rstride,
    int32_t* __restrict__ meta_out) {
  constexpr int CH = KPT * 256;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int c0 = blockIdx.x * CPB;
  const int nc = (CPB == 2 && c0 + 1 < nchunks) ? 2 : 1;
  __shared__ float s_P[kPtabLds];
  __shared__ uint16_t s_list[2 * CH];
  __shared__ uint2 s_w2[4];
  __shared__ uint32_t s_mm[8];
  // global reads first
  int T = 0;
  int64_t Q = 0;
  uint32_t off_c[2] = {0, 0}, tieb_c[2] = {0, 0};
  if constexpr (!FT) {
    T = meta[bh * 4 + 0];
    Q = meta[bh * 4 + 2];
  }
  uint8_t sc[2][KPT];
  uint2 raw[2] = {make_uint2(0, 0), make_uint2(0, 0)};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int chunk = c0 + (h < nc ? h : 0);
    if constexpr (!FT) {
      off_c[h] = coff[((int64_t)bh * chunk_stride + chunk) * 2 + 0];
      tieb_c[h] = coff[((int64_t)bh * chunk_stride + chunk) * 2 + 1];
    }
    const uint8_t* sp = scores + bh * Epad + (int64_t)chunk * CH + tid * KPT;
    if constexpr (KPT == 8) {
      raw[h] = load_stream(reinterpret_cast<const uint2*>(sp));
#pragma unroll
      for (int t = 0; t < 8; ++t) sc[h][t] = (uint8_t)(((t < 4) ? raw[h].x : raw[h].y) >> ((t & 3) * 8));
    } else {
      load_scores<KPT>(sp, sc[h]);
    }
  }
  {
    // table [b][j][code] (2048 floats) -> LDS rows of kPtabRow floats per subspace
    const float4* src = reinterpret_cast<const float4*>(ptab + (int64_t)bh * 2048);
    const float4 v0 = src[tid], v1 = src[tid + 256];
    reinterpret_cast<float4*>(s_P + (tid >> 5) * kPtabRow)[tid & 31] = v0;
    reinterpret_cast<float4*>(s_P + ((tid + 256) >> 5) * kPtabRow)[tid & 31] = v1;
  }
  if constexpr (FT) {
    __shared__ uint32_t s_tot[260];
    __shared__ int s_T;
    const uint32_t* hb = chist + (int64_t)bh * chunk_stride * rstride;
    // column sums as K4a: thread = (row r0, group g of 4 bins), 16-byte loads,
    // 8 rows in flight per thread, summed in registers, then LDS atomics
    s_tot[tid] = 0u;
    if (tid < 4) s_tot[256 + tid] = 0u;
    const int ng = rstride >> 2, rpp = 256 / ng;
    const int g = tid % ng, r0 = tid / ng;
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
    if (r0 < rpp) {
      const uint4* h4 = reinterpret_cast<const uint4*>(hb);
      for (int rb = r0; rb < nchunks; rb += 8 * rpp) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = rb + u * rpp;
          v[u] = h4[(int64_t)(row < nchunks ? row : nchunks - 1) * ng + g];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (rb + u * rpp < nchunks) {
            acc[0] += v[u].x;
            acc[1] += v[u].y;
            acc[2] += v[u].z;
            acc[3] += v[u].w;
          }
        }
      }
    }
    __syncthreads();
    if (r0 < rpp) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (acc[i] && 4 * g + i < nbins) atomicAdd(&s_tot[4 * g + i], acc[i]);
    }
    __syncthreads();
    if (tid < nbins && (int64_t)s_tot[tid] >= C && (int64_t)s_tot[tid + 1] < C) s_T = tid;
    __syncthreads();
    T = s_T;
    Q = C - (int64_t)s_tot[T + 1];
    if (blockIdx.x == 0 && tid == 0) {
      meta_out[bh * 4 + 0] = T;
      meta_out[bh * 4 + 1] = (int32_t)s_tot[T + 1];
      meta_out[bh * 4 + 2] = (int32_t)Q;
      meta_out[bh * 4 + 3] = (int32_t)C;
    }
    // row r = tid: ties before it and its output offset (as K4a)
    uint32_t gt = 0, eq = 0;
    if (tid < nchunks) {
      const uint32_t* hc = hb + (int64_t)tid * rstride;
      gt = (T + 1 < nbins) ? hc[T + 1] : 0u;
      eq = hc[T] - gt;
    }
    // one scan of (ties, keys above T): the chunks before this one hold
    // min(#ties before it, Q) of the kept ties
    uint2 tot;
    const uint2 ex = block_exscan2<256, false>(make_uint2(eq, gt), s_w2, tot);
    const int64_t taken = (int64_t)ex.x < Q ? (int64_t)ex.x : Q;
    // hand the two chunks' values to every thread
    __shared__ uint32_t s_co[4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (tid == c0 + (h < nc ? h : 0)) {
        s_co[2 * h] = ex.y + (uint32_t)taken;
        s_co[2 * h + 1] = ex.x;
      }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      off_c[h] = s_co[2 * h];
      tieb_c[h] = s_co[2 * h + 1];
    }
  }
  // candidate masks and counts of both chunks, one block scan
  int64_t quota[2];
  uint32_t gtm[2], eqm[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    quota[h] = Q - (int64_t)tieb_c[h];
    if (quota[h] < 0) quota[h] = 0;
    gtm[h] = 0;
    eqm[h] = 0;
    if (h < nc) {
      // keys of this thread below E: 0..KPT (one 64-bit compare per chunk)
      const int64_t rem = E - ((int64_t)(c0 + h) * CH + tid * KPT);
      const int nval = rem <= 0 ? 0 : (rem >= KPT ? KPT : (int)rem);
      score_masks<KPT>(sc[h], raw[h], T, nval, swar != 0, gtm[h], eqm[h]);
    }
  }
  // counts packed two per word: (gt, eq) of chunk 0 and of chunk 1
  uint2 tot;
  const uint2 ex = block_exscan_packed<256>(
      make_uint2((uint32_t)__popc(gtm[0]) | ((uint32_t)__popc(eqm[0]) << 16),
                 (uint32_t)__popc(gtm[1]) | ((uint32_t)__popc(eqm[1]) << 16)),
      s_w2, tot);
  const uint32_t tg0 = tot.x & 0xFFFFu, tq0 = tot.x >> 16, tg1 = tot.y & 0xFFFFu, tq1 = tot.y >> 16;
  const uint32_t nsel0 = tg0 + (uint32_t)((int64_t)tq0 < quota[0] ? tq0 : quota[0]);
  const uint32_t nsel1 = tg1 + (uint32_t)((int64_t)tq1 < quota[1] ? tq1 : quota[1]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h >= nc) continue;
    const uint32_t exw = h ? ex.y : ex.x;
    const uint32_t exg = exw & 0xFFFFu, exq = exw >> 16;
    // ties of this thread inside the quota: the lowest r of its tie keys
    const int64_t left = quota[h] - (int64_t)exq;
    const uint32_t r = left <= 0 ? 0u : (uint32_t)(left < 32 ? left : 32);
    uint32_t sel = gtm[h] | lowest_bits(eqm[h], r);
    uint32_t pos = (h ? nsel0 : 0u) + exg + (uint32_t)((int64_t)exq < quota[h] ? exq : quota[h]);
    while (sel) {
      const int t = __builtin_ctz(sel);
      s_list[pos++] = (uint16_t)((h << 14) | (tid * KPT + t));
      sel &= sel - 1u;
    }
  }
  __syncthreads();

  const uint32_t ntot = nsel0 + nsel1;
  // 4 lanes per candidate: the lane of quarter q reads the codes of
  // coordinates 32 q .. 32 q + 31 (16 B) and the w of their 32 / M
  // subspaces from the candidate's record and forms w_b p_b for them;
  // quarter 0's lane adds all B terms in b order.  Lane 32 h + 2 c + b of
  // wave w takes quarter q = 2 h + b of candidate slot 16 w + c (see
  // rerank_estimate_halves).  Up to 4 candidates per slot are fetched before
  // any is used.
  using WT = typename std::conditional<M == 8, uint2, uint4>::type;
  const int lane = tid & 63;
  const int q = 2 * (lane >> 5) + (lane & 1);
  const int slot = 16 * (tid >> 6) + ((lane >> 1) & 15);
  const uint32_t* rq = rec + (int64_t)(bh / unit_div) * cap * 32;  // the unit's KV head
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;  // order keys of this block's estimates
  for (uint32_t j0 = 0; j0 < ntot; j0 += 256) {
    uint4 cw[4];
    WT ww[4];
    int64_t pi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t j = j0 + r * 64 + slot;
      const bool has = j < ntot;
      const uint32_t ent = has ? s_list[j] : 0u;
      const int h = (int)(ent >> 14);
      pi[r] = S + (int64_t)(c0 + h) * CH + (ent & 0x3FFFu);
      // unconditional loads (idle lanes read record 0), so each round's wait
      // covers only the loads issued before it
      const uint32_t* rp = rq + (has ? pi[r] : 0) * 32;
      cw[r] = reinterpret_cast<const uint4*>(rp)[q];
      ww[r] = reinterpret_cast<const WT*>(rp + 16)[q];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (j0 + r * 64 >= ntot) break;  // uniform across the block
      const uint32_t j = j0 + r * 64 + slot;
      const float e = rerank_estimate_halves<M>(cw[r], ww[r], s_P, q);
      // the range update is unconditional (masked by selects), so the sum's
      // additions stay beside their lane moves and fold into DPP adds; only
      // quarter 0's lane holds the estimate
      const bool valid = j < ntot && q == 0;
      const uint32_t ok = order_key(e);
      kmn = min(kmn, valid ? ok : 0xFFFFFFFFu);
      kmx = max(kmx, valid ? ok : 0u);
      if (valid) {
        const uint32_t o = (j >= nsel0) ? off_c[1] + (j - nsel0) : off_c[0] + j;
        if ((int64_t)o < C) {  // always true when K4a and this kernel agree
          cand[bh * cstride + o] = (int32_t)pi[r];
          est[bh * cstride + o] = e;
        }
      }
    }
  }
  // this block's estimate range (order keys; no candidates: max key 0 < min)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, off));
    kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, off));
  }
  if ((tid & 63) == 0) { s_mm[tid >> 6] = kmn; s_mm[4 + (tid >> 6)] = kmx; }
  __syncthreads();
  if (tid < 2) {
    const int chunk = c0 + (tid < nc ? tid : 0);
    mm[((int64_t)bh * chunk_stride + chunk) * 2 + 0] = min(min(s_mm[0], s_mm[1]), min(s_mm[2], s_mm[3]));
    mm[((int64_t)bh * chunk_stride + chunk) * 2 + 1] = max(max(s_mm[4], s_mm[5]), max(s_mm[6], s_mm[7]));
  }
}

// The m = 8 separate-threshold form is held to 72 VGPRs (7 waves per SIMD, 7
// blocks per CU) by its launch bounds, one more resident block per CU than
// the 74 it would take; the other forms keep what they need (held to 72, the
// fused-threshold and m = 4 forms spill).
#define PKV_CR_PARAMS                                                                          \
  const uint8_t* __restrict__ scores, int64_t Epad, int64_t S, int64_t E,                      \
      const int32_t* __restrict__ meta, const uint32_t* __restrict__ coff, int chunk_stride,   \
      int nchunks, const float* __restrict__ ptab, const uint32_t* __restrict__ rec,           \
      int64_t cap, int32_t* __restrict__ cand, float* __restrict__ est, int64_t cstride,       \
      int64_t C, uint32_t* __restrict__ mm, int swar, int unit_div,                            \
      const uint32_t* __restrict__ chist, int nbins, int rstride, int32_t* __restrict__ meta_out
#define PKV_CR_ARGS                                                                            \
  scores, Epad, S, E, meta, coff, chunk_stride, nchunks, ptab, rec, cap, cand, est, cstride, C, \
      mm, swar, unit_div, chist, nbins, rstride, meta_out
template <int KPT, int CPB>
__global__ __launch_bounds__(256, 7) void k_compact_rerank_m8(PKV_CR_PARAMS) {
  compact_rerank<KPT, CPB, 8, false>(PKV_CR_ARGS);
}
template <int KPT, int CPB, int M, bool FT>
__global__ __launch_bounds__(256) void k_compact_rerank(PKV_CR_PARAMS) {
  compact_rerank<KPT, CPB, M, FT>(PKV_CR_ARGS);
}
#undef PKV_CR_PARAMS
#undef PKV_CR_ARGS

// ---------------------------------------------------------------------------
// K6 exact top-k over the reranked candidates ([TS] Key Contributions 2:
// Top-k selection on the compressed codes).  Order: (est desc, position asc),
// -0 == +0.  Two kernels over blocks of TK_SL candidates, no atomics on
// global memory and no cross-block waiting:
//  * k_topk_hist: every block reduces the per-chunk estimate ranges that
//    K4b+K5 wrote to this (b, h)'s minimum and maximum, bins its candidates
//    linearly between them (fp32: bin = min(2047, trunc((e - min) * 2047 /
//    (max - min))), monotone non-decreasing in e, -0 and +0 alike) and writes
//    a cumulative row #(bin >= b) of 16-bit entries (a block holds at most
//    TK_SL candidates).
//  * k_topk_select: every block sums the rows, finds the bin b1 holding rank
//    k', gathers b1's members (usually a few dozen; the counting sort in
//    k_topk_hist left each block's members contiguous), ranks them exactly
//    by (est desc, position asc) and keeps the first `remaining` -- the same
//    result in every block -- then writes its own selected candidates (bin >
//    b1, or a kept member of b1) in position order at its offset, after the
//    sinks.  A bin with more than TK_MAXMEM members is resolved instead by a
//    whole-(b, h) radix select in block 0.
// ---------------------------------------------------------------------------
constexpr int TK_SL = kTopkSlice;           // candidates per block (1024 threads x 4)
constexpr int TK_MAXMEM = kTopkMaxMembers;  // largest threshold bin ranked pairwise

__device__ __forceinline__ void range_scale(uint32_t kmin, uint32_t kmax, float& fmin,
                                            float& scale) {
  fmin = key_float(kmin);
  const float fmax = key_float(kmax);
  scale = (fmax > fmin) ? 2047.0f / (fmax - fmin) : 0.0f;
  if (!(scale < INFINITY)) scale = 0.0f;
}
__device__ __forceinline__ uint32_t est_bin(float f, float fmin, float scale) {
  return (uint32_t)fminf((f - fmin) * scale, 2047.0f);
}
// one 64-bit key per member: larger means earlier in (est desc, position asc)
__device__ __forceinline__ uint64_t member_key(uint32_t okey, uint32_t pos) {
  return ((uint64_t)okey << 32) | (uint64_t)(~pos);
}

// Whole-(b, h) exact selection by an 11 + 11 + 10-bit radix select of the
// order keys, for 1024 threads; writes sinks, positions and estimates.
__device__ void topk_radix_block(const float* __restrict__ e, const int32_t* __restrict__ cd,
                                 int C, int kprime, int S, int32_t* __restrict__ oi,
                                 float* __restrict__ oe, uint32_t* s_hist, uint2* s_w,
                                 uint32_t* s_sel) {
  const int tid = threadIdx.x;
  for (int t = tid; t < S; t += 1024) oi[t] = t;
  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)kprime;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass], nb = 1 << widths[pass];
    for (int i = tid; i < nb; i += 1024) s_hist[i] = 0;
    __syncthreads();
#pragma nounroll
    for (int c = tid; c < C; c += 1024) {
      const uint32_t o = order_key(e[c]);
      if ((o & pmask) == prefix) atomicAdd(&s_hist[(o >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    const int bpt = nb / 1024;
    uint32_t mine = 0;
    for (int q = 0; q < bpt; ++q) mine += s_hist[nb - 1 - (tid * bpt + q)];
    uint2 tot;
    const uint2 ex = block_exscan2<1024>(make_uint2(mine, 0), s_w, tot);
    uint32_t above = ex.x;
    for (int q = 0; q < bpt; ++q) {
      const int bin = nb - 1 - (tid * bpt + q);
      const uint32_t cnt = s_hist[bin];
      if (above < remaining && remaining <= above + cnt) { s_sel[0] = bin; s_sel[1] = remaining - above; }
      above += cnt;
    }
    __syncthreads();
    prefix |= s_sel[0] << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    remaining = s_sel[1];
    __syncthreads();
  }
  const uint32_t thr = prefix;
  const int per = (C + 1023) / 1024;
  const int c0 = tid * per;
  const int c1 = (c0 + per < C) ? c0 + per : C;
  uint32_t ngt = 0, neq = 0;
#pragma nounroll
  for (int c = c0; c < c1; ++c) {
    const uint32_t o = order_key(e[c]);
    ngt += o > thr;
    neq += o == thr;
  }
  uint2 tot;
  const uint2 ex = block_exscan2<1024>(make_uint2(ngt, neq), s_w, tot);
  uint32_t pos = ex.x + (ex.y < remaining ? ex.y : remaining);
  uint32_t tie_seen = ex.y;
#pragma nounroll
  for (int c = c0; c < c1; ++c) {
    const float ev = e[c];
    const uint32_t o = order_key(ev);
    bool sel = o > thr;
    if (o == thr) { sel = tie_seen < remaining; ++tie_seen; }
    if (sel && pos < (uint32_t)kprime) {  // bound holds by construction
      oi[S + pos] = cd[c];
      if (oe) oe[pos] = ev;
      ++pos;
    }
  }
}

__device__ __forceinline__ void topk_hist_slice(
    const float* __restrict__ est, int64_t cstride, int C, int P,
    const uint32_t* __restrict__ mmc, int chunk_stride, int nchunks,
    uint16_t* __restrict__ rows, uint32_t* __restrict__ range, uint2* __restrict__ sorted,
    int p) {
  const int bh = blockIdx.y, tid = threadIdx.x;
  const float* e = est + bh * cstride;
  __shared__ uint32_t s_hist[2048];
  __shared__ uint2 s_w[16];
  __shared__ uint32_t s_r[32];
  // this block's candidates first (independent of the range), 4 at a time
  // at an index clamped into the row of cstride (a multiple of 64); entries
  // past C are not used
  const int c0 = p * TK_SL + tid * 4;
  const float4 fv = *reinterpret_cast<const float4*>(e + min(c0, (int)cstride - 4));
  const float f[4] = {fv.x, fv.y, fv.z, fv.w};
  // this (b, h)'s estimate range from the per-chunk ranges
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  const uint2* mb = reinterpret_cast<const uint2*>(mmc + (int64_t)bh * chunk_stride * 2);
  for (int c = tid; c < nchunks; c += 1024) {
    const uint2 r = mb[c];
    kmin = min(kmin, r.x);
    kmax = max(kmax, r.y);
  }
  for (int i = tid; i < 2048; i += 1024) s_hist[i] = 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if ((tid & 63) == 0) { s_r[tid >> 6] = kmin; s_r[16 + (tid >> 6)] = kmax; }
  __syncthreads();
  kmin = s_r[0];
  kmax = s_r[16];
#pragma unroll
  for (int w = 1; w < 16; ++w) { kmin = min(kmin, s_r[w]); kmax = max(kmax, s_r[16 + w]); }
  if (p == 0 && tid == 0) { range[2 * bh] = kmin; range[2 * bh + 1] = kmax; }
  float fmin, scale;
  range_scale(kmin, kmax, fmin, scale);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (c0 + r < C) atomicAdd(&s_hist[est_bin(f[r], fmin, scale)], 1u);
  __syncthreads();
  // cumulative row #(bin >= b); thread t owns bins 2047 - 2t and 2046 - 2t
  const uint32_t hh = s_hist[2047 - 2 * tid], hl = s_hist[2046 - 2 * tid];
  uint2 tot;
  const uint2 ex = block_exscan2<1024, false>(make_uint2(hh + hl, 0), s_w, tot);
  // 16-bit entries: a slice holds at most TK_SL candidates
  uint16_t* row = rows + ((int64_t)bh * P + p) * 2048;
  row[2047 - 2 * tid] = (uint16_t)(ex.x + hh);
  row[2046 - 2 * tid] = (uint16_t)(ex.x + hh + hl);
  // counting sort of the block's candidates by bin, descending: bin b's
  // entries start at #(bin > b), so a bin's members are contiguous
  s_hist[2047 - 2 * tid] = ex.x;
  s_hist[2046 - 2 * tid] = ex.x + hh;
  __syncthreads();
  // sorted in LDS, then written out coalesced
  __shared__ uint2 s_sorted[TK_SL];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (c0 + r < C) {
      const uint32_t slot = atomicAdd(&s_hist[est_bin(f[r], fmin, scale)], 1u);
      s_sorted[slot] = make_uint2(order_key(f[r]), (uint32_t)(c0 + r));
    }
  }
  __syncthreads();
  uint2* out = sorted + ((int64_t)bh * P + p) * TK_SL;
  const int nb = min(TK_SL, C - p * TK_SL);  // the block's candidates
  for (int i = tid; i < nb; i += 1024) out[i] = s_sorted[i];
}

// cmeta (optional): this unit's candidate count is cmeta[bh * 4 + 3], at
// most P slices; the grid may be narrower than the unit's slices, each block
// then takes slices blockIdx.x, blockIdx.x + gridDim.x, ...
__global__ __launch_bounds__(1024) void k_topk_hist(
    const float* __restrict__ est, int64_t cstride, int C, int P,
    const uint32_t* __restrict__ mmc, int chunk_stride, int nchunks,
    uint16_t* __restrict__ rows, uint32_t* __restrict__ range, uint2* __restrict__ sorted,
    const int32_t* __restrict__ cmeta) {
  int Pu = P;
  if (cmeta) {
    C = cmeta[blockIdx.y * 4 + 3];
    Pu = (C + TK_SL - 1) / TK_SL;
  }
  for (int p = blockIdx.x; p < Pu; p += gridDim.x) {
    topk_hist_slice(est, cstride, C, P, mmc, chunk_stride, nchunks, rows, range, sorted, p);
    __syncthreads();  // LDS is reused by the next slice
  }
}

__device__ __forceinline__ void topk_select_slice(
    const float* __restrict__ est, const int32_t* __restrict__ cand, int64_t cstride, int C,
    int kprime, int S, int k, int P, int Pu, const uint32_t* __restrict__ range,
    const uint16_t* __restrict__ rows, const uint2* __restrict__ sorted,
    int32_t* __restrict__ tkmeta, int32_t* __restrict__ out_idx, float* __restrict__ out_est,
    int p) {
  // rows are laid out for P slices; Pu of them are this unit's
  const int bh = blockIdx.y, tid = threadIdx.x;
  const float* e = est + bh * cstride;
  const int32_t* cd = cand + bh * cstride;
  int32_t* oi = out_idx + (int64_t)bh * k;
  __shared__ uint32_t s_hist[2049];
  __shared__ uint64_t s_mem[TK_MAXMEM];
  __shared__ uint32_t s_pref[1024];
  __shared__ uint32_t s_start[1024];
  __shared__ uint32_t s_bits[TK_SL / 32];
  __shared__ uint2 s_w[16];
  __shared__ uint32_t s_sel[4];
  // this block's candidates: loads go out first
  const int c0 = p * TK_SL + tid * 4;
  const int cl = min(c0, (int)cstride - 4);  // in the row; entries past C unused
  const float4 fv = *reinterpret_cast<const float4*>(e + cl);
  const int4 cv = *reinterpret_cast<const int4*>(cd + cl);
  const float f[4] = {fv.x, fv.y, fv.z, fv.w};
  const int32_t ci[4] = {cv.x, cv.y, cv.z, cv.w};
  // resolve (every block of this (b, h) does it, identically): the bin b1
  // holding rank k' and the kept members of b1
  const uint16_t* rb = rows + (int64_t)bh * P * 2048;
  for (int b = tid; b < 2048; b += 1024) {
    uint32_t acc = 0;
    for (int q0 = 0; q0 < Pu; q0 += 8) {  // 8 rows in flight
      uint32_t v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = (q0 + r < Pu) ? rb[(int64_t)(q0 + r) * 2048 + b] : 0u;
#pragma unroll
      for (int r = 0; r < 8; ++r) acc += v[r];
    }
    s_hist[b] = acc;
  }
  if (tid == 0) { s_hist[2048] = 0; s_sel[2] = 0; s_sel[3] = 0; }
  if (tid < TK_SL / 32) s_bits[tid] = 0;
  __syncthreads();
  for (int b = tid; b < 2048; b += 1024)
    if (s_hist[b] >= (uint32_t)kprime && s_hist[b + 1] < (uint32_t)kprime) s_sel[0] = b;
  __syncthreads();
  const uint32_t b1 = s_sel[0];
  const uint32_t above_tot = s_hist[b1 + 1];
  const uint32_t M = s_hist[b1] - above_tot;
  const uint32_t remaining = (uint32_t)kprime - above_tot;
  if (M > (uint32_t)TK_MAXMEM) {
    // tie-heavy threshold bin: block 0 selects exactly for the whole (b, h)
    if (p == 0) {
      __syncthreads();
      topk_radix_block(e, cd, C, kprime, S, oi,
                       out_est ? out_est + (int64_t)bh * kprime : nullptr, s_hist, s_w, s_sel);
    }
    if (p == 0 && tid == 0) {
      tkmeta[bh * 4 + 0] = (int32_t)b1;
      tkmeta[bh * 4 + 1] = (int32_t)remaining;
      tkmeta[bh * 4 + 2] = 1;
      tkmeta[bh * 4 + 3] = (int32_t)M;
    }
    return;
  }
  // gather b1's members: block q holds them contiguously in its sorted array
  // from #(bin > b1) on; also the rows-above counts of the blocks before p
  uint32_t above_before = 0;
  {
    const int q = tid;
    uint32_t nq = 0, sq = 0;
    if (q < Pu) {
      sq = (b1 + 1 < 2048) ? rb[(int64_t)q * 2048 + b1 + 1] : 0u;
      nq = rb[(int64_t)q * 2048 + b1] - sq;
    }
    uint2 tt;
    const uint2 ex = block_exscan2<1024, false>(make_uint2(nq, q < p ? sq : 0u), s_w, tt);
    s_pref[q] = ex.x;
    s_start[q] = sq;
    above_before = tt.y;
  }
  __syncthreads();
  for (uint32_t j = tid; j < M; j += 1024) {
    int lo = 0, hi = Pu - 1;  // last block q with s_pref[q] <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= j) lo = mid; else hi = mid - 1;
    }
    const uint2 pr = sorted[((int64_t)bh * P + lo) * TK_SL + s_start[lo] + (j - s_pref[lo])];
    s_mem[j] = member_key(pr.x, pr.y);
  }
  __syncthreads();
  // rank the members by (est desc, position asc); keep the first `remaining`
  for (uint32_t j = tid; j < M; j += 1024) {
    const uint64_t mj = s_mem[j];
    const uint32_t cj = ~(uint32_t)mj;
    uint32_t rank = 0;
#pragma unroll 8
    for (uint32_t q = 0; q < M; ++q) rank += (s_mem[q] > mj) ? 1u : 0u;
    if (rank < remaining) {
      const uint32_t qb = cj / TK_SL;
      if (qb < (uint32_t)p) atomicAdd(&s_sel[3], 1u);
      else if (qb == (uint32_t)p) atomicOr(&s_bits[(cj % TK_SL) >> 5], 1u << (cj & 31));
    }
  }
  __syncthreads();
  if (p == 0) {
    for (int t = tid; t < S; t += 1024) oi[t] = t;
    if (tid == 0) {
      tkmeta[bh * 4 + 0] = (int32_t)b1;
      tkmeta[bh * 4 + 1] = (int32_t)remaining;
      tkmeta[bh * 4 + 2] = 0;
      tkmeta[bh * 4 + 3] = (int32_t)M;
    }
  }
  // ordered compaction of this block's selection at its offset
  float fmin, scale;
  range_scale(range[2 * bh], range[2 * bh + 1], fmin, scale);
  uint32_t selm = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = c0 + r;
    if (c < C) {
      const uint32_t bn = est_bin(f[r], fmin, scale);
      if (bn > b1 || (bn == b1 && ((s_bits[(c % TK_SL) >> 5] >> (c & 31)) & 1u)))
        selm |= 1u << r;
    }
  }
  uint2 tot;
  const uint2 ex = block_exscan2<1024, false>(make_uint2((uint32_t)__popc(selm), 0), s_w, tot);
  uint32_t pos = above_before + s_sel[3] + ex.x;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (((selm >> r) & 1u) && pos < (uint32_t)kprime) {  // bound holds by construction
      oi[S + pos] = ci[r];
      if (out_est) out_est[(int64_t)bh * kprime + pos] = f[r];
      ++pos;
    }
  }
}

// cmeta as for k_topk_hist; every slice a block takes repeats the resolve
__global__ __launch_bounds__(1024) void k_topk_select(
    const float* __restrict__ est, const int32_t* __restrict__ cand, int64_t cstride, int C,
    int kprime, int S, int k, int P, const uint32_t* __restrict__ range,
    const uint16_t* __restrict__ rows, const uint2* __restrict__ sorted,
    int32_t* __restrict__ tkmeta, int32_t* __restrict__ out_idx, float* __restrict__ out_est,
    const int32_t* __restrict__ cmeta) {
  int Pu = P;
  if (cmeta) {
    C = cmeta[blockIdx.y * 4 + 3];
    Pu = (C + TK_SL - 1) / TK_SL;
  }
  for (int p = blockIdx.x; p < Pu; p += gridDim.x) {
    topk_select_slice(est, cand, cstride, C, kprime, S, k, P, Pu, range, rows, sorted, tkmeta,
                      out_idx, out_est, p);
    __syncthreads();  // LDS is reused by the next slice
  }
}

// k_topk_select for P <= MAXP slices: every global read the resolve needs
// goes out at once (this block's candidates, the range, and the rows of
// bins 2t, 2t+1 of every slice, kept in registers), so b1's per-slice
// counts come from the registers of the threads owning b1 and b1 + 1, and
// only the gather of b1's members waits on a second round of loads.
template <int MAXP>
__global__ __launch_bounds__(1024) void k_topk_select_few(
    const float* __restrict__ est, const int32_t* __restrict__ cand, int64_t cstride, int C,
    int kprime, int S, int k, int P, const uint32_t* __restrict__ range,
    const uint16_t* __restrict__ rows, const uint2* __restrict__ sorted,
    int32_t* __restrict__ tkmeta, int32_t* __restrict__ out_idx, float* __restrict__ out_est) {
  const int p = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const float* e = est + bh * cstride;
  const int32_t* cd = cand + bh * cstride;
  int32_t* oi = out_idx + (int64_t)bh * k;
  __shared__ uint32_t s_hist[2049];
  __shared__ uint64_t s_mem[TK_MAXMEM];
  __shared__ uint32_t s_cnt[MAXP], s_start[MAXP], s_pref[MAXP + 1], s_cnt16[16];
  __shared__ uint32_t s_bits[TK_SL / 32];
  __shared__ uint2 s_w[16];
  __shared__ uint32_t s_sel[4];
  // All loads are unconditional (one wait covers them all): rows past P
  // re-read row P - 1 and are masked; this block's candidates are read 4 at
  // a time at an index clamped into the row of cstride (a multiple of 64).
  const uint16_t* rb = rows + (int64_t)bh * P * 2048;
  // rows of 16-bit entries: thread t holds bins 2t (low half) and 2t + 1
  uint32_t rv[MAXP];
#pragma unroll
  for (int q = 0; q < MAXP; ++q)
    rv[q] = reinterpret_cast<const uint32_t*>(rb + (int64_t)(q < P ? q : P - 1) * 2048)[tid];
  const int c0 = p * TK_SL + tid * 4;
  const int cl = min(c0, (int)cstride - 4);
  const float4 fv = *reinterpret_cast<const float4*>(e + cl);
  const int4 cv = *reinterpret_cast<const int4*>(cd + cl);
  const float f[4] = {fv.x, fv.y, fv.z, fv.w};
  const int32_t ci[4] = {cv.x, cv.y, cv.z, cv.w};
  const uint32_t kmin = range[2 * bh], kmax = range[2 * bh + 1];
  uint32_t a0 = 0, a1 = 0;
#pragma unroll
  for (int q = 0; q < MAXP; ++q) {
    if (q < P) { a0 += rv[q] & 0xFFFFu; a1 += rv[q] >> 16; }
  }
  s_hist[2 * tid] = a0;
  s_hist[2 * tid + 1] = a1;
  if (tid == 0) { s_hist[2048] = 0; s_sel[3] = 0; }
  if (tid < TK_SL / 32) s_bits[tid] = 0;
  // #(bin >= b) falls as b grows and is C >= k' at b = 0, so b1, the last
  // bin where it is still >= k', is the number of such bins minus one:
  // counted by ballots, summed over the waves
  {
    const uint32_t nge = (uint32_t)__popcll(__ballot(a0 >= (uint32_t)kprime)) +
                         (uint32_t)__popcll(__ballot(a1 >= (uint32_t)kprime));
    if ((tid & 63) == 0) s_cnt16[tid >> 6] = nge;
  }
  __syncthreads();
  uint32_t b1 = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) b1 += s_cnt16[w];
  b1 -= 1u;
  const uint32_t above_tot = s_hist[b1 + 1];
  const uint32_t M = s_hist[b1] - above_tot;
  const uint32_t remaining = (uint32_t)kprime - above_tot;
  if (M > (uint32_t)TK_MAXMEM) {
    if (p == 0) {
      __syncthreads();  // s_hist is reused below
      topk_radix_block(e, cd, C, kprime, S, oi,
                       out_est ? out_est + (int64_t)bh * kprime : nullptr, s_hist, s_w, s_sel);
      if (tid == 0) {
        tkmeta[bh * 4 + 0] = (int32_t)b1;
        tkmeta[bh * 4 + 1] = (int32_t)remaining;
        tkmeta[bh * 4 + 2] = 1;
        tkmeta[bh * 4 + 3] = (int32_t)M;
      }
    }
    return;
  }
  // per slice q: #(bin >= b1) and #(bin > b1), from the owners' registers
  // (separate loops for the even and odd bin keep rv[] in registers)
  if (tid == (int)(b1 >> 1)) {
    if (b1 & 1u) {
#pragma unroll
      for (int q = 0; q < MAXP; ++q)
        if (q < P) s_cnt[q] = rv[q] >> 16;
    } else {
#pragma unroll
      for (int q = 0; q < MAXP; ++q)
        if (q < P) s_cnt[q] = rv[q] & 0xFFFFu;
    }
  }
  if (b1 + 1 < 2048u) {
    if (tid == (int)((b1 + 1) >> 1)) {
      if ((b1 + 1) & 1u) {
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
          if (q < P) s_start[q] = rv[q] >> 16;
      } else {
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
          if (q < P) s_start[q] = rv[q] & 0xFFFFu;
      }
    }
  } else if (tid < P) {
    s_start[tid] = 0;
  }
  __syncthreads();
  if (tid < 64) {
    // wave 0: prefix of the per-slice member counts, and #(bin > b1) in the
    // slices before p
    const uint32_t nq = (tid < P) ? s_cnt[tid] - s_start[tid] : 0u;
    const uint32_t sb = (tid < P && tid < p) ? s_start[tid] : 0u;
    const uint32_t inc = wave_incl_scan(nq), sbs = wave_incl_scan(sb);
    if (tid < P) s_pref[tid + 1] = inc;
    if (tid == 0) s_pref[0] = 0;
    if (tid == 63) s_sel[2] = sbs;
  }
  __syncthreads();
  const uint32_t above_before = s_sel[2];
  // b1's members: slice q holds them contiguously in its sorted array from
  // #(bin > b1) on
  for (uint32_t j = tid; j < M; j += 1024) {
    // the last slice q with s_pref[q] <= j (s_pref does not fall, s_pref[0] = 0)
    int q = 0;
#pragma unroll
    for (int qq = 1; qq < MAXP; ++qq) q += (qq < P && s_pref[qq] <= j) ? 1 : 0;
    const uint2 pr = sorted[((int64_t)bh * P + q) * TK_SL + s_start[q] + (j - s_pref[q])];
    s_mem[j] = member_key(pr.x, pr.y);
  }
  __syncthreads();
  // rank the members by (est desc, position asc); keep the first `remaining`
  for (uint32_t j = tid; j < M; j += 1024) {
    const uint64_t mj = s_mem[j];
    const uint32_t cj = ~(uint32_t)mj;
    uint32_t rank = 0;
#pragma unroll 8
    for (uint32_t q = 0; q < M; ++q) rank += (s_mem[q] > mj) ? 1u : 0u;
    if (rank < remaining) {
      const uint32_t qb = cj / TK_SL;
      if (qb < (uint32_t)p) atomicAdd(&s_sel[3], 1u);
      else if (qb == (uint32_t)p) atomicOr(&s_bits[(cj % TK_SL) >> 5], 1u << (cj & 31));
    }
  }
  __syncthreads();
  if (p == 0) {
    for (int t = tid; t < S; t += 1024) oi[t] = t;
    if (tid == 0) {
      tkmeta[bh * 4 + 0] = (int32_t)b1;
      tkmeta[bh * 4 + 1] = (int32_t)remaining;
      tkmeta[bh * 4 + 2] = 0;
      tkmeta[bh * 4 + 3] = (int32_t)M;
    }
  }
  // ordered compaction of this block's selection at its offset
  float fmin, scale;
  range_scale(kmin, kmax, fmin, scale);
  uint32_t selm = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = c0 + r;
    if (c < C) {
      const uint32_t bn = est_bin(f[r], fmin, scale);
      if (bn > b1 || (bn == b1 && ((s_bits[(c % TK_SL) >> 5] >> (c & 31)) & 1u)))
        selm |= 1u << r;
    }
  }
  uint2 tot;
  const uint2 ex = block_exscan2<1024, false>(make_uint2((uint32_t)__popc(selm), 0), s_w, tot);
  uint32_t pos = above_before + s_sel[3] + ex.x;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (((selm >> r) & 1u) && pos < (uint32_t)kprime) {  // bound holds by construction
      oi[S + pos] = ci[r];
      if (out_est) out_est[(int64_t)bh * kprime + pos] = f[r];
      ++pos;
    }
  }
}

// ---------------------------------------------------------------------------
// K6, single kernel for C <= TK_SL * MAXS candidates per (b, h).  Every
// block loads all C estimates of its (b, h) (at most 256 KB, L2-resident)
// and resolves the selection by itself -- the same result in every block:
// range = min/max of the estimates, linear 2048-bin histogram (same binning
// as above), cumulative counts, the bin b1 holding rank k', exact ranking of
// b1's members by (est desc, position asc).  Then block p writes the
// selected candidates of its slice [p TK_SL, (p + 1) TK_SL) in position
// order at offset S + #(selected before the slice).  A bin with more than
// TK_MAXMEM members goes to the whole-(b, h) radix select in block 0.
// ---------------------------------------------------------------------------
template <int MAXS>
__global__ __launch_bounds__(1024) void k_topk_fused(
    const float* __restrict__ est, const int32_t* __restrict__ cand, int64_t cstride, int C,
    int kprime, int S, int k, int32_t* __restrict__ tkmeta, int32_t* __restrict__ out_idx,
    float* __restrict__ out_est) {
  const int p = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const float* e = est + bh * cstride;
  const int32_t* cd = cand + bh * cstride;
  int32_t* oi = out_idx + (int64_t)bh * k;
  __shared__ uint32_t s_hist[2049];
  __shared__ uint64_t s_mem[TK_MAXMEM];
  __shared__ uint32_t s_bits[MAXS * TK_SL / 32];
  __shared__ uint2 s_w[16];
  __shared__ uint32_t s_r[32];
  __shared__ uint32_t s_sel[4];
  // all estimates: thread t holds candidates sl TK_SL + 4 t .. + 3 of every slice sl
  // (unconditional loads, 4 at a time at an index clamped into the row of
  // cstride, a multiple of 64; entries past C are not used)
  float f[MAXS][4];
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl) {
    const int c0 = sl * TK_SL + tid * 4;
    const float4 t = *reinterpret_cast<const float4*>(e + min(c0, (int)cstride - 4));
    f[sl][0] = t.x; f[sl][1] = t.y; f[sl][2] = t.z; f[sl][3] = t.w;
  }
  const int cp = p * TK_SL + tid * 4;
  const int4 cv = *reinterpret_cast<const int4*>(cd + min(cp, (int)cstride - 4));
  const int32_t ci[4] = {cv.x, cv.y, cv.z, cv.w};
  for (int i = tid; i < 2049; i += 1024) s_hist[i] = 0;
  for (int i = tid; i < MAXS * TK_SL / 32; i += 1024) s_bits[i] = 0;
  if (tid < 4) s_sel[tid] = 0;
  // range of the estimates (order keys)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (sl * TK_SL + tid * 4 + r < C) {
        const uint32_t o = order_key(f[sl][r]);
        kmin = min(kmin, o);
        kmax = max(kmax, o);
      }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if ((tid & 63) == 0) { s_r[tid >> 6] = kmin; s_r[16 + (tid >> 6)] = kmax; }
  __syncthreads();
  kmin = s_r[0];
  kmax = s_r[16];
#pragma unroll
  for (int w = 1; w < 16; ++w) { kmin = min(kmin, s_r[w]); kmax = max(kmax, s_r[16 + w]); }
  float fmin, scale;
  range_scale(kmin, kmax, fmin, scale);
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (sl * TK_SL + tid * 4 + r < C) atomicAdd(&s_hist[est_bin(f[sl][r], fmin, scale)], 1u);
  __syncthreads();
  {
    // cumulative #(bin >= b); thread t owns bins 2047 - 2t and 2046 - 2t
    const uint32_t hh = s_hist[2047 - 2 * tid], hl = s_hist[2046 - 2 * tid];
    uint2 tot;
    const uint2 ex = block_exscan2<1024>(make_uint2(hh + hl, 0), s_w, tot);
    s_hist[2047 - 2 * tid] = ex.x + hh;
    s_hist[2046 - 2 * tid] = ex.x + hh + hl;
  }
  __syncthreads();
  for (int b = tid; b < 2048; b += 1024)
    if (s_hist[b] >= (uint32_t)kprime && s_hist[b + 1] < (uint32_t)kprime) s_sel[0] = b;
  __syncthreads();
  const uint32_t b1 = s_sel[0];
  const uint32_t above_tot = s_hist[b1 + 1];
  const uint32_t M = s_hist[b1] - above_tot;
  const uint32_t remaining = (uint32_t)kprime - above_tot;
  if (M > (uint32_t)TK_MAXMEM) {
    if (p == 0) {
      __syncthreads();  // s_hist is reused below
      topk_radix_block(e, cd, C, kprime, S, oi,
                       out_est ? out_est + (int64_t)bh * kprime : nullptr, s_hist, s_w, s_sel);
      if (tid == 0) {
        tkmeta[bh * 4 + 0] = (int32_t)b1;
        tkmeta[bh * 4 + 1] = (int32_t)remaining;
        tkmeta[bh * 4 + 2] = 1;
        tkmeta[bh * 4 + 3] = (int32_t)M;
      }
    }
    return;
  }
  // b1's members, then their exact ranks; kept members are marked in s_bits
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = sl * TK_SL + tid * 4 + r;
      if (c < C && est_bin(f[sl][r], fmin, scale) == b1) {
        const uint32_t slot = atomicAdd(&s_sel[2], 1u);
        s_mem[slot] = member_key(order_key(f[sl][r]), (uint32_t)c);
      }
    }
  __syncthreads();
  for (uint32_t j = tid; j < M; j += 1024) {
    const uint64_t mj = s_mem[j];
    const uint32_t cj = ~(uint32_t)mj;
    uint32_t rank = 0;
#pragma unroll 8
    for (uint32_t q = 0; q < M; ++q) rank += (s_mem[q] > mj) ? 1u : 0u;
    if (rank < remaining) atomicOr(&s_bits[cj >> 5], 1u << (cj & 31));
  }
  __syncthreads();
  // selected flags: count those of the slices before p, keep this slice's
  uint32_t before = 0, selm = 0;
  float fo[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = sl * TK_SL + tid * 4 + r;
      if (c < C && sl <= p) {
        const uint32_t bn = est_bin(f[sl][r], fmin, scale);
        const bool sel = bn > b1 || (bn == b1 && ((s_bits[c >> 5] >> (c & 31)) & 1u));
        if (sl < p) before += sel ? 1u : 0u;
        else if (sel) selm |= 1u << r;
      }
      if (sl == p) fo[r] = f[sl][r];
    }
  uint2 tot;
  const uint2 ex = block_exscan2<1024>(make_uint2((uint32_t)__popc(selm), before), s_w, tot);
  uint32_t pos = tot.y + ex.x;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (((selm >> r) & 1u) && pos < (uint32_t)kprime) {  // bound holds by construction
      oi[S + pos] = ci[r];
      if (out_est) out_est[(int64_t)bh * kprime + pos] = fo[r];
      ++pos;
    }
  }
  if (p == 0) {
    for (int t = tid; t < S; t += 1024) oi[t] = t;
    if (tid == 0) {
      tkmeta[bh * 4 + 0] = (int32_t)b1;
      tkmeta[bh * 4 + 1] = (int32_t)remaining;
      tkmeta[bh * 4 + 2] = 0;
      tkmeta[bh * 4 + 3] = (int32_t)M;
    }
  }
}

// ---------------------------------------------------------------------------
// Small-N retrieval in one kernel ([TS] Two-Stage GPU-Native Retrieval
// Pipeline, every stage): one 1024-thread block per retrieval unit (a (b, KV
// head); shared retrieval) encodes the keys appended since the last
// retrieval, prepares the query, scans the ids, finds the threshold, lists
// the candidates in index order, reranks them and selects the exact top-k,
// with block barriers between the stages instead of kernel boundaries.  Each
// stage is the fp32 operation sequence of its multi-kernel counterpart, and
// the workspace receives the same vote table, yq, scores, threshold meta,
// candidates and estimates.  For at most kSmallTopkSlices * 4096 candidates
// (the top-k holds every estimate in registers).  Opt-in: one block
// serialises every dependent memory round trip of the stages (query, ids,
// scores, candidates, records, estimates), which costs more than the kernel
// boundaries it removes, from 4K keys per unit up.
// ---------------------------------------------------------------------------
template <typename T, int M>
__global__ __launch_bounds__(1024) void k_retrieve_small(
    const T* __restrict__ Q, int n_kv_heads, int G, float invG, SignMask sg, float c, int rho,
    Tiers tw, AppendJob app, const uint4* __restrict__ ids, const uint32_t* __restrict__ rec,
    int64_t cap, int64_t S, int64_t E, int64_t C, int kprime, int k, int nbins,
    uint8_t* __restrict__ lut_out, float* __restrict__ yq_out, uint8_t* __restrict__ scores,
    int64_t Epad, int32_t* __restrict__ meta, int32_t* __restrict__ cand, float* __restrict__ est,
    int64_t cstride, int32_t* __restrict__ out_idx, float* __restrict__ out_est) {
  constexpr int MAXS = kSmallTopkSlices;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = bh / n_kv_heads, h = bh - b * n_kv_heads, Hq = n_kv_heads * G;
  __shared__ float s_yq[128];
  __shared__ float s_lv[8];  // codebook levels for the product table
  __shared__ uint8_t s_lut[16 * 256];
  __shared__ float s_P[kPtabLds];
  __shared__ uint32_t s_wh[16][256];  // per-wave score histograms, then the top-k bins
  __shared__ uint32_t s_ge[257];
  __shared__ uint2 s_w[16];
  __shared__ uint32_t s_sel[4];
  __shared__ uint32_t s_r[32];
  __shared__ uint64_t s_mem[TK_MAXMEM];
  __shared__ uint32_t s_bits[MAXS * TK_SL / 32];

  // (1) appended keys: 16 lanes per key into the index, before the scan reads
  // them (the barriers below order this block's stores before its loads)
  if ((tid >> 4) < app.n)
    encode_key<T, M>((const T*)app.K, app.rows_per_head, bh, tid >> 4, app.lo + (tid >> 4),
                     app.cap, app.ids, app.rec, sg, c, tid & 15);
  // (2) query: mean of the G query rows (summed in head order), SRHT
  if (tid < 16) {
    const int sub = tid;
    const T* q0 = Q + ((int64_t)(b * Hq + h * G) << 7) + sub * 8;
    float x[8];
    load8(q0, x);
    for (int g = 1; g < G; ++g) {
      float xg[8];
      load8(q0 + ((int64_t)g << 7), xg);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = x[j] + xg[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = x[j] * invG;
    srht16(x, sign_byte_of(sg, sub), sub, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) s_yq[sub * 8 + j] = x[j];
    reinterpret_cast<float4*>(yq_out + (int64_t)bh * 128 + sub * 8)[0] =
        make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(yq_out + (int64_t)bh * 128 + sub * 8)[1] =
        make_float4(x[4], x[5], x[6], x[7]);
  }
  if (tid == 0) {
#pragma unroll
    for (int l = 0; l < 8; ++l) s_lv[l] = cb_level<M>(l);
  }
  for (int i = tid; i < 16 * 256; i += 1024) (&s_wh[0][0])[i] = 0u;
  __threadfence_block();
  __syncthreads();
  // signed product table (rows of kPtabRow floats) and the vote table, row
  // s = wave s
  for (int e = tid; e < 2048; e += 1024) {
    const float pr = s_lv[e & 7] * s_yq[e >> 4];
    s_P[(e >> 7) * kPtabRow + (e & 127)] = (e & 8) ? -pr : pr;
  }
  {
    const uint32_t word = vote_table_word<M>(s_yq, wv, lane, rho, tw);
    reinterpret_cast<uint32_t*>(s_lut)[wv * 64 + lane] = word;
    reinterpret_cast<uint32_t*>(lut_out + (int64_t)bh * 4096)[wv * 64 + lane] = word;
  }
  __syncthreads();

  // (3) vote scan over the eligible keys [S, S + E): score bytes out, zeros by
  // wave ballot, other scores by per-wave LDS atomics
  const uint4* src = ids + (int64_t)bh * cap + S;
  uint8_t* dst = scores + (int64_t)bh * Epad;
  {
    constexpr int U = 8;  // keys per thread in flight
    uint32_t zeros = 0;
    for (int64_t base = 0; base < E; base += 1024 * U) {
      uint4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t p = base + u * 1024 + tid;
        x[u] = src[p < E ? p : E - 1];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t p = base + u * 1024 + tid;
        const bool valid = p < E;
        const uint32_t w4[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
        uint32_t sc = 0;
#pragma unroll
        for (int bb = 0; bb < 16; ++bb)
          sc += s_lut[bb * 256 + ((w4[bb >> 2] >> ((bb & 3) * 8)) & 0xFFu)];
        zeros += (uint32_t)__popcll(__ballot(valid && sc == 0));
        if (valid) {
          dst[p] = (uint8_t)sc;
          if (sc != 0) atomicAdd(&s_wh[wv][sc], 1u);
        }
      }
    }
    if (lane == 0) s_wh[wv][0] = zeros;
  }
  __threadfence_block();
  __syncthreads();

  // (4) threshold: Tv = the largest v with #(score >= v) >= C, ties quota
  // Qt = C - #(score > Tv)
  if (tid < 256) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) a += s_wh[w][tid];
    s_ge[tid] = a;
  }
  __syncthreads();
  if (wv == 0) {
    uint32_t hc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) hc[r] = s_ge[4 * lane + r];
    const uint32_t loc = hc[0] + hc[1] + hc[2] + hc[3];
    uint32_t inc = loc;  // sum over lanes >= this one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_down(inc, off);
      if (lane + off < 64) inc += t;
    }
    const uint32_t g3 = inc - loc + hc[3], g2 = g3 + hc[2], g1 = g2 + hc[1], g0 = g1 + hc[0];
    s_ge[4 * lane + 0] = g0;
    s_ge[4 * lane + 1] = g1;
    s_ge[4 * lane + 2] = g2;
    s_ge[4 * lane + 3] = g3;
    if (lane == 0) s_ge[256] = 0u;
  }
  __syncthreads();
  if (tid < 256 && (int64_t)s_ge[tid] >= C && (int64_t)s_ge[tid + 1] < C) s_sel[0] = (uint32_t)tid;
  __syncthreads();
  const int Tv = (int)s_sel[0];
  const int64_t n_gt = s_ge[Tv + 1];
  const int64_t Qt = C - n_gt;
  if (tid == 0) {
    meta[bh * 4 + 0] = Tv;
    meta[bh * 4 + 1] = (int32_t)n_gt;
    meta[bh * 4 + 2] = (int32_t)Qt;
    meta[bh * 4 + 3] = (int32_t)C;
  }

  // (5) candidates in index order: tiles of 8192 keys, 8 per thread; every
  // key with score > Tv and the first Qt keys with score == Tv
  int32_t* cb = cand + (int64_t)bh * cstride;
  {
    const bool swar = nbins <= 128;
    int64_t eq_seen = 0, out_base = 0;  // uniform across the block
    for (int64_t base = 0; base < E; base += 8192) {
      const int64_t p0 = base + (int64_t)tid * 8;
      const int64_t rem = E - p0;
      const int nval = rem <= 0 ? 0 : (rem >= 8 ? 8 : (int)rem);
      const uint2 raw = nval > 0 ? *reinterpret_cast<const uint2*>(dst + p0) : make_uint2(0u, 0u);
      uint8_t sc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) sc[t] = (uint8_t)(((t < 4) ? raw.x : raw.y) >> ((t & 3) * 8));
      uint32_t gtm, eqm;
      score_masks<8>(sc, raw, Tv, nval, swar, gtm, eqm);
      uint2 tot;
      const uint2 ex = block_exscan2<1024>(
          make_uint2((uint32_t)__popc(gtm), (uint32_t)__popc(eqm)), s_w, tot);
      const int64_t qleft = Qt - eq_seen;  // ties still to keep at the tile start
      const int64_t mine = qleft - (int64_t)ex.y;
      const uint32_t r = mine <= 0 ? 0u : (uint32_t)(mine < 32 ? mine : 32);
      uint32_t sel = gtm | lowest_bits(eqm, r);
      const int64_t keep_before = (int64_t)ex.y < qleft ? (int64_t)ex.y : (qleft > 0 ? qleft : 0);
      int64_t o = out_base + ex.x + keep_before;
      while (sel) {
        const int t = __builtin_ctz(sel);
        if (o < C) cb[o] = (int32_t)(S + p0 + t);
        ++o;
        sel &= sel - 1u;
      }
      out_base += (int64_t)tot.x + ((int64_t)tot.y < qleft ? (int64_t)tot.y : (qleft > 0 ? qleft : 0));
      eq_seen += tot.y;
    }
  }
  __threadfence_block();
  __syncthreads();

  // (6) RSQ-IP estimates, 4 lanes per candidate, 4 candidates per lane group
  // fetched before any is used
  float* eb = est + (int64_t)bh * cstride;
  {
    using WT = typename std::conditional<M == 8, uint2, uint4>::type;
    const int q = tid & 3;
    const uint32_t* rq = rec + (int64_t)bh * cap * 32;
    for (int64_t j0 = 0; j0 < C; j0 += 1024) {
      int32_t pi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t j = j0 + r * 256 + (tid >> 2);
        pi[r] = cb[j < C ? j : C - 1];
      }
      uint4 cw[4];
      WT ww[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t* rp = rq + (int64_t)pi[r] * 32;
        cw[r] = reinterpret_cast<const uint4*>(rp)[q];
        ww[r] = reinterpret_cast<const WT*>(rp + 16)[q];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (j0 + r * 256 >= C) break;  // uniform: no candidates left
        const int64_t j = j0 + r * 256 + (tid >> 2);
        const float e = rerank_estimate<M>(cw[r], ww[r], s_P, q);
        if (j < C && q == 0) eb[j] = e;
      }
    }
  }
  __threadfence_block();
  __syncthreads();

  // (7) exact top-k' by (est desc, position asc), as k_topk_fused with every
  // slice written by this block
  int32_t* oi = out_idx + (int64_t)bh * k;
  float* oe = out_est ? out_est + (int64_t)bh * kprime : nullptr;
  const int Ci = (int)C, P = (Ci + TK_SL - 1) / TK_SL;
  uint32_t* s_hist = &s_wh[0][0];
  float f[MAXS][4];
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl) {
    const int c0 = sl * TK_SL + tid * 4;
    const float4 t = *reinterpret_cast<const float4*>(eb + min(c0, (int)cstride - 4));
    f[sl][0] = t.x; f[sl][1] = t.y; f[sl][2] = t.z; f[sl][3] = t.w;
  }
  for (int i = tid; i < 2049; i += 1024) s_hist[i] = 0u;
  for (int i = tid; i < MAXS * TK_SL / 32; i += 1024) s_bits[i] = 0u;
  if (tid < 4) s_sel[tid] = 0u;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (sl * TK_SL + tid * 4 + r < Ci) {
        const uint32_t o = order_key(f[sl][r]);
        kmin = min(kmin, o);
        kmax = max(kmax, o);
      }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) { s_r[wv] = kmin; s_r[16 + wv] = kmax; }
  __syncthreads();
  kmin = s_r[0];
  kmax = s_r[16];
#pragma unroll
  for (int w = 1; w < 16; ++w) { kmin = min(kmin, s_r[w]); kmax = max(kmax, s_r[16 + w]); }
  float fmin, scale;
  range_scale(kmin, kmax, fmin, scale);
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (sl * TK_SL + tid * 4 + r < Ci) atomicAdd(&s_hist[est_bin(f[sl][r], fmin, scale)], 1u);
  __syncthreads();
  {
    // cumulative #(bin >= b); thread t owns bins 2047 - 2t and 2046 - 2t
    const uint32_t hh = s_hist[2047 - 2 * tid], hl = s_hist[2046 - 2 * tid];
    uint2 tot;
    const uint2 ex = block_exscan2<1024>(make_uint2(hh + hl, 0), s_w, tot);
    s_hist[2047 - 2 * tid] = ex.x + hh;
    s_hist[2046 - 2 * tid] = ex.x + hh + hl;
  }
  __syncthreads();
  for (int bn = tid; bn < 2048; bn += 1024)
    if (s_hist[bn] >= (uint32_t)kprime && s_hist[bn + 1] < (uint32_t)kprime) s_sel[0] = bn;
  __syncthreads();
  const uint32_t b1 = s_sel[0];
  const uint32_t above_tot = s_hist[b1 + 1];
  const uint32_t Mb = s_hist[b1] - above_tot;
  const uint32_t remaining = (uint32_t)kprime - above_tot;
  if (Mb > (uint32_t)TK_MAXMEM) {
    // tie-heavy threshold bin: whole-unit radix select
    __syncthreads();  // s_hist is reused
    topk_radix_block(eb, cb, Ci, kprime, (int)S, oi, oe, s_hist, s_w, s_sel);
    return;
  }
  // b1's members, then their exact ranks; kept members are marked in s_bits
#pragma unroll
  for (int sl = 0; sl < MAXS; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int cc = sl * TK_SL + tid * 4 + r;
      if (cc < Ci && est_bin(f[sl][r], fmin, scale) == b1) {
        const uint32_t slot = atomicAdd(&s_sel[2], 1u);
        s_mem[slot] = member_key(order_key(f[sl][r]), (uint32_t)cc);
      }
    }
  __syncthreads();
  for (uint32_t j = tid; j < Mb; j += 1024) {
    const uint64_t mj = s_mem[j];
    const uint32_t cj = ~(uint32_t)mj;
    uint32_t rank = 0;
#pragma unroll 8
    for (uint32_t qq = 0; qq < Mb; ++qq) rank += (s_mem[qq] > mj) ? 1u : 0u;
    if (rank < remaining) atomicOr(&s_bits[cj >> 5], 1u << (cj & 31));
  }
  __syncthreads();
  for (int t = tid; t < (int)S; t += 1024) oi[t] = t;
  // every slice's selection in position order after the sinks
  uint32_t done = 0;  // selected candidates of the slices before
  for (int p = 0; p < P; ++p) {
    const int cp = p * TK_SL + tid * 4;
    const int4 cv = *reinterpret_cast<const int4*>(cb + min(cp, (int)cstride - 4));
    const int32_t ci[4] = {cv.x, cv.y, cv.z, cv.w};
    uint32_t selm = 0;
    float fo[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sl = 0; sl < MAXS; ++sl) {
      if (sl != p) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cc = sl * TK_SL + tid * 4 + r;
        fo[r] = f[sl][r];
        if (cc < Ci) {
          const uint32_t bn = est_bin(f[sl][r], fmin, scale);
          if (bn > b1 || (bn == b1 && ((s_bits[cc >> 5] >> (cc & 31)) & 1u))) selm |= 1u << r;
        }
      }
    }
    uint2 tot;
    const uint2 ex = block_exscan2<1024>(make_uint2((uint32_t)__popc(selm), 0u), s_w, tot);
    uint32_t pos = done + ex.x;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (((selm >> r) & 1u) && pos < (uint32_t)kprime) {  // bound holds by construction
        oi[S + pos] = ci[r];
        if (oe) oe[pos] = fo[r];
        ++pos;
      }
    }
    done += tot.x;
  }
}

// ---------------------------------------------------------------------------
// The single-kernel retrieval for tiny units (E <= kTinyKeys eligible keys,
// C <= kTinyCands candidates): as k_retrieve_small, with everything resident.
// The ids are loaded into registers at the start (8 keys per thread, the
// keys appended by this call patched in from the encoding lanes through
// LDS), and scores, candidates and estimates stay in LDS, so the record
// gathers are the only global round trip after the query.  The workspace
// receives the same intermediates.  The top-k ranks every member of the
// threshold bin exactly (at most C of them, all in LDS).
// ---------------------------------------------------------------------------
template <typename T, int M>
__global__ __launch_bounds__(1024) void k_retrieve_tiny(
    const T* __restrict__ Q, int n_kv_heads, int G, float invG, SignMask sg, float c, int rho,
    Tiers tw, AppendJob app, const uint4* __restrict__ ids, const uint32_t* __restrict__ rec,
    int64_t cap, int64_t S, int64_t E, int64_t C, int kprime, int k, int nbins,
    uint8_t* __restrict__ lut_out, float* __restrict__ yq_out, uint8_t* __restrict__ scores,
    int64_t Epad, int32_t* __restrict__ meta, int32_t* __restrict__ cand, float* __restrict__ est,
    int64_t cstride, int32_t* __restrict__ out_idx, float* __restrict__ out_est) {
  constexpr int U = kTinyKeys / 1024;  // keys per thread
  constexpr int CM = kTinyCands;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = bh / n_kv_heads, h = bh - b * n_kv_heads, Hq = n_kv_heads * G;
  const int Ei = (int)E, Ci = (int)C;
  __shared__ float s_yq[128];
  __shared__ float s_lv[8];  // codebook levels for the product table
  __shared__ uint8_t s_lut[16 * 256];
  __shared__ float s_P[kPtabLds];
  __shared__ uint32_t s_wh[16][256];  // per-wave score histograms, then the top-k bins
  __shared__ uint32_t s_ge[257];
  __shared__ __align__(16) uint8_t s_sc[kTinyKeys];
  __shared__ int32_t s_cand[CM];
  __shared__ float s_est[CM];
  __shared__ uint64_t s_mem[CM];
  __shared__ uint32_t s_bits[CM / 32];
  __shared__ __align__(16) uint8_t s_app[64 * 16];
  __shared__ uint2 s_w[16];
  __shared__ uint32_t s_sel[4];
  __shared__ uint32_t s_r[32];

  // (1) every eligible key's ids first (unconditional loads at clamped
  // positions), then the appended keys' encode, whose lanes also leave the
  // id bytes in LDS, and the query
  const uint4* src = ids + (int64_t)bh * cap + S;
  uint4 x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = u * 1024 + tid;
    x[u] = src[p < Ei ? p : Ei - 1];
  }
  if ((tid >> 4) < app.n)
    s_app[tid] = (uint8_t)encode_key<T, M>((const T*)app.K, app.rows_per_head, bh, tid >> 4,
                                           app.lo + (tid >> 4), app.cap, app.ids, app.rec, sg, c,
                                           tid & 15);
  if (tid < 16) {
    const int sub = tid;
    const T* q0 = Q + ((int64_t)(b * Hq + h * G) << 7) + sub * 8;
    float xq[8];
    load8(q0, xq);
    for (int g = 1; g < G; ++g) {
      float xg[8];
      load8(q0 + ((int64_t)g << 7), xg);
#pragma unroll
      for (int j = 0; j < 8; ++j) xq[j] = xq[j] + xg[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) xq[j] = xq[j] * invG;
    srht16(xq, sign_byte_of(sg, sub), sub, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) s_yq[sub * 8 + j] = xq[j];
    reinterpret_cast<float4*>(yq_out + (int64_t)bh * 128 + sub * 8)[0] =
        make_float4(xq[0], xq[1], xq[2], xq[3]);
    reinterpret_cast<float4*>(yq_out + (int64_t)bh * 128 + sub * 8)[1] =
        make_float4(xq[4], xq[5], xq[6], xq[7]);
  }
  if (tid == 0) {
#pragma unroll
    for (int l = 0; l < 8; ++l) s_lv[l] = cb_level<M>(l);
  }
  for (int i = tid; i < 16 * 256; i += 1024) (&s_wh[0][0])[i] = 0u;
  __threadfence_block();
  __syncthreads();
  // keys appended by this call: their ids from the encoding lanes
  if (app.n > 0) {
    const int64_t a0 = app.lo - S;  // eligible index of the first appended key
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = u * 1024 + tid;
      if (p >= a0 && p < a0 + app.n)
        x[u] = reinterpret_cast<const uint4*>(s_app)[p - a0];
    }
  }
  // (2) signed product table and vote table (row s = wave s)
  for (int e = tid; e < 2048; e += 1024) {
    const float pr = s_lv[e & 7] * s_yq[e >> 4];
    s_P[(e >> 7) * kPtabRow + (e & 127)] = (e & 8) ? -pr : pr;
  }
  {
    const uint32_t word = vote_table_word<M>(s_yq, wv, lane, rho, tw);
    reinterpret_cast<uint32_t*>(s_lut)[wv * 64 + lane] = word;
    reinterpret_cast<uint32_t*>(lut_out + (int64_t)bh * 4096)[wv * 64 + lane] = word;
  }
  __syncthreads();

  // (3) vote scan from registers: scores into LDS (and the workspace)
  uint8_t* dst = scores + (int64_t)bh * Epad;
  {
    uint32_t zeros = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u * 1024 >= Ei) break;  // uniform: the rest of the key slots are empty
      const int p = u * 1024 + tid;
      const bool valid = p < Ei;
      const uint32_t w4[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
      uint32_t sc = 0;
#pragma unroll
      for (int bb = 0; bb < 16; ++bb)
        sc += s_lut[bb * 256 + ((w4[bb >> 2] >> ((bb & 3) * 8)) & 0xFFu)];
      zeros += (uint32_t)__popcll(__ballot(valid && sc == 0));
      s_sc[p] = valid ? (uint8_t)sc : (uint8_t)0;
      if (valid) {
        dst[p] = (uint8_t)sc;
        if (sc != 0) atomicAdd(&s_wh[wv][sc], 1u);
      }
    }
    if (lane == 0) s_wh[wv][0] = zeros;
  }
  __syncthreads();

  // (4) threshold: Tv = the largest v with #(score >= v) >= C
  if (tid < 256) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) a += s_wh[w][tid];
    s_ge[tid] = a;
  }
  __syncthreads();
  if (wv == 0) {
    uint32_t hc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) hc[r] = s_ge[4 * lane + r];
    const uint32_t loc = hc[0] + hc[1] + hc[2] + hc[3];
    uint32_t inc = loc;  // sum over lanes >= this one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_down(inc, off);
      if (lane + off < 64) inc += t;
    }
    const uint32_t g3 = inc - loc + hc[3], g2 = g3 + hc[2], g1 = g2 + hc[1], g0 = g1 + hc[0];
    s_ge[4 * lane + 0] = g0;
    s_ge[4 * lane + 1] = g1;
    s_ge[4 * lane + 2] = g2;
    s_ge[4 * lane + 3] = g3;
    if (lane == 0) s_ge[256] = 0u;
  }
  __syncthreads();
  if (tid < 256 && (int)s_ge[tid] >= Ci && (int)s_ge[tid + 1] < Ci) s_sel[0] = (uint32_t)tid;
  __syncthreads();
  const int Tv = (int)s_sel[0];
  const int n_gt = (int)s_ge[Tv + 1];
  const int Qt = Ci - n_gt;
  if (tid == 0) {
    meta[bh * 4 + 0] = Tv;
    meta[bh * 4 + 1] = n_gt;
    meta[bh * 4 + 2] = Qt;
    meta[bh * 4 + 3] = Ci;
  }

  // (5) candidates in index order: thread t owns keys 8 t .. 8 t + 7
  int32_t* cb = cand + (int64_t)bh * cstride;
  {
    const int p0 = tid * 8;
    const int rem = Ei - p0;
    const int nval = rem <= 0 ? 0 : (rem >= 8 ? 8 : rem);
    const uint2 raw = reinterpret_cast<const uint2*>(s_sc)[tid];
    uint8_t sc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) sc[t] = (uint8_t)(((t < 4) ? raw.x : raw.y) >> ((t & 3) * 8));
    uint32_t gtm, eqm;
    score_masks<8>(sc, raw, Tv, nval, nbins <= 128, gtm, eqm);
    uint2 tot;
    const uint2 ex = block_exscan2<1024>(
        make_uint2((uint32_t)__popc(gtm), (uint32_t)__popc(eqm)), s_w, tot);
    const int mine = Qt - (int)ex.y;  // ties of this thread still within the quota
    const uint32_t r = mine <= 0 ? 0u : (uint32_t)(mine < 32 ? mine : 32);
    uint32_t sel = gtm | lowest_bits(eqm, r);
    int o = (int)ex.x + ((int)ex.y < Qt ? (int)ex.y : (Qt > 0 ? Qt : 0));
    while (sel) {
      const int t = __builtin_ctz(sel);
      if (o < Ci) {
        s_cand[o] = (int32_t)(S + p0 + t);
        cb[o] = (int32_t)(S + p0 + t);
      }
      ++o;
      sel &= sel - 1u;
    }
  }
  __syncthreads();

  // (6) RSQ-IP estimates, 4 lanes per candidate, 4 candidates per lane group
  // fetched before any is used
  float* eb = est + (int64_t)bh * cstride;
  {
    using WT = typename std::conditional<M == 8, uint2, uint4>::type;
    const int q = tid & 3;
    const uint32_t* rq = rec + (int64_t)bh * cap * 32;
    for (int j0 = 0; j0 < Ci; j0 += 1024) {
      int32_t pi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + r * 256 + (tid >> 2);
        pi[r] = s_cand[j < Ci ? j : Ci - 1];
      }
      uint4 cw[4];
      WT ww[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t* rp = rq + (int64_t)pi[r] * 32;
        cw[r] = reinterpret_cast<const uint4*>(rp)[q];
        ww[r] = reinterpret_cast<const WT*>(rp + 16)[q];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (j0 + r * 256 >= Ci) break;  // uniform: no candidates left
        const int j = j0 + r * 256 + (tid >> 2);
        const float e = rerank_estimate<M>(cw[r], ww[r], s_P, q);
        if (j < Ci && q == 0) {
          s_est[j] = e;
          eb[j] = e;
        }
      }
    }
  }
  __syncthreads();

  // (7) exact top-k' by (est desc, position asc)
  int32_t* oi = out_idx + (int64_t)bh * k;
  float* oe = out_est ? out_est + (int64_t)bh * kprime : nullptr;
  // linear 2048-bin histogram between the estimates' extremes, the bin b1
  // holding rank k', exact ranks of b1's members; thread t owns candidates
  // 2 t and 2 t + 1
  uint32_t* s_hist = &s_wh[0][0];
  float f[2];
  bool has[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int cc = 2 * tid + r;
    has[r] = cc < Ci;
    f[r] = has[r] ? s_est[cc] : 0.0f;
  }
  for (int i = tid; i < 2049; i += 1024) s_hist[i] = 0u;
  if (tid < CM / 32) s_bits[tid] = 0u;
  if (tid < 4) s_sel[tid] = 0u;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (has[r]) {
      const uint32_t ok = order_key(f[r]);
      kmin = min(kmin, ok);
      kmax = max(kmax, ok);
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) { s_r[wv] = kmin; s_r[16 + wv] = kmax; }
  __syncthreads();
  kmin = s_r[0];
  kmax = s_r[16];
#pragma unroll
  for (int w = 1; w < 16; ++w) { kmin = min(kmin, s_r[w]); kmax = max(kmax, s_r[16 + w]); }
  float fmin, scale;
  range_scale(kmin, kmax, fmin, scale);
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (has[r]) atomicAdd(&s_hist[est_bin(f[r], fmin, scale)], 1u);
  __syncthreads();
  {
    // cumulative #(bin >= b); thread t owns bins 2047 - 2t and 2046 - 2t
    const uint32_t hh = s_hist[2047 - 2 * tid], hl = s_hist[2046 - 2 * tid];
    uint2 tot;
    const uint2 ex = block_exscan2<1024>(make_uint2(hh + hl, 0), s_w, tot);
    s_hist[2047 - 2 * tid] = ex.x + hh;
    s_hist[2046 - 2 * tid] = ex.x + hh + hl;
  }
  __syncthreads();
  for (int bn = tid; bn < 2048; bn += 1024)
    if (s_hist[bn] >= (uint32_t)kprime && s_hist[bn + 1] < (uint32_t)kprime) s_sel[0] = bn;
  __syncthreads();
  const uint32_t b1 = s_sel[0];
  const uint32_t above_tot = s_hist[b1 + 1];
  const uint32_t Mb = s_hist[b1] - above_tot;
  const uint32_t remaining = (uint32_t)kprime - above_tot;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int cc = 2 * tid + r;
    if (has[r] && est_bin(f[r], fmin, scale) == b1) {
      const uint32_t slot = atomicAdd(&s_sel[2], 1u);
      s_mem[slot] = member_key(order_key(f[r]), (uint32_t)cc);
    }
  }
  __syncthreads();
  for (uint32_t j = tid; j < Mb; j += 1024) {
    const uint64_t mj = s_mem[j];
    const uint32_t cj = ~(uint32_t)mj;
    uint32_t rank = 0;
#pragma unroll 8
    for (uint32_t qq = 0; qq < Mb; ++qq) rank += (s_mem[qq] > mj) ? 1u : 0u;
    if (rank < remaining) atomicOr(&s_bits[cj >> 5], 1u << (cj & 31));
  }
  __syncthreads();
  for (int t = tid; t < (int)S; t += 1024) oi[t] = t;
  uint32_t selm = 0;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int cc = 2 * tid + r;
    if (has[r]) {
      const uint32_t bn = est_bin(f[r], fmin, scale);
      if (bn > b1 || (bn == b1 && ((s_bits[cc >> 5] >> (cc & 31)) & 1u))) selm |= 1u << r;
    }
  }
  uint2 tot;
  const uint2 ex = block_exscan2<1024>(make_uint2((uint32_t)__popc(selm), 0u), s_w, tot);
  uint32_t pos = ex.x;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (((selm >> r) & 1u) && pos < (uint32_t)kprime) {  // bound holds by construction
      oi[S + pos] = s_cand[2 * tid + r];
      if (oe) oe[pos] = f[r];
      ++pos;
    }
  }
}

// ---------------------------------------------------------------------------
// K7 split-K sparse attention ([TS] Problem Statement; System-Level
// Innovations 1: only the selected rows are fetched).  Block = a chunk of
// 16 RPL selected rows of one (b, h) (RPL = 2 or 4: attn_rows_per_lane); 16
// lanes per row (16 B of K and of V per lane), 16 row slots x RPL rows.  The G query heads of the KV head are held in registers
// (pre-multiplied by scale * log2 e), logits summed across the 16 lanes of a
// row with DPP, softmax statistics per slot; the 16 slots are combined in
// LDS (wave 0, one row of 16 lanes per query head, forms each slot's factor
// and the total denominator once).  Writes per query head a partial
// (o[128], m, l) in the log2 domain.  The weights exp2(logit - max) use the
// hardware exp2 directly: every argument is <= 0, and a weight below 2^-126
// (flushed to zero there) is far below the attention's tolerance.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  // every source lane of these patterns lies in the same row of 16, so the
  // bound-control zero fill never applies; it lets the move fold into the
  // add or max that consumes it
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// sum / maximum over the 16 lanes of a row, received by all of them
__device__ __forceinline__ float row_sum16(float v) {
  v += dppf<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dppf<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dppf<0x141>(v);  // row_half_mirror
  v += dppf<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  return v;
}

// WIN: rows may come from the near store or its ring (a sliding window);
// without it every row is a listed position in the far store.
template <typename T, int G, int RPL, bool WIN>
__global__ __launch_bounds__(256) void k_attn_split(const T* __restrict__ Q, AttnRows rs,
                                                    const int32_t* __restrict__ idx, int k,
                                                    int n_kv_heads, float qscale,
                                                    float* __restrict__ part, int nch) {
  const int bh = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int b = bh / n_kv_heads, h = bh - b * n_kv_heads;
  const int Hq = n_kv_heads * G;
  const int slot = tid >> 4, sub = tid & 15;
  __shared__ float s_m[16][G], s_l[16][G], s_f[16][G];
  __shared__ float s_M[G], s_L[G];
  __shared__ float s_o[16][G][128];

  // rows r < k are the positions idx[r] (positions below n_near_head in the
  // near store, the rest in the far store); rows k .. k + tail_n - 1 are the
  // positions tail_lo + (r - k), in the near store's ring
  const int n_rows = k + (WIN ? rs.tail_n : 0);
  const int32_t* ib = idx + (int64_t)bh * k;
  int64_t row[RPL];
  bool valid[RPL], near[RPL];
#pragma unroll
  for (int it = 0; it < RPL; ++it) {
    const int r = chunk * (16 * RPL) + slot + 16 * it;
    valid[it] = r < n_rows;
    const int32_t li = ib[r < k ? r : k - 1];  // unconditional load
    if constexpr (WIN) {
      const bool listed = r < k;
      const int64_t p = listed ? (int64_t)li : rs.tail_lo + (r - k);
      if (listed) {
        near[it] = p < rs.n_near_head;
        row[it] = p;
      } else {
        near[it] = true;
        row[it] = rs.n_near_head + (p - rs.n_near_head) % rs.ring;
      }
    } else {
      near[it] = false;
      row[it] = li;
    }
    if (!valid[it]) { near[it] = false; row[it] = 0; }
  }
  float q[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    load8(Q + ((int64_t)(b * Hq + h * G + g) << 7) + sub * 8, q[g]);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[g][j] *= qscale;
  }
  const int64_t kvh = bh / rs.unit_div;  // the KV head whose rows this block reads
  const T* Kf = (const T*)rs.K + ((int64_t)kvh * rs.rows << 7) + sub * 8;
  const T* Vf = (const T*)rs.V + ((int64_t)kvh * rs.rows << 7) + sub * 8;
  const T* Kn = (const T*)rs.K_near + ((int64_t)kvh * rs.near_rows << 7) + sub * 8;
  const T* Vn = (const T*)rs.V_near + ((int64_t)kvh * rs.near_rows << 7) + sub * 8;
  float kx[RPL][8], vx[RPL][8];
#pragma unroll
  for (int it = 0; it < RPL; ++it) {
    load8_stream((WIN && near[it] ? Kn : Kf) + (row[it] << 7), kx[it]);
    load8_stream((WIN && near[it] ? Vn : Vf) + (row[it] << 7), vx[it]);
  }
  float lg[RPL][G];
#pragma unroll
  for (int it = 0; it < RPL; ++it)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float sdot = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) sdot = __builtin_fmaf(q[g][j], kx[it][j], sdot);
      sdot = row_sum16(sdot);
      lg[it][g] = valid[it] ? sdot : -INFINITY;
    }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = lg[0][g];
#pragma unroll
    for (int it = 1; it < RPL; ++it) m = fmaxf(m, lg[it][g]);
    float l = 0.0f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (m != -INFINITY) {
#pragma unroll
      for (int it = 0; it < RPL; ++it) {
        const float pw = __builtin_amdgcn_exp2f(lg[it][g] - m);  // argument <= 0
        l += pw;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = __builtin_fmaf(pw, vx[it][j], o[j]);
      }
    }
    if (sub == 0) { s_m[slot][g] = m; s_l[slot][g] = l; }
    reinterpret_cast<float4*>(&s_o[slot][g][sub * 8])[0] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<float4*>(&s_o[slot][g][sub * 8])[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
  __syncthreads();
  if (tid < 16 * G) {
    // row g of 16 lanes, lane s: slot s's factor exp2(m_s - M) and the sum of
    // the scaled denominators (some slot of the chunk has a valid row)
    const int g = tid >> 4, sl = tid & 15;
    const float ms = s_m[sl][g];
    const float M = row_max16(ms);
    const float f = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
    const float lt = row_sum16(f * s_l[sl][g]);
    s_f[sl][g] = f;
    if (sl == 0) { s_M[g] = M; s_L[g] = lt; }
  }
  __syncthreads();
  for (int e = tid; e < G * 128; e += 256) {
    const int g = e >> 7, j = e & 127;
    float o = 0.0f;
#pragma unroll
    for (int sl = 0; sl < 16; ++sl) o = __builtin_fmaf(s_f[sl][g], s_o[sl][g][j], o);
    float* pp = part + (((int64_t)(b * Hq + h * G + g)) * nch + chunk) * kPartStride;
    pp[j] = o;
    if (j == 0) { pp[128] = s_M[g]; pp[129] = s_L[g]; }
  }
}

// K8 log-sum-exp merge of the split-K partials -> output row per query head,
// for fewer than kMergeSplitRows (b, query head) pairs.  Four blocks per
// (b, query head), block q for output coordinates 32 q ..
// 32 q + 31: thread (g = tid / 32, j = tid % 32) takes chunks g, g + 8, ...
// of coordinate 32 q + j, up to 16 of them (m, l and o) loaded in one round;
// the block's maximum M by wave reductions, then each thread's sum of
// exp2(m_c - M) o_c and exp2(m_c - M) l_c over its chunks (rescaled by the
// running maximum from one round of 16 chunks to the next), and the 8 chunk
// groups added in group order.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part, int nch,
                                                    T* __restrict__ out) {
  constexpr int NB = 16;
  const int bq = blockIdx.x, q = blockIdx.y, tid = threadIdx.x;
  const int j = tid & 31, g = tid >> 5, lane = tid & 63, wv = tid >> 6;
  const int d = 32 * q + j;
  const float* pp = part + (int64_t)bq * nch * kPartStride;
  __shared__ float s_w[4], s_a[8][32], s_l[8];
  float M = -INFINITY, acc = 0.0f, lac = 0.0f;
  for (int c0 = 0; c0 < nch; c0 += 8 * NB) {
    float mv[NB], lv[NB], ov[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int c = c0 + g + 8 * u;
      const int cc = c < nch ? c : nch - 1;  // in the buffer; masked below
      const float* pc = pp + (int64_t)cc * kPartStride;
      mv[u] = pc[128];
      lv[u] = pc[129];
      ov[u] = pc[d];
      if (c >= nch) mv[u] = -INFINITY;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < NB; ++u) bm = fmaxf(bm, mv[u]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
    __syncthreads();  // s_w of the previous batch has been read
    if (lane == 0) s_w[wv] = bm;
    __syncthreads();
    bm = fmaxf(fmaxf(s_w[0], s_w[1]), fmaxf(s_w[2], s_w[3]));
    const float Mn = fmaxf(M, bm);
    if (Mn != -INFINITY) {
      // hardware exp2: every argument is <= 0 (a factor below 2^-126 is
      // flushed to zero, far below the attention's tolerance)
      const float r = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
      acc *= r;
      lac *= r;
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const float f = (mv[u] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mv[u] - Mn);
        acc = __builtin_fmaf(f, ov[u], acc);
        lac = __builtin_fmaf(f, lv[u], lac);
      }
      M = Mn;
    }
  }
  s_a[g][j] = acc;
  if (j == 0) s_l[g] = lac;
  __syncthreads();
  if (g == 0) {
    float A = 0.0f, L = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      A += s_a[t][j];
      L += s_l[t];
    }
    const float r = A / L;
    if constexpr (sizeof(T) == 2) {
      // fp32 -> bf16, round to nearest even
      uint32_t u = __float_as_uint(r);
      u += 0x7FFFu + ((u >> 16) & 1u);
      out[(int64_t)bq * 128 + d] = (T)(u >> 16);
    } else {
      out[(int64_t)bq * 128 + d] = r;
    }
  }
}

// K8 for many query heads (kMergeSplitRows or more): one block per (b, query
// head).  Partials are staged in LDS 64 chunks at a time (one round of
// 16-byte loads); wave 0 forms the tile's maximum and each chunk's factor
// exp2(m_c - M) once, then threads 0..127 combine the chunks for their
// output element in chunk order, rescaling by the running maximum across
// tiles.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_merge_row(const float* __restrict__ part, int nch,
                                                        T* __restrict__ out) {
  constexpr int R4 = kPartStride / 4;  // float4 per partial record
  constexpr int TILE = 64;
  constexpr int NLD = (TILE * R4 + 255) / 256;
  const int bq = blockIdx.x, tid = threadIdx.x;
  const float* pp = part + (int64_t)bq * nch * kPartStride;
  __shared__ float4 s_p4[TILE * R4];
  __shared__ float s_f[TILE], s_m[1];
  const float* s_p = reinterpret_cast<const float*>(s_p4);
  float o = 0.0f, l = 0.0f, M = -INFINITY;
  for (int t0 = 0; t0 < nch; t0 += TILE) {
    const int nt = min(TILE, nch - t0);
    const int n4 = nt * R4;
    const float4* src = reinterpret_cast<const float4*>(pp + (int64_t)t0 * kPartStride);
    float4 v[NLD];
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int i = tid + 256 * u;
      v[u] = (i < n4) ? src[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    __syncthreads();  // the previous tile has been consumed
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int i = tid + 256 * u;
      if (i < n4) s_p4[i] = v[u];
    }
    __syncthreads();
    if (tid < 64) {
      // lane c: chunk c's maximum; the tile's by a wave reduction
      const float mc = tid < nt ? s_p[tid * kPartStride + 128] : -INFINITY;
      float tm = mc;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) tm = fmaxf(tm, __shfl_xor(tm, off));
      const float Mn = fmaxf(M, tm);
      if (tid < nt) s_f[tid] = (Mn == -INFINITY || mc == -INFINITY) ? 0.0f : exp2f(mc - Mn);
      if (tid == 0) s_m[0] = Mn;
    }
    __syncthreads();
    if (tid < 128) {
      const float Mn = s_m[0];
      if (Mn != -INFINITY) {
        const float r = (M == -INFINITY) ? 0.0f : exp2f(M - Mn);
        o *= r;
        l *= r;
        M = Mn;
        for (int c = 0; c < nt; ++c) {
          const float f = s_f[c];
          o = __builtin_fmaf(f, s_p[c * kPartStride + tid], o);
          l = __builtin_fmaf(f, s_p[c * kPartStride + 129], l);
        }
      }
    }
  }
  if (tid < 128) {
    const float r = o / l;
    if constexpr (sizeof(T) == 2) {
      // fp32 -> bf16, round to nearest even
      uint32_t u = __float_as_uint(r);
      u += 0x7FFFu + ((u >> 16) & 1u);
      out[(int64_t)bq * 128 + tid] = (T)(u >> 16);
    } else {
      out[(int64_t)bq * 128 + tid] = r;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers (host side, called from the C ABI).  Every launch goes through
// hipExtLaunchKernelGGL: with a non-null start/stop event pair the dispatch
// itself timestamps the kernel's execution (exact per-kernel durations even
// when launches are host-bound); with null events it is a plain launch.
// ---------------------------------------------------------------------------
hipError_t launch_encode(int m, int dtype, const void* K, int64_t rows_per_head, int64_t lo,
                         int64_t n, int BH, int64_t cap, uint8_t* ids, uint32_t* rec,
                         const SignMask& sg, float c, hipStream_t st, const EvPair& ev) {
  const int64_t total = (int64_t)BH * n;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 15) / 16));
#define PKV_ENC(T, MM)                                                                       \
  return launch(k_encode<T, MM>, grid, dim3(256), st, ev, (const T*)K, rows_per_head, lo, n, \
                total, cap, ids, rec, sg, c)
  if (m == 8) {
    if (dtype == 0) PKV_ENC(uint16_t, 8);
    PKV_ENC(float, 8);
  }
  if (m == 4) {
    if (dtype == 0) PKV_ENC(uint16_t, 4);
    PKV_ENC(float, 4);
  }
#undef PKV_ENC
  return hipErrorInvalidValue;
}

template <int M>
static hipError_t launch_qprep_m(int dtype, const void* Q, int BH, int n_kv_heads, int G,
                                 const SignMask& sg, float c, int rho, const Tiers& tw,
                                 uint8_t* lut, float* yq, float* ptab, const AppendJob& app,
                                 int unit_div, hipStream_t st, const EvPair& ev) {
  const float invG = 1.0f / (float)G;
  // encode blocks: 4 (KV head, key) pairs each
  const int nenc = app.n > 0 ? (int)(((int64_t)(BH / unit_div) * app.n + 3) / 4) : 0;
#define PKV_QP(T, GG)                                                                           \
  return launch(k_qprep<T, GG, M>, dim3(16 * BH + nenc), dim3(64), st, ev, (const T*)Q,         \
                n_kv_heads, invG, sg, c, rho, tw, lut, yq, ptab, app, unit_div, BH)
  if (dtype == 0) {
    switch (G) {
      case 1: PKV_QP(uint16_t, 1);
      case 2: PKV_QP(uint16_t, 2);
      case 4: PKV_QP(uint16_t, 4);
      case 8: PKV_QP(uint16_t, 8);
      default: return hipErrorInvalidValue;
    }
  }
  switch (G) {
    case 1: PKV_QP(float, 1);
    case 2: PKV_QP(float, 2);
    case 4: PKV_QP(float, 4);
    case 8: PKV_QP(float, 8);
    default: return hipErrorInvalidValue;
  }
#undef PKV_QP
}

hipError_t launch_qprep(int m, int dtype, const void* Q, int BH, int n_kv_heads, int G,
                        const SignMask& sg, float c, int rho, const Tiers& tw, uint8_t* lut,
                        float* yq, float* ptab, const AppendJob& app, int unit_div,
                        hipStream_t st, const EvPair& ev) {
  if (m == 8)
    return launch_qprep_m<8>(dtype, Q, BH, n_kv_heads, G, sg, c, rho, tw, lut, yq, ptab, app,
                             unit_div, st, ev);
  if (m == 4)
    return launch_qprep_m<4>(dtype, Q, BH, n_kv_heads, G, sg, c, rho, tw, lut, yq, ptab, app,
                             unit_div, st, ev);
  return hipErrorInvalidValue;
}

hipError_t launch_scan(int kpt, int nchunks, int BH, const uint8_t* ids, int64_t cap, int64_t S,
                       int64_t E, const uint8_t* lut, uint8_t* scores, int64_t Epad,
                       uint32_t* chist, int chunk_stride, int nbins, int rstride, int unit_div,
                       hipStream_t st, const EvPair& ev) {
  // a chunk is kpt * 256 keys; the scan covers it with kScanThreads threads
  const dim3 grid(nchunks, BH);
  const uint4* id4 = (const uint4*)ids;
  constexpr int NT = kScanThreads;
  if (unit_div > 1 && kpt >= 2) {
    // unshared retrieval: one pass per KV head for its unit_div query heads
    const dim3 gg(nchunks, BH / unit_div);
#define PKV_SG(K, GU)                                                                           \
  return launch(k_scan_group<(K * 256) / NT, NT, GU>, gg, dim3(NT), st, ev, id4, cap, S, E, lut, \
                scores, Epad, chist, chunk_stride, nbins, rstride)
#define PKV_SGK(GU)        \
  switch (kpt) {           \
    case 2: PKV_SG(2, GU); \
    case 4: PKV_SG(4, GU); \
    case 8: PKV_SG(8, GU); \
    case 16: PKV_SG(16, GU); \
    default: return hipErrorInvalidValue; \
  }
    switch (unit_div) {
      case 2: PKV_SGK(2);
      case 4: PKV_SGK(4);
      case 8: PKV_SGK(8);
      default: return hipErrorInvalidValue;
    }
#undef PKV_SGK
#undef PKV_SG
  }
  switch (kpt) {
#define PKV_SCAN(K)                                                                          \
  case K:                                                                                    \
    return launch(k_scan<(K * 256) / NT, NT>, grid, dim3(NT), st, ev, id4, cap, S, E, lut,   \
                  scores, Epad, chist, chunk_stride, nbins, rstride, unit_div);
    PKV_SCAN(4) PKV_SCAN(8) PKV_SCAN(16)
#undef PKV_SCAN
    case 1:
      return launch(k_scan<1, 256>, grid, dim3(256), st, ev, id4, cap, S, E, lut, scores, Epad,
                    chist, chunk_stride, nbins, rstride, unit_div);
    case 2:
      return launch(k_scan<2, 256>, grid, dim3(256), st, ev, id4, cap, S, E, lut, scores, Epad,
                    chist, chunk_stride, nbins, rstride, unit_div);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_thresh(int BH, const uint32_t* chist, int chunk_stride, int nchunks, int nbins,
                         int rstride, int64_t C, int all_ties, int32_t* meta, uint32_t* coff,
                         hipStream_t st, const EvPair& ev) {
  return launch(k_thresh, dim3(BH), dim3(1024), st, ev, chist, chunk_stride, nchunks, nbins,
                rstride, C, all_ties, meta, coff);
}

hipError_t launch_compact_rerank(int m, int kpt, int nchunks, int BH, const uint8_t* scores,
                                 int64_t Epad, int64_t S, int64_t E, const int32_t* meta,
                                 const uint32_t* coff, int chunk_stride, const float* ptab,
                                 const uint32_t* rec, int64_t cap, int32_t* cand, float* est,
                                 int64_t cstride, int64_t C, uint32_t* mm, int nbins,
                                 int unit_div, const uint32_t* chist, int rstride,
                                 int32_t* meta_out, hipStream_t st, const EvPair& ev) {
  // chist: fold the threshold into this kernel (nchunks <= kFusedThreshChunks)
  const bool ft = chist != nullptr;
  const int swar = nbins <= 128 ? 1 : 0;  // every score below 128
  const dim3 grid((nchunks + kCompactChunks - 1) / kCompactChunks, BH);
#define PKV_CR(K, MM, FT)                                                                     \
  case K:                                                                                     \
    if constexpr (MM == 8 && !(FT))                                                           \
      return launch(k_compact_rerank_m8<K, kCompactChunks>, grid, dim3(256), st, ev, scores,  \
                    Epad, S, E, meta, coff, chunk_stride, nchunks, ptab, rec, cap, cand, est, \
                    cstride, C, mm, swar, unit_div, chist, nbins, rstride, meta_out);         \
    else                                                                                      \
      return launch(k_compact_rerank<K, kCompactChunks, MM, FT>, grid, dim3(256), st, ev,     \
                    scores, Epad, S, E, meta, coff, chunk_stride, nchunks, ptab, rec, cap,    \
                    cand, est, cstride, C, mm, swar, unit_div, chist, nbins, rstride,         \
                    meta_out);
#define PKV_CRK(MM, FT)                                                                      \
  switch (kpt) {                                                                             \
    PKV_CR(1, MM, FT) PKV_CR(2, MM, FT) PKV_CR(4, MM, FT) PKV_CR(8, MM, FT) PKV_CR(16, MM, FT) \
    default: return hipErrorInvalidValue;                                                    \
  }
  if (ft && nchunks > kFusedThreshChunks) return hipErrorInvalidValue;
  if (m == 8) {
    if (ft) PKV_CRK(8, true);
    PKV_CRK(8, false);
  }
  if (m == 4) {
    if (ft) PKV_CRK(4, true);
    PKV_CRK(4, false);
  }
#undef PKV_CRK
#undef PKV_CR
  return hipErrorInvalidValue;
}

hipError_t launch_topk(int BH, const float* est, const int32_t* cand, int64_t cstride, int C,
                       int kprime, int S, int k, int P, const uint32_t* mmc, int chunk_stride,
                       int nchunks, uint32_t* range, uint16_t* rows, int32_t* tkmeta,
                       uint2* sorted, int32_t* out_idx, float* out_est, hipStream_t st,
                       const EvPair& ev_hist, const EvPair& ev_select) {
  const dim3 grid(P, BH);
  if (P <= kTopkFusedSlices) {
    // few slices: the whole top-k in one kernel
    static_assert(kTopkFusedSlices <= 4, "k_topk_fused instances");
    hipError_t e;
    if (P == 1)
      e = launch(k_topk_fused<1>, grid, dim3(1024), st, ev_hist, est, cand, cstride, C, kprime, S,
                 k, tkmeta, out_idx, out_est);
    else if (P == 2)
      e = launch(k_topk_fused<2>, grid, dim3(1024), st, ev_hist, est, cand, cstride, C, kprime, S,
                 k, tkmeta, out_idx, out_est);
    else
      e = launch(k_topk_fused<4>, grid, dim3(1024), st, ev_hist, est, cand, cstride, C, kprime, S,
                 k, tkmeta, out_idx, out_est);
    if (e != hipSuccess || !ev_select.start) return e;
    // the second stage does not run: its events are recorded back to back
    e = hipEventRecord(ev_select.start, st);
    if (e != hipSuccess) return e;
    return hipEventRecord(ev_select.stop, st);
  }
  hipError_t e = launch(k_topk_hist, grid, dim3(1024), st, ev_hist, est, cstride, C, P, mmc,
                        chunk_stride, nchunks, rows, range, sorted, (const int32_t*)nullptr);
  if (e != hipSuccess) return e;
  if (P <= kTopkFewSlices)
    return launch(k_topk_select_few<kTopkFewSlices>, grid, dim3(1024), st, ev_select, est, cand,
                  cstride, C, kprime, S, k, P, (const uint32_t*)range, (const uint16_t*)rows,
                  (const uint2*)sorted, tkmeta, out_idx, out_est);
  return launch(k_topk_select, grid, dim3(1024), st, ev_select, est, cand, cstride, C, kprime, S,
                k, P, (const uint32_t*)range, (const uint16_t*)rows, (const uint2*)sorted, tkmeta,
                out_idx, out_est, (const int32_t*)nullptr);
}

hipError_t launch_topk_counted(int BH, const float* est, const int32_t* cand, int64_t cstride,
                               const int32_t* cmeta, int Cmax, int grid_slices, int kprime,
                               int S, int k, const uint32_t* mmc, int chunk_stride, int nchunks,
                               uint32_t* range, uint16_t* rows, int32_t* tkmeta, uint2* sorted,
                               int32_t* out_idx, float* out_est, hipStream_t st,
                               const EvPair& ev_hist, const EvPair& ev_select) {
  // per-unit candidate counts known on the device only: rows laid out for
  // the largest (P slices), a grid of grid_slices blocks per unit looping
  // over the unit's own slices; the general select (any number of slices)
  const int P = (Cmax + kTopkSlice - 1) / kTopkSlice;
  const dim3 grid(grid_slices < P ? grid_slices : P, BH);
  hipError_t e = launch(k_topk_hist, grid, dim3(1024), st, ev_hist, est, cstride, Cmax, P, mmc,
                        chunk_stride, nchunks, rows, range, sorted, cmeta);
  if (e != hipSuccess) return e;
  return launch(k_topk_select, grid, dim3(1024), st, ev_select, est, cand, cstride, Cmax, kprime,
                S, k, P, (const uint32_t*)range, (const uint16_t*)rows, (const uint2*)sorted,
                tkmeta, out_idx, out_est, cmeta);
}

hipError_t launch_retrieve_small(int m, int dtype, const void* Q, int BH, int n_kv_heads, int G,
                                 const SignMask& sg, float c, int rho, const Tiers& tw,
                                 const AppendJob& app, const uint8_t* ids, const uint32_t* rec,
                                 int64_t cap, int64_t S, int64_t E, int64_t C, int kprime, int k,
                                 int nbins, uint8_t* lut, float* yq, uint8_t* scores, int64_t Epad,
                                 int32_t* meta, int32_t* cand, float* est, int64_t cstride,
                                 int32_t* out_idx, float* out_est, hipStream_t st,
                                 const EvPair& ev) {
  // one block per unit; appended keys take 16 lanes each of the block
  if (E < 1 || C < 1 || C > E || C > (int64_t)kSmallTopkSlices * kTopkSlice || app.n > 64 ||
      nbins > 256 || kprime < 1 || (int64_t)kprime > C)
    return hipErrorInvalidValue;
  const float invG = 1.0f / (float)G;
  const uint4* id4 = (const uint4*)ids;
  const bool tiny = E <= kTinyKeys && C <= kTinyCands;
#define PKV_RS(TT, MM)                                                                          \
  return tiny ? launch(k_retrieve_tiny<TT, MM>, dim3(BH), dim3(1024), st, ev, (const TT*)Q,     \
                       n_kv_heads, G, invG, sg, c, rho, tw, app, id4, rec, cap, S, E, C, kprime, \
                       k, nbins, lut, yq, scores, Epad, meta, cand, est, cstride, out_idx,       \
                       out_est)                                                                 \
              : launch(k_retrieve_small<TT, MM>, dim3(BH), dim3(1024), st, ev, (const TT*)Q,    \
                       n_kv_heads, G, invG, sg, c, rho, tw, app, id4, rec, cap, S, E, C, kprime, \
                       k, nbins, lut, yq, scores, Epad, meta, cand, est, cstride, out_idx,       \
                       out_est)
  if (m == 8) {
    if (dtype == 0) PKV_RS(uint16_t, 8);
    PKV_RS(float, 8);
  }
  if (m == 4) {
    if (dtype == 0) PKV_RS(uint16_t, 4);
    PKV_RS(float, 4);
  }
#undef PKV_RS
  return hipErrorInvalidValue;
}

hipError_t launch_attn_split(int dtype, int G, int rpl, const void* Q, const AttnRows& rs,
                             const int32_t* idx, int k, int batch, int n_kv_heads, float qscale,
                             float* part, int nch, hipStream_t st, const EvPair& ev) {
  const dim3 grid(nch, batch * n_kv_heads);
  if (rpl != 2 && rpl != 4) return hipErrorInvalidValue;
  const bool win = rs.n_near_head > 0 || rs.tail_n > 0;
#define PKV_ASW(T, GG, R)                                                                      \
  (win ? launch(k_attn_split<T, GG, R, true>, grid, dim3(256), st, ev, (const T*)Q, rs, idx,   \
                k, n_kv_heads, qscale, part, nch)                                              \
       : launch(k_attn_split<T, GG, R, false>, grid, dim3(256), st, ev, (const T*)Q, rs, idx,  \
                k, n_kv_heads, qscale, part, nch))
#define PKV_AS(T, GG) return rpl == 2 ? PKV_ASW(T, GG, 2) : PKV_ASW(T, GG, 4)
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
#undef PKV_ASW
}

hipError_t launch_attn_merge(int dtype, const float* part, int nch, int rows, void* out,
                             hipStream_t st, const EvPair& ev) {
  // four blocks per (b, query head) while they are few, else one
  if (rows < kMergeSplitRows) {
    if (dtype == 0)
      return launch(k_attn_merge<uint16_t>, dim3(rows, 4), dim3(256), st, ev, part, nch,
                    (uint16_t*)out);
    return launch(k_attn_merge<float>, dim3(rows, 4), dim3(256), st, ev, part, nch, (float*)out);
  }
  if (dtype == 0)
    return launch(k_attn_merge_row<uint16_t>, dim3(rows), dim3(256), st, ev, part, nch,
                  (uint16_t*)out);
  return launch(k_attn_merge_row<float>, dim3(rows), dim3(256), st, ev, part, nch, (float*)out);
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
