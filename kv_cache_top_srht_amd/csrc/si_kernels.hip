// HIP kernels (gfx950 / CDNA4) for the Self-Indexing retrieval workload:
// one-pass sign-based vector quantisation of the keys and LUT-GEMV scoring in
// the compressed domain.
//
// Method: "Self-Indexing KVCache: Predicting Sparse Attention from Compressed
// Keys" (gist.science/paper/2603.14224), cited as [SI] with section names.
// Keys are centred by their channel means (Methodology A.4), split into 32
// sub-vectors of 4 coordinates (A.1), each coded by its sign pattern, one of
// 16 clusters (A.2); a cluster's centroid is the mean of its members (A.3).
// A query's LUT holds its inner product with every centroid and a key's
// score is the sum of its LUT entries (B).  The top-k by score and the sinks
// are attended with the library's split-K attention.
//
// Exactness: channel and cluster sums are accumulated in fp64 (per-chunk
// partials reduced in chunk order) and rounded once to fp32; ids, LUT and
// scores follow the fp32 operation order stated at each kernel (no
// contraction), so the selection is exact given those fp32 tables.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pariskv_device.h"
#include "pariskv_internal.h"

#pragma clang fp contract(off)

namespace pkv {

// ---------------------------------------------------------------------------
// SI1 channel sums of one chunk of kSiChunk keys: 16 lanes per key (8
// channels each), 16 keys side by side; each thread sums its keys
// sequentially in fp64, then the 16 row slots are added in slot order.
// partial[bh][chunk][c], over keys [lo, hi) of each (b, h).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_si_colsum(const T* __restrict__ K, int64_t rows_per_head,
                                                   int64_t lo, int64_t hi,
                                                   double* __restrict__ partial, int nchunk) {
  const int chunk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int sub = tid & 15, slot = tid >> 4;
  __shared__ double s_p[16][129];
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  const int64_t r0 = lo + (int64_t)chunk * kSiChunk;
  const int64_t r1 = (r0 + kSiChunk < hi) ? r0 + kSiChunk : hi;
  for (int64_t r = r0 + slot; r < r1; r += 16) {
    float x[8];
    load8(K + (((int64_t)bh * rows_per_head + r) << 7) + sub * 8, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += (double)x[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) s_p[slot][sub * 8 + j] = acc[j];
  __syncthreads();
  if (tid < 128) {
    double a = s_p[0][tid];
#pragma unroll
    for (int s = 1; s < 16; ++s) a += s_p[s][tid];
    partial[((int64_t)bh * nchunk + chunk) * 128 + tid] = a;
  }
}

// SI2 channel means mu_c = fp32((sum over chunks, in order) / n); n = 0
// gives mu = 0.  One 128-thread block per (b, h).
__global__ __launch_bounds__(128) void k_si_mean(const double* __restrict__ partial, int nchunk,
                                                 int64_t n, float* __restrict__ mean) {
  const int bh = blockIdx.x, c = threadIdx.x;
  double a = 0.0;
  for (int k = 0; k < nchunk; ++k) a += partial[((int64_t)bh * nchunk + k) * 128 + c];
  mean[bh * 128 + c] = n > 0 ? (float)(a / (double)n) : 0.0f;
}

// ---------------------------------------------------------------------------
// Sign ids of centred keys.  Coordinate c of a key: y_c = fp32(x_c - mu_c);
// sub-vector b (coordinates 4 b .. 4 b + 3) has id_b = sum_j [y_{4b+j} < 0] 2^j
// (a zero goes to the + side).  Byte s of a key's 16-byte id row holds id_2s
// in its low nibble and id_2s+1 in its high nibble, i.e. it is the sign
// pattern of coordinates 8 s .. 8 s + 7.
// ---------------------------------------------------------------------------

// SI3 (build) ids of keys [0, n) and the per-chunk cluster sums of the keys
// in [lo, n): thread c owns coordinate c; for each key in order it adds y_c
// to its cluster's fp64 sum in LDS (column c of s_acc, so threads never
// share a word), and lane j = 0 of a sub-vector counts the key.
// psum[bh][chunk][p][c] (fp64), pcnt[bh][chunk][p][b].
template <typename T>
__global__ __launch_bounds__(128) void k_si_encode_sums(const T* __restrict__ K,
                                                        int64_t rows_per_head, int64_t lo,
                                                        int64_t n, const float* __restrict__ mean,
                                                        int64_t cap, uint8_t* __restrict__ ids,
                                                        double* __restrict__ psum,
                                                        uint32_t* __restrict__ pcnt, int nchunk) {
  const int chunk = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const int lane = c & 63, b = c >> 2, j = c & 3;
  __shared__ double s_acc[16][128];
  __shared__ uint32_t s_cnt[16][32];
  for (int p = 0; p < 16; ++p) s_acc[p][c] = 0.0;
  for (int i = c; i < 16 * 32; i += 128) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  const float mu = mean[bh * 128 + c];
  const int64_t r0 = (int64_t)chunk * kSiChunk;
  const int64_t r1 = (r0 + kSiChunk < n) ? r0 + kSiChunk : n;
  const T* kp = K + (int64_t)bh * rows_per_head * 128 + c;
  for (int64_t r = r0; r < r1; ++r) {
    const float x = to_f32(kp[r * 128]);
    const float y = x - mu;
    const uint64_t neg = __ballot(y < 0.0f);
    const uint32_t id = (uint32_t)(neg >> (lane & ~3)) & 15u;
    if ((c & 7) == 0) {
      const uint32_t idn = (uint32_t)(neg >> ((lane & ~7) + 4)) & 15u;
      ids[((int64_t)bh * cap + r) * 16 + (c >> 3)] = (uint8_t)(id | (idn << 4));
    }
    if (r >= lo) {
      s_acc[id][c] += (double)y;
      if (j == 0) s_cnt[id][b] += 1u;
    }
  }
  __syncthreads();
  double* ps = psum + ((int64_t)bh * nchunk + chunk) * 2048;
  for (int p = 0; p < 16; ++p) ps[p * 128 + c] = s_acc[p][c];
  uint32_t* pc = pcnt + ((int64_t)bh * nchunk + chunk) * 512;
  for (int i = c; i < 512; i += 128) pc[i] = (&s_cnt[0][0])[i];
}

// SI4 codebook: centroid (b, p) = fp32((sum over chunks, in order) / count),
// 0 for an empty cluster.  cb[bh][b][p][j] (j = coordinate within the
// sub-vector).  One 256-thread block per (b, h).
__global__ __launch_bounds__(256) void k_si_codebook(const double* __restrict__ psum,
                                                     const uint32_t* __restrict__ pcnt,
                                                     int nchunk, float* __restrict__ cb) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < 2048; e += 256) {
    const int p = e >> 7, c = e & 127, b = c >> 2, j = c & 3;
    double a = 0.0;
    uint32_t cnt = 0;
    for (int k = 0; k < nchunk; ++k) {
      a += psum[((int64_t)bh * nchunk + k) * 2048 + e];
      cnt += pcnt[((int64_t)bh * nchunk + k) * 512 + p * 32 + b];
    }
    cb[(int64_t)bh * 2048 + (b * 16 + p) * 4 + j] = cnt ? (float)(a / (double)cnt) : 0.0f;
  }
}

// SI5 (append) ids of keys [lo, lo + n) with the stored means: 16 lanes per
// key, lane s forming byte s from coordinates 8 s .. 8 s + 7.
template <typename T>
__global__ __launch_bounds__(256) void k_si_encode(const T* __restrict__ K, int64_t rows_per_head,
                                                   int64_t lo, int64_t n, int64_t total,
                                                   const float* __restrict__ mean, int64_t cap,
                                                   uint8_t* __restrict__ ids) {
  const int sub = threadIdx.x & 15;
  const int64_t g = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (g >= total) return;
  const int64_t bh = g / n, r = g - bh * n;
  float x[8];
  load8(K + ((bh * rows_per_head + r) << 7) + sub * 8, x);
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float y = x[j] - mean[bh * 128 + sub * 8 + j];
    v |= (y < 0.0f ? 1u : 0u) << j;
  }
  ids[(bh * cap + lo + r) * 16 + sub] = (uint8_t)v;
}

// ---------------------------------------------------------------------------
// SI6 query LUT ([SI] Methodology B): the unit's query qbar (mean of its G
// query heads, (q_0 + ... + q_{G-1}) * fp32(1/G) in head order);
//   lut_b[p] = ((0 + qbar_{4b} c_{b,p,0}) + qbar_{4b+1} c_{b,p,1}) + ...
// then the byte table the scan reads, one row per id byte s:
//   tab[s][v] = lut_2s[v & 15] + lut_2s+1[v >> 4]
// and the score range: lo = sum_s min_v tab[s][v], hi = sum_s max_v tab[s][v]
// (fp32, s ascending, the scan's order, so every score lies in [lo, hi]);
// bin scale = 255 / (hi - lo) (0 if not finite and positive).
// One 512-thread block per unit: thread (b, p) = (tid >> 4, tid & 15).
// ---------------------------------------------------------------------------
template <typename T, int G>
__global__ __launch_bounds__(512) void k_si_lut(const T* __restrict__ Q, int n_kv_heads,
                                                float invG, const float* __restrict__ cb,
                                                float* __restrict__ lut_out,
                                                float* __restrict__ tab_out,
                                                float* __restrict__ range_out) {
  const int u = blockIdx.x, tid = threadIdx.x;
  const int bb = u / n_kv_heads, h = u - bb * n_kv_heads;
  const int b = tid >> 4, p = tid & 15;
  __shared__ float s_lut[32][16];
  __shared__ float s_mn[16], s_mx[16];
  const T* q0 = Q + ((int64_t)(bb * n_kv_heads + h) * G << 7) + 4 * b;
  float qb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = to_f32(q0[j]);
#pragma unroll
    for (int g = 1; g < G; ++g) a = a + to_f32(q0[(g << 7) + j]);
    qb[j] = a * invG;
  }
  const float* c = cb + (int64_t)u * 2048 + (b * 16 + p) * 4;
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s = s + qb[j] * c[j];
  s_lut[b][p] = s;
  lut_out[(int64_t)u * 512 + tid] = s;
  __syncthreads();
  // byte table: 4096 entries, 8 per thread; row minima and maxima
  float* tb = tab_out + (int64_t)u * 4096;
  for (int e = tid; e < 4096; e += 512) {
    const int r = e >> 8, v = e & 255;
    tb[e] = s_lut[2 * r][v & 15] + s_lut[2 * r + 1][v >> 4];
  }
  if (tid < 16) {
    float mn0 = s_lut[2 * tid][0], mx0 = mn0, mn1 = s_lut[2 * tid + 1][0], mx1 = mn1;
    for (int q = 1; q < 16; ++q) {
      mn0 = fminf(mn0, s_lut[2 * tid][q]);
      mx0 = fmaxf(mx0, s_lut[2 * tid][q]);
      mn1 = fminf(mn1, s_lut[2 * tid + 1][q]);
      mx1 = fmaxf(mx1, s_lut[2 * tid + 1][q]);
    }
    // the smallest (largest) table entry of row tid is the sum of the
    // smallest (largest) entries of its two sub-vectors (fp32 addition is
    // monotone in each operand)
    s_mn[tid] = mn0 + mn1;
    s_mx[tid] = mx0 + mx1;
  }
  __syncthreads();
  if (tid == 0) {
    float lo = 0.0f, hi = 0.0f;
    for (int r = 0; r < 16; ++r) {
      lo = lo + s_mn[r];
      hi = hi + s_mx[r];
    }
    float scale = 255.0f / (hi - lo);
    if (!(scale < INFINITY) || !(scale > 0.0f)) scale = 0.0f;
    range_out[u * 2 + 0] = lo;
    range_out[u * 2 + 1] = scale;
  }
}

// bin of a score in [lo, hi]: monotone non-decreasing in the score
__device__ __forceinline__ uint32_t si_bin(float s, float lo, float scale) {
  return (uint32_t)fminf((s - lo) * scale, 255.0f);
}

// A key's LUT-GEMV score from its 16 id bytes and the unit's byte table
// (LDS or global): (((0 + tab[0][byte_0]) + tab[1][byte_1]) + ...) in fp32.
__device__ __forceinline__ float si_score(const uint4 x, const float* tab) {
  const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s = s + tab[r * 256 + ((w4[r >> 2] >> ((r & 3) * 8)) & 0xFFu)];
  return s;
}

// ---------------------------------------------------------------------------
// SI7 LUT-GEMV scan ([SI] Methodology B): for keys i in [S, N)
//   score_i = (((0 + tab[0][byte_0]) + tab[1][byte_1]) + ...) + tab[15][byte_15]
// (fp32, 16 LDS reads per key); writes its bin (one byte) and a cumulative
// per-chunk row #(bin >= v) of the bins, as the vote scan does for vote
// scores, so the threshold and compaction kernels serve both.  The fp32 score
// itself is not stored: the compaction recomputes it for the candidates.
// Grid (chunks, units), KPT * NT keys per chunk.
// ---------------------------------------------------------------------------
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void k_si_scan(const uint4* __restrict__ ids, int64_t cap,
                                                int64_t S, int64_t E,
                                                const float* __restrict__ tab,
                                                const float* __restrict__ range,
                                                uint8_t* __restrict__ bins, int64_t Epad,
                                                uint32_t* __restrict__ chist, int chunk_stride) {
  constexpr int NW = NT / 64;
  const int u = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  __shared__ float s_tab[16 * 256];
  __shared__ uint32_t s_hist[NW][256];
  float4 tv[4096 / 4 / NT];
#pragma unroll
  for (int i = 0; i < 4096 / 4 / NT; ++i)
    tv[i] = reinterpret_cast<const float4*>(tab + (int64_t)u * 4096)[tid + i * NT];
  const float lo = range[2 * u], scale = range[2 * u + 1];
  const uint4* src = ids + (int64_t)u * cap + S;
  const int64_t p0 = (int64_t)chunk * (KPT * NT) + tid;
  uint4 x[KPT];
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int64_t p = p0 + t * NT;
    x[t] = load_stream(&src[p < E ? p : E - 1]);
  }
#pragma unroll
  for (int i = 0; i < 4096 / 4 / NT; ++i) reinterpret_cast<float4*>(s_tab)[tid + i * NT] = tv[i];
  for (int i = tid; i < NW * 256; i += NT) (&s_hist[0][0])[i] = 0;
  __syncthreads();
  uint32_t zeros = 0;
#pragma unroll
  for (int t = 0; t < KPT; ++t) {
    const int64_t p = p0 + t * NT;
    const bool valid = p < E;
    const uint32_t bn = si_bin(si_score(x[t], s_tab), lo, scale);
    zeros += (uint32_t)__popcll(__ballot(valid && bn == 0));
    if (valid) {
      bins[(int64_t)u * Epad + p] = (uint8_t)bn;
      if (bn != 0) atomicAdd(&s_hist[wv][bn], 1u);
    }
  }
  if (lane == 0) s_hist[wv][0] = zeros;
  __syncthreads();
  for (int v = tid; v < 256; v += NT) {
    uint32_t a = s_hist[0][v];
#pragma unroll
    for (int w = 1; w < NW; ++w) a += s_hist[w][v];
    s_hist[0][v] = a;
  }
  __syncthreads();
  if (wv == 0) {
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = s_hist[0][4 * lane + r];
    const uint32_t loc = h[0] + h[1] + h[2] + h[3];
    uint32_t inc = wave_incl_scan(loc);   // sum over lanes <= this one
    const uint32_t total = (uint32_t)__shfl((int)inc, 63);
    const uint32_t above = total - inc;   // sum over lanes > this one
    uint32_t ge[4];
    ge[3] = above + h[3];
    ge[2] = ge[3] + h[2];
    ge[1] = ge[2] + h[1];
    ge[0] = ge[1] + h[0];
    uint32_t* row = chist + ((int64_t)u * chunk_stride + chunk) * 256;
    reinterpret_cast<uint4*>(row)[lane] = make_uint4(ge[0], ge[1], ge[2], ge[3]);
  }
}

// ---------------------------------------------------------------------------
// SI8 candidates of two consecutive chunks: every key whose bin is >= T (the
// bin holding rank k', found by the threshold kernel with all of T's keys
// kept), listed in ascending position order at the chunk's offset with its
// fp32 score (recomputed from the key's ids and the byte table in global
// memory, the scan's order of additions); plus the block's score range
// (order keys) for the top-k.
// Grid (ceil(chunks / 2), units), 256 threads, KPT keys per thread.
// ---------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(256) void k_si_compact(const uint8_t* __restrict__ bins,
                                                    const uint4* __restrict__ ids, int64_t cap,
                                                    const float* __restrict__ tab,
                                                    int64_t Epad, int64_t S, int64_t E,
                                                    const int32_t* __restrict__ meta,
                                                    const uint32_t* __restrict__ coff,
                                                    int chunk_stride, int nchunks,
                                                    int32_t* __restrict__ cand,
                                                    float* __restrict__ est, int64_t cstride,
                                                    uint32_t* __restrict__ mm) {
  constexpr int CH = KPT * 256;
  const int u = blockIdx.y, tid = threadIdx.x;
  const int c0 = blockIdx.x * 2;
  const int nc = (c0 + 1 < nchunks) ? 2 : 1;
  __shared__ uint16_t s_list[2 * CH];
  __shared__ uint2 s_w2[4];
  __shared__ uint32_t s_mm[8];
  const int T = meta[u * 4 + 0];
  uint32_t off_c[2], msk[2];
  uint8_t bv[2][KPT];
  // loads first, unconditional (bins past E lie inside the padded row)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int chunk = c0 + (h < nc ? h : 0);
    off_c[h] = coff[((int64_t)u * chunk_stride + chunk) * 2 + 0];
    load_scores<KPT>(bins + (int64_t)u * Epad + (int64_t)chunk * CH + tid * KPT, bv[h]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    msk[h] = 0;
    const int64_t base = (int64_t)(c0 + h) * CH + tid * KPT;
#pragma unroll
    for (int t = 0; t < KPT; ++t)
      if (h < nc && base + t < E && (int)bv[h][t] >= T) msk[h] |= 1u << t;
  }
  uint2 tot;
  const uint2 ex = block_exscan_packed<256>(
      make_uint2((uint32_t)__popc(msk[0]), (uint32_t)__popc(msk[1])), s_w2, tot);
  const uint32_t n0 = tot.x, ntot = tot.x + tot.y;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t sel = msk[h];
    uint32_t pos = (h ? n0 + ex.y : ex.x);
    while (sel) {
      const int t = __builtin_ctz(sel);
      s_list[pos++] = (uint16_t)((h << 14) | (tid * KPT + t));
      sel &= sel - 1u;
    }
  }
  __syncthreads();
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
  const uint4* src = ids + (int64_t)u * cap + S;
  const float* tb = tab + (int64_t)u * 4096;
  for (uint32_t j = tid; j < ntot; j += 256) {
    const uint32_t ent = s_list[j];
    const int h = (int)(ent >> 14);
    const int64_t q = (int64_t)(c0 + h) * CH + (ent & 0x3FFFu);  // eligible index
    const float e = si_score(src[q], tb);
    const uint32_t o = (j >= n0) ? off_c[1] + (j - n0) : off_c[0] + j;
    cand[(int64_t)u * cstride + o] = (int32_t)(S + q);
    est[(int64_t)u * cstride + o] = e;
    const uint32_t ok = order_key(e);
    kmn = min(kmn, ok);
    kmx = max(kmx, ok);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, off));
    kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, off));
  }
  if ((tid & 63) == 0) { s_mm[tid >> 6] = kmn; s_mm[4 + (tid >> 6)] = kmx; }
  __syncthreads();
  if (tid < 2) {
    const int chunk = c0 + (tid < nc ? tid : 0);
    mm[((int64_t)u * chunk_stride + chunk) * 2 + 0] = min(min(s_mm[0], s_mm[1]), min(s_mm[2], s_mm[3]));
    mm[((int64_t)u * chunk_stride + chunk) * 2 + 1] = max(max(s_mm[4], s_mm[5]), max(s_mm[6], s_mm[7]));
  }
}

// Every eligible key's fp32 score, for parity introspection only (the
// retrieval keeps bins): the scan's arithmetic from the table in global
// memory.  Grid (ceil(E / 256), units).
__global__ __launch_bounds__(256) void k_si_scores(const uint4* __restrict__ ids, int64_t cap,
                                                   int64_t S, int64_t E,
                                                   const float* __restrict__ tab,
                                                   float* __restrict__ fscore, int64_t Epad) {
  const int u = blockIdx.y;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p < E) fscore[(int64_t)u * Epad + p] = si_score(ids[(int64_t)u * cap + S + p],
                                                      tab + (int64_t)u * 4096);
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_si_build(int dtype, const void* K, int64_t rows_per_head, int64_t S, int64_t n,
                           int BH, int64_t cap, uint8_t* ids, float* mean, float* cb,
                           void* build_ws, hipStream_t st) {
  // keys [S, n) define the means and the codebook; ids cover [0, n)
  const int64_t m = n > S ? n - S : 0;
  const int nck = (int)((m + kSiChunk - 1) / kSiChunk);
  const int nce = (int)((n + kSiChunk - 1) / kSiChunk);
  const int ncb = nck > 1 ? nck : 1;
  double* colp = (double*)build_ws;
  double* psum = colp + (size_t)BH * ncb * 128;
  uint32_t* pcnt = (uint32_t*)(psum + (size_t)BH * (nce > 0 ? nce : 1) * 2048);
  const EvPair none{};
  hipError_t e = hipSuccess;
  if (nck > 0) {
    e = dtype == 0 ? launch(k_si_colsum<uint16_t>, dim3(nck, BH), dim3(256), st, none,
                            (const uint16_t*)K, rows_per_head, S, n, colp, nck)
                   : launch(k_si_colsum<float>, dim3(nck, BH), dim3(256), st, none,
                            (const float*)K, rows_per_head, S, n, colp, nck);
    if (e != hipSuccess) return e;
  }
  e = launch(k_si_mean, dim3(BH), dim3(128), st, none, (const double*)colp, nck, m, mean);
  if (e != hipSuccess || nce == 0) return e;
  e = dtype == 0 ? launch(k_si_encode_sums<uint16_t>, dim3(nce, BH), dim3(128), st, none,
                          (const uint16_t*)K, rows_per_head, S, n, (const float*)mean, cap, ids,
                          psum, pcnt, nce)
                 : launch(k_si_encode_sums<float>, dim3(nce, BH), dim3(128), st, none,
                          (const float*)K, rows_per_head, S, n, (const float*)mean, cap, ids,
                          psum, pcnt, nce);
  if (e != hipSuccess) return e;
  return launch(k_si_codebook, dim3(BH), dim3(256), st, none, (const double*)psum,
                (const uint32_t*)pcnt, nce, cb);
}

size_t si_build_ws_bytes(int BH, int64_t S, int64_t n) {
  const int64_t m = n > S ? n - S : 0;
  const int64_t nck = (m + kSiChunk - 1) / kSiChunk, nce = (n + kSiChunk - 1) / kSiChunk;
  return (size_t)BH * (nck > 1 ? nck : 1) * 128 * 8 + (size_t)BH * (nce > 0 ? nce : 1) * 2048 * 8 +
         (size_t)BH * (nce > 0 ? nce : 1) * 512 * 4;
}

hipError_t launch_si_encode(int dtype, const void* K, int64_t rows_per_head, int64_t lo, int64_t n,
                            int BH, const float* mean, int64_t cap, uint8_t* ids, hipStream_t st) {
  const int64_t total = (int64_t)BH * n;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 15) / 16));
  const EvPair none{};
  if (dtype == 0)
    return launch(k_si_encode<uint16_t>, grid, dim3(256), st, none, (const uint16_t*)K,
                  rows_per_head, lo, n, total, mean, cap, ids);
  return launch(k_si_encode<float>, grid, dim3(256), st, none, (const float*)K, rows_per_head, lo,
                n, total, mean, cap, ids);
}

hipError_t launch_si_lut(int dtype, const void* Q, int units, int n_kv_heads, int G,
                         const float* cb, float* lut, float* tab, float* range, hipStream_t st,
                         const EvPair& ev) {
  const float invG = 1.0f / (float)G;
#define PKV_SL(T, GG)                                                                            \
  return launch(k_si_lut<T, GG>, dim3(units), dim3(512), st, ev, (const T*)Q, n_kv_heads, invG, \
                cb, lut, tab, range)
  if (dtype == 0) {
    switch (G) {
      case 1: PKV_SL(uint16_t, 1);
      case 2: PKV_SL(uint16_t, 2);
      case 4: PKV_SL(uint16_t, 4);
      case 8: PKV_SL(uint16_t, 8);
      default: return hipErrorInvalidValue;
    }
  }
  switch (G) {
    case 1: PKV_SL(float, 1);
    case 2: PKV_SL(float, 2);
    case 4: PKV_SL(float, 4);
    case 8: PKV_SL(float, 8);
    default: return hipErrorInvalidValue;
  }
#undef PKV_SL
}

hipError_t launch_si_scan(int kpt, int nchunks, int units, const uint8_t* ids, int64_t cap,
                          int64_t S, int64_t E, const float* tab, const float* range,
                          uint8_t* bins, int64_t Epad, uint32_t* chist, int chunk_stride,
                          hipStream_t st, const EvPair& ev) {
  const dim3 grid(nchunks, units);
  const uint4* id4 = (const uint4*)ids;
  switch (kpt) {
#define PKV_SS(K, NT)                                                                          \
  case K:                                                                                      \
    return launch(k_si_scan<(K * 256) / NT, NT>, grid, dim3(NT), st, ev, id4, cap, S, E, tab, \
                  range, bins, Epad, chist, chunk_stride);
    PKV_SS(1, 256) PKV_SS(2, 256) PKV_SS(4, 512) PKV_SS(8, 512) PKV_SS(16, 512)
#undef PKV_SS
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_si_compact(int kpt, int nchunks, int units, const uint8_t* bins,
                             const uint8_t* ids, int64_t cap, const float* tab, int64_t Epad,
                             int64_t S, int64_t E, const int32_t* meta, const uint32_t* coff,
                             int chunk_stride, int32_t* cand, float* est, int64_t cstride,
                             uint32_t* mm, hipStream_t st, const EvPair& ev) {
  const dim3 grid((nchunks + 1) / 2, units);
  switch (kpt) {
#define PKV_SC(K)                                                                              \
  case K:                                                                                      \
    return launch(k_si_compact<K>, grid, dim3(256), st, ev, bins, (const uint4*)ids, cap, tab, \
                  Epad, S, E, meta, coff, chunk_stride, nchunks, cand, est, cstride, mm);
    PKV_SC(1) PKV_SC(2) PKV_SC(4) PKV_SC(8) PKV_SC(16)
#undef PKV_SC
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_si_scores(int units, const uint8_t* ids, int64_t cap, int64_t S, int64_t E,
                            const float* tab, float* fscore, int64_t Epad, hipStream_t st) {
  if (E <= 0) return hipSuccess;
  const dim3 grid((unsigned)((E + 255) / 256), units);
  return launch(k_si_scores, grid, dim3(256), st, EvPair{}, (const uint4*)ids, cap, S, E, tab,
                fscore, Epad);
}

}  // namespace pkv
