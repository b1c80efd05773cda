// Internal declarations shared by the kernels and the C ABI host code of the
// ParisKV retrieval library (not installed; the public ABI is pariskv.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Rotation signs D as a bitmask (bit j set <=> D_j = -1), d <= 128.
struct SignMask {
  uint32_t w[4];
};

// Vote weight of the s-th ranked centroid.
struct Tiers {
  int32_t w[8];
};

// Keys appended to the index but not yet encoded: rows [0, n) of each (b, h)
// of K go to positions [lo, lo + n).  The query-prep kernel of the next
// retrieval encodes them (n <= kMaxFusedAppend).
struct AppendJob {
  const void* K = nullptr;
  int64_t rows_per_head = 0;
  int64_t lo = 0;
  int64_t cap = 0;
  uint8_t* ids = nullptr;
  uint32_t* rec = nullptr;
  int n = 0;
};
constexpr int kMaxFusedAppend = 48;
// scan chunks per compact + rerank block (1 or 2)
constexpr int kCompactChunks = 2;
// up to this many chunks per unit, compact + rerank finds the threshold itself
constexpr int kFusedThreshChunks = 256;
// threads of a vote-scan block (256 or 512; chunks of 4+ keys per 256 threads)
constexpr int kScanThreads = 512;

// Optional timing events stamped by a kernel's own dispatch (null: none).
struct EvPair {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_encode(int m, int dtype, const void* K, int64_t rows_per_head, int64_t lo,
                         int64_t n, int BH, int64_t cap, uint8_t* ids, uint32_t* rec,
                         const SignMask& sg, float c, hipStream_t st, const EvPair& ev);
hipError_t launch_qprep(int m, int dtype, const void* Q, int BH, int n_kv_heads, int G,
                        const SignMask& sg, float c, int rho, const Tiers& tw, uint8_t* lut,
                        float* yq, float* ptab, const AppendJob& app, int unit_div,
                        hipStream_t st, const EvPair& ev);
hipError_t launch_scan(int kpt, int nchunks, int BH, const uint8_t* ids, int64_t cap, int64_t S,
                       int64_t E, const uint8_t* lut, uint8_t* scores, int64_t Epad,
                       uint32_t* chist, int chunk_stride, int nbins, int rstride,
                       int unit_div, hipStream_t st, const EvPair& ev);
hipError_t launch_thresh(int BH, const uint32_t* chist, int chunk_stride, int nchunks, int nbins,
                         int rstride, int64_t C, int all_ties, int32_t* meta, uint32_t* coff,
                         hipStream_t st, const EvPair& ev);
// chist (optional, nchunks <= kFusedThreshChunks): the chunk rows, read
// instead of meta / coff (no threshold kernel); meta_out then receives meta
hipError_t launch_compact_rerank(int m, int kpt, int nchunks, int BH, const uint8_t* scores,
                                 int64_t Epad, int64_t S, int64_t E, const int32_t* meta,
                                 const uint32_t* coff, int chunk_stride, const float* ptab,
                                 const uint32_t* rec, int64_t cap, int32_t* cand, float* est,
                                 int64_t cstride, int64_t C, uint32_t* mm, int nbins,
                                 int unit_div, const uint32_t* chist, int rstride,
                                 int32_t* meta_out, hipStream_t st, const EvPair& ev);
hipError_t launch_topk(int BH, const float* est, const int32_t* cand, int64_t cstride, int C,
                       int kprime, int S, int k, int P, const uint32_t* mmc, int chunk_stride,
                       int nchunks, uint32_t* range, uint16_t* rows, int32_t* tkmeta,
                       uint2* sorted, int32_t* out_idx, float* out_est, hipStream_t st,
                       const EvPair& ev_hist, const EvPair& ev_select);
// top-k with per-unit candidate counts read from cmeta[unit * 4 + 3] on the
// device (at most Cmax); hist + general select, grid_slices blocks per unit
// The whole retrieval of every unit in one kernel (shared retrieval, E >= 1,
// 1 <= k' <= C <= kSmallTopkSlices * kTopkSlice, at most 64 appended keys).
hipError_t launch_retrieve_small(int m, int dtype, const void* Q, int BH, int n_kv_heads, int G,
                                 const SignMask& sg, float c, int rho, const Tiers& tw,
                                 const AppendJob& app, const uint8_t* ids, const uint32_t* rec,
                                 int64_t cap, int64_t S, int64_t E, int64_t C, int kprime, int k,
                                 int nbins, uint8_t* lut, float* yq, uint8_t* scores, int64_t Epad,
                                 int32_t* meta, int32_t* cand, float* est, int64_t cstride,
                                 int32_t* out_idx, float* out_est, hipStream_t st,
                                 const EvPair& ev);
hipError_t launch_topk_counted(int BH, const float* est, const int32_t* cand, int64_t cstride,
                               const int32_t* cmeta, int Cmax, int grid_slices, int kprime,
                               int S, int k,
                               const uint32_t* mmc, int chunk_stride, int nchunks,
                               uint32_t* range, uint16_t* rows, int32_t* tkmeta, uint2* sorted,
                               int32_t* out_idx, float* out_est, hipStream_t st,
                               const EvPair& ev_hist, const EvPair& ev_select);

// Self-Indexing workload: keys per build chunk (channel and cluster sums)
constexpr int kSiChunk = 4096;
size_t si_build_ws_bytes(int BH, int64_t S, int64_t n);
hipError_t launch_si_build(int dtype, const void* K, int64_t rows_per_head, int64_t S, int64_t n,
                           int BH, int64_t cap, uint8_t* ids, float* mean, float* cb,
                           void* build_ws, hipStream_t st);
hipError_t launch_si_encode(int dtype, const void* K, int64_t rows_per_head, int64_t lo, int64_t n,
                            int BH, const float* mean, int64_t cap, uint8_t* ids, hipStream_t st);
hipError_t launch_si_lut(int dtype, const void* Q, int units, int n_kv_heads, int G,
                         const float* cb, float* lut, float* tab, float* range, hipStream_t st,
                         const EvPair& ev);
hipError_t launch_si_scan(int kpt, int nchunks, int units, const uint8_t* ids, int64_t cap,
                          int64_t S, int64_t E, const float* tab, const float* range,
                          uint8_t* bins, int64_t Epad, uint32_t* chist, int chunk_stride,
                          hipStream_t st, const EvPair& ev);
hipError_t launch_si_compact(int kpt, int nchunks, int units, const uint8_t* bins,
                             const uint8_t* ids, int64_t cap, const float* tab, int64_t Epad,
                             int64_t S, int64_t E, const int32_t* meta, const uint32_t* coff,
                             int chunk_stride, int32_t* cand, float* est, int64_t cstride,
                             uint32_t* mm, hipStream_t st, const EvPair& ev);
// every eligible key's fp32 score (parity introspection)
hipError_t launch_si_scores(int units, const uint8_t* ids, int64_t cap, int64_t S, int64_t E,
                            const float* tab, float* fscore, int64_t Epad, hipStream_t st);

// candidates per top-k block and the largest threshold bin ranked pairwise
constexpr int kTopkSlice = 4096;
constexpr int kTopkMaxMembers = 4096;
// up to this many slices per (b, h), top-k runs as one kernel (every block
// reads all of its (b, h)'s estimates: cheaper than a second kernel while
// the slices are few)
constexpr int kTopkFusedSlices = 4;
// the single-kernel retrieval holds up to this many slices of candidates
constexpr int kSmallTopkSlices = 4;
// up to these sizes per unit it keeps every key's ids and score and every
// candidate in registers and LDS (the resident variant)
constexpr int kTinyKeys = 8192;
constexpr int kTinyCands = 2048;
// up to this many slices, the select kernel loads all histogram rows at once
constexpr int kTopkFewSlices = 16;
// split-K attention partial per (query head, chunk): o[128], m, l, 2 unused
constexpr int kPartStride = 132;
// Split attention: a block of 16 row slots takes rpl rows per slot, a chunk
// of 16 rpl selected rows (one split-K partial per query head and chunk).
// rpl = 2 (32-row chunks) when the grid of 64-row chunks would hold fewer
// than kAttnSmallGrid blocks, else 4; workspaces are sized for the smaller
// chunk.
constexpr int kAttnChunkRowsMin = 32;
constexpr int64_t kAttnSmallGrid = 1024;
inline int attn_rows_per_lane(int64_t rows, int64_t units) {
  return units * ((rows + 63) / 64) < kAttnSmallGrid ? 2 : 4;
}
// the merge takes four blocks per (b, query head) below this many of them
constexpr int kMergeSplitRows = 128;
// Where attention rows come from.  Listed positions p (from idx) are read
// from the near store when p < n_near_head, else from the far store; the
// tail_n rows after the list are positions tail_lo + t, read from the near
// store's ring at n_near_head + (p - n_near_head) % ring.  Plain sparse
// attention: far store only (n_near_head = 0, tail_n = 0).
struct AttnRows {
  const void* K = nullptr;       // far store [b][h][rows][d]
  const void* V = nullptr;
  int64_t rows = 0;
  const void* K_near = nullptr;  // near store [b][h][near_rows][d]
  const void* V_near = nullptr;
  int64_t near_rows = 0;
  int64_t n_near_head = 0;       // positions [0, n_near_head) live in the near store
  int64_t ring = 1;
  int64_t tail_lo = 0;
  int tail_n = 0;
  int unit_div = 1;              // attention units (blocks.y) per KV head of K and V
};
hipError_t launch_attn_split(int dtype, int G, int rpl, const void* Q, const AttnRows& rs,
                             const int32_t* idx, int k, int batch, int n_kv_heads, float qscale,
                             float* part, int nch, hipStream_t st, const EvPair& ev);
hipError_t launch_attn_merge(int dtype, const float* part, int nch, int rows, void* out,
                             hipStream_t st,
                         const EvPair& ev);
// Device scratch of the entry point that allocates nothing: a file-scope
// array of this many bytes per GPU; noalloc_scratch() returns its address on
// the current device (resolved once per device, then kept).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** out);

void codebook_m8(float* L, float* tau);
void codebook_m4(float* L, float* tau);

}  // namespace pkv
