// Host-only stand-ins for the library's kernel launchers, so that the
// C-ABI sources (pariskv_api.cpp, si_api.cpp) build with g++ under the
// address and undefined-behaviour sanitizers and their validation, layout,
// handle and error paths run without a GPU.  Every launcher succeeds
// without touching memory.  Host buffers the driver registers with
// stub_track() are checked: a 2-D copy (hipMemcpy2DAsync, replaced here by
// a host memcpy) or an encode that reads rows of such a buffer must stay
// inside it, and every encode is recorded.  Test infrastructure only.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "codebook_tables.h"
#include "launch_stubs.h"
#include "pariskv_internal.h"

namespace {
struct Tracked {
  const uint8_t* p;
  size_t n;
};
std::vector<Tracked> g_tracked;
std::vector<StubEncode> g_encodes;

// the tracked buffer holding [p, p + n), or null when p is in none
const Tracked* find_tracked(const void* p) {
  const uint8_t* b = (const uint8_t*)p;
  for (const Tracked& t : g_tracked)
    if (b >= t.p && b < t.p + t.n) return &t;
  return nullptr;
}
void check_range(const void* p, size_t n, const char* what) {
  const Tracked* t = find_tracked(p);
  if (!t) return;
  if ((const uint8_t*)p + n > t->p + t->n) {
    std::printf("out of bounds: %s reads/writes %zu bytes past its buffer\n", what,
                (size_t)((const uint8_t*)p + n - (t->p + t->n)));
    std::abort();
  }
}
}  // namespace

void stub_track(const void* p, size_t bytes) { g_tracked.push_back({(const uint8_t*)p, bytes}); }
void stub_untrack_all() { g_tracked.clear(); }
const std::vector<StubEncode>& stub_encodes() { return g_encodes; }
void stub_clear_encodes() { g_encodes.clear(); }

extern "C" hipError_t hipMemcpy2DAsync(void* dst, size_t dpitch, const void* src, size_t spitch,
                                       size_t width, size_t height, hipMemcpyKind kind,
                                       hipStream_t stream) {
  (void)kind;
  (void)stream;
  if (height == 0 || width == 0) return hipSuccess;
  if (!find_tracked(dst) || !find_tracked(src)) return hipErrorInvalidValue;
  check_range(dst, (height - 1) * dpitch + width, "copy destination");
  check_range(src, (height - 1) * spitch + width, "copy source");
  for (size_t r = 0; r < height; ++r)
    std::memmove((uint8_t*)dst + r * dpitch, (const uint8_t*)src + r * spitch, width);
  return hipSuccess;
}

namespace pkv {

hipError_t launch_encode(int m, int dtype, const void* K, int64_t rows_per_head, int64_t lo,
                         int64_t n, int BH, int64_t cap, uint8_t* ids, uint32_t* rec,
                         const SignMask& sg, float c, hipStream_t st, const EvPair& ev) {
  const size_t rb = (dtype == 0 ? 2 : 4) * 128;  // d = 128 rows of bf16 or fp32
  if (lo < 0 || n < 0 || lo + n > cap) {
    std::printf("encode past the index capacity: [%lld, %lld) of %lld\n", (long long)lo,
                (long long)(lo + n), (long long)cap);
    std::abort();
  }
  if (n > 0) check_range(K, ((size_t)(BH - 1) * rows_per_head + n) * rb, "encode");
  g_encodes.push_back({K, rows_per_head, lo, n});
  return hipSuccess;
}

hipError_t launch_qprep(int m, int dtype, const void* Q, int BH, int n_kv_heads, int G,
                        const SignMask& sg, float c, int rho, const Tiers& tw, uint8_t* lut,
                        float* yq, float* ptab, const AppendJob& app, int unit_div,
                        hipStream_t st, const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_scan(int kpt, int nchunks, int BH, const uint8_t* ids, int64_t cap, int64_t S,
                       int64_t E, const uint8_t* lut, uint8_t* scores, int64_t Epad,
                       uint32_t* chist, int chunk_stride, int nbins, int rstride,
                       int unit_div, hipStream_t st, const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_thresh(int BH, const uint32_t* chist, int chunk_stride, int nchunks, int nbins,
                         int rstride, int64_t C, int all_ties, int32_t* meta, uint32_t* coff,
                         hipStream_t st, const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_compact_rerank(int m, int kpt, int nchunks, int BH, const uint8_t* scores,
                                 int64_t Epad, int64_t S, int64_t E, const int32_t* meta,
                                 const uint32_t* coff, int chunk_stride, const float* ptab,
                                 const uint32_t* rec, int64_t cap, int32_t* cand, float* est,
                                 int64_t cstride, int64_t C, uint32_t* mm, int nbins,
                                 int unit_div, const uint32_t* chist, int rstride,
                                 int32_t* meta_out, hipStream_t st, const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_topk(int BH, const float* est, const int32_t* cand, int64_t cstride, int C,
                       int kprime, int S, int k, int P, const uint32_t* mmc, int chunk_stride,
                       int nchunks, uint32_t* range, uint16_t* rows, int32_t* tkmeta,
                       uint2* sorted, int32_t* out_idx, float* out_est, hipStream_t st,
                       const EvPair& ev_hist, const EvPair& ev_select) {
  return hipSuccess;
}

hipError_t launch_topk_counted(int BH, const float* est, const int32_t* cand, int64_t cstride,
                               const int32_t* cmeta, int Cmax, int grid_slices, int kprime,
                               int S, int k,
                               const uint32_t* mmc, int chunk_stride, int nchunks,
                               uint32_t* range, uint16_t* rows, int32_t* tkmeta, uint2* sorted,
                               int32_t* out_idx, float* out_est, hipStream_t st,
                               const EvPair& ev_hist, const EvPair& ev_select) {
  return hipSuccess;
}

hipError_t launch_si_build(int dtype, const void* K, int64_t rows_per_head, int64_t S, int64_t n,
                           int BH, int64_t cap, uint8_t* ids, float* mean, float* cb,
                           void* build_ws, hipStream_t st) {
  return hipSuccess;
}

hipError_t launch_si_encode(int dtype, const void* K, int64_t rows_per_head, int64_t lo, int64_t n,
                            int BH, const float* mean, int64_t cap, uint8_t* ids, hipStream_t st) {
  return hipSuccess;
}

hipError_t launch_si_lut(int dtype, const void* Q, int units, int n_kv_heads, int G,
                         const float* cb, float* lut, float* tab, float* range, hipStream_t st,
                         const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_si_scan(int kpt, int nchunks, int units, const uint8_t* ids, int64_t cap,
                          int64_t S, int64_t E, const float* tab, const float* range,
                          uint8_t* bins, int64_t Epad, uint32_t* chist, int chunk_stride,
                          hipStream_t st, const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_si_compact(int kpt, int nchunks, int units, const uint8_t* bins,
                             const uint8_t* ids, int64_t cap, const float* tab, int64_t Epad,
                             int64_t S, int64_t E, const int32_t* meta, const uint32_t* coff,
                             int chunk_stride, int32_t* cand, float* est, int64_t cstride,
                             uint32_t* mm, hipStream_t st, const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_si_scores(int units, const uint8_t* ids, int64_t cap, int64_t S, int64_t E,
                            const float* tab, float* fscore, int64_t Epad, hipStream_t st) {
  return hipSuccess;
}

hipError_t launch_attn_split(int dtype, int G, int rpl, const void* Q, const AttnRows& rs,
                             const int32_t* idx, int k, int batch, int n_kv_heads, float qscale,
                             float* part, int nch, hipStream_t st, const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_attn_merge(int dtype, const float* part, int nch, int rows, void* out,
                             hipStream_t st,
                         const EvPair& ev) {
  return hipSuccess;
}

hipError_t launch_retrieve_small(int m, int dtype, const void* Q, int BH, int n_kv_heads, int G,
                                 const SignMask& sg, float c, int rho, const Tiers& tw,
                                 const AppendJob& app, const uint8_t* ids, const uint32_t* rec,
                                 int64_t cap, int64_t S, int64_t E, int64_t C, int kprime, int k,
                                 int nbins, uint8_t* lut, float* yq, uint8_t* scores, int64_t Epad,
                                 int32_t* meta, int32_t* cand, float* est, int64_t cstride,
                                 int32_t* out_idx, float* out_est, hipStream_t st,
                                 const EvPair& ev) {
  return hipSuccess;
}

hipError_t noalloc_scratch(void** out) {
  *out = reinterpret_cast<void*>(uintptr_t(0x7f) << 24);  // never dereferenced
  return hipSuccess;
}

size_t si_build_ws_bytes(int BH, int64_t S, int64_t n) {
  return (size_t)BH * (size_t)(n > S ? n - S : 1) * 32 + 4096;
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
