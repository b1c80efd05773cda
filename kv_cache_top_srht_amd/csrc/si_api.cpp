// C ABI of the Self-Indexing retrieval workload ("Self-Indexing KVCache:
// Predicting Sparse Attention from Compressed Keys", Methodology A-C):
// validation, buffer layouts and launch sequencing.  Declarations and their
// contracts are in include/pariskv.h; the kernels are in si_kernels.hip, the
// threshold and top-k kernels are shared with the ParisKV path.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>
#include <vector>

#include "pariskv.h"
#include "pariskv_internal.h"

struct pariskv_si_index {
  pariskv_si_config cfg;
  uint8_t* ids;  // [BH][cap][16]  two 4-bit sign ids per byte
  float* mean;   // [BH][128]      channel means of the indexed prefill keys
  float* cb;     // [BH][32][16][4] cluster centroids
  int64_t n;     // keys per (b, h)
};

namespace {

constexpr size_t kAlign = 256;
// top-k slices per unit the general select handles
constexpr int64_t kMaxSlices = 1024;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int32_t hip_status(hipError_t e) { return e == hipSuccess ? PARISKV_OK : PARISKV_ERR_HIP; }

int32_t check_si_cfg(const pariskv_si_config* c) {
  if (!c) return PARISKV_ERR_INVALID_ARG;
  if (c->head_dim < 2 || c->head_dim > 1024 || (c->head_dim & (c->head_dim - 1)))
    return PARISKV_ERR_INVALID_ARG;
  if (c->n_sink < 0 || c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return PARISKV_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads) return PARISKV_ERR_INVALID_ARG;
  if (c->key_dtype != PARISKV_DTYPE_BF16 && c->key_dtype != PARISKV_DTYPE_FP32)
    return PARISKV_ERR_INVALID_ARG;
  if (c->capacity < 1 || c->capacity > 0x7FFFFFFFll || c->n_sink >= c->capacity)
    return PARISKV_ERR_INVALID_ARG;
  // kernels of this build: d = 128 (32 sub-vectors of 4), G in {1, 2, 4, 8},
  // at most 1024 top-k slices of candidates per (b, h)
  if (c->head_dim != 128) return PARISKV_ERR_UNSUPPORTED;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PARISKV_ERR_UNSUPPORTED;
  if ((int64_t)c->batch * c->n_kv_heads > 65535) return PARISKV_ERR_UNSUPPORTED;
  if (c->capacity - c->n_sink > kMaxSlices * pkv::kTopkSlice) return PARISKV_ERR_UNSUPPORTED;
  return PARISKV_OK;
}

int64_t bh_of(const pariskv_si_config* c) { return (int64_t)c->batch * c->n_kv_heads; }

struct SiIndexLayout {
  size_t ids, mean, cb, total;
};

SiIndexLayout si_index_layout(const pariskv_si_config* c) {
  const size_t BH = (size_t)bh_of(c);
  SiIndexLayout L;
  L.ids = 0;
  L.mean = align_up(BH * (size_t)c->capacity * 16, kAlign);
  L.cb = L.mean + align_up(BH * 128 * 4, kAlign);
  L.total = L.cb + align_up(BH * 2048 * 4, kAlign);
  return L;
}

struct SiWsLayout {
  size_t lut, tab, range, fscore, bins, chist, coff, meta, cand, est, mmc, tkrange, tkmeta, rows,
      sorted, total;
  int64_t Epad, nchunks_max, cstride, pmax;
};

SiWsLayout si_ws_layout(const pariskv_si_config* c) {
  const size_t BH = (size_t)bh_of(c);
  const int64_t Emax = c->capacity - c->n_sink;
  SiWsLayout L;
  L.Epad = (int64_t)align_up((size_t)Emax, 4096);
  L.nchunks_max = ceil_div(Emax, 256);
  L.cstride = (int64_t)align_up((size_t)Emax, 64);
  L.pmax = ceil_div(Emax, pkv::kTopkSlice);
  size_t off = 0;
  L.lut = off;    off += align_up(BH * 512 * 4, kAlign);
  L.tab = off;    off += align_up(BH * 4096 * 4, kAlign);
  L.range = off;  off += align_up(BH * 2 * 4, kAlign);
  L.fscore = off; off += align_up(BH * (size_t)L.Epad * 4, kAlign);
  L.bins = off;   off += align_up(BH * (size_t)L.Epad, kAlign);
  L.chist = off;  off += align_up(BH * (size_t)L.nchunks_max * 256 * 4, kAlign);
  L.coff = off;   off += align_up(BH * (size_t)L.nchunks_max * 2 * 4, kAlign);
  L.meta = off;   off += align_up(BH * 4 * 4, kAlign);
  L.cand = off;   off += align_up(BH * (size_t)L.cstride * 4, kAlign);
  L.est = off;    off += align_up(BH * (size_t)L.cstride * 4, kAlign);
  L.mmc = off;    off += align_up(BH * (size_t)L.nchunks_max * 2 * 4, kAlign);
  L.tkrange = off; off += align_up(BH * 2 * 4, kAlign);
  L.tkmeta = off; off += align_up(BH * 4 * 4, kAlign);
  L.rows = off;   off += align_up(BH * (size_t)L.pmax * 2048 * 2, kAlign);
  L.sorted = off; off += align_up(BH * (size_t)L.pmax * pkv::kTopkSlice * 8, kAlign);
  L.total = off;
  return L;
}

int pick_kpt(int64_t E, int64_t BH) {
  int kpt = 8;
  while (kpt > 1 && ceil_div(E, 256 * kpt) * BH < 2048) kpt >>= 1;
  return kpt;
}

int32_t si_retrieve_impl(const pariskv_si_index* ix, const void* Q, int32_t k, int32_t* out_idx,
                         float* out_score, void* ws, size_t ws_bytes, hipStream_t st,
                         void** events) {
  if (!ix || !Q || !out_idx || !ws) return PARISKV_ERR_INVALID_ARG;
  const pariskv_si_config* c = &ix->cfg;
  const int64_t S = c->n_sink, N = ix->n;
  if (k <= S || (int64_t)k > N) return PARISKV_ERR_INVALID_ARG;
  const SiWsLayout L = si_ws_layout(c);
  if (ws_bytes < L.total) return PARISKV_ERR_WORKSPACE;
  const int BH = (int)bh_of(c);
  const int G = c->n_q_heads / c->n_kv_heads;
  const int64_t E = N - S, kp = k - S;
  const int kpt = pick_kpt(E, BH);
  const int nch = (int)ceil_div(E, 256 * kpt);
  uint8_t* base = (uint8_t*)ws;
  float* lut = (float*)(base + L.lut);
  float* tab = (float*)(base + L.tab);
  float* range = (float*)(base + L.range);
  uint8_t* bins = base + L.bins;
  uint32_t* chist = (uint32_t*)(base + L.chist);
  uint32_t* coff = (uint32_t*)(base + L.coff);
  int32_t* meta = (int32_t*)(base + L.meta);
  int32_t* cand = (int32_t*)(base + L.cand);
  float* est = (float*)(base + L.est);
  uint32_t* mmc = (uint32_t*)(base + L.mmc);
  uint32_t* tkrange = (uint32_t*)(base + L.tkrange);
  int32_t* tkmeta = (int32_t*)(base + L.tkmeta);
  uint16_t* rows = (uint16_t*)(base + L.rows);
  uint2* sorted = (uint2*)(base + L.sorted);
  auto ev = [&](int s) {
    pkv::EvPair p;
    if (events) {
      p.start = (hipEvent_t)events[2 * s];
      p.stop = (hipEvent_t)events[2 * s + 1];
    }
    return p;
  };
  (void)hipGetLastError();
  hipError_t e;
  e = pkv::launch_si_lut(c->key_dtype, Q, BH, c->n_kv_heads, G, ix->cb, lut, tab, range, st,
                         ev(0));
  if (e != hipSuccess) return hip_status(e);
  e = pkv::launch_si_scan(kpt, nch, BH, ix->ids, c->capacity, S, E, tab, range, bins, L.Epad,
                          chist, (int)L.nchunks_max, st, ev(1));
  if (e != hipSuccess) return hip_status(e);
  // the bin holding rank k', every key of it kept
  e = pkv::launch_thresh(BH, chist, (int)L.nchunks_max, nch, 256, 256, kp, 1, meta, coff, st,
                         ev(2));
  if (e != hipSuccess) return hip_status(e);
  e = pkv::launch_si_compact(kpt, nch, BH, bins, ix->ids, c->capacity, tab, L.Epad, S, E, meta,
                             coff, (int)L.nchunks_max, cand, est, L.cstride, mmc, st, ev(3));
  if (e != hipSuccess) return hip_status(e);
  // candidates are usually a little over k' (the keys of the bins down to
  // the one holding rank k'): blocks for twice that, more slices are looped
  const int grid_slices = (int)ceil_div(2 * kp, pkv::kTopkSlice) + 1;
  e = pkv::launch_topk_counted(BH, est, cand, L.cstride, meta, (int)E, grid_slices, (int)kp,
                               (int)S, k, mmc, (int)L.nchunks_max, nch, tkrange, rows, tkmeta,
                               sorted, out_idx, out_score, st, ev(4), ev(5));
  return hip_status(e);
}

}  // namespace

extern "C" {

int32_t pariskv_si_index_bytes(const pariskv_si_config* cfg, size_t* bytes) {
  if (!bytes) return PARISKV_ERR_INVALID_ARG;
  if (int32_t rc = check_si_cfg(cfg)) return rc;
  *bytes = si_index_layout(cfg).total;
  return PARISKV_OK;
}

int32_t pariskv_si_build_workspace_bytes(const pariskv_si_config* cfg, int64_t n_keys,
                                         size_t* bytes) {
  if (!bytes) return PARISKV_ERR_INVALID_ARG;
  if (int32_t rc = check_si_cfg(cfg)) return rc;
  if (n_keys < 0 || n_keys > cfg->capacity) return PARISKV_ERR_INVALID_ARG;
  *bytes = pkv::si_build_ws_bytes((int)bh_of(cfg), cfg->n_sink, n_keys);
  return PARISKV_OK;
}

int32_t pariskv_si_retrieve_workspace_bytes(const pariskv_si_config* cfg, int32_t k,
                                            size_t* bytes) {
  if (!bytes) return PARISKV_ERR_INVALID_ARG;
  if (int32_t rc = check_si_cfg(cfg)) return rc;
  if (k <= cfg->n_sink || (int64_t)k > cfg->capacity) return PARISKV_ERR_INVALID_ARG;
  *bytes = si_ws_layout(cfg).total;
  return PARISKV_OK;
}

int32_t pariskv_si_build_index(const pariskv_si_config* cfg, void* index_buf, size_t index_bytes,
                               const void* K, int64_t k_rows_per_head, int64_t n_keys,
                               void* build_ws, size_t build_ws_bytes, void* stream,
                               pariskv_si_index** out) {
  if (!out) return PARISKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (int32_t rc = check_si_cfg(cfg)) return rc;
  if (!index_buf || n_keys < 0) return PARISKV_ERR_INVALID_ARG;
  if (n_keys > cfg->capacity) return PARISKV_ERR_CAPACITY;
  if (n_keys > 0 && (!K || k_rows_per_head < n_keys)) return PARISKV_ERR_INVALID_ARG;
  const SiIndexLayout L = si_index_layout(cfg);
  if (index_bytes < L.total) return PARISKV_ERR_WORKSPACE;
  const int BH = (int)bh_of(cfg);
  const size_t need = pkv::si_build_ws_bytes(BH, cfg->n_sink, n_keys);
  if (!build_ws || build_ws_bytes < need) return PARISKV_ERR_WORKSPACE;
  pariskv_si_index* ix = new (std::nothrow) pariskv_si_index;
  if (!ix) return PARISKV_ERR_NOMEM;
  ix->cfg = *cfg;
  ix->ids = (uint8_t*)index_buf + L.ids;
  ix->mean = (float*)((uint8_t*)index_buf + L.mean);
  ix->cb = (float*)((uint8_t*)index_buf + L.cb);
  ix->n = n_keys;
  (void)hipGetLastError();
  const hipError_t e = pkv::launch_si_build(cfg->key_dtype, K, k_rows_per_head, cfg->n_sink,
                                            n_keys, BH, cfg->capacity, ix->ids, ix->mean, ix->cb,
                                            build_ws, (hipStream_t)stream);
  if (e != hipSuccess) {
    delete ix;
    return PARISKV_ERR_HIP;
  }
  *out = ix;
  return PARISKV_OK;
}

int32_t pariskv_si_append_keys(pariskv_si_index* ix, const void* K_new,
                               int64_t new_rows_per_head, int64_t n_new, void* stream) {
  if (!ix || n_new < 0) return PARISKV_ERR_INVALID_ARG;
  if (n_new == 0) return PARISKV_OK;
  if (!K_new || new_rows_per_head < n_new) return PARISKV_ERR_INVALID_ARG;
  if (ix->n + n_new > ix->cfg.capacity) return PARISKV_ERR_CAPACITY;
  (void)hipGetLastError();
  const hipError_t e = pkv::launch_si_encode(ix->cfg.key_dtype, K_new, new_rows_per_head, ix->n,
                                             n_new, (int)bh_of(&ix->cfg), ix->mean,
                                             ix->cfg.capacity, ix->ids, (hipStream_t)stream);
  if (e != hipSuccess) return PARISKV_ERR_HIP;
  ix->n += n_new;
  return PARISKV_OK;
}

int64_t pariskv_si_index_size(const pariskv_si_index* ix) { return ix ? ix->n : -1; }

void pariskv_si_index_destroy(pariskv_si_index* ix) { delete ix; }

int32_t pariskv_si_retrieve_topk(const pariskv_si_index* ix, const void* Q, int32_t k,
                                 int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                                 void* stream) {
  return si_retrieve_impl(ix, Q, k, out_idx, out_score, ws, ws_bytes, (hipStream_t)stream,
                          nullptr);
}

int32_t pariskv_si_retrieve_topk_profiled(const pariskv_si_index* ix, const void* Q, int32_t k,
                                          int32_t* out_idx, float* out_score, void* ws,
                                          size_t ws_bytes, void* stream, void** events) {
  if (!events) return PARISKV_ERR_INVALID_ARG;
  for (int s = 0; s < 2 * PARISKV_SI_STAGES; ++s)
    if (!events[s]) return PARISKV_ERR_INVALID_ARG;
  return si_retrieve_impl(ix, Q, k, out_idx, out_score, ws, ws_bytes, (hipStream_t)stream,
                          events);
}

int32_t pariskv_si_debug_export(const pariskv_si_index* ix, int64_t lo, int64_t hi,
                                uint8_t* ids_host, float* mean_host, float* codebook_host) {
  if (!ix || lo < 0 || hi < lo || hi > ix->cfg.capacity) return PARISKV_ERR_INVALID_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return PARISKV_ERR_HIP;
  const int64_t BH = bh_of(&ix->cfg), cap = ix->cfg.capacity, n = hi - lo;
  std::vector<uint8_t> packed((size_t)n * 16);
  for (int64_t bh = 0; bh < BH && ids_host && n > 0; ++bh) {
    if (hipMemcpy(packed.data(), ix->ids + (bh * cap + lo) * 16, n * 16,
                  hipMemcpyDeviceToHost) != hipSuccess)
      return PARISKV_ERR_HIP;
    for (int64_t i = 0; i < n * 16; ++i) {
      ids_host[bh * n * 32 + 2 * i] = packed[i] & 15u;
      ids_host[bh * n * 32 + 2 * i + 1] = packed[i] >> 4;
    }
  }
  if (mean_host &&
      hipMemcpy(mean_host, ix->mean, BH * 128 * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return PARISKV_ERR_HIP;
  if (codebook_host &&
      hipMemcpy(codebook_host, ix->cb, BH * 2048 * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return PARISKV_ERR_HIP;
  return PARISKV_OK;
}

int32_t pariskv_si_debug_intermediate(const pariskv_si_index* ix, int32_t k, const void* ws,
                                      size_t ws_bytes, int32_t which, void* dst,
                                      size_t dst_bytes) {
  if (!ix || !ws || !dst) return PARISKV_ERR_INVALID_ARG;
  const pariskv_si_config* c = &ix->cfg;
  const SiWsLayout L = si_ws_layout(c);
  if (ws_bytes < L.total) return PARISKV_ERR_WORKSPACE;
  if (k <= c->n_sink || (int64_t)k > ix->n) return PARISKV_ERR_INVALID_ARG;
  const int64_t BH = bh_of(c), E = ix->n - c->n_sink;
  const uint8_t* base = (const uint8_t*)ws;
  if (hipDeviceSynchronize() != hipSuccess) return PARISKV_ERR_HIP;
  auto rows = [&](size_t off, size_t stride, size_t row) -> int32_t {
    if (dst_bytes < (size_t)BH * row) return PARISKV_ERR_INVALID_ARG;
    if (row == 0) return PARISKV_OK;
    return hipMemcpy2D(dst, row, base + off, stride, row, BH, hipMemcpyDeviceToHost) == hipSuccess
               ? PARISKV_OK
               : PARISKV_ERR_HIP;
  };
  switch (which) {
    case 0: return rows(L.lut, 512 * 4, 512 * 4);
    case 1: {
      // recomputed from the ids and this workspace's byte table
      uint8_t* wsb = const_cast<uint8_t*>(base);
      if (pkv::launch_si_scores((int)BH, ix->ids, c->capacity, c->n_sink, E,
                                (const float*)(wsb + L.tab), (float*)(wsb + L.fscore), L.Epad,
                                nullptr) != hipSuccess ||
          hipDeviceSynchronize() != hipSuccess)
        return PARISKV_ERR_HIP;
      return rows(L.fscore, (size_t)L.Epad * 4, (size_t)E * 4);
    }
    case 2: return rows(L.meta, 16, 16);
    default: return PARISKV_ERR_INVALID_ARG;
  }
}

}  // extern "C"
