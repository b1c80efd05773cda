// C ABI of the ParisKV retrieval library: argument validation, buffer
// layouts and launch sequencing.  Declarations and their contracts are in
// include/pariskv.h; the kernels are in pariskv_kernels.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "pariskv.h"
#include "pariskv_internal.h"

struct pariskv_index {
  pariskv_config cfg;
  pkv::SignMask signs;
  float rot_c;
  uint8_t* ids;    // [BH][cap][16]  bucket id per subspace
  uint32_t* rec;   // [BH][cap][32]  128-byte record: 16 code dwords, 16 fp16 w, pad
  int64_t n;       // keys per (b, h), including appended keys not yet encoded
  hipStream_t last;
  pkv::AppendJob pending;       // appended rows the next retrieval encodes
  hipStream_t pending_stream;
  int32_t path;                 // PARISKV_PATH_*
};

// Four-region window over one index (sinks, retrieval, local, update buffer).
struct pariskv_window {
  pariskv_index* ix;
  int64_t S, L, U, ring;  // ring = L + U slots after the S sink rows of the near store
  uint8_t* Kn;            // near store [BH][S + ring][d]
  uint8_t* Vn;
  uint8_t* Kf;            // far store [BH][far_rows][d]
  uint8_t* Vf;
  int64_t far_rows;
  int64_t R;              // keys in the retrieval region [S, S + R): the index holds S + R
  int64_t u;              // tokens in the update buffer
  size_t rb;              // bytes per row
};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// retrieval units: one per (b, KV head), or per (b, query head) when unshared
int64_t units_of(const pariskv_config* c) {
  return (int64_t)c->batch * (c->per_query_head ? c->n_q_heads : c->n_kv_heads);
}
int unit_div_of(const pariskv_config* c) {
  return c->per_query_head ? c->n_q_heads / c->n_kv_heads : 1;
}

int64_t cand_count(int64_t E, int64_t kprime, int64_t num, int64_t den) {
  int64_t c = (E * num + den - 1) / den;
  if (c < kprime) c = kprime;
  if (c > E) c = E;
  return c;
}

int max_tier(const pariskv_config* c) {
  int mx = 0;
  for (int s = 0; s < c->rho; ++s) mx = c->tier_w[s] > mx ? c->tier_w[s] : mx;
  return mx;
}

// coordinates per subspace
int m_of(const pariskv_config* c) { return c->head_dim / c->n_subspaces; }

int32_t check_cfg(const pariskv_config* c) {
  if (!c) return PARISKV_ERR_INVALID_ARG;
  const int d = c->head_dim;
  if (d < 2 || d > 1024 || (d & (d - 1))) return PARISKV_ERR_INVALID_ARG;
  if (c->n_subspaces < 1 || d % c->n_subspaces) return PARISKV_ERR_INVALID_ARG;
  const int m = d / c->n_subspaces;
  if (m < 2 || m > 8) return PARISKV_ERR_INVALID_ARG;
  if (c->rho < 1 || c->rho > 8 || c->rho > (1 << m)) return PARISKV_ERR_INVALID_ARG;
  for (int s = 0; s < c->rho; ++s)
    if (c->tier_w[s] < 0 || c->tier_w[s] > 255) return PARISKV_ERR_INVALID_ARG;
  if ((int64_t)c->n_subspaces * max_tier(c) > 255) return PARISKV_ERR_INVALID_ARG;
  if (c->cand_num < 1 || c->cand_den < c->cand_num) return PARISKV_ERR_INVALID_ARG;
  if (c->n_sink < 0 || c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return PARISKV_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads) return PARISKV_ERR_INVALID_ARG;
  if (c->key_dtype != PARISKV_DTYPE_BF16 && c->key_dtype != PARISKV_DTYPE_FP32)
    return PARISKV_ERR_INVALID_ARG;
  if (c->capacity < 1 || c->capacity > 0x7FFFFFFFll || c->n_sink >= c->capacity)
    return PARISKV_ERR_INVALID_ARG;
  if (c->per_query_head != 0 && c->per_query_head != 1) return PARISKV_ERR_INVALID_ARG;
  if ((int64_t)c->batch * c->n_kv_heads > 65535) return PARISKV_ERR_UNSUPPORTED;
  if (units_of(c) > 65535) return PARISKV_ERR_UNSUPPORTED;
  // kernels of this build: d = 128 split into 16 subspaces of 8 or 32 of 4,
  // and 1, 2, 4 or 8 query heads per KV head
  if (d != 128 || (m != 8 && m != 4)) return PARISKV_ERR_UNSUPPORTED;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PARISKV_ERR_UNSUPPORTED;
  return PARISKV_OK;
}

struct IndexLayout {
  size_t ids, rec, total;
};

IndexLayout index_layout(const pariskv_config* c) {
  const size_t keys = (size_t)c->batch * c->n_kv_heads * (size_t)c->capacity;
  IndexLayout L;
  L.ids = 0;
  L.rec = align_up(keys * 16, kAlign);
  L.total = L.rec + align_up(keys * 128, kAlign);
  return L;
}

struct WsLayout {
  size_t lut, yq, ptab, scores, chist, coff, meta, cand, est, mmc, range, tkmeta, rows, sorted,
      total;
  int64_t Epad, nchunks_max, cstride, tk_blocks_max;
  int nbins, rstride;
};

WsLayout ws_layout(const pariskv_config* c, int64_t k) {
  const int64_t BH = units_of(c);  // workspace rows: one per retrieval unit
  const int64_t Emax = c->capacity - c->n_sink;
  int64_t kp = k - c->n_sink;
  if (kp > Emax) kp = Emax;
  const int64_t Cmax = cand_count(Emax, kp, c->cand_num, c->cand_den);
  WsLayout L;
  L.nbins = c->n_subspaces * max_tier(c) + 1;
  L.rstride = (int)align_up((size_t)L.nbins, 4);  // chunk rows are 16-byte aligned
  L.nchunks_max = ceil_div(Emax, 256);
  L.Epad = (int64_t)align_up((size_t)Emax, 4096);
  L.cstride = (int64_t)align_up((size_t)(Cmax > 0 ? Cmax : 1), 64);  // 256-byte rows
  size_t off = 0;
  L.lut = off;    off += align_up((size_t)BH * 16 * 256, kAlign);
  L.yq = off;     off += align_up((size_t)BH * 128 * 4, kAlign);
  L.ptab = off;   off += align_up((size_t)BH * 2048 * 4, kAlign);
  L.scores = off; off += align_up((size_t)BH * L.Epad, kAlign);
  L.chist = off;  off += align_up((size_t)BH * L.nchunks_max * L.rstride * 4, kAlign);
  L.coff = off;   off += align_up((size_t)BH * L.nchunks_max * 8, kAlign);
  L.meta = off;   off += align_up((size_t)BH * 16, kAlign);
  L.cand = off;   off += align_up((size_t)BH * L.cstride * 4, kAlign);
  L.est = off;    off += align_up((size_t)BH * L.cstride * 4, kAlign);
  L.tk_blocks_max = ceil_div(L.cstride, pkv::kTopkSlice);
  L.mmc = off;    off += align_up((size_t)BH * L.nchunks_max * 8, kAlign);
  L.range = off;  off += align_up((size_t)BH * 8, kAlign);
  L.tkmeta = off; off += align_up((size_t)BH * 16, kAlign);
  L.rows = off;   off += align_up((size_t)BH * L.tk_blocks_max * 2048 * 2, kAlign);
  L.sorted = off; off += align_up((size_t)BH * L.tk_blocks_max * pkv::kTopkSlice * 8, kAlign);
  L.total = off;
  return L;
}

// Keys per thread of the scan/compaction chunks: the largest power of two
// <= 8 that still gives >= 2048 blocks (8 per CU on 256 CUs).  8 keys per
// thread keeps the scan at 8 waves per SIMD, so a full wave of blocks fits.
int pick_kpt(int64_t E, int64_t BH) {
  int kpt = 8;
  while (kpt > 1 && ceil_div(E, 256 * kpt) * BH < 2048) kpt >>= 1;
  return kpt;
}

float rot_scale(int d) { return (float)(1.0L / std::sqrt((long double)d)); }

// Split-K partial slots per query head of a retrieval + attention: the
// attention's chunks, at their smallest.
int64_t attend_part_chunks(int64_t k) { return ceil_div(k, pkv::kAttnChunkRowsMin); }
size_t attend_part_bytes(const pariskv_config* c, int64_t k) {
  return align_up((size_t)c->batch * c->n_q_heads * attend_part_chunks(k) * pkv::kPartStride * 4,
                  kAlign);
}

// Attention after a retrieval: K, V ([kv heads][rows][d], key_dtype), the
// output [b][H_q][d] and the split-K partial buffer.
struct AttnSpec {
  const void* K = nullptr;
  const void* V = nullptr;
  int64_t rows = 0;
  float scale = 0.0f;
  void* out = nullptr;
  float* part = nullptr;
  int64_t part_chunks = 0;  // partial slots per query head
};

int32_t hip_status(hipError_t e) { return e == hipSuccess ? PARISKV_OK : PARISKV_ERR_HIP; }

// Encodes deferred appended keys now, on the stream they were appended on.
int32_t flush_pending(pariskv_index* ix) {
  if (ix->pending.n == 0) return PARISKV_OK;
  const pkv::AppendJob job = ix->pending;
  ix->pending.n = 0;
  const int BH = ix->cfg.batch * ix->cfg.n_kv_heads;
  (void)hipGetLastError();
  return hip_status(pkv::launch_encode(m_of(&ix->cfg), ix->cfg.key_dtype, job.K,
                                       job.rows_per_head, job.lo, job.n, BH, ix->cfg.capacity,
                                       ix->ids, ix->rec, ix->signs, ix->rot_c,
                                       ix->pending_stream, pkv::EvPair{}));
}

// The retrieval path for C candidates per unit: the single kernel, when
// asked for, serves shared retrieval with at most kSmallTopkSlices top-k
// slices; otherwise the pipeline.
int32_t choose_path(const pariskv_index* ix, int64_t C) {
  if (ix->path != PARISKV_PATH_SINGLE) return PARISKV_PATH_PIPELINE;
  const bool fits = !ix->cfg.per_query_head &&
                    C <= (int64_t)pkv::kSmallTopkSlices * pkv::kTopkSlice;
  return fits ? PARISKV_PATH_SINGLE : PARISKV_ERR_UNSUPPORTED;
}

int32_t attn_core(const void* Q, const pkv::AttnRows& rs, const int32_t* idx, int32_t k,
                  int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                  int32_t dtype, float scale, void* out, void* ws, size_t ws_bytes, void* stream,
                  void** events);

// Split-K attention over the k selected rows of every unit, with the partial
// buffer of a retrieval + attention call; events (optional) as
// retrieve_impl's, the attention pairs after the retrieval stages.
int32_t attend_selected(const pariskv_index* ix, const void* Q, int32_t k, const int32_t* idx,
                        const AttnSpec& att, hipStream_t st, void** events) {
  const pariskv_config* c = &ix->cfg;
  pkv::AttnRows rs;
  rs.K = att.K;
  rs.V = att.V;
  rs.rows = att.rows;
  rs.K_near = att.K;
  rs.V_near = att.V;
  rs.near_rows = att.rows;
  rs.unit_div = unit_div_of(c);
  const int Hu = c->per_query_head ? c->n_q_heads : c->n_kv_heads;
  // the partial buffer as the workspace reserves it (256-byte aligned size)
  const size_t bytes =
      align_up((size_t)c->batch * c->n_q_heads * att.part_chunks * pkv::kPartStride * 4, kAlign);
  return attn_core(Q, rs, idx, k, c->batch, c->n_q_heads, Hu, c->head_dim, c->key_dtype,
                   att.scale, att.out, att.part, bytes, st,
                   events ? events + 2 * PARISKV_RETRIEVE_STAGES : nullptr);
}

// events: 2 per retrieval stage; with attention 4 more (split, merge)
int32_t retrieve_impl(const pariskv_index* ix, const void* Q, int32_t k, int32_t* out_idx,
                      float* out_est, void* ws, size_t ws_bytes, void* stream, void** events,
                      const AttnSpec* att = nullptr) {
  if (!ix || !Q || !out_idx || !ws) return PARISKV_ERR_INVALID_ARG;
  const pariskv_config* c = &ix->cfg;
  const int64_t N = ix->n, S = c->n_sink;
  if (k <= S || (int64_t)k > N) return PARISKV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return PARISKV_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(c, k);
  if (ws_bytes < L.total) return PARISKV_ERR_WORKSPACE;
  // every refusal comes before the deferred appends are taken over below
  const int64_t E = N - S, kp = k - S;
  const int64_t C = cand_count(E, kp, c->cand_num, c->cand_den);
  if (C > 1024ll * pkv::kTopkSlice) return PARISKV_ERR_UNSUPPORTED;  // > 4M candidates per head
  const int32_t path = choose_path(ix, C);
  if (path < 0) return path;
  hipStream_t st = (hipStream_t)stream;
  pariskv_index* mix = const_cast<pariskv_index*>(ix);
  mix->last = st;
  // deferred appends: encoded by this retrieval's first kernel, on its own
  // stream, which the caller has ordered after the appended rows were
  // written (whichever stream the append was issued on), so the scan that
  // follows on this stream sees them
  pkv::AppendJob app;
  if (mix->pending.n > 0) {
    app = mix->pending;
    mix->pending.n = 0;
  }
  const int BH = (int)units_of(c);  // retrieval units
  const int udiv = unit_div_of(c);
  // a unit's query: the mean of its G query heads, or its own head when unshared
  const int G = c->per_query_head ? 1 : c->n_q_heads / c->n_kv_heads;
  const int units_per_batch = c->per_query_head ? c->n_q_heads : c->n_kv_heads;
  const int kpt = pick_kpt(E, BH);
  const int P = (int)ceil_div(C, pkv::kTopkSlice);
  const int nch = (int)ceil_div(E, 256 * kpt);
  uint8_t* base = (uint8_t*)ws;
  uint8_t* lut = base + L.lut;
  float* yq = (float*)(base + L.yq);
  float* ptab = (float*)(base + L.ptab);
  uint8_t* scores = base + L.scores;
  uint32_t* chist = (uint32_t*)(base + L.chist);
  uint32_t* coff = (uint32_t*)(base + L.coff);
  int32_t* meta = (int32_t*)(base + L.meta);
  int32_t* cand = (int32_t*)(base + L.cand);
  float* est = (float*)(base + L.est);
  uint32_t* mmc = (uint32_t*)(base + L.mmc);
  uint32_t* range = (uint32_t*)(base + L.range);
  int32_t* tkmeta = (int32_t*)(base + L.tkmeta);
  uint16_t* rows = (uint16_t*)(base + L.rows);
  uint2* sorted = (uint2*)(base + L.sorted);
  pkv::Tiers tw;
  for (int s = 0; s < 8; ++s) tw.w[s] = c->tier_w[s];

  // events (optional): start/stop pair per stage, stamped by the dispatch
  auto ev = [&](int s) {
    pkv::EvPair p;
    if (events) {
      p.start = (hipEvent_t)events[2 * s];
      p.stop = (hipEvent_t)events[2 * s + 1];
    }
    return p;
  };
  (void)hipGetLastError();  // launches below report only their own errors
  hipError_t e;
  if (path == PARISKV_PATH_SINGLE) {
    // one kernel, stamped as stage 1; the other stages' events back to back
    for (int s = 0; s < PARISKV_RETRIEVE_STAGES; ++s) {
      if (s == 1) continue;
      const pkv::EvPair p = ev(s);
      if (p.start && (e = hipEventRecord(p.start, st)) != hipSuccess) return hip_status(e);
      if (p.stop && (e = hipEventRecord(p.stop, st)) != hipSuccess) return hip_status(e);
    }
    e = pkv::launch_retrieve_small(
        m_of(c), c->key_dtype, Q, BH, units_per_batch, G, ix->signs, ix->rot_c, c->rho, tw, app,
        ix->ids, ix->rec, c->capacity, S, E, C, (int)kp, k, L.nbins, lut, yq, scores, L.Epad,
        meta, cand, est, L.cstride, out_idx, out_est, st, ev(1));
    if (e != hipSuccess || !att) return hip_status(e);
    return attend_selected(ix, Q, k, out_idx, *att, st, events);
  }
  e = pkv::launch_qprep(m_of(c), c->key_dtype, Q, BH, units_per_batch, G, ix->signs, ix->rot_c,
                        c->rho, tw, lut, yq, ptab, app, udiv, st, ev(0));
  if (e != hipSuccess) return hip_status(e);
  e = pkv::launch_scan(kpt, nch, BH, ix->ids, c->capacity, S, E, lut, scores, L.Epad, chist,
                       (int)L.nchunks_max, L.nbins, L.rstride, udiv, st, ev(1));
  if (e != hipSuccess) return hip_status(e);
  // up to kFusedThreshChunks chunks per unit the compaction finds the
  // threshold itself (the stage's events are then recorded back to back)
  const bool fused_thresh = nch <= pkv::kFusedThreshChunks;
  if (fused_thresh) {
    const pkv::EvPair tp = ev(2);
    if (tp.start && (e = hipEventRecord(tp.start, st)) != hipSuccess) return hip_status(e);
    if (tp.stop && (e = hipEventRecord(tp.stop, st)) != hipSuccess) return hip_status(e);
  } else {
    e = pkv::launch_thresh(BH, chist, (int)L.nchunks_max, nch, L.nbins, L.rstride, C, 0, meta,
                           coff, st, ev(2));
    if (e != hipSuccess) return hip_status(e);
  }
  e = pkv::launch_compact_rerank(m_of(c), kpt, nch, BH, scores, L.Epad, S, E, meta, coff,
                                 (int)L.nchunks_max, ptab, ix->rec, c->capacity, cand, est,
                                 L.cstride, C, mmc, L.nbins, udiv, fused_thresh ? chist : nullptr,
                                 L.rstride, meta, st, ev(3));
  if (e != hipSuccess) return hip_status(e);
  e = pkv::launch_topk(BH, est, cand, L.cstride, (int)C, (int)kp, (int)S, k, P, mmc,
                       (int)L.nchunks_max, nch, range, rows, tkmeta, sorted, out_idx, out_est, st,
                       ev(4), ev(5));
  if (e != hipSuccess) return hip_status(e);
  if (!att) return PARISKV_OK;
  return attend_selected(ix, Q, k, out_idx, *att, st, events);
}

// Split-K attention over k listed rows plus rs.tail_n tail rows.
int32_t attn_core(const void* Q, const pkv::AttnRows& rs, const int32_t* idx, int32_t k,
                  int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                  int32_t dtype, float scale, void* out, void* ws, size_t ws_bytes, void* stream,
                  void** events) {
  if (!Q || !rs.K || !rs.V || !idx || !out || !ws) return PARISKV_ERR_INVALID_ARG;
  if (k < 1 || batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || rs.rows < 1 || rs.tail_n < 0)
    return PARISKV_ERR_INVALID_ARG;
  if (n_q_heads % n_kv_heads) return PARISKV_ERR_INVALID_ARG;
  if (dtype != PARISKV_DTYPE_BF16 && dtype != PARISKV_DTYPE_FP32) return PARISKV_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PARISKV_ERR_INVALID_ARG;
  const int G = n_q_heads / n_kv_heads;
  if (head_dim != 128 || (G != 1 && G != 2 && G != 4 && G != 8)) return PARISKV_ERR_UNSUPPORTED;
  if ((int64_t)batch * n_kv_heads > 65535) return PARISKV_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)k + rs.tail_n;
  if (rows > 0x7FFFFFFFll) return PARISKV_ERR_INVALID_ARG;
  size_t need = 0;
  pariskv_attn_workspace_bytes(batch, n_q_heads, (int32_t)rows, head_dim, &need);
  if (ws_bytes < need) return PARISKV_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int rpl = pkv::attn_rows_per_lane(rows, (int64_t)batch * n_kv_heads);
  const int nch = (int)ceil_div(rows, 16 * rpl);
  const float qscale = scale * 1.4426950408889634f;
  pkv::EvPair e0, e1;
  if (events) {
    e0.start = (hipEvent_t)events[0];
    e0.stop = (hipEvent_t)events[1];
    e1.start = (hipEvent_t)events[2];
    e1.stop = (hipEvent_t)events[3];
  }
  (void)hipGetLastError();
  hipError_t e = pkv::launch_attn_split(dtype, G, rpl, Q, rs, idx, k, batch, n_kv_heads,
                                        qscale, (float*)ws, nch, st, e0);
  if (e != hipSuccess) return hip_status(e);
  e = pkv::launch_attn_merge(dtype, (const float*)ws, nch, batch * n_q_heads, out, st, e1);
  if (e != hipSuccess) return hip_status(e);
  return PARISKV_OK;
}

int32_t attn_impl(const void* Q, const void* K, const void* V, int64_t rows_per_head,
                  const int32_t* idx, int32_t k, int32_t batch, int32_t n_q_heads,
                  int32_t n_kv_heads, int32_t head_dim, int32_t dtype, float scale, void* out,
                  void* ws, size_t ws_bytes, void* stream, void** events) {
  pkv::AttnRows rs;
  rs.K = K;
  rs.V = V;
  rs.rows = rows_per_head;
  rs.K_near = K;  // unused: no near rows, no tail
  rs.V_near = V;
  rs.near_rows = rows_per_head;
  return attn_core(Q, rs, idx, k, batch, n_q_heads, n_kv_heads, head_dim, dtype, scale, out, ws,
                   ws_bytes, stream, events);
}

}  // namespace

extern "C" {

int32_t pariskv_index_bytes(const pariskv_config* cfg, size_t* bytes) {
  const int32_t rc = check_cfg(cfg);
  if (rc) return rc;
  if (!bytes) return PARISKV_ERR_INVALID_ARG;
  *bytes = index_layout(cfg).total;
  return PARISKV_OK;
}

int32_t pariskv_retrieve_workspace_bytes(const pariskv_config* cfg, int32_t k, size_t* bytes) {
  const int32_t rc = check_cfg(cfg);
  if (rc) return rc;
  if (!bytes || k <= cfg->n_sink || (int64_t)k > cfg->capacity) return PARISKV_ERR_INVALID_ARG;
  *bytes = ws_layout(cfg, k).total;
  return PARISKV_OK;
}

int32_t pariskv_attn_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t k,
                                     int32_t head_dim, size_t* bytes) {
  if (!bytes || batch < 1 || n_q_heads < 1 || k < 1 || head_dim < 1)
    return PARISKV_ERR_INVALID_ARG;
  const size_t chunks = (size_t)ceil_div(k, pkv::kAttnChunkRowsMin);
  *bytes = align_up((size_t)batch * n_q_heads * chunks * (head_dim + 4) * 4, kAlign);
  return PARISKV_OK;
}

int32_t pariskv_build_index(const pariskv_config* cfg, const int8_t* srht_signs, void* index_buf,
                            size_t index_bytes, const void* K, int64_t k_rows_per_head,
                            int64_t n_keys, void* stream, pariskv_index** out) {
  if (out) *out = nullptr;
  const int32_t rc = check_cfg(cfg);
  if (rc) return rc;
  if (!srht_signs || !index_buf || !out || (n_keys > 0 && !K) || n_keys < 0)
    return PARISKV_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(index_buf) & (kAlign - 1)) != 0) return PARISKV_ERR_INVALID_ARG;
  if (n_keys > 0 && k_rows_per_head < n_keys) return PARISKV_ERR_INVALID_ARG;
  if (n_keys > cfg->capacity) return PARISKV_ERR_CAPACITY;
  const IndexLayout L = index_layout(cfg);
  if (index_bytes < L.total) return PARISKV_ERR_WORKSPACE;
  pkv::SignMask sg{};
  for (int j = 0; j < cfg->head_dim; ++j) {
    if (srht_signs[j] == -1) sg.w[j >> 5] |= 1u << (j & 31);
    else if (srht_signs[j] != 1) return PARISKV_ERR_INVALID_ARG;
  }
  pariskv_index* ix = new (std::nothrow) pariskv_index;
  if (!ix) return PARISKV_ERR_NOMEM;
  ix->cfg = *cfg;
  ix->signs = sg;
  ix->rot_c = rot_scale(cfg->head_dim);
  uint8_t* base = (uint8_t*)index_buf;
  ix->ids = base + L.ids;
  ix->rec = (uint32_t*)(base + L.rec);
  ix->n = 0;
  ix->last = (hipStream_t)stream;
  ix->pending = pkv::AppendJob{};
  ix->pending_stream = nullptr;
  ix->path = PARISKV_PATH_AUTO;
  const int BH = cfg->batch * cfg->n_kv_heads;
  (void)hipGetLastError();
  hipError_t e = pkv::launch_encode(m_of(cfg), cfg->key_dtype, K, k_rows_per_head, 0, n_keys, BH,
                                    cfg->capacity, ix->ids, ix->rec, ix->signs, ix->rot_c,
                                    (hipStream_t)stream, pkv::EvPair{});
  if (e != hipSuccess) {
    delete ix;
    return PARISKV_ERR_HIP;
  }
  ix->n = n_keys;
  *out = ix;
  return PARISKV_OK;
}

int32_t pariskv_append_keys(pariskv_index* ix, const void* K_new, int64_t new_rows_per_head,
                            int64_t n_new, void* stream) {
  if (!ix || n_new < 0 || (n_new > 0 && (!K_new || new_rows_per_head < n_new)))
    return PARISKV_ERR_INVALID_ARG;
  if (ix->n + n_new > ix->cfg.capacity) return PARISKV_ERR_CAPACITY;
  if (n_new == 0) return PARISKV_OK;
  if (int32_t rc = flush_pending(ix)) return rc;
  ix->last = (hipStream_t)stream;
  if (n_new <= pkv::kMaxFusedAppend) {
    // a decode step's few keys: encoded by the next retrieval's first kernel
    pkv::AppendJob job;
    job.K = K_new;
    job.rows_per_head = new_rows_per_head;
    job.lo = ix->n;
    job.cap = ix->cfg.capacity;
    job.ids = ix->ids;
    job.rec = ix->rec;
    job.n = (int)n_new;
    ix->pending = job;
    ix->pending_stream = (hipStream_t)stream;
    ix->n += n_new;
    return PARISKV_OK;
  }
  const int BH = ix->cfg.batch * ix->cfg.n_kv_heads;
  (void)hipGetLastError();
  hipError_t e = pkv::launch_encode(m_of(&ix->cfg), ix->cfg.key_dtype, K_new, new_rows_per_head,
                                    ix->n, n_new, BH, ix->cfg.capacity, ix->ids, ix->rec,
                                    ix->signs, ix->rot_c, (hipStream_t)stream, pkv::EvPair{});
  if (e != hipSuccess) return PARISKV_ERR_HIP;
  ix->n += n_new;
  return PARISKV_OK;
}

int64_t pariskv_index_size(const pariskv_index* ix) { return ix ? ix->n : -1; }

void pariskv_index_destroy(pariskv_index* ix) {
  if (ix) (void)flush_pending(ix);  // the caller's index buffer gets every key
  delete ix;
}

int32_t pariskv_retrieve_topk(const pariskv_index* ix, const void* Q, int32_t k, int32_t* out_idx,
                              float* out_est, void* ws, size_t ws_bytes, void* stream) {
  return retrieve_impl(ix, Q, k, out_idx, out_est, ws, ws_bytes, stream, nullptr);
}

int32_t pariskv_retrieve_attend_workspace_bytes(const pariskv_config* cfg, int32_t k,
                                                size_t* bytes) {
  size_t r = 0;
  if (int32_t rc = pariskv_retrieve_workspace_bytes(cfg, k, &r)) return rc;
  *bytes = align_up(r, kAlign) + align_up(attend_part_bytes(cfg, k), kAlign);
  return PARISKV_OK;
}

static int32_t retrieve_attend_impl(const pariskv_index* ix, const void* Q, const void* K,
                                    const void* V, int64_t kv_rows_per_head, int32_t k,
                                    float scale, int32_t* out_idx, float* out_est, void* out,
                                    void* ws, size_t ws_bytes, void* stream, void** events) {
  if (!ix || !Q || !K || !V || !out || !out_idx || !ws) return PARISKV_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || kv_rows_per_head < ix->n) return PARISKV_ERR_INVALID_ARG;
  const pariskv_config* c = &ix->cfg;
  size_t need = 0;
  if (int32_t rc = pariskv_retrieve_attend_workspace_bytes(c, k, &need)) return rc;
  if (ws_bytes < need) return PARISKV_ERR_WORKSPACE;
  AttnSpec att;
  att.K = K;
  att.V = V;
  att.rows = kv_rows_per_head;
  att.scale = scale;
  att.out = out;
  att.part = (float*)((uint8_t*)ws + align_up(ws_layout(c, k).total, kAlign));
  att.part_chunks = attend_part_chunks(k);
  return retrieve_impl(ix, Q, k, out_idx, out_est, ws, ws_bytes, stream, events, &att);
}

int32_t pariskv_retrieve_attend(const pariskv_index* ix, const void* Q, const void* K,
                                const void* V, int64_t kv_rows_per_head, int32_t k, float scale,
                                int32_t* out_idx, float* out_est, void* out, void* ws,
                                size_t ws_bytes, void* stream) {
  return retrieve_attend_impl(ix, Q, K, V, kv_rows_per_head, k, scale, out_idx, out_est, out, ws,
                              ws_bytes, stream, nullptr);
}

int32_t pariskv_retrieve_attend_profiled(const pariskv_index* ix, const void* Q, const void* K,
                                         const void* V, int64_t kv_rows_per_head, int32_t k,
                                         float scale, int32_t* out_idx, float* out_est,
                                         void* out, void* ws, size_t ws_bytes, void* stream,
                                         void** events) {
  if (!events) return PARISKV_ERR_INVALID_ARG;
  for (int s = 0; s < 2 * PARISKV_RETRIEVE_STAGES + 4; ++s)
    if (!events[s]) return PARISKV_ERR_INVALID_ARG;
  return retrieve_attend_impl(ix, Q, K, V, kv_rows_per_head, k, scale, out_idx, out_est, out, ws,
                              ws_bytes, stream, events);
}

int32_t pariskv_retrieve_topk_noalloc(const pariskv_index* ix, const void* Q, int32_t k,
                                      int32_t* out_idx, float* out_est, void* stream) {
  if (!ix || !Q || !out_idx) return PARISKV_ERR_INVALID_ARG;
  size_t need = 0;
  if (int32_t rc = pariskv_retrieve_workspace_bytes(&ix->cfg, k, &need)) return rc;
  if (need > pkv::kNoAllocScratchBytes) return PARISKV_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (pkv::noalloc_scratch(&scratch) != hipSuccess) return PARISKV_ERR_HIP;
  return retrieve_impl(ix, Q, k, out_idx, out_est, scratch, pkv::kNoAllocScratchBytes, stream,
                       nullptr);
}

int32_t pariskv_retrieve_topk_profiled(const pariskv_index* ix, const void* Q, int32_t k,
                                       int32_t* out_idx, float* out_est, void* ws,
                                       size_t ws_bytes, void* stream, void** events) {
  if (!events) return PARISKV_ERR_INVALID_ARG;
  for (int s = 0; s < 2 * PARISKV_RETRIEVE_STAGES; ++s)
    if (!events[s]) return PARISKV_ERR_INVALID_ARG;
  return retrieve_impl(ix, Q, k, out_idx, out_est, ws, ws_bytes, stream, events);
}

static int32_t attn_per_head_impl(const void* Q, const void* K, const void* V,
                                  int64_t kv_rows_per_head, const int32_t* idx, int32_t k,
                                  int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t dtype, float scale, void* out,
                                  void* ws, size_t ws_bytes, void* stream, void** events) {
  if (n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads) return PARISKV_ERR_INVALID_ARG;
  pkv::AttnRows rs;
  rs.K = K;
  rs.V = V;
  rs.rows = kv_rows_per_head;
  rs.K_near = K;
  rs.V_near = V;
  rs.near_rows = kv_rows_per_head;
  rs.unit_div = n_q_heads / n_kv_heads;  // query head q reads KV head q / G
  // each query head is its own attention unit with one query row
  return attn_core(Q, rs, idx, k, batch, n_q_heads, n_q_heads, head_dim, dtype, scale, out, ws,
                   ws_bytes, stream, events);
}

int32_t pariskv_sparse_attn_per_query_head(const void* Q, const void* K, const void* V,
                                           int64_t kv_rows_per_head, const int32_t* idx,
                                           int32_t k, int32_t batch, int32_t n_q_heads,
                                           int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                                           float scale, void* out, void* ws, size_t ws_bytes,
                                           void* stream) {
  return attn_per_head_impl(Q, K, V, kv_rows_per_head, idx, k, batch, n_q_heads, n_kv_heads,
                            head_dim, dtype, scale, out, ws, ws_bytes, stream, nullptr);
}

int32_t pariskv_sparse_attn_per_query_head_profiled(
    const void* Q, const void* K, const void* V, int64_t kv_rows_per_head, const int32_t* idx,
    int32_t k, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
    int32_t dtype, float scale, void* out, void* ws, size_t ws_bytes, void* stream,
    void** events) {
  if (!events) return PARISKV_ERR_INVALID_ARG;
  for (int s = 0; s < 4; ++s)
    if (!events[s]) return PARISKV_ERR_INVALID_ARG;
  return attn_per_head_impl(Q, K, V, kv_rows_per_head, idx, k, batch, n_q_heads, n_kv_heads,
                            head_dim, dtype, scale, out, ws, ws_bytes, stream, events);
}

const char* pariskv_stage_name(int32_t s) {
  static const char* names[PARISKV_RETRIEVE_STAGES] = {
      "query_prep", "vote_scan", "threshold", "compact_rerank", "topk", "topk_second_pass"};
  return (s >= 0 && s < PARISKV_RETRIEVE_STAGES) ? names[s] : nullptr;
}

int32_t pariskv_sparse_attn(const void* Q, const void* K, const void* V, int64_t kv_rows_per_head,
                            const int32_t* idx, int32_t k, int32_t batch, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, int32_t dtype, float scale,
                            void* out, void* ws, size_t ws_bytes, void* stream) {
  return attn_impl(Q, K, V, kv_rows_per_head, idx, k, batch, n_q_heads, n_kv_heads, head_dim,
                   dtype, scale, out, ws, ws_bytes, stream, nullptr);
}

int32_t pariskv_sparse_attn_profiled(const void* Q, const void* K, const void* V,
                                     int64_t kv_rows_per_head, const int32_t* idx, int32_t k,
                                     int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t head_dim, int32_t dtype, float scale, void* out,
                                     void* ws, size_t ws_bytes, void* stream, void** events) {
  if (!events || !events[0] || !events[1] || !events[2] || !events[3])
    return PARISKV_ERR_INVALID_ARG;
  return attn_impl(Q, K, V, kv_rows_per_head, idx, k, batch, n_q_heads, n_kv_heads, head_dim,
                   dtype, scale, out, ws, ws_bytes, stream, events);
}

int32_t pariskv_debug_export(const pariskv_index* ix, int64_t lo, int64_t hi, uint8_t* ids_host,
                             uint8_t* nib_host, uint16_t* w_host) {
  if (!ix || lo < 0 || hi < lo || hi > ix->cfg.capacity) return PARISKV_ERR_INVALID_ARG;
  if (flush_pending(const_cast<pariskv_index*>(ix))) return PARISKV_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return PARISKV_ERR_HIP;
  const int64_t BH = (int64_t)ix->cfg.batch * ix->cfg.n_kv_heads;
  const int64_t cap = ix->cfg.capacity, n = hi - lo;
  const int B = ix->cfg.n_subspaces;  // 16 (m = 8) or 32 (m = 4)
  if (n == 0) return PARISKV_OK;
  std::vector<uint8_t> packed(B == 16 ? 0 : (size_t)n * 16);
  for (int64_t bh = 0; bh < BH; ++bh) {
    const int64_t key = bh * cap + lo;
    if (ids_host) {
      // device byte s holds the sign bits of coordinates 8 s .. 8 s + 7:
      // one id (m = 8), or the ids of subspaces 2 s and 2 s + 1 (m = 4)
      uint8_t* dst = B == 16 ? ids_host + bh * n * 16 : packed.data();
      if (hipMemcpy(dst, ix->ids + key * 16, n * 16, hipMemcpyDeviceToHost) != hipSuccess)
        return PARISKV_ERR_HIP;
      if (B == 32)
        for (int64_t i = 0; i < n * 16; ++i) {
          ids_host[bh * n * 32 + 2 * i] = packed[i] & 15u;
          ids_host[bh * n * 32 + 2 * i + 1] = packed[i] >> 4;
        }
    }
    const uint8_t* rec = (const uint8_t*)ix->rec + key * 128;
    if (nib_host && hipMemcpy2D(nib_host + bh * n * 64, 64, rec, 128, 64, n,
                                hipMemcpyDeviceToHost) != hipSuccess)
      return PARISKV_ERR_HIP;
    if (w_host && hipMemcpy2D(w_host + bh * n * B, 2 * B, rec + 64, 128, 2 * B, n,
                              hipMemcpyDeviceToHost) != hipSuccess)
      return PARISKV_ERR_HIP;
  }
  return PARISKV_OK;
}

int32_t pariskv_retrieve_sizes(const pariskv_index* ix, int32_t k, int64_t* E, int64_t* C) {
  if (!ix || !E || !C) return PARISKV_ERR_INVALID_ARG;
  const int64_t S = ix->cfg.n_sink;
  if (k <= S || (int64_t)k > ix->n) return PARISKV_ERR_INVALID_ARG;
  *E = ix->n - S;
  *C = cand_count(*E, k - S, ix->cfg.cand_num, ix->cfg.cand_den);
  return PARISKV_OK;
}

int32_t pariskv_set_retrieval_path(pariskv_index* ix, int32_t path) {
  if (!ix || (path != PARISKV_PATH_AUTO && path != PARISKV_PATH_PIPELINE &&
              path != PARISKV_PATH_SINGLE))
    return PARISKV_ERR_INVALID_ARG;
  ix->path = path;
  return PARISKV_OK;
}

int32_t pariskv_retrieval_path(const pariskv_index* ix, int32_t k) {
  int64_t E = 0, C = 0;
  const int32_t rc = pariskv_retrieve_sizes(ix, k, &E, &C);
  if (rc) return rc;
  return choose_path(ix, C);
}

int32_t pariskv_debug_intermediate(const pariskv_index* ix, int32_t k, const void* ws,
                                   size_t ws_bytes, int32_t which, void* host_dst,
                                   size_t dst_bytes) {
  int64_t E = 0, C = 0;
  int32_t rc = pariskv_retrieve_sizes(ix, k, &E, &C);
  if (rc) return rc;
  if (!ws || !host_dst) return PARISKV_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(&ix->cfg, k);
  if (ws_bytes < L.total) return PARISKV_ERR_WORKSPACE;
  const int64_t BH = units_of(&ix->cfg);  // one row per retrieval unit
  const uint8_t* base = (const uint8_t*)ws;
  if (hipDeviceSynchronize() != hipSuccess) return PARISKV_ERR_HIP;
  auto rows = [&](size_t off, int64_t stride, int64_t len, int64_t elem) -> int32_t {
    if (dst_bytes < (size_t)(BH * len * elem)) return PARISKV_ERR_INVALID_ARG;
    for (int64_t bh = 0; bh < BH; ++bh)
      if (hipMemcpy((uint8_t*)host_dst + bh * len * elem, base + off + bh * stride * elem,
                    len * elem, hipMemcpyDeviceToHost) != hipSuccess)
        return PARISKV_ERR_HIP;
    return PARISKV_OK;
  };
  switch (which) {
    case 0: return rows(L.lut, 16 * 256, 16 * 256, 1);
    case 1: return rows(L.yq, 128, 128, 4);
    case 2: return rows(L.scores, L.Epad, E, 1);
    case 3: return rows(L.cand, L.cstride, C, 4);
    case 4: return rows(L.est, L.cstride, C, 4);
    case 5: return rows(L.meta, 4, 4, 4);
    default: return PARISKV_ERR_INVALID_ARG;
  }
}

int32_t pariskv_window_create(pariskv_index* ix, int64_t n_local, int64_t n_update, void* K_near,
                              void* V_near, void* K_far, void* V_far, int64_t far_rows_per_head,
                              pariskv_window** out) {
  if (out) *out = nullptr;
  if (!ix || !out || !K_near || !V_near || !K_far || !V_far) return PARISKV_ERR_INVALID_ARG;
  const int64_t S = ix->cfg.n_sink;
  if (n_update < 1 || n_local < n_update || n_local % n_update) return PARISKV_ERR_INVALID_ARG;
  if (ix->n < S || far_rows_per_head < ix->cfg.capacity) return PARISKV_ERR_INVALID_ARG;
  if (n_local + n_update > 0x7FFFFFFFll) return PARISKV_ERR_INVALID_ARG;
  pariskv_window* w = new (std::nothrow) pariskv_window;
  if (!w) return PARISKV_ERR_NOMEM;
  w->ix = ix;
  w->S = S;
  w->L = n_local;
  w->U = n_update;
  w->ring = n_local + n_update;
  w->Kn = (uint8_t*)K_near;
  w->Vn = (uint8_t*)V_near;
  w->Kf = (uint8_t*)K_far;
  w->Vf = (uint8_t*)V_far;
  w->far_rows = far_rows_per_head;
  w->R = ix->n - S;
  w->u = 0;
  w->rb = (size_t)ix->cfg.head_dim * (ix->cfg.key_dtype == PARISKV_DTYPE_BF16 ? 2 : 4);
  *out = w;
  return PARISKV_OK;
}

int32_t pariskv_window_append(pariskv_window* w, const void* K_new, const void* V_new,
                              int64_t new_rows_per_head, void* stream) {
  if (!w || !K_new || !V_new || new_rows_per_head < 1) return PARISKV_ERR_INVALID_ARG;
  pariskv_index* ix = w->ix;
  if (w->u + 1 == w->U && ix->n + w->U > ix->cfg.capacity) return PARISKV_ERR_CAPACITY;
  const int64_t BH = (int64_t)ix->cfg.batch * ix->cfg.n_kv_heads;
  const size_t rb = w->rb, near_pitch = (size_t)(w->S + w->ring) * rb;
  hipStream_t st = (hipStream_t)stream;
  // the new token's row goes to its ring slot in the near store
  const int64_t p = w->S + w->R + w->L + w->u;
  const int64_t slot = w->S + (p - w->S) % w->ring;
  (void)hipGetLastError();
  hipError_t e = hipMemcpy2DAsync(w->Kn + slot * rb, near_pitch, K_new, new_rows_per_head * rb, rb,
                                  BH, hipMemcpyDefault, st);
  if (e == hipSuccess)
    e = hipMemcpy2DAsync(w->Vn + slot * rb, near_pitch, V_new, new_rows_per_head * rb, rb, BH,
                         hipMemcpyDefault, st);
  if (e != hipSuccess) return PARISKV_ERR_HIP;
  if (++w->u < w->U) return PARISKV_OK;
  // update buffer full: the U oldest local tokens [S + R, S + R + U) move to the
  // retrieval region: their rows are copied to the far store and their keys
  // encoded into the index now (the next token reuses the first slot).  Their
  // ring slots start at S + R % ring and wrap to S at the end of the ring, so
  // the copy and the encode run in at most two contiguous pieces.
  const int64_t pos0 = w->S + w->R, r0 = w->R % w->ring;
  const int64_t n1 = (w->U < w->ring - r0) ? w->U : w->ring - r0;
  const size_t far_pitch = (size_t)w->far_rows * rb;
  if (int32_t rc = flush_pending(ix)) return rc;
  for (int piece = 0; piece < 2; ++piece) {
    const int64_t cnt = piece ? w->U - n1 : n1;
    if (cnt == 0) continue;
    const int64_t slot0 = w->S + (piece ? 0 : r0), pos = pos0 + (piece ? n1 : 0);
    e = hipMemcpy2DAsync(w->Kf + pos * rb, far_pitch, w->Kn + slot0 * rb, near_pitch, cnt * rb,
                         BH, hipMemcpyDefault, st);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(w->Vf + pos * rb, far_pitch, w->Vn + slot0 * rb, near_pitch,
                           cnt * rb, BH, hipMemcpyDefault, st);
    if (e == hipSuccess)
      e = pkv::launch_encode(m_of(&ix->cfg), ix->cfg.key_dtype, w->Kn + slot0 * rb,
                             w->S + w->ring, ix->n + (piece ? n1 : 0), cnt, (int)BH,
                             ix->cfg.capacity, ix->ids, ix->rec, ix->signs, ix->rot_c, st,
                             pkv::EvPair{});
    if (e != hipSuccess) return PARISKV_ERR_HIP;
  }
  ix->n += w->U;
  ix->last = st;
  w->R += w->U;
  w->u = 0;
  return PARISKV_OK;
}

int32_t pariskv_window_state(const pariskv_window* w, int64_t* n_tokens, int64_t* n_retrieval,
                             int64_t* n_tail) {
  if (!w) return PARISKV_ERR_INVALID_ARG;
  if (n_tokens) *n_tokens = w->S + w->R + w->L + w->u;
  if (n_retrieval) *n_retrieval = w->R;
  if (n_tail) *n_tail = w->L + w->u;
  return PARISKV_OK;
}

int32_t pariskv_window_attn_workspace_bytes(const pariskv_window* w, int32_t k, size_t* bytes) {
  if (!w || !bytes || k < 1) return PARISKV_ERR_INVALID_ARG;
  const pariskv_config* c = &w->ix->cfg;
  const int64_t rows = (int64_t)k + w->L + w->U;
  if (rows > 0x7FFFFFFFll) return PARISKV_ERR_INVALID_ARG;
  return pariskv_attn_workspace_bytes(c->batch, c->n_q_heads, (int32_t)rows, c->head_dim, bytes);
}

static int32_t window_attn_impl(const pariskv_window* w, const void* Q, const int32_t* idx, int32_t k,
                         float scale, void* out, void* ws, size_t ws_bytes, void* stream,
                         void** events) {
  if (!w) return PARISKV_ERR_INVALID_ARG;
  const pariskv_config* c = &w->ix->cfg;
  pkv::AttnRows rs;
  rs.K = w->Kf;
  rs.V = w->Vf;
  rs.rows = w->far_rows;
  rs.K_near = w->Kn;
  rs.V_near = w->Vn;
  rs.near_rows = w->S + w->ring;
  rs.n_near_head = w->S;
  rs.ring = w->ring;
  rs.tail_lo = w->S + w->R;
  rs.tail_n = (int)(w->L + w->u);
  return attn_core(Q, rs, idx, k, c->batch, c->n_q_heads, c->n_kv_heads, c->head_dim,
                   c->key_dtype, scale, out, ws, ws_bytes, stream, events);
}

int32_t pariskv_window_attn(const pariskv_window* w, const void* Q, const int32_t* idx, int32_t k,
                            float scale, void* out, void* ws, size_t ws_bytes, void* stream) {
  return window_attn_impl(w, Q, idx, k, scale, out, ws, ws_bytes, stream, nullptr);
}

int32_t pariskv_window_attn_profiled(const pariskv_window* w, const void* Q, const int32_t* idx,
                                     int32_t k, float scale, void* out, void* ws,
                                     size_t ws_bytes, void* stream, void** events) {
  if (!events) return PARISKV_ERR_INVALID_ARG;
  for (int s = 0; s < 4; ++s)
    if (!events[s]) return PARISKV_ERR_INVALID_ARG;
  return window_attn_impl(w, Q, idx, k, scale, out, ws, ws_bytes, stream, events);
}

void pariskv_window_destroy(pariskv_window* w) { delete w; }

int32_t pariskv_codebook(int32_t m, float* L, float* tau) {
  if (!L || !tau) return PARISKV_ERR_INVALID_ARG;
  if (m == 8) pkv::codebook_m8(L, tau);
  else if (m == 4) pkv::codebook_m4(L, tau);
  else return PARISKV_ERR_UNSUPPORTED;
  return PARISKV_OK;
}

float pariskv_rot_scale(int32_t head_dim) { return head_dim > 0 ? rot_scale(head_dim) : 0.0f; }

int32_t pariskv_srht_signs_from_seed(uint64_t seed, int32_t head_dim, int8_t* signs) {
  if (!signs || head_dim < 1 || head_dim > 1024) return PARISKV_ERR_INVALID_ARG;
  // SplitMix64: Weyl-sequence state, output mixed by two multiply rounds
  constexpr uint64_t kGamma = 0x9e3779b97f4a7c15ull;
  constexpr uint64_t kMul1 = 0xbf58476d1ce4e5b9ull, kMul2 = 0x94d049bb133111ebull;
  for (int32_t j = 0; j < head_dim; ++j) {
    uint64_t x = seed + kGamma * (uint64_t)(j + 1);
    x = (x ^ (x >> 30)) * kMul1;
    x = (x ^ (x >> 27)) * kMul2;
    x ^= x >> 31;
    signs[j] = (int8_t)(1 - 2 * (int)(x >> 63));
  }
  return PARISKV_OK;
}

const char* pariskv_status_string(int32_t s) {
  switch (s) {
    case PARISKV_OK: return "ok";
    case PARISKV_ERR_INVALID_ARG: return "invalid argument";
    case PARISKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PARISKV_ERR_CAPACITY: return "index capacity exceeded";
    case PARISKV_ERR_WORKSPACE: return "workspace or index buffer too small";
    case PARISKV_ERR_HIP: return "HIP runtime error";
    case PARISKV_ERR_NOMEM: return "host allocation failed";
    default: return "unknown status";
  }
}

}  // extern "C"
