// Test driver for the C-ABI sources built host-only with the address and
// undefined-behaviour sanitizers (kernel launchers replaced by
// launch_stubs.cpp): configuration checks, sizing, index and window handles,
// argument errors and the launch sequencing of every entry point, with
// device pointers that the host code never dereferences.  Prints "ok" when
// every expectation holds.  Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "launch_stubs.h"
#include "pariskv.h"

namespace {

int fails = 0;
#define EXPECT(x)                                                   \
  do {                                                              \
    if (!(x)) {                                                     \
      std::printf("failed: %s (line %d)\n", #x, __LINE__);         \
      ++fails;                                                      \
    }                                                               \
  } while (0)

// a device address stand-in, 1 MiB aligned, never dereferenced here (the
// stubs launch nothing, and no entry point called below copies memory)
void* dev(uintptr_t a) { return reinterpret_cast<void*>(a << 20); }

pariskv_config base_cfg() {
  pariskv_config c{};
  c.head_dim = 128;
  c.n_subspaces = 16;
  c.rho = 4;
  const int tw[4] = {4, 3, 2, 1};
  for (int i = 0; i < 4; ++i) c.tier_w[i] = tw[i];
  c.cand_num = 1;
  c.cand_den = 20;
  c.n_sink = 16;
  c.batch = 2;
  c.n_kv_heads = 4;
  c.n_q_heads = 16;
  c.key_dtype = PARISKV_DTYPE_BF16;
  c.capacity = 100000;
  c.per_query_head = 0;
  return c;
}

void run_index(const pariskv_config& c, int32_t k) {
  size_t ib = 0, ws = 0;
  EXPECT(pariskv_index_bytes(&c, &ib) == PARISKV_OK && ib > 0);
  EXPECT(pariskv_retrieve_workspace_bytes(&c, k, &ws) == PARISKV_OK && ws > 0);
  std::vector<int8_t> signs(128);
  for (int j = 0; j < 128; ++j) signs[j] = (j * 7) % 3 ? 1 : -1;
  pariskv_index* ix = nullptr;
  EXPECT(pariskv_build_index(&c, signs.data(), dev(1), ib, dev(2), c.capacity, 50000, nullptr,
                             &ix) == PARISKV_OK);
  if (!ix) return;
  EXPECT(pariskv_append_keys(ix, dev(3), c.capacity, 1, nullptr) == PARISKV_OK);   // deferred
  EXPECT(pariskv_append_keys(ix, dev(3), c.capacity, 3, nullptr) == PARISKV_OK);   // flush + defer
  EXPECT(pariskv_append_keys(ix, dev(3), c.capacity, 100, nullptr) == PARISKV_OK); // encoded now
  EXPECT(pariskv_index_size(ix) == 50104);
  EXPECT(pariskv_append_keys(ix, dev(3), c.capacity, c.capacity, nullptr) == PARISKV_ERR_CAPACITY);
  EXPECT(pariskv_retrieve_topk(ix, dev(4), k, (int32_t*)dev(5), (float*)dev(6), dev(7), ws,
                               nullptr) == PARISKV_OK);
  EXPECT(pariskv_retrieve_topk(ix, dev(4), k, (int32_t*)dev(5), nullptr, dev(7), ws - 1,
                               nullptr) == PARISKV_ERR_WORKSPACE);
  EXPECT(pariskv_retrieve_topk(ix, dev(4), 60000, (int32_t*)dev(5), nullptr, dev(7), ws,
                               nullptr) == PARISKV_ERR_INVALID_ARG);
  EXPECT(pariskv_retrieve_topk(ix, dev(4), c.n_sink, (int32_t*)dev(5), nullptr, dev(7), ws,
                               nullptr) == PARISKV_ERR_INVALID_ARG);
  // the entry point that allocates nothing: this workspace fits its scratch
  EXPECT(ws <= PARISKV_NOALLOC_SCRATCH_BYTES);
  EXPECT(pariskv_retrieve_topk_noalloc(ix, dev(4), k, (int32_t*)dev(5), (float*)dev(6),
                                       nullptr) == PARISKV_OK);
  EXPECT(pariskv_retrieve_topk_noalloc(ix, dev(4), c.n_sink, (int32_t*)dev(5), nullptr,
                                       nullptr) == PARISKV_ERR_INVALID_ARG);
  EXPECT(pariskv_retrieve_topk_noalloc(nullptr, dev(4), k, (int32_t*)dev(5), nullptr,
                                       nullptr) == PARISKV_ERR_INVALID_ARG);
  int64_t E = 0, C = 0;
  EXPECT(pariskv_retrieve_sizes(ix, k, &E, &C) == PARISKV_OK && E == 50104 - c.n_sink && C > 0);
  // retrieval paths: the pipeline by default; the single kernel, when asked
  // for, serves shared retrieval with at most 16384 candidates
  EXPECT(pariskv_retrieval_path(ix, k) == PARISKV_PATH_PIPELINE);
  EXPECT(pariskv_set_retrieval_path(ix, 7) == PARISKV_ERR_INVALID_ARG);
  EXPECT(pariskv_set_retrieval_path(nullptr, PARISKV_PATH_SINGLE) == PARISKV_ERR_INVALID_ARG);
  EXPECT(pariskv_set_retrieval_path(ix, PARISKV_PATH_SINGLE) == PARISKV_OK);
  if (c.per_query_head) {
    EXPECT(pariskv_retrieval_path(ix, k) == PARISKV_ERR_UNSUPPORTED);
    // a refused retrieval leaves a deferred append pending (encoded at destroy)
    EXPECT(pariskv_append_keys(ix, dev(3), c.capacity, 1, nullptr) == PARISKV_OK);
    EXPECT(pariskv_retrieve_topk(ix, dev(4), k, (int32_t*)dev(5), nullptr, dev(7), ws,
                                 nullptr) == PARISKV_ERR_UNSUPPORTED);
    EXPECT(pariskv_index_size(ix) == 50105);
  } else {
    EXPECT(pariskv_retrieval_path(ix, k) == PARISKV_PATH_SINGLE);
    EXPECT(pariskv_retrieve_topk(ix, dev(4), k, (int32_t*)dev(5), (float*)dev(6), dev(7), ws,
                                 nullptr) == PARISKV_OK);
  }
  EXPECT(pariskv_retrieval_path(ix, c.n_sink) == PARISKV_ERR_INVALID_ARG);
  EXPECT(pariskv_set_retrieval_path(ix, PARISKV_PATH_AUTO) == PARISKV_OK);
  // a window over the index
  if (!c.per_query_head) {
    pariskv_window* w = nullptr;
    EXPECT(pariskv_window_create(ix, 1024, 128, dev(8), dev(9), dev(10), dev(11), c.capacity,
                                 &w) == PARISKV_OK);
    pariskv_window* bad = w;
    EXPECT(pariskv_window_create(ix, 1000, 128, dev(8), dev(9), dev(10), dev(11), c.capacity,
                                 &bad) == PARISKV_ERR_INVALID_ARG && bad == nullptr);
    EXPECT(pariskv_window_create(ix, 1024, 128, dev(8), dev(9), dev(10), dev(11), c.capacity - 1,
                                 &bad) == PARISKV_ERR_INVALID_ARG && bad == nullptr);
    if (w) {
      int64_t nt = 0, nr = 0, nl = 0;
      EXPECT(pariskv_window_state(w, &nt, &nr, &nl) == PARISKV_OK && nl == 1024);
      size_t aws = 0;
      EXPECT(pariskv_window_attn_workspace_bytes(w, k, &aws) == PARISKV_OK && aws > 0);
      EXPECT(pariskv_window_attn(w, dev(4), (const int32_t*)dev(5), k, 0.088f, dev(12), dev(13),
                                 aws, nullptr) == PARISKV_OK);
      pariskv_window_destroy(w);
    }
  }
  pariskv_index_destroy(ix);
}

// A window whose retrieval region R0 is not a multiple of the update buffer
// U: promotions take ring rows that wrap past the ring's end.  Host buffers
// stand in for the near and far stores (the copy stub copies host memory and
// aborts on any access outside a registered buffer); every row carries its
// (head, position) tag, so the far store and the encoded rows can be checked
// position by position.
void run_window_wrap() {
  pariskv_config c = base_cfg();
  c.capacity = 4096;
  const int64_t S = c.n_sink, L = 64, U = 32, ring = L + U, N0 = 2013;
  const int64_t R0 = N0 - S, BH = (int64_t)c.batch * c.n_kv_heads, d = 128;
  EXPECT(R0 % U != 0 && R0 % ring + U > ring);
  size_t ib = 0;
  EXPECT(pariskv_index_bytes(&c, &ib) == PARISKV_OK);
  std::vector<int8_t> signs(128, 1);
  pariskv_index* ix = nullptr;
  EXPECT(pariskv_build_index(&c, signs.data(), dev(1), ib, dev(2), c.capacity, N0, nullptr,
                             &ix) == PARISKV_OK);
  if (!ix) return;
  auto tag = [&](uint16_t* row, int64_t h, int64_t p) {
    row[0] = (uint16_t)h;
    row[1] = (uint16_t)(p & 0xFFFF);
    row[2] = (uint16_t)(p >> 16);
  };
  auto has_tag = [&](const uint16_t* row, int64_t h, int64_t p) {
    return row[0] == (uint16_t)h && row[1] == (uint16_t)(p & 0xFFFF) &&
           row[2] == (uint16_t)(p >> 16);
  };
  const int64_t nrows = S + ring;
  std::vector<uint16_t> Kn(BH * nrows * d, 0xFFFF), Vn(Kn), Kf(BH * c.capacity * d, 0xFFFF),
      Vf(Kf), Kx(BH * d), Vx(BH * d);
  for (auto* v : {&Kn, &Vn, &Kf, &Vf, &Kx, &Vx}) stub_track(v->data(), v->size() * 2);
  for (int64_t h = 0; h < BH; ++h) {
    for (int64_t p = 0; p < S; ++p) tag(&Kn[(h * nrows + p) * d], h, p);
    for (int64_t p = S + R0; p < S + R0 + L; ++p)
      tag(&Kn[(h * nrows + S + (p - S) % ring) * d], h, p);
  }
  Vn = Kn;
  pariskv_window* w = nullptr;
  EXPECT(pariskv_window_create(ix, L, U, Kn.data(), Vn.data(), Kf.data(), Vf.data(), c.capacity,
                               &w) == PARISKV_OK);
  if (!w) return;
  stub_clear_encodes();
  int promotions = 0;
  size_t seen = 0;
  int64_t next = S + R0, pieces = 0;
  for (int64_t t = 0; t < 100; ++t) {
    const int64_t p = S + R0 + L + t;
    for (int64_t h = 0; h < BH; ++h) tag(&Kx[h * d], h, p);
    Vx = Kx;
    EXPECT(pariskv_window_append(w, Kx.data(), Vx.data(), 1, nullptr) == PARISKV_OK);
    int64_t nt = 0, R = 0, tail = 0;
    EXPECT(pariskv_window_state(w, &nt, &R, &tail) == PARISKV_OK && nt == p + 1);
    if (R == R0 + (promotions + 1) * U) ++promotions;
    EXPECT(pariskv_index_size(ix) == S + R);
    // encodes issued by this call: each reads its own tokens' ring rows
    for (; seen < stub_encodes().size(); ++seen) {
      const StubEncode& e = stub_encodes()[seen];
      EXPECT(e.lo == next && e.rows_per_head == nrows);
      const int64_t r0 = ((const uint16_t*)e.K - Kn.data()) / d;
      for (int64_t h = 0; h < BH; ++h)
        for (int64_t i = 0; i < e.n; ++i) EXPECT(has_tag(&Kn[(h * nrows + r0 + i) * d], h, e.lo + i));
      next += e.n;
      ++pieces;
    }
  }
  EXPECT(promotions == 3);
  EXPECT(next == S + R0 + 3 * U && pieces == 4);  // the first promotion in two pieces
  // the far store holds positions [S + R0, S + R0 + 3U) of every head
  for (int64_t h = 0; h < BH; ++h)
    for (int64_t p = S + R0; p < S + R0 + 3 * U; ++p) {
      EXPECT(has_tag(&Kf[(h * c.capacity + p) * d], h, p));
      EXPECT(has_tag(&Vf[(h * c.capacity + p) * d], h, p));
    }
  pariskv_window_destroy(w);
  pariskv_index_destroy(ix);
  stub_untrack_all();
}

}  // namespace

int main() {
  pariskv_config c = base_cfg();
  run_index(c, 1024);
  run_window_wrap();
  c.n_subspaces = 32;  // subspaces of 4
  run_index(c, 300);
  c = base_cfg();
  c.per_query_head = 1;
  run_index(c, 512);
  // a retrieval workspace beyond the no-alloc scratch is refused before any launch
  {
    pariskv_config big = base_cfg();
    big.capacity = 2000000;  // 8 heads x 2M keys: about 45 MiB of workspace at k = 1024
    size_t ib = 0, ws = 0;
    EXPECT(pariskv_index_bytes(&big, &ib) == PARISKV_OK);
    EXPECT(pariskv_retrieve_workspace_bytes(&big, 1024, &ws) == PARISKV_OK &&
           ws > PARISKV_NOALLOC_SCRATCH_BYTES);
    std::vector<int8_t> signs(128, 1);
    pariskv_index* ix = nullptr;
    EXPECT(pariskv_build_index(&big, signs.data(), dev(1), ib, dev(2), big.capacity, 5000,
                               nullptr, &ix) == PARISKV_OK);
    if (ix) {
      EXPECT(pariskv_retrieve_topk_noalloc(ix, dev(4), 1024, (int32_t*)dev(5), nullptr,
                                           nullptr) == PARISKV_ERR_WORKSPACE);
      pariskv_index_destroy(ix);
    }
  }
  // configuration errors
  c = base_cfg();
  size_t n = 0;
  c.rho = 9;
  EXPECT(pariskv_index_bytes(&c, &n) == PARISKV_ERR_INVALID_ARG);
  c = base_cfg();
  c.n_q_heads = 12;
  EXPECT(pariskv_index_bytes(&c, &n) == PARISKV_ERR_UNSUPPORTED);
  c = base_cfg();
  c.head_dim = 64;
  EXPECT(pariskv_index_bytes(&c, &n) == PARISKV_ERR_UNSUPPORTED);
  // attention
  size_t aws = 0;
  EXPECT(pariskv_attn_workspace_bytes(2, 16, 1000, 128, &aws) == PARISKV_OK);
  EXPECT(pariskv_sparse_attn(dev(1), dev(2), dev(3), 5000, (const int32_t*)dev(4), 1000, 2, 16, 4,
                             128, PARISKV_DTYPE_BF16, 0.088f, dev(5), dev(6), aws,
                             nullptr) == PARISKV_OK);
  EXPECT(pariskv_sparse_attn_per_query_head(dev(1), dev(2), dev(3), 5000, (const int32_t*)dev(4),
                                            1000, 2, 16, 4, 128, PARISKV_DTYPE_BF16, 0.088f,
                                            dev(5), dev(6), aws, nullptr) == PARISKV_OK);
  EXPECT(pariskv_sparse_attn(dev(1), dev(2), dev(3), 5000, (const int32_t*)dev(4), 1000, 2, 16, 4,
                             128, PARISKV_DTYPE_BF16, 0.088f, dev(5), dev(6), aws - 1,
                             nullptr) == PARISKV_ERR_WORKSPACE);
  // the Self-Indexing workload
  pariskv_si_config s{};
  s.head_dim = 128;
  s.n_sink = 8;
  s.batch = 2;
  s.n_kv_heads = 4;
  s.n_q_heads = 16;
  s.key_dtype = PARISKV_DTYPE_FP32;
  s.capacity = 70000;
  size_t sib = 0, sbw = 0, srw = 0;
  EXPECT(pariskv_si_index_bytes(&s, &sib) == PARISKV_OK);
  EXPECT(pariskv_si_build_workspace_bytes(&s, 60000, &sbw) == PARISKV_OK);
  EXPECT(pariskv_si_retrieve_workspace_bytes(&s, 500, &srw) == PARISKV_OK);
  pariskv_si_index* si = nullptr;
  EXPECT(pariskv_si_build_index(&s, dev(20), sib, dev(21), s.capacity, 60000, dev(22), sbw,
                                nullptr, &si) == PARISKV_OK);
  if (si) {
    EXPECT(pariskv_si_append_keys(si, dev(23), s.capacity, 10, nullptr) == PARISKV_OK);
    EXPECT(pariskv_si_index_size(si) == 60010);
    EXPECT(pariskv_si_retrieve_topk(si, dev(24), 500, (int32_t*)dev(25), (float*)dev(26), dev(27),
                                    srw, nullptr) == PARISKV_OK);
    EXPECT(pariskv_si_retrieve_topk(si, dev(24), 8, (int32_t*)dev(25), nullptr, dev(27), srw,
                                    nullptr) == PARISKV_ERR_INVALID_ARG);
    pariskv_si_index_destroy(si);
  }
  std::printf(fails ? "FAILED\n" : "ok\n");
  return fails != 0;
}
