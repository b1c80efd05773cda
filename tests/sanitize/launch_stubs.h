// Checks the host-only launcher stubs (launch_stubs.cpp) offer the driver:
// registered host buffers are bounds-checked by the 2-D copy and the encode
// stubs, and every encode call is recorded.  Test infrastructure only.
#pragma once
#include <cstddef>
#include <cstdint>
#include <vector>

struct StubEncode {
  const void* K;
  int64_t rows_per_head;
  int64_t lo;
  int64_t n;
};

void stub_track(const void* p, size_t bytes);
void stub_untrack_all();
const std::vector<StubEncode>& stub_encodes();
void stub_clear_encodes();
