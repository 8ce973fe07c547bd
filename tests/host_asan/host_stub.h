// Recorder of the host-only stand-ins (host_stub.cpp).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "kernels.h"

namespace hoststub {
struct Call {
  std::string name;          // launcher name without "launch_"
  moba::Dims d;              // its problem dimensions (when it takes them)
  bool has_d = false;
  std::vector<uintptr_t> ptrs;   // pointer arguments in order
  std::vector<int64_t> ints;     // integer / flag arguments in order
  uintptr_t stream = 0;
};
extern std::vector<Call> g_calls;
extern int g_events_created, g_streams_created, g_event_records, g_stream_waits;
extern int g_mallocs, g_frees;
void record(const Call& c);
void reset();
}  // namespace hoststub
