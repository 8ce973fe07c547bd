// Host-only stand-ins for the GPU side of libmoba.so, for the sanitizer
// build of the C ABI layer (csrc/api.cpp with csrc/plan.cpp): every kernel
// launcher records its call (name, problem dimensions, pointer and integer
// arguments, stream) instead of launching, and the few HIP runtime calls the
// ABI layer makes are answered on the host (no device is touched; workspace
// "allocations" hand out addresses that nothing dereferences).  Used by
// tests/host_asan/host_checks.cpp.
#include <cstdint>
#include <cstdlib>
#include <string>
#include <vector>

#include "host_stub.h"
#include "kernels.h"

namespace hoststub {
std::vector<Call> g_calls;
int g_events_created = 0, g_streams_created = 0, g_event_records = 0, g_stream_waits = 0;
int g_mallocs = 0, g_frees = 0;
void record(const Call& c) { g_calls.push_back(c); }
void reset() {
  g_calls.clear();
  g_events_created = g_streams_created = g_event_records = g_stream_waits = 0;
  g_mallocs = g_frees = 0;
}
}  // namespace hoststub

using hoststub::Call;
using hoststub::record;

// ------------------------------------------------------------ HIP runtime
static uintptr_t g_next_handle = 0x1000;
static uintptr_t g_next_addr = (uintptr_t)1 << 44;

extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* stream, unsigned int) {
  ++hoststub::g_streams_created;
  *stream = reinterpret_cast<hipStream_t>(g_next_handle += 16);
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t* event) {
  ++hoststub::g_events_created;
  *event = reinterpret_cast<hipEvent_t>(g_next_handle += 16);
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned) {
  return hipEventCreate(event);
}
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  ++hoststub::g_event_records;
  return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) {
  ++hoststub::g_stream_waits;
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 0.f;
  return hipSuccess;
}
hipError_t hipMallocAsync(void** ptr, size_t size, hipStream_t) {
  ++hoststub::g_mallocs;
  *ptr = reinterpret_cast<void*>(g_next_addr);
  g_next_addr += (size + 4095) & ~(size_t)4095;
  return hipSuccess;
}
hipError_t hipFreeAsync(void*, hipStream_t) {
  ++hoststub::g_frees;
  return hipSuccess;
}
hipError_t hipMemsetAsync(void*, int, size_t, hipStream_t) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "host stub"; }
}  // extern "C"

// ------------------------------------------------------------- launchers
namespace moba {

hipError_t noalloc_scratch(void** out) {
  *out = reinterpret_cast<void*>((uintptr_t)0x7f0000000000);
  Call c;
  c.name = "noalloc_scratch";
  record(c);
  return hipSuccess;
}

hipError_t launch_block_mean(const void* k, float* kbar, float* partial, const Dims& d, hipStream_t st, bool defer_finalize, int j0) {
  Call c;
  c.name = "block_mean";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(kbar));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(partial));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  c.ints.push_back((int64_t)defer_finalize);
  c.ints.push_back((int64_t)j0);
  record(c);
  return hipSuccess;
}

hipError_t launch_pool_transpose(const void* k, const void* v, float* kbar, float* partial, void* vt, void* ktail, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "pool_transpose";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(kbar));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(partial));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(vt));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ktail));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_block_mean_finalize(float* kbar, const float* partial, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "block_mean_finalize";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(kbar));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(partial));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_transpose_v(const void* k, const void* v, void* vt, void* ktail, const Dims& d, hipStream_t st, const float* bm_partial, float* kbar) {
  Call c;
  c.name = "transpose_v";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(vt));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ktail));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bm_partial));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(kbar));
  record(c);
  return hipSuccess;
}

hipError_t launch_gate_topk(const void* q, const float* kbar, int32_t* sel, const Dims& d, hipStream_t st, uint32_t* counts) {
  Call c;
  c.name = "gate_topk";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(kbar));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(sel));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(counts));
  record(c);
  return hipSuccess;
}

hipError_t launch_route_count(const int32_t* sel, uint32_t* counts, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "route_count";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(sel));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(counts));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_route_scan_rows(uint32_t* counts, uint32_t* bucket_total, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "route_scan_rows";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(counts));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_total));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_route_scan_buckets(const uint32_t* bucket_total, uint32_t* bucket_off, uint32_t* tile_off, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "route_scan_buckets";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_total));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(tile_off));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_route_scan_small(uint32_t* counts, uint32_t* bucket_off, uint32_t* tile_off, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "route_scan_small";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(counts));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(tile_off));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_route_scatter(const int32_t* sel, const uint32_t* counts, const uint32_t* bucket_off, uint32_t* list, const Dims& d, hipStream_t st, bool counts_global) {
  Call c;
  c.name = "route_scatter";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(sel));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(counts));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(list));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  c.ints.push_back((int64_t)counts_global);
  record(c);
  return hipSuccess;
}

hipError_t launch_attn_routed_bf16(const void* q, const void* k, const void* vt, const uint32_t* list, const uint32_t* bucket_off, const uint32_t* tile_off, void* part_o, float* part_lse, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "attn_routed_bf16";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(vt));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(list));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(tile_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part_o));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part_lse));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_attn_routed_f32(const void* q, const void* k, const void* v, const uint32_t* list, const uint32_t* bucket_off, const uint32_t* tile_off, void* part_o, float* part_lse, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "attn_routed_f32";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(list));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(tile_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part_o));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part_lse));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_attn_query_bf16(const void* q, const void* k, const void* vt, const void* ktail, const void* part_o, const float* part_lse, void* out, int mode, const Dims& d, hipStream_t st, int nparts, float* lse_out) {
  Call c;
  c.name = "attn_query_bf16";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(vt));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ktail));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part_o));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part_lse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(out));
  c.ints.push_back((int64_t)mode);
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  c.ints.push_back((int64_t)nparts);
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse_out));
  record(c);
  return hipSuccess;
}

hipError_t launch_merge_partials_bf16(const void* own_o, const float* own_lse, int nown, const void* po, const float* plse, void* out, const Dims& d, hipStream_t st, float* lse_out) {
  Call c;
  c.name = "merge_partials_bf16";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(own_o));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(own_lse));
  c.ints.push_back((int64_t)nown);
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(po));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(plse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(out));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse_out));
  record(c);
  return hipSuccess;
}

hipError_t launch_attn_query_f32(const void* q, const void* k, const void* v, const void* part_o, const float* part_lse, void* out, int mode, const Dims& d, hipStream_t st, float* lse_out) {
  Call c;
  c.name = "attn_query_f32";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part_o));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part_lse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(out));
  c.ints.push_back((int64_t)mode);
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse_out));
  record(c);
  return hipSuccess;
}

hipError_t launch_decode_plan(const int32_t* sel, int32_t* ublk, uint32_t* umask, int32_t* ucount, bool all_blocks, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "decode_plan";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(sel));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ublk));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(umask));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ucount));
  c.ints.push_back((int64_t)all_blocks);
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_decode_attn(const void* q, const void* k, const void* v, const int32_t* ublk, const uint32_t* umask, const int32_t* ucount, float* part, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "decode_attn";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ublk));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(umask));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ucount));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_decode_merge(const float* part, const int32_t* ublk, const uint32_t* umask, const int32_t* ucount, void* out, const Dims& d, hipStream_t st, float* lse_out) {
  Call c;
  c.name = "decode_merge";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(part));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ublk));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(umask));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ucount));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(out));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse_out));
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_dot(const void* out, const void* dout, const float* lse, float* dvec, void* rowstat, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_dot";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(out));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dout));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dvec));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(rowstat));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_tail(const void* k, const void* v, void* ktail, void* vtail, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_tail";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ktail));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(vtail));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_dq_routed(const void* q, const void* dout, const void* k, const void* v, const float* lse, const float* dvec, const uint32_t* list, const uint32_t* bucket_off, const uint32_t* tile_off, void* dqp, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_dq_routed";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dout));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dvec));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(list));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(tile_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dqp));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_dq_own(const void* q, const void* dout, const void* k, const void* v, const void* ktail, const void* vtail, const float* lse, const float* dvec, const void* dqp, void* dq, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_dq_own";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dout));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ktail));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(vtail));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dvec));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dqp));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dq));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_entry_rows(const uint32_t* list, const uint32_t* bucket_off, void* ent, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_entries";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(list));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ent));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_dkdv(const void* q, const void* dout, const void* k, const void* v, const void* rowstat, const void* ent, const uint32_t* bucket_off, void* dk, void* dv, float* kvpart, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_dkdv";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dout));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(rowstat));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(ent));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dk));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dv));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(kvpart));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_dot_f32(const void* out, const void* dout, float* dvec, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_dot_f32";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(out));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dout));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dvec));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_dq_routed_f32(const void* q, const void* dout, const void* k, const void* v, const float* lse, const float* dvec, const uint32_t* list, const uint32_t* bucket_off, const uint32_t* tile_off, float* dqp, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_dq_routed_f32";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dout));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dvec));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(list));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(tile_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dqp));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_dq_own_f32(const void* q, const void* dout, const void* k, const void* v, const float* lse, const float* dvec, const float* dqp, void* dq, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_dq_own_f32";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dout));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dvec));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dqp));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dq));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_bwd_dkdv_f32(const void* q, const void* dout, const void* k, const void* v, const float* lse, const float* dvec, const uint32_t* list, const uint32_t* bucket_off, void* dk, void* dv, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "bwd_dkdv_f32";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dout));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(v));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(lse));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dvec));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(list));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(bucket_off));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dk));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(dv));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_naive_scores(const void* q, const void* k, float* sc, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "naive_scores";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(q));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(k));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(sc));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_naive_softmax(const float* sc, const int32_t* sel, void* p, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "naive_softmax";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(sc));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(sel));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(p));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

hipError_t launch_naive_pv(const void* p, const void* vt, void* out, const Dims& d, hipStream_t st) {
  Call c;
  c.name = "naive_pv";
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(p));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(vt));
  c.ptrs.push_back(reinterpret_cast<uintptr_t>(out));
  c.d = d; c.has_d = true;
  c.stream = reinterpret_cast<uintptr_t>(st);
  record(c);
  return hipSuccess;
}

}  // namespace moba
