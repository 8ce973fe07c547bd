// Host-only checks of the C ABI layer (csrc/api.cpp + csrc/plan.cpp) built
// with AddressSanitizer and UndefinedBehaviorSanitizer against the recording
// stand-ins of host_stub.cpp: argument checks, structs of every ABI version
// read from buffers of exactly their size, host arrays of exactly their
// length, and the launch sequences the planning rules choose.  No GPU.
// Prints one line per check; the exit status counts the failures.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "host_stub.h"
#include "moba.h"

using hoststub::Call;
using hoststub::g_calls;

static int failures = 0;

static void expect(bool ok, const char* what) {
  std::printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) {
    ++failures;
    std::printf("     last error: %s\n", moba_last_error());
  }
}

static const uintptr_t kFake = (uintptr_t)1 << 40;   // device addresses, never dereferenced

static moba_args make_args(int32_t batch, int64_t q_len, int64_t kv_len, int32_t H, int32_t Hkv,
                           int32_t D, int32_t B, int32_t topk, moba_dtype dt = MOBA_DTYPE_BF16) {
  moba_args a;
  std::memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(moba_args);
  a.q = a.k = a.v = (const void*)kFake;
  a.out = (void*)(kFake + ((uintptr_t)1 << 36));
  a.batch = batch; a.n_heads = H; a.n_kv_heads = Hkv; a.head_dim = D;
  a.block_size = B; a.topk = topk; a.q_len = q_len; a.kv_len = kv_len; a.dtype = dt;
  return a;
}

static int count(const char* name) {
  int n = 0;
  for (const Call& c : g_calls) n += c.name == name;
  return n;
}

static int first(const char* name) {
  for (size_t i = 0; i < g_calls.size(); ++i)
    if (g_calls[i].name == name) return (int)i;
  return -1;
}

// Structs of the older ABI versions, copied into heap buffers of exactly
// their size: the library must read nothing past struct_size.
static void check_struct_versions() {
  const moba_args full = make_args(1, 4096, 4096, 8, 2, 128, 512, 4);
  const size_t sizes[] = {offsetof(moba_args, lse_out), offsetof(moba_args, kv_lens),
                          offsetof(moba_args, routed_bytes_limit), sizeof(moba_args)};
  size_t ref = 0;
  for (size_t n : sizes) {
    unsigned char* buf = static_cast<unsigned char*>(std::malloc(n));
    std::memcpy(buf, &full, n);
    reinterpret_cast<moba_args*>(buf)->struct_size = n;
    const size_t ws = moba_workspace_size(reinterpret_cast<const moba_args*>(buf));
    if (ref == 0) ref = ws;
    char what[128];
    std::snprintf(what, sizeof(what), "struct of %zu bytes read within its size (workspace %zu)",
                  n, ws);
    expect(ws > 0 && ws == ref, what);
    std::free(buf);
  }
  unsigned char* buf = static_cast<unsigned char*>(std::malloc(sizeof(size_t)));
  const size_t bad = 24;
  std::memcpy(buf, &bad, sizeof(size_t));
  expect(moba_workspace_size(reinterpret_cast<const moba_args*>(buf)) == 0 &&
             std::strstr(moba_last_error(), "struct_size") != nullptr,
         "an unknown struct_size is refused after reading struct_size alone");
  std::free(buf);
}

static void check_validation_enqueues_nothing() {
  moba_args a = make_args(1, 1024, 1024, 4, 2, 96, 128, 3);
  hoststub::reset();
  expect(moba_forward_ex(&a) == MOBA_ERR_UNSUPPORTED && g_calls.empty() &&
             hoststub::g_mallocs == 0,
         "head_dim 96: UNSUPPORTED, nothing launched or allocated");
  a = make_args(1, 2048, 1024, 4, 2, 128, 128, 3);
  expect(moba_forward_ex(&a) == MOBA_ERR_INVALID_ARGUMENT && g_calls.empty(),
         "q_len > kv_len: INVALID_ARGUMENT, nothing launched");
  a = make_args(1, 1024, 1024, 4, 2, 128, 128, 3);
  a.workspace = (void*)kFake;
  a.workspace_bytes = 16;
  expect(moba_forward_ex(&a) == MOBA_ERR_INVALID_ARGUMENT && g_calls.empty(),
         "a short workspace: INVALID_ARGUMENT, nothing launched");
}

// bf16 q_len 1 with 64 query heads per KV head: the decode kernels do not
// take the group, the call routes, and the gate that runs (the decode gate)
// writes no routing histogram -> the gate gets no counts buffer and
// route_count runs before the scans.
static void check_decode_gate_routing() {
  moba_args a = make_args(2, 1, 4096, 64, 1, 128, 64, 4);
  hoststub::reset();
  const moba_status st = moba_forward_ex(&a);
  const int gi = first("gate_topk"), ci = first("route_count");
  const int si = first("route_scan_small") >= 0 ? first("route_scan_small")
                                                : first("route_scan_rows");
  expect(st == MOBA_OK && gi >= 0 && g_calls[gi].ptrs.size() == 4 && g_calls[gi].ptrs[3] == 0,
         "q_len 1, 64 heads per KV head: the gate gets no counts buffer");
  expect(ci > gi && si > ci && first("decode_attn") < 0,
         "... and route_count runs after it, before the scans (not the decode kernels)");
  // a prefill with the 128-row gate: it writes the histogram itself
  a = make_args(1, 2048, 2048, 16, 1, 128, 64, 4);
  hoststub::reset();
  moba_forward_ex(&a);
  const int g2 = first("gate_topk");
  expect(g2 >= 0 && g_calls[g2].ptrs[3] != 0 && count("route_count") == 0,
         "a bf16 prefill: the gate writes the histogram, no route_count");
}

// 1M tokens, 32/8 heads: the routed partials pass the default limit, so the
// call routes one KV head at a time: one gate and one column scan, then per
// pass the bucket scan, the scatter, the routed tiles and the own block.
static void check_grouped_passes() {
  moba_args a = make_args(1, 1 << 20, 1 << 20, 32, 8, 128, 4096, 12);
  a.workspace = (void*)kFake;
  a.workspace_bytes = moba_workspace_size(&a);
  hoststub::reset();
  expect(moba_forward_ex(&a) == MOBA_OK, "1M-token prefill with a caller workspace");
  expect(count("gate_topk") == 1 && count("route_scan_rows") == 1 &&
             count("route_scan_buckets") == 8 && count("route_scatter") == 8 &&
             count("attn_routed_bf16") == 8 && count("attn_query_bf16") == 8,
         "... one gate and column scan, eight passes of scan, scatter, routed, own+merge");
  bool ok = true;
  int pass = 0;
  for (const Call& c : g_calls) {
    if (c.name != "attn_routed_bf16") continue;
    const moba::Dims& d = c.d;
    ok = ok && d.ps0 == 0 && d.pS == 1 && d.ph0 == 4 * pass && d.pH == 4 &&
         d.prow0 == 256 * pass && d.pnrows == 256 &&
         d.pslots == (int64_t)4 * (1 << 20) * 11;
    ++pass;
  }
  expect(ok && pass == 8, "... pass p covers query heads 4p..4p+3 and buckets 256p..256p+255");
  a.routed_bytes_limit = (size_t)1 << 40;
  a.workspace_bytes = moba_workspace_size(&a);
  hoststub::reset();
  moba_forward_ex(&a);
  expect(count("attn_routed_bf16") == 1 && g_calls[first("attn_routed_bf16")].d.pH == 32,
         "a limit above all partials: one pass over every head");
  expect(hoststub::g_mallocs == 0, "a caller workspace: nothing allocated");
}

// The entry point that allocates nothing: no allocation, stream or event;
// the own block runs on the caller's stream; too large problems refused.
static void check_noalloc() {
  moba_args a = make_args(1, 32768, 32768, 1, 1, 128, 2048, 3);
  a.stream = (void*)0x4440;
  hoststub::reset();
  const moba_status st = moba_forward_noalloc(&a);
  bool own_here = false;
  for (const Call& c : g_calls)
    if (c.name == "attn_query_bf16" && c.ints.size() >= 1 && c.ints[0] == 2)
      own_here = c.stream == 0x4440;
  expect(st == MOBA_OK && count("noalloc_scratch") == 1, "noalloc: the 32K workload runs");
  expect(hoststub::g_mallocs == 0 && hoststub::g_events_created == 0 &&
             hoststub::g_streams_created == 0 && hoststub::g_stream_waits == 0,
         "... with no allocation, event or stream");
  expect(own_here, "... and the own block on the caller's stream");
  // the stand-in scratch array starts at 0x7f0000000000; every workspace
  // buffer handed to the routed kernel lies inside its 64 MiB (q and k are
  // the caller's, below it)
  const uintptr_t base = 0x7f0000000000, end = base + ((uintptr_t)64 << 20);
  int inside = 0;
  bool outside = false;
  for (const Call& c : g_calls)
    if (c.name == "attn_routed_bf16")
      for (uintptr_t p : c.ptrs) {
        if (p >= base && p < end) ++inside;
        if (p >= end) outside = true;
      }
  expect(inside >= 5 && !outside, "... its buffers inside the 64 MiB scratch array");
  a = make_args(1, 1 << 17, 1 << 17, 32, 8, 128, 4096, 12);
  hoststub::reset();
  expect(moba_forward_noalloc(&a) == MOBA_ERR_UNSUPPORTED && g_calls.empty(),
         "noalloc: a 128K problem is refused before anything runs");
  hoststub::reset();
  a = make_args(1, 32768, 32768, 1, 1, 128, 2048, 3);
  moba_forward_ex(&a);
  expect(hoststub::g_events_created == 2 && hoststub::g_stream_waits == 2,
         "moba_forward_ex at 32K: the own block on the internal stream (fork and join)");
}

// Packed variable-length calls read exactly batch + 1 host offsets.
static void check_varlen_host_arrays() {
  const int batch = 5;
  int64_t* cq = static_cast<int64_t*>(std::malloc((batch + 1) * sizeof(int64_t)));
  int64_t* ck = static_cast<int64_t*>(std::malloc((batch + 1) * sizeof(int64_t)));
  const int64_t lq[batch] = {300, 0, 77, 1, 129}, lk[batch] = {300, 50, 1234, 700, 129};
  cq[0] = ck[0] = 0;
  for (int s = 0; s < batch; ++s) {
    cq[s + 1] = cq[s] + lq[s];
    ck[s + 1] = ck[s] + lk[s];
  }
  moba_varlen_args v;
  std::memset(&v, 0, sizeof(v));
  v.struct_size = sizeof(v);
  v.q = v.k = v.v = (const void*)kFake;
  v.out = (void*)kFake;
  v.cu_seqlens_q = cq;
  v.cu_seqlens_k = ck;
  v.batch = batch; v.n_heads = 4; v.n_kv_heads = 2; v.head_dim = 128; v.block_size = 128;
  v.topk = 3; v.dtype = MOBA_DTYPE_BF16;
  const size_t ws = moba_varlen_workspace_size(&v, 0);
  hoststub::reset();
  const moba_status st = moba_forward_varlen(&v);
  expect(ws > 0 && st == MOBA_OK && count("gate_topk") == 4,
         "varlen: exact-size host offsets, one call per non-empty sequence");
  cq[2] = cq[1] - 1;   // decreasing
  hoststub::reset();
  expect(moba_forward_varlen(&v) == MOBA_ERR_INVALID_ARGUMENT && g_calls.empty(),
         "varlen: decreasing offsets refused before anything runs");
  std::free(cq);
  std::free(ck);
}

static void check_route_and_backward() {
  hoststub::reset();
  const moba_status st = moba_route((const int32_t*)kFake, 2, 6, 2, 700, 1500, 64, 5,
                                    (uint32_t*)kFake, (uint32_t*)kFake, nullptr, 0, nullptr);
  expect(st == MOBA_OK && count("route_count") == 1 && count("route_scatter") == 1 &&
             hoststub::g_mallocs == 1 && hoststub::g_frees == 1,
         "moba_route: count, scan, scatter on a stream-ordered workspace");
  moba_bwd_args b;
  std::memset(&b, 0, sizeof(b));
  b.struct_size = sizeof(b);
  b.q = b.k = b.v = b.out = b.dout = (const void*)kFake;
  b.lse = (const float*)kFake;
  b.sel = (const int32_t*)kFake;
  b.dq = b.dk = b.dv = (void*)kFake;
  b.batch = 1; b.n_heads = 8; b.n_kv_heads = 2; b.head_dim = 128; b.block_size = 128;
  b.topk = 4; b.q_len = 4096; b.kv_len = 4096; b.dtype = MOBA_DTYPE_BF16;
  hoststub::reset();
  expect(moba_backward_ex(&b) == MOBA_OK && count("bwd_dkdv") == 1 && count("bwd_dq_own") == 1,
         "backward: dq and dk/dv launched");
  // bf16 dk/dv reads the entry rows written from the routing list
  expect(count("bwd_entries") == 1 && first("route_scatter") < first("bwd_entries") &&
             first("bwd_entries") < first("bwd_dkdv") && count("bwd_tail") == 0,
         "backward: entry rows after the scatter and before dk/dv; no tail copy at 4096 keys");
  b.kv_len = 4100; b.q_len = 4100;
  hoststub::reset();
  expect(moba_backward_ex(&b) == MOBA_OK && count("bwd_tail") == 1,
         "backward: the last partial K/V tile copied when kv_len % 64 != 0");
  b.dtype = MOBA_DTYPE_F32;
  hoststub::reset();
  expect(moba_backward_ex(&b) == MOBA_OK && count("bwd_entries") == 0 && count("bwd_tail") == 0,
         "backward fp32: no entry rows, no tail copy");
}

int main() {
  check_struct_versions();
  check_validation_enqueues_nothing();
  check_decode_gate_routing();
  check_grouped_passes();
  check_noalloc();
  check_varlen_host_arrays();
  check_route_and_backward();
  std::printf("%s\n", failures ? "FAILED" : "passed");
  return failures;
}
