// C ABI of libmoba.so: argument checks, workspace layout and the launch
// sequence of the MoBA forward.  Every entry point checks all arguments
// before it enqueues anything and never lets a C++ exception cross the ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "moba.h"

using moba::Dims;

namespace {

thread_local std::string g_last_error;

// Sizes of the version-1 moba_args (without lse_out and kv_lens) and of the
// version-2 one (without kv_lens), still accepted.
constexpr size_t kArgsV1Size = offsetof(moba_args, lse_out);
constexpr size_t kArgsV2Size = offsetof(moba_args, kv_lens);
constexpr size_t kArgsV3Size = offsetof(moba_args, routed_bytes_limit);
// Routed partial outputs (with their log-sum-exps and list entries) a bf16
// prefill holds at once unless moba_args.routed_bytes_limit says otherwise;
// above it the routing runs one (sequence, KV head) at a time.
constexpr size_t kDefaultRoutedBytes = (size_t)12 << 30;

// Copies the caller's struct (any version) into a full one, so that no field
// past the caller's struct_size is read; later fields default to NULL.
moba_args load_args(const moba_args* a) {
  moba_args b;
  std::memset(&b, 0, sizeof(b));
  size_t n = 0;
  std::memcpy(&n, a, sizeof(size_t));   // struct_size comes first in every version
  if (n == sizeof(moba_args) || n == kArgsV1Size || n == kArgsV2Size || n == kArgsV3Size)
    std::memcpy(&b, a, n);
  else b.struct_size = n;               // rejected by check_common
  return b;
}

moba_status fail(moba_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

// ---------------------------------------------------------------- profiling
enum KernelId {
  K_BLOCK_MEAN, K_TRANSPOSE_V, K_GATE, K_RCOUNT, K_RSCAN_ROWS, K_RSCAN_BUCKETS, K_RSCATTER,
  K_ATTN_ROUTED, K_ATTN_OWN, K_ATTN_FULL, K_DEC_PLAN, K_DEC_ATTN, K_DEC_MERGE, K_MERGE,
  K_POOL_TRANSPOSE, K_MEAN_FINALIZE, K_RSCAN_SMALL, K_BWD_DOT, K_BWD_TAIL,
  K_BWD_DQ_ROUTED, K_BWD_DQ_OWN, K_BWD_DKDV, K_NAIVE_SCORES, K_NAIVE_SOFTMAX, K_NAIVE_PV,
  K_BWD_ENTRIES, K_COUNT
};
const char* const kKernelNames[K_COUNT] = {
    "block_mean", "transpose_v", "gate_topk", "route_count", "route_scan_rows",
    "route_scan_buckets", "route_scatter", "attn_routed", "attn_own_merge", "attn_full",
    "decode_plan", "decode_attn", "decode_merge", "merge_partials", "pool_transpose",
    "block_mean_finalize", "route_scan_small", "bwd_dot", "bwd_tail", "bwd_dq_routed",
    "bwd_dq_own", "bwd_dkdv", "naive_scores", "naive_softmax", "naive_pv", "bwd_entries"};

struct ProfRecord {
  int id;
  hipEvent_t a, b;
};

struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<ProfRecord> recs;
  double total_ms[K_COUNT] = {};
  int64_t launches[K_COUNT] = {};
};
Profiler g_prof;

struct Launch {
  hipStream_t st;
  hipError_t err = hipSuccess;
  const char* what = nullptr;
  template <class F>
  void run(int id, F&& f) {
    if (err != hipSuccess) return;
    hipEvent_t a = nullptr, b = nullptr;
    bool prof = false;
    {
      std::lock_guard<std::mutex> g(g_prof.mu);
      prof = g_prof.on;
    }
    if (prof) {
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess ||
          hipEventRecord(a, st) != hipSuccess) {
        err = hipErrorUnknown;
        what = "profiling event";
        return;
      }
    }
    err = f();
    if (err != hipSuccess) {
      what = kKernelNames[id];
      return;
    }
    if (prof) {
      (void)hipEventRecord(b, st);
      std::lock_guard<std::mutex> g(g_prof.mu);
      g_prof.recs.push_back({id, a, b});
    }
  }
};

// ------------------------------------------------------------ side stream
// One non-blocking stream per device (default priority), created on first use
// and kept for the life of the process.  The own-block attention runs on it
// concurrently with the gate and routing; fork/join events are per call.
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
hipStream_t g_side[kMaxDevices] = {};

hipError_t side_stream(hipStream_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_side_mu);
  if (!g_side[dev]) {
    e = hipStreamCreateWithFlags(&g_side[dev], hipStreamNonBlocking);
    if (e != hipSuccess) {
      g_side[dev] = nullptr;
      return e;
    }
  }
  *out = g_side[dev];
  return hipSuccess;
}

// ------------------------------------------------------------------ checks
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

struct Plan {
  Dims d;
  bool need_kbar = false, need_vt = false, need_sel = false, routed = false, decode = false;
  size_t off_kbar = 0, off_vt = 0, off_sel = 0, off_counts = 0, off_btotal = 0, off_boff = 0,
         off_toff = 0, off_list = 0, off_po = 0, off_plse = 0, total = 0;
  size_t off_ublk = 0, off_umask = 0, off_ucount = 0, off_part = 0, off_bmpart = 0;
  size_t off_own_o = 0, off_own_lse = 0;
  size_t off_ktail = 0;    // bf16 with L % 64 != 0: last K tile, zero padded
  size_t off_sc = 0, off_p = 0;  // mask-based form: dense scores and probabilities
  bool need_ktail = false;
  bool split_own = false;  // own block on the side stream + separate merge
  int full_parts = 0;      // split full attention: key chunks per row (0: whole rows)
  bool grouped = false;    // routing pass by pass: group_kv KV heads of one sequence each
  int group_kv = 0;
};

moba_status check_common(const moba_args* a, bool full, Plan* p) {
  if (!a) return fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(moba_args) && a->struct_size != kArgsV1Size &&
      a->struct_size != kArgsV2Size && a->struct_size != kArgsV3Size)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "struct_size %zu != sizeof(moba_args) %zu",
                a->struct_size, sizeof(moba_args));
  if (!a->q || !a->k || !a->v || !a->out)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "q, k, v and out must be non-NULL");
  if (a->batch < 1 || a->n_heads < 1 || a->n_kv_heads < 1 || a->head_dim < 1 || a->q_len < 1 ||
      a->kv_len < 1)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (!full && (a->block_size < 1 || a->topk < 1))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "block_size and topk must be >= 1");
  if (a->n_heads % a->n_kv_heads != 0)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "n_heads %% n_kv_heads != 0");
  if (a->q_len > a->kv_len) return fail(MOBA_ERR_INVALID_ARGUMENT, "q_len > kv_len");
  if (a->dtype != MOBA_DTYPE_F32 && a->dtype != MOBA_DTYPE_BF16)
    return fail(MOBA_ERR_UNSUPPORTED, "unknown dtype %d", (int)a->dtype);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(MOBA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", a->head_dim);
  const uintptr_t align = (uintptr_t)a->q | (uintptr_t)a->k | (uintptr_t)a->v |
                          (uintptr_t)a->out | (uintptr_t)a->k_block_mean |
                          (uintptr_t)a->workspace;
  if (align & 15) return fail(MOBA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (a->sel_out && ((uintptr_t)a->sel_out & 3))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "sel_out must be 4-byte aligned");
  if (a->lse_out && ((uintptr_t)a->lse_out & 3))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "lse_out must be 4-byte aligned");
  if (a->kv_lens && ((uintptr_t)a->kv_lens & 3))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "kv_lens must be 4-byte aligned");
  if (a->kv_lens && a->q_len != 1)
    return fail(MOBA_ERR_UNSUPPORTED, "kv_lens needs q_len 1 (a decode batch)");

  Dims& d = p->d;
  d.S = a->batch; d.H = a->n_heads; d.Hkv = a->n_kv_heads; d.G = d.H / d.Hkv; d.D = a->head_dim;
  d.Lq = a->q_len; d.L = a->kv_len; d.q_off = d.L - d.Lq; d.bf16 = a->dtype == MOBA_DTYPE_BF16;
  d.kv_lens = a->kv_lens;
  moba::whole_pass(d);
  int64_t t = 0;
  if (!mul_ok(d.S, d.Lq, &t) || !mul_ok(t, d.H, &t) || !mul_ok(t, d.D, &t) ||
      !mul_ok(d.S, d.L, &t) || !mul_ok(t, d.Hkv, &t) || !mul_ok(t, d.D, &t) ||
      !mul_ok(t, 4, &t))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "tensor size overflows int64");
  if ((int64_t)d.S * d.H > 65535)
    return fail(MOBA_ERR_UNSUPPORTED, "batch * n_heads > 65535");
  if (d.L >= ((int64_t)1 << 31)) return fail(MOBA_ERR_UNSUPPORTED, "kv_len >= 2^31");
  d.Lv = (d.L + 63) / 64 * 64;
  // bf16 prefill kernels address the transposed V [.., D, Lv] with 32-bit offsets
  if (d.bf16 && d.Lq > 1 && d.Lv * d.D >= ((int64_t)1 << 31))
    return fail(MOBA_ERR_UNSUPPORTED, "kv_len * head_dim >= 2^31 with bf16 and q_len > 1");
  return MOBA_OK;
}

// Argument checks and the dimensions shared by the forward and the backward.
moba_status forward_dims(const moba_args* a, Plan* p) {
  moba_status st = check_common(a, false, p);
  if (st != MOBA_OK) return st;
  Dims& d = p->d;
  if (a->block_size % 64 != 0)
    return fail(MOBA_ERR_UNSUPPORTED, "block_size %d is not a multiple of 64", a->block_size);
  if (a->topk > moba::kMaxTopk)
    return fail(MOBA_ERR_UNSUPPORTED, "topk %d > %d", a->topk, moba::kMaxTopk);
  const int64_t nb = (d.L + a->block_size - 1) / a->block_size;  // last block may be partial
  if (nb > moba::kMaxBlocks) return fail(MOBA_ERR_UNSUPPORTED, "more than %d blocks", moba::kMaxBlocks);
  d.B = a->block_size;
  d.topk = a->topk;
  d.kp = d.topk - 1;
  d.nb = (int)nb;
  d.nchunk_r = (int)((d.Lq + moba::kRouteChunkRows - 1) / moba::kRouteChunkRows);
  d.ncols = d.G * d.nchunk_r;
  d.nrows = d.S * d.Hkv * d.nb;
  int64_t slots = 0;
  if (!mul_ok((int64_t)d.S * d.H, d.Lq, &slots) || !mul_ok(slots, d.kp, &slots))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "slot count overflows");
  if (slots >= ((int64_t)1 << 32))
    return fail(MOBA_ERR_UNSUPPORTED, "more than 2^32 routed slots");
  d.slots = slots;
  // Routed tiles of 256 entries (8-wave workgroups, one per CU, twice the
  // work per K/V tile load) unless there would be too few of them to spread
  // over the chip; the fp32 path always uses 128.
  d.tile_m = (d.bf16 && slots / 256 >= 128) ? 256 : 128;
  moba::whole_pass(d);
  if ((int64_t)d.S * d.H * d.nchunk_r >= ((int64_t)1 << 31))
    return fail(MOBA_ERR_UNSUPPORTED, "too many routing chunks");
  return MOBA_OK;
}

moba_status plan_forward(const moba_args* a, Plan* p) {
  moba_status st = forward_dims(a, p);
  if (st != MOBA_OK) return st;
  Dims& d = p->d;
  const int64_t esz = d.bf16 ? 2 : 4;
  p->need_kbar = a->k_block_mean == nullptr;
  p->need_sel = a->sel_out == nullptr;
  p->decode = moba::decode_supported(d);
  if (d.kv_lens && !p->decode)
    return fail(MOBA_ERR_UNSUPPORTED,
                "kv_lens needs the decode kernels (block_size a multiple of 512, at most 8 "
                "query heads per KV head)");
  p->need_vt = d.bf16 && !p->decode;
  p->routed = !p->decode && d.kp > 0 && d.nb > 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  if (p->need_kbar) {
    p->off_kbar = take((size_t)d.S * d.Hkv * d.nb * d.D * 4);
    p->off_bmpart = take(moba::block_mean_partial_floats(d) * 4);
  }
  if (p->decode) {
    const size_t nu = (size_t)d.S * d.Hkv * moba::decode_umax(d);
    p->off_ublk = take(nu * 4);
    p->off_umask = take(nu * 4);
    p->off_ucount = take((size_t)d.S * d.Hkv * 4);
    p->off_part = take(moba::decode_part_floats(d) * 4);
  }
  if (p->need_vt) p->off_vt = take((size_t)d.S * d.Hkv * d.D * d.Lv * 2);
  p->need_ktail = p->need_vt && d.L % 64 != 0;
  if (p->need_ktail) p->off_ktail = take((size_t)d.S * 64 * d.Hkv * d.D * 2);
  if (p->need_sel) p->off_sel = take((size_t)d.S * d.H * d.Lq * d.topk * 4);
  if (p->routed) {
    // Large bf16 problems whose routed partials pass the limit route one
    // (sequence, KV head) at a time: list and partials then hold one pass.
    const size_t limit = a->routed_bytes_limit ? a->routed_bytes_limit : kDefaultRoutedBytes;
    const bool small = d.bf16 && (int64_t)d.S * d.H * d.Lq <= ((int64_t)1 << 20);
    const size_t routed_bytes = (size_t)d.slots * (d.D * esz + 8);
    p->grouped = d.bf16 && !small && d.S * d.Hkv > 1 && routed_bytes > limit;
    Dims dp = d;
    if (p->grouped) {
      // as many KV heads of one sequence per pass as fit the limit (at least one)
      const size_t per_kv = (size_t)d.G * d.Lq * d.kp * (d.D * esz + 8);
      size_t ng = limit / per_kv;
      if (ng < 1) ng = 1;
      if (ng > (size_t)d.Hkv) ng = d.Hkv;
      p->group_kv = (int)ng;
      moba::group_pass(dp, 0, 0, p->group_kv);
    }
    p->off_counts = take((size_t)d.nrows * d.ncols * 4);
    p->off_btotal = take((size_t)d.nrows * 4);
    p->off_boff = take((size_t)(dp.pnrows + 1) * 4);
    p->off_toff = take((size_t)(dp.pnrows + 1) * 4);
    p->off_list = take((size_t)dp.pslots * 4);
    p->off_po = take((size_t)dp.pslots * d.D * esz);
    p->off_plse = take((size_t)dp.pslots * 4);
    // Small problems: run the own block concurrently with the routing (its
    // workgroups alone do not fill the chip).  Large ones fill the chip with
    // the routed attention already, and the fused own-block + merge is cheaper.
    if (d.bf16 && (int64_t)d.S * d.H * d.Lq <= ((int64_t)1 << 20)) {
      p->split_own = true;
      const size_t nqh = (size_t)d.S * d.H * d.Lq;
      p->off_own_o = take(2 * nqh * d.D * 2);   // two halves of a split own block
      p->off_own_lse = take(2 * nqh * 4);
    }
  }
  p->total = off;
  if (a->workspace && a->workspace_bytes < p->total)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes",
                a->workspace_bytes, p->total);
  return MOBA_OK;
}

// Mask-based form: the forward's gate, then dense scores, masked softmax and
// P.V.  Workspace: block means (when not given), the selection (when not
// requested), V^T (+ the K tail tile), fp32 scores and bf16 probabilities of
// every (query, key) pair.
moba_status plan_naive(const moba_args* a, Plan* p) {
  moba_status st = forward_dims(a, p);
  if (st != MOBA_OK) return st;
  Dims& d = p->d;
  if (!d.bf16) return fail(MOBA_ERR_UNSUPPORTED, "moba_naive_ex: bf16 only");
  if (d.kv_lens) return fail(MOBA_ERR_UNSUPPORTED, "moba_naive_ex: no kv_lens");
  int64_t pairs = 0;
  if (!mul_ok((int64_t)d.S * d.H, d.Lq, &pairs) || pairs >= ((int64_t)1 << 31) ||
      !mul_ok(pairs, d.Lv, &pairs) || !mul_ok(pairs, 6, &pairs))
    return fail(MOBA_ERR_UNSUPPORTED, "moba_naive_ex: score matrix too large");
  p->need_kbar = a->k_block_mean == nullptr;
  p->need_sel = a->sel_out == nullptr;
  p->need_vt = true;
  p->need_ktail = d.L % 64 != 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  if (p->need_kbar) {
    p->off_kbar = take((size_t)d.S * d.Hkv * d.nb * d.D * 4);
    p->off_bmpart = take(moba::block_mean_partial_floats(d) * 4);
  }
  if (p->need_sel) p->off_sel = take((size_t)d.S * d.H * d.Lq * d.topk * 4);
  p->off_vt = take((size_t)d.S * d.Hkv * d.D * d.Lv * 2);
  if (p->need_ktail) p->off_ktail = take((size_t)d.S * 64 * d.Hkv * d.D * 2);
  const size_t n = (size_t)d.S * d.H * d.Lq * d.Lv;
  p->off_sc = take(n * 4);
  p->off_p = take(n * 2);
  p->total = off;
  if (a->workspace && a->workspace_bytes < p->total)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes",
                a->workspace_bytes, p->total);
  return MOBA_OK;
}

moba_status plan_full(const moba_args* a, Plan* p) {
  moba_status st = check_common(a, true, p);
  if (st != MOBA_OK) return st;
  Dims& d = p->d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  // q_len 1: split-K over 512-key chunks with every chunk kept by every head
  Dims dd = d;
  dd.B = moba::decode_chunk();
  dd.nb = (int)((d.L + dd.B - 1) / dd.B);
  dd.topk = dd.nb;
  if (d.kv_lens && !(dd.nb <= moba::kMaxBlocks && moba::decode_supported(dd)))
    return fail(MOBA_ERR_UNSUPPORTED, "kv_lens needs the decode kernels (at most 8 query "
                "heads per KV head)");
  if (dd.nb <= moba::kMaxBlocks && moba::decode_supported(dd)) {
    d = dd;
    d.kp = 0;
    p->decode = true;
    const size_t nu = (size_t)d.S * d.Hkv * moba::decode_umax(d);
    p->off_ublk = take(nu * 4);
    p->off_umask = take(nu * 4);
    p->off_ucount = take((size_t)d.S * d.Hkv * 4);
    p->off_part = take(moba::decode_part_floats(d) * 4);
  } else {
    d.B = 64;
    d.topk = 1;
    d.kp = 0;
    d.nb = (int)((d.L + 63) / 64);
    p->need_vt = d.bf16;
    if (p->need_vt) p->off_vt = take((size_t)d.S * d.Hkv * d.D * d.Lv * 2);
    p->need_ktail = p->need_vt && d.L % 64 != 0;
    if (p->need_ktail) p->off_ktail = take((size_t)d.S * 64 * d.Hkv * d.D * 2);
    // small problems: key chunks + merge (whole row tiles would leave the chip idle)
    p->full_parts = moba::full_split_parts(d);
    if (p->full_parts > 0) {
      const size_t nqh = (size_t)d.S * d.H * d.Lq;
      p->off_own_o = take((size_t)p->full_parts * nqh * d.D * 2);
      p->off_own_lse = take((size_t)p->full_parts * nqh * 4);
    }
  }
  p->total = off;
  if (a->workspace && a->workspace_bytes < p->total)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes",
                a->workspace_bytes, p->total);
  return MOBA_OK;
}

struct Workspace {
  char* base = nullptr;
  bool owned = false;
  hipStream_t st = nullptr;
  ~Workspace() {
    if (owned && base) (void)hipFreeAsync(base, st);
  }
};

moba_status get_workspace(const moba_args* a, const Plan& p, Workspace* ws) {
  ws->st = (hipStream_t)a->stream;
  if (p.total == 0) return MOBA_OK;
  if (a->workspace) {
    ws->base = (char*)a->workspace;
    return MOBA_OK;
  }
  void* ptr = nullptr;
  const hipError_t e = hipMallocAsync(&ptr, p.total, ws->st);
  if (e != hipSuccess || !ptr) {
    (void)hipGetLastError();
    return fail(MOBA_ERR_OUT_OF_MEMORY, "hipMallocAsync(%zu bytes) failed: %s", p.total,
                hipGetErrorString(e));
  }
  ws->base = (char*)ptr;
  ws->owned = true;
  return MOBA_OK;
}

// Makes `main` wait for the side stream's last event when a call leaves early,
// so that the stream-ordered free of a library workspace (and the caller's next
// work) comes after the side stream's kernels.
struct SideJoin {
  hipStream_t main = nullptr;
  hipEvent_t done = nullptr;
  ~SideJoin() {
    if (done) {
      (void)hipStreamWaitEvent(main, done, 0);
      (void)hipEventDestroy(done);
    }
  }
};

moba_status hip_fail(const Launch& l) {
  return fail(MOBA_ERR_HIP, "launch of %s failed: %s", l.what ? l.what : "?",
              hipGetErrorString(l.err));
}

// fixed_ws (nullable): device memory of fixed_bytes used as the workspace
// instead of the caller's or an allocation; the call then also keeps off the
// internal stream (no stream or event is created) and allocates nothing.
moba_status forward_impl(const moba_args* a, void* fixed_ws = nullptr, size_t fixed_bytes = 0) {
  Plan p;
  moba_status st = plan_forward(a, &p);
  if (st != MOBA_OK) return st;
  Workspace ws;
  if (fixed_ws) {
    if (p.total > fixed_bytes)
      return fail(MOBA_ERR_UNSUPPORTED,
                  "the problem needs %zu bytes of scratch; the entry point that allocates "
                  "nothing holds at most %zu (use moba_forward_ex with a workspace)",
                  p.total, fixed_bytes);
    ws.base = (char*)fixed_ws;
    ws.st = (hipStream_t)a->stream;
  } else {
    st = get_workspace(a, p, &ws);
    if (st != MOBA_OK) return st;
  }
  const Dims& d = p.d;
  char* w = ws.base;
  float* kbar = p.need_kbar ? (float*)(w + p.off_kbar) : const_cast<float*>(a->k_block_mean);
  void* vt = p.need_vt ? (void*)(w + p.off_vt) : nullptr;
  void* ktail = p.need_ktail ? (void*)(w + p.off_ktail) : nullptr;
  int32_t* sel = p.need_sel ? (int32_t*)(w + p.off_sel) : a->sel_out;
  uint32_t* counts = (uint32_t*)(w + p.off_counts);
  uint32_t* btotal = (uint32_t*)(w + p.off_btotal);
  uint32_t* boff = (uint32_t*)(w + p.off_boff);
  uint32_t* toff = (uint32_t*)(w + p.off_toff);
  uint32_t* list = (uint32_t*)(w + p.off_list);
  void* po = (void*)(w + p.off_po);
  float* plse = (float*)(w + p.off_plse);

  Launch l{(hipStream_t)a->stream};
  float* bm_partial = (float*)(w + p.off_bmpart);
  void* own_o = (void*)(w + p.off_own_o);
  float* own_lse = (float*)(w + p.off_own_lse);

  // Small bf16 problems: one launch pools K and writes V^T; then the own-block
  // attention (which needs only Q, K and V^T) runs on the side stream while
  // the gate and the routing run here, and the merge waits for both.
  SideJoin join;
  join.main = l.st;
  if (p.split_own) {
    if (p.need_kbar)
      l.run(K_POOL_TRANSPOSE, [&] {
        return moba::launch_pool_transpose(a->k, a->v, kbar, bm_partial, vt, ktail, d, l.st);
      });
    else
      l.run(K_TRANSPOSE_V,
            [&] { return moba::launch_transpose_v(a->k, a->v, vt, ktail, d, l.st); });
    if (l.err != hipSuccess) return hip_fail(l);
    if (fixed_ws) {
      // no internal stream: the own block runs here, ahead of the gate (the
      // same kernels and partials, so the same output bits)
      l.run(K_ATTN_OWN, [&] {
        return moba::launch_attn_query_bf16(a->q, a->k, vt, ktail, own_o, own_lse, nullptr, 2,
                                            d, l.st);
      });
    } else {
      hipStream_t side = nullptr;
      hipEvent_t fork = nullptr;
      hipError_t e = side_stream(&side);
      // device-scope release: the events only order work on this device
      const unsigned evf = hipEventDisableTiming | hipEventReleaseToDevice;
      if (e == hipSuccess) e = hipEventCreateWithFlags(&fork, evf);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&join.done, evf);
      if (e == hipSuccess) e = hipEventRecord(fork, l.st);
      if (e == hipSuccess) e = hipStreamWaitEvent(side, fork, 0);
      if (fork) (void)hipEventDestroy(fork);
      if (e != hipSuccess) {
        if (join.done) (void)hipEventDestroy(join.done);
        join.done = nullptr;
        return fail(MOBA_ERR_HIP, "side stream setup failed: %s", hipGetErrorString(e));
      }
      Launch ls{side};
      ls.run(K_ATTN_OWN, [&] {
        return moba::launch_attn_query_bf16(a->q, a->k, vt, ktail, own_o, own_lse, nullptr, 2,
                                            d, side);
      });
      const hipError_t ed = hipEventRecord(join.done, side);
      if (ls.err == hipSuccess) ls.err = ed;
      if (ls.err != hipSuccess) return hip_fail(ls);
    }
    if (p.need_kbar)
      l.run(K_MEAN_FINALIZE,
            [&] { return moba::launch_block_mean_finalize(kbar, bm_partial, d, l.st); });
  } else {
    // The V transform finishes the block means when both run (one launch less).
    const bool fold_mean =
        p.need_kbar && p.need_vt && moba::block_mean_partial_floats(d) > 0;
    if (p.need_kbar)
      l.run(K_BLOCK_MEAN, [&] {
        return moba::launch_block_mean(a->k, kbar, bm_partial, d, l.st, fold_mean);
      });
    if (p.need_vt)
      l.run(K_TRANSPOSE_V, [&] {
        return moba::launch_transpose_v(a->k, a->v, vt, ktail, d, l.st,
                                        fold_mean ? bm_partial : nullptr,
                                        fold_mean ? kbar : nullptr);
      });
  }
  if (l.err != hipSuccess) return hip_fail(l);

  // the gate writes the routing histogram itself when it can
  const bool gate_counts = p.routed && moba::gate_writes_counts(d);
  l.run(K_GATE, [&] {
    return moba::launch_gate_topk(a->q, kbar, sel, d, l.st, gate_counts ? counts : nullptr);
  });
  if (p.decode) {
    int32_t* ublk = (int32_t*)(w + p.off_ublk);
    uint32_t* umask = (uint32_t*)(w + p.off_umask);
    int32_t* ucount = (int32_t*)(w + p.off_ucount);
    float* part = (float*)(w + p.off_part);
    l.run(K_DEC_PLAN,
          [&] { return moba::launch_decode_plan(sel, ublk, umask, ucount, false, d, l.st); });
    l.run(K_DEC_ATTN, [&] {
      return moba::launch_decode_attn(a->q, a->k, a->v, ublk, umask, ucount, part, d, l.st);
    });
    l.run(K_DEC_MERGE, [&] {
      return moba::launch_decode_merge(part, ublk, umask, ucount, a->out, d, l.st, a->lse_out);
    });
    if (l.err != hipSuccess) return hip_fail(l);
    return MOBA_OK;
  }
  // One routed pass (the whole problem, or one (sequence, KV head) when
  // grouped): scans of the pass's buckets, its scatter and routed tiles;
  // with `own`, the own block and the merge of the pass's heads follow.
  // (grouped passes scan with route_scan_buckets: the column scans of every
  // bucket run once before the passes)
  const bool small_scan = p.routed && !p.grouped && moba::route_scan_small_fits(d);
  auto routed_pass = [&](const Dims& dp, bool own) {
    if (small_scan) {
      l.run(K_RSCAN_SMALL,
            [&] { return moba::launch_route_scan_small(counts, boff, toff, dp, l.st); });
    } else {
      l.run(K_RSCAN_BUCKETS,
            [&] { return moba::launch_route_scan_buckets(btotal, boff, toff, dp, l.st); });
    }
    l.run(K_RSCATTER, [&] {
      return moba::launch_route_scatter(sel, counts, boff, list, dp, l.st, small_scan);
    });
    l.run(K_ATTN_ROUTED, [&] {
      return dp.bf16 ? moba::launch_attn_routed_bf16(a->q, a->k, vt, list, boff, toff, po, plse,
                                                     dp, l.st)
                     : moba::launch_attn_routed_f32(a->q, a->k, a->v, list, boff, toff, po,
                                                    plse, dp, l.st);
    });
    if (own)
      l.run(K_ATTN_OWN, [&] {
        return dp.bf16 ? moba::launch_attn_query_bf16(a->q, a->k, vt, ktail, po, plse, a->out, 0,
                                                      dp, l.st, 0, a->lse_out)
                       : moba::launch_attn_query_f32(a->q, a->k, a->v, po, plse, a->out, 0, dp,
                                                     l.st, a->lse_out);
      });
  };
  if (p.routed) {
    if (!gate_counts)
      l.run(K_RCOUNT, [&] { return moba::launch_route_count(sel, counts, d, l.st); });
    // per-bucket column scans of every bucket at once (the small scan does
    // them itself, pass by pass)
    if (!small_scan)
      l.run(K_RSCAN_ROWS, [&] { return moba::launch_route_scan_rows(counts, btotal, d, l.st); });
    if (p.grouped) {
      for (int s = 0; s < d.S && l.err == hipSuccess; ++s)
        for (int g = 0; g < d.Hkv && l.err == hipSuccess; g += p.group_kv) {
          Dims dp = d;
          moba::group_pass(dp, s, g, g + p.group_kv <= d.Hkv ? p.group_kv : d.Hkv - g);
          routed_pass(dp, true);
        }
      if (l.err != hipSuccess) return hip_fail(l);
      return MOBA_OK;
    }
    routed_pass(d, false);
  }
  if (p.split_own) {
    if (l.err == hipSuccess && join.done) {
      l.err = hipStreamWaitEvent(l.st, join.done, 0);
      if (l.err == hipSuccess) {
        (void)hipEventDestroy(join.done);
        join.done = nullptr;
      }
    }
    l.run(K_MERGE, [&] {
      return moba::launch_merge_partials_bf16(own_o, own_lse, 2, po, plse, a->out, d, l.st,
                                              a->lse_out);
    });
    if (l.err != hipSuccess) return hip_fail(l);
    return MOBA_OK;
  }
  Dims dq = d;
  if (!p.routed) dq.kp = 0;  // nothing to merge
  l.run(K_ATTN_OWN, [&] {
    return d.bf16 ? moba::launch_attn_query_bf16(a->q, a->k, vt, ktail, po, plse, a->out, 0, dq,
                                                 l.st, 0, a->lse_out)
                  : moba::launch_attn_query_f32(a->q, a->k, a->v, po, plse, a->out, 0, dq,
                                                l.st, a->lse_out);
  });
  if (l.err != hipSuccess) return hip_fail(l);
  return MOBA_OK;
}

moba_status naive_impl(const moba_args* a) {
  Plan p;
  moba_status st = plan_naive(a, &p);
  if (st != MOBA_OK) return st;
  Workspace ws;
  st = get_workspace(a, p, &ws);
  if (st != MOBA_OK) return st;
  const Dims& d = p.d;
  char* w = ws.base;
  float* kbar = p.need_kbar ? (float*)(w + p.off_kbar) : const_cast<float*>(a->k_block_mean);
  float* bm_partial = (float*)(w + p.off_bmpart);
  int32_t* sel = p.need_sel ? (int32_t*)(w + p.off_sel) : a->sel_out;
  void* vt = (void*)(w + p.off_vt);
  void* ktail = p.need_ktail ? (void*)(w + p.off_ktail) : nullptr;
  float* sc = (float*)(w + p.off_sc);
  void* prob = (void*)(w + p.off_p);
  Launch l{(hipStream_t)a->stream};
  if (p.need_kbar)
    l.run(K_BLOCK_MEAN, [&] { return moba::launch_block_mean(a->k, kbar, bm_partial, d, l.st); });
  l.run(K_TRANSPOSE_V, [&] { return moba::launch_transpose_v(a->k, a->v, vt, ktail, d, l.st); });
  l.run(K_GATE, [&] { return moba::launch_gate_topk(a->q, kbar, sel, d, l.st); });
  l.run(K_NAIVE_SCORES, [&] { return moba::launch_naive_scores(a->q, a->k, sc, d, l.st); });
  l.run(K_NAIVE_SOFTMAX, [&] { return moba::launch_naive_softmax(sc, sel, prob, d, l.st); });
  l.run(K_NAIVE_PV, [&] { return moba::launch_naive_pv(prob, vt, a->out, d, l.st); });
  if (l.err != hipSuccess) return hip_fail(l);
  return MOBA_OK;
}

moba_status full_impl(const moba_args* a) {
  Plan p;
  moba_status st = plan_full(a, &p);
  if (st != MOBA_OK) return st;
  Workspace ws;
  st = get_workspace(a, p, &ws);
  if (st != MOBA_OK) return st;
  const Dims& d = p.d;
  void* vt = p.need_vt ? (void*)(ws.base + p.off_vt) : nullptr;
  void* ktail = p.need_ktail ? (void*)(ws.base + p.off_ktail) : nullptr;
  Launch l{(hipStream_t)a->stream};
  if (p.decode) {
    char* w = ws.base;
    int32_t* ublk = (int32_t*)(w + p.off_ublk);
    uint32_t* umask = (uint32_t*)(w + p.off_umask);
    int32_t* ucount = (int32_t*)(w + p.off_ucount);
    float* part = (float*)(w + p.off_part);
    l.run(K_DEC_PLAN,
          [&] { return moba::launch_decode_plan(nullptr, ublk, umask, ucount, true, d, l.st); });
    l.run(K_DEC_ATTN, [&] {
      return moba::launch_decode_attn(a->q, a->k, a->v, ublk, umask, ucount, part, d, l.st);
    });
    l.run(K_DEC_MERGE, [&] {
      return moba::launch_decode_merge(part, ublk, umask, ucount, a->out, d, l.st);
    });
    if (l.err != hipSuccess) return hip_fail(l);
    return MOBA_OK;
  }
  if (p.need_vt)
    l.run(K_TRANSPOSE_V,
          [&] { return moba::launch_transpose_v(a->k, a->v, vt, ktail, d, l.st); });
  if (p.full_parts > 0) {
    void* part_o = (void*)(ws.base + p.off_own_o);
    float* part_lse = (float*)(ws.base + p.off_own_lse);
    l.run(K_ATTN_FULL, [&] {
      return moba::launch_attn_query_bf16(a->q, a->k, vt, ktail, part_o, part_lse, nullptr, 3,
                                          d, l.st, p.full_parts);
    });
    l.run(K_MERGE, [&] {
      return moba::launch_merge_partials_bf16(part_o, part_lse, p.full_parts, nullptr, nullptr,
                                              a->out, d, l.st);
    });
    if (l.err != hipSuccess) return hip_fail(l);
    return MOBA_OK;
  }
  l.run(K_ATTN_FULL, [&] {
    return d.bf16 ? moba::launch_attn_query_bf16(a->q, a->k, vt, ktail, nullptr, nullptr, a->out,
                                                 1, d, l.st)
                  : moba::launch_attn_query_f32(a->q, a->k, a->v, nullptr, nullptr, a->out, 1,
                                                d, l.st);
  });
  if (l.err != hipSuccess) return hip_fail(l);
  return MOBA_OK;
}

// ------------------------------------------------------------------ backward
struct BwdPlan {
  Plan f;                  // dims (forward_dims) and the routing-table offsets
  bool routed = false, need_tail = false;
  size_t off_dvec = 0, off_rowstat = 0, off_ktail = 0, off_vtail = 0, off_dqp = 0, off_ent = 0,
         off_kvpart = 0,
         total = 0;
  bool need_kvpart = false;
};

moba_status plan_backward(const moba_bwd_args* b, BwdPlan* bp) {
  if (!b) return fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (b->struct_size != sizeof(moba_bwd_args))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "struct_size %zu != sizeof(moba_bwd_args) %zu",
                b->struct_size, sizeof(moba_bwd_args));
  if (!b->dout || !b->lse || !b->sel || !b->dq || !b->dk || !b->dv)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "dout, lse, sel, dq, dk and dv must be non-NULL");
  if (((uintptr_t)b->dout | (uintptr_t)b->dq | (uintptr_t)b->dk | (uintptr_t)b->dv) & 15)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (((uintptr_t)b->lse | (uintptr_t)b->sel) & 3)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "lse and sel must be 4-byte aligned");
  moba_args a;
  std::memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(moba_args);
  a.q = b->q; a.k = b->k; a.v = b->v; a.out = const_cast<void*>(b->out);
  a.batch = b->batch; a.n_heads = b->n_heads; a.n_kv_heads = b->n_kv_heads;
  a.head_dim = b->head_dim; a.block_size = b->block_size; a.topk = b->topk;
  a.q_len = b->q_len; a.kv_len = b->kv_len; a.dtype = b->dtype; a.stream = b->stream;
  moba_status st = forward_dims(&a, &bp->f);
  if (st != MOBA_OK) return st;
  Dims& d = bp->f.d;
  // routed dq tiles: eight waves (two per SIMD) in bf16, 128 queries per
  // fp32 workgroup
  d.tile_m = d.bf16 ? 256 : 128;
  if (d.bf16 && d.Lv * d.D >= ((int64_t)1 << 31))
    return fail(MOBA_ERR_UNSUPPORTED, "kv_len * head_dim >= 2^31");
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  Plan& p = bp->f;
  bp->off_dvec = take((size_t)d.S * d.H * d.Lq * 4);
  if (d.bf16) bp->off_rowstat = take((size_t)d.S * d.H * d.Lq * 8);
  // fp32 reads K and V as given (no tail tiles)
  bp->need_tail = d.bf16 && d.L % 64 != 0;
  if (bp->need_tail) {
    bp->off_ktail = take((size_t)d.S * 64 * d.Hkv * d.D * 2);
    bp->off_vtail = take((size_t)d.S * 64 * d.Hkv * d.D * 2);
  }
  bp->routed = d.kp > 0 && d.nb > 1;
  if (bp->routed) {
    p.off_counts = take((size_t)d.nrows * d.ncols * 4);
    p.off_btotal = take((size_t)d.nrows * 4);
    p.off_boff = take((size_t)(d.nrows + 1) * 4);
    p.off_toff = take((size_t)(d.nrows + 1) * 4);
    p.off_list = take((size_t)d.slots * 4);
    bp->off_dqp = take((size_t)d.slots * d.D * (d.bf16 ? 2 : 4));
    // bf16 dk/dv reads every entry's Q / dO row index
    if (d.bf16) bp->off_ent = take((size_t)d.slots * 4);
  }
  const size_t kvp = d.bf16 ? moba::bwd_dkdv_partial_floats(d) : 0;
  bp->need_kvpart = kvp > 0;
  if (bp->need_kvpart) bp->off_kvpart = take(kvp * 4);
  bp->total = off;
  if (b->workspace && b->workspace_bytes < bp->total)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes",
                b->workspace_bytes, bp->total);
  if (b->workspace && ((uintptr_t)b->workspace & 15))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  return MOBA_OK;
}

moba_status backward_impl(const moba_bwd_args* b) {
  BwdPlan bp;
  moba_status st = plan_backward(b, &bp);
  if (st != MOBA_OK) return st;
  const Dims& d = bp.f.d;
  Workspace ws;
  ws.st = (hipStream_t)b->stream;
  if (b->workspace) {
    ws.base = (char*)b->workspace;
  } else if (bp.total) {
    void* ptr = nullptr;
    const hipError_t e = hipMallocAsync(&ptr, bp.total, ws.st);
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(MOBA_ERR_OUT_OF_MEMORY, "hipMallocAsync(%zu bytes) failed: %s", bp.total,
                  hipGetErrorString(e));
    }
    ws.base = (char*)ptr;
    ws.owned = true;
  }
  char* w = ws.base;
  float* dvec = (float*)(w + bp.off_dvec);
  void* rowstat = d.bf16 ? (void*)(w + bp.off_rowstat) : nullptr;
  void* ktail = bp.need_tail ? (void*)(w + bp.off_ktail) : nullptr;
  void* vtail = bp.need_tail ? (void*)(w + bp.off_vtail) : nullptr;
  const Plan& p = bp.f;
  uint32_t* counts = bp.routed ? (uint32_t*)(w + p.off_counts) : nullptr;
  uint32_t* btotal = bp.routed ? (uint32_t*)(w + p.off_btotal) : nullptr;
  uint32_t* boff = bp.routed ? (uint32_t*)(w + p.off_boff) : nullptr;
  uint32_t* toff = bp.routed ? (uint32_t*)(w + p.off_toff) : nullptr;
  uint32_t* list = bp.routed ? (uint32_t*)(w + p.off_list) : nullptr;
  void* dqp = bp.routed ? (void*)(w + bp.off_dqp) : nullptr;

  Launch l{ws.st};
  l.run(K_BWD_DOT, [&] {
    return d.bf16 ? moba::launch_bwd_dot(b->out, b->dout, b->lse, dvec, rowstat, d, l.st)
                  : moba::launch_bwd_dot_f32(b->out, b->dout, dvec, d, l.st);
  });
  if (bp.need_tail)
    l.run(K_BWD_TAIL, [&] { return moba::launch_bwd_tail(b->k, b->v, ktail, vtail, d, l.st); });
  if (bp.routed) {
    l.run(K_RCOUNT, [&] { return moba::launch_route_count(b->sel, counts, d, l.st); });
    const bool small_scan = moba::route_scan_small_fits(d);
    if (small_scan) {
      l.run(K_RSCAN_SMALL,
            [&] { return moba::launch_route_scan_small(counts, boff, toff, d, l.st); });
    } else {
      l.run(K_RSCAN_ROWS, [&] { return moba::launch_route_scan_rows(counts, btotal, d, l.st); });
      l.run(K_RSCAN_BUCKETS,
            [&] { return moba::launch_route_scan_buckets(btotal, boff, toff, d, l.st); });
    }
    l.run(K_RSCATTER, [&] {
      return moba::launch_route_scatter(b->sel, counts, boff, list, d, l.st, small_scan);
    });
    l.run(K_BWD_DQ_ROUTED, [&] {
      return d.bf16 ? moba::launch_bwd_dq_routed(b->q, b->dout, b->k, b->v, b->lse, dvec,
                                                 list, boff, toff, dqp, d, l.st)
                    : moba::launch_bwd_dq_routed_f32(b->q, b->dout, b->k, b->v, b->lse, dvec,
                                                     list, boff, toff, (float*)dqp, d, l.st);
    });
  }
  l.run(K_BWD_DQ_OWN, [&] {
    return d.bf16 ? moba::launch_bwd_dq_own(b->q, b->dout, b->k, b->v, ktail, vtail, b->lse,
                                            dvec, dqp, b->dq, d, l.st)
                  : moba::launch_bwd_dq_own_f32(b->q, b->dout, b->k, b->v, b->lse, dvec,
                                                (const float*)dqp, b->dq, d, l.st);
  });
  void* ent = (bp.routed && d.bf16) ? (void*)(w + bp.off_ent) : nullptr;
  if (ent)
    l.run(K_BWD_ENTRIES,
          [&] { return moba::launch_bwd_entry_rows(list, boff, ent, d, l.st); });
  l.run(K_BWD_DKDV, [&] {
    if (!d.bf16)
      return moba::launch_bwd_dkdv_f32(b->q, b->dout, b->k, b->v, b->lse, dvec, list, boff,
                                       b->dk, b->dv, d, l.st);
    float* kvpart = bp.need_kvpart ? (float*)(w + bp.off_kvpart) : nullptr;
    return moba::launch_bwd_dkdv(b->q, b->dout, b->k, b->v, rowstat, ent, boff, b->dk,
                                 b->dv, kvpart, d, l.st);
  });
  if (l.err != hipSuccess) return hip_fail(l);
  return MOBA_OK;
}

// ------------------------------------------------------------------ varlen
// One batch-1 call per sequence on slices of the packed tensors, sharing one
// workspace sized for the largest sequence (calls are ordered on the stream).
struct VarlenPlan {
  std::vector<moba_args> fwd;        // per sequence with queries (forward)
  std::vector<moba_bwd_args> bwd;    // per sequence with queries (backward)
  std::vector<std::pair<int64_t, int64_t>> zero_kv;  // backward: (first key, keys) to zero
  size_t ws = 0;
};

moba_status plan_varlen(const moba_varlen_args* a, bool backward, VarlenPlan* vp) {
  if (!a) return fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->struct_size != sizeof(moba_varlen_args))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "struct_size %zu != sizeof(moba_varlen_args) %zu",
                a->struct_size, sizeof(moba_varlen_args));
  if (!a->q || !a->k || !a->v || !a->out)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "q, k, v and out must be non-NULL");
  if (backward && (!a->dout || !a->dq || !a->dk || !a->dv || !a->sel || !a->lse))
    return fail(MOBA_ERR_INVALID_ARGUMENT, "dout, dq, dk, dv, sel and lse must be non-NULL");
  if (!a->cu_seqlens_q || !a->cu_seqlens_k)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens_q and cu_seqlens_k must be non-NULL");
  if (a->batch < 1) return fail(MOBA_ERR_INVALID_ARGUMENT, "batch must be >= 1");
  if (a->n_heads < 1 || a->n_kv_heads < 1 || a->head_dim < 1 || a->topk < 1)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (a->dtype != MOBA_DTYPE_F32 && a->dtype != MOBA_DTYPE_BF16)
    return fail(MOBA_ERR_UNSUPPORTED, "unknown dtype %d", (int)a->dtype);
  const int64_t esz = a->dtype == MOBA_DTYPE_BF16 ? 2 : 4;
  const int64_t qrow = (int64_t)a->n_heads * a->head_dim * esz;     // bytes per query row
  const int64_t krow = (int64_t)a->n_kv_heads * a->head_dim * esz;  // bytes per key row
  const int64_t* cq = a->cu_seqlens_q;
  const int64_t* ck = a->cu_seqlens_k;
  if (cq[0] != 0 || ck[0] != 0)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens must start at 0");
  for (int32_t s = 0; s < a->batch; ++s) {
    const int64_t qn = cq[s + 1] - cq[s], kn = ck[s + 1] - ck[s];
    if (qn < 0 || kn < 0)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "cu_seqlens decrease at sequence %d", s);
    if (qn > kn)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "sequence %d: q_len %lld > kv_len %lld", s,
                  (long long)qn, (long long)kn);
    if (qn == 0) {
      if (backward && kn > 0) vp->zero_kv.push_back({ck[s], kn});
      continue;
    }
    const char* q = (const char*)a->q + cq[s] * qrow;
    const char* k = (const char*)a->k + ck[s] * krow;
    const char* v = (const char*)a->v + ck[s] * krow;
    char* out = (char*)a->out + cq[s] * qrow;
    int32_t* sel = a->sel ? a->sel + (int64_t)a->n_heads * cq[s] * a->topk : nullptr;
    float* lse = a->lse ? a->lse + (int64_t)a->n_heads * cq[s] : nullptr;
    moba_status st;
    size_t need = 0;
    if (!backward) {
      moba_args f;
      std::memset(&f, 0, sizeof(f));
      f.struct_size = sizeof(f);
      f.q = q; f.k = k; f.v = v; f.out = out; f.sel_out = sel; f.lse_out = lse;
      f.batch = 1; f.n_heads = a->n_heads; f.n_kv_heads = a->n_kv_heads;
      f.head_dim = a->head_dim; f.block_size = a->block_size; f.topk = a->topk;
      f.q_len = qn; f.kv_len = kn; f.dtype = a->dtype; f.stream = a->stream;
      Plan p;
      st = plan_forward(&f, &p);
      need = p.total;
      vp->fwd.push_back(f);
    } else {
      moba_bwd_args b;
      std::memset(&b, 0, sizeof(b));
      b.struct_size = sizeof(b);
      b.q = q; b.k = k; b.v = v; b.out = out;
      b.dout = (const char*)a->dout + cq[s] * qrow;
      b.lse = lse; b.sel = sel;
      b.dq = (char*)a->dq + cq[s] * qrow;
      b.dk = (char*)a->dk + ck[s] * krow;
      b.dv = (char*)a->dv + ck[s] * krow;
      b.batch = 1; b.n_heads = a->n_heads; b.n_kv_heads = a->n_kv_heads;
      b.head_dim = a->head_dim; b.block_size = a->block_size; b.topk = a->topk;
      b.q_len = qn; b.kv_len = kn; b.dtype = a->dtype; b.stream = a->stream;
      BwdPlan bp;
      st = plan_backward(&b, &bp);
      need = bp.total;
      vp->bwd.push_back(b);
    }
    if (st != MOBA_OK) {
      const std::string why = g_last_error;
      return fail(st, "sequence %d: %s", s, why.c_str());
    }
    if (need > vp->ws) vp->ws = need;
  }
  if (a->workspace && a->workspace_bytes < vp->ws)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes",
                a->workspace_bytes, vp->ws);
  return MOBA_OK;
}

moba_status varlen_impl(const moba_varlen_args* a, bool backward) {
  VarlenPlan vp;
  moba_status st = plan_varlen(a, backward, &vp);
  if (st != MOBA_OK) return st;
  Workspace ws;
  ws.st = (hipStream_t)a->stream;
  if (a->workspace) {
    ws.base = (char*)a->workspace;
  } else if (vp.ws) {
    void* ptr = nullptr;
    const hipError_t e = hipMallocAsync(&ptr, vp.ws, ws.st);
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(MOBA_ERR_OUT_OF_MEMORY, "hipMallocAsync(%zu bytes) failed: %s", vp.ws,
                  hipGetErrorString(e));
    }
    ws.base = (char*)ptr;
    ws.owned = true;
  }
  for (auto& f : vp.fwd) {
    f.workspace = ws.base;
    f.workspace_bytes = vp.ws;
    st = forward_impl(&f);
    if (st != MOBA_OK) return st;
  }
  for (auto& b : vp.bwd) {
    b.workspace = ws.base;
    b.workspace_bytes = vp.ws;
    st = backward_impl(&b);
    if (st != MOBA_OK) return st;
  }
  const int64_t krow = (int64_t)a->n_kv_heads * a->head_dim * (a->dtype == MOBA_DTYPE_BF16 ? 2 : 4);
  for (const auto& z : vp.zero_kv) {
    hipError_t e = hipMemsetAsync((char*)a->dk + z.first * krow, 0, z.second * krow, ws.st);
    if (e == hipSuccess) e = hipMemsetAsync((char*)a->dv + z.first * krow, 0, z.second * krow, ws.st);
    if (e != hipSuccess) return fail(MOBA_ERR_HIP, "hipMemsetAsync failed: %s", hipGetErrorString(e));
  }
  return MOBA_OK;
}

moba_args simple_args(const void* q, const void* k, const void* v, int64_t seq_len,
                      int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t topk, void* out, moba_dtype dtype, void* stream) {
  moba_args a;
  std::memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(moba_args);
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.batch = 1; a.n_heads = n_heads; a.n_kv_heads = n_kv_heads; a.head_dim = head_dim;
  a.block_size = block_size; a.topk = topk; a.q_len = seq_len; a.kv_len = seq_len;
  a.dtype = dtype; a.stream = stream;
  return a;
}

// ------------------------------------------------------------ routing alone

// Dims and workspace layout of moba_route (a moba_args view of its arguments
// through forward_dims, so the limits are the forward's).
moba_status plan_route(int32_t batch, int32_t n_heads, int32_t n_kv_heads, int64_t q_len,
                       int64_t kv_len, int32_t block_size, int32_t topk, Plan* p) {
  moba_args a;
  std::memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(moba_args);
  const uintptr_t fake = (uintptr_t)1 << 40;   // checked, never dereferenced
  a.q = a.k = a.v = (const void*)fake;
  a.out = (void*)fake;
  a.batch = batch; a.n_heads = n_heads; a.n_kv_heads = n_kv_heads; a.head_dim = 128;
  a.block_size = block_size; a.topk = topk; a.q_len = q_len; a.kv_len = kv_len;
  a.dtype = MOBA_DTYPE_BF16;
  moba_status st = forward_dims(&a, p);
  if (st != MOBA_OK) return st;
  const Dims& d = p->d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  p->off_counts = take((size_t)d.nrows * d.ncols * 4);
  p->off_btotal = take((size_t)d.nrows * 4);
  p->off_toff = take((size_t)(d.nrows + 1) * 4);
  p->total = off;
  return MOBA_OK;
}


template <class F>
moba_status guarded(F&& f) {
  g_last_error.clear();
  try {
    return f();
  } catch (const std::exception& e) {
    return fail(MOBA_ERR_HIP, "internal error: %s", e.what());
  } catch (...) {
    return fail(MOBA_ERR_HIP, "internal error");
  }
}

}  // namespace

extern "C" {

moba_status moba_forward(const void* q, const void* k, const void* v, int64_t seq_len,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t topk, void* out, moba_dtype dtype,
                         void* stream) {
  return guarded([&] {
    const moba_args a = simple_args(q, k, v, seq_len, n_heads, n_kv_heads, head_dim, block_size,
                                    topk, out, dtype, stream);
    return forward_impl(&a);
  });
}

moba_status moba_full_attention(const void* q, const void* k, const void* v, int64_t seq_len,
                                int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                void* out, moba_dtype dtype, void* stream) {
  return guarded([&] {
    const moba_args a =
        simple_args(q, k, v, seq_len, n_heads, n_kv_heads, head_dim, 64, 1, out, dtype, stream);
    return full_impl(&a);
  });
}

moba_status moba_forward_ex(const moba_args* a) {
  return guarded([&]() -> moba_status {
    if (!a) return fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
    const moba_args b = load_args(a);
    return forward_impl(&b);
  });
}

moba_status moba_forward_noalloc(const moba_args* a) {
  return guarded([&]() -> moba_status {
    if (!a) return fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
    moba_args b = load_args(a);
    b.workspace = nullptr;    // the scratch array replaces any workspace
    b.workspace_bytes = 0;
    Plan p;
    moba_status st = plan_forward(&b, &p);   // every argument check first
    if (st != MOBA_OK) return st;
    if (p.total > moba::kNoAllocScratchBytes)
      return fail(MOBA_ERR_UNSUPPORTED,
                  "the problem needs %zu bytes of scratch; moba_forward_noalloc holds at most "
                  "%zu (use moba_forward_ex with a workspace)",
                  p.total, moba::kNoAllocScratchBytes);
    void* scratch = nullptr;
    const hipError_t e = moba::noalloc_scratch(&scratch);
    if (e != hipSuccess)
      return fail(MOBA_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
    return forward_impl(&b, scratch, moba::kNoAllocScratchBytes);
  });
}

moba_status moba_full_attention_ex(const moba_args* a) {
  return guarded([&]() -> moba_status {
    if (!a) return fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
    const moba_args b = load_args(a);
    return full_impl(&b);
  });
}

moba_status moba_naive_ex(const moba_args* a) {
  return guarded([&]() -> moba_status {
    if (!a) return fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
    const moba_args b = load_args(a);
    return naive_impl(&b);
  });
}

size_t moba_naive_workspace_size(const moba_args* a) {
  g_last_error.clear();
  try {
    if (!a) {
      fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
      return 0;
    }
    moba_args b = load_args(a);
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    Plan p;
    if (plan_naive(&b, &p) != MOBA_OK) return 0;
    return p.total;
  } catch (...) {
    return 0;
  }
}

size_t moba_workspace_size(const moba_args* a) {
  g_last_error.clear();
  try {
    if (!a) {
      fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
      return 0;
    }
    moba_args b = load_args(a);
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    Plan p;
    if (plan_forward(&b, &p) != MOBA_OK) return 0;
    return p.total;
  } catch (...) {
    return 0;
  }
}

moba_status moba_backward_ex(const moba_bwd_args* a) {
  return guarded([&] { return backward_impl(a); });
}

size_t moba_backward_workspace_size(const moba_bwd_args* a) {
  g_last_error.clear();
  try {
    if (!a) {
      fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
      return 0;
    }
    if (a->struct_size != sizeof(moba_bwd_args)) {
      fail(MOBA_ERR_INVALID_ARGUMENT, "struct_size %zu != sizeof(moba_bwd_args) %zu",
           a->struct_size, sizeof(moba_bwd_args));
      return 0;
    }
    moba_bwd_args b = *a;
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    BwdPlan bp;
    if (plan_backward(&b, &bp) != MOBA_OK) return 0;
    return bp.total;
  } catch (...) {
    return 0;
  }
}

moba_status moba_forward_varlen(const moba_varlen_args* a) {
  return guarded([&] { return varlen_impl(a, false); });
}

moba_status moba_backward_varlen(const moba_varlen_args* a) {
  return guarded([&] { return varlen_impl(a, true); });
}

size_t moba_varlen_workspace_size(const moba_varlen_args* a, int32_t backward) {
  g_last_error.clear();
  try {
    if (!a) {
      fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
      return 0;
    }
    if (a->struct_size != sizeof(moba_varlen_args)) {
      fail(MOBA_ERR_INVALID_ARGUMENT, "struct_size %zu != sizeof(moba_varlen_args) %zu",
           a->struct_size, sizeof(moba_varlen_args));
      return 0;
    }
    moba_varlen_args b = *a;
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    VarlenPlan vp;
    if (plan_varlen(&b, backward != 0, &vp) != MOBA_OK) return 0;
    return vp.ws;
  } catch (...) {
    return 0;
  }
}

size_t moba_full_workspace_size(const moba_args* a) {
  g_last_error.clear();
  try {
    if (!a) {
      fail(MOBA_ERR_INVALID_ARGUMENT, "args is NULL");
      return 0;
    }
    moba_args b = load_args(a);
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    Plan p;
    if (plan_full(&b, &p) != MOBA_OK) return 0;
    return p.total;
  } catch (...) {
    return 0;
  }
}

static moba_status block_mean_impl(const void* k, int32_t batch, int64_t kv_len,
                                   int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t first_block, float* k_block_mean, moba_dtype dtype,
                                   void* stream) {
  return guarded([&]() -> moba_status {
    if (!k || !k_block_mean)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "k and k_block_mean must be non-NULL");
    if (batch < 1 || kv_len < 1 || n_kv_heads < 1 || head_dim < 1 || block_size < 1)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
    if (((uintptr_t)k | (uintptr_t)k_block_mean) & 15)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    if (dtype != MOBA_DTYPE_F32 && dtype != MOBA_DTYPE_BF16)
      return fail(MOBA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (head_dim != 64 && head_dim != 128)
      return fail(MOBA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (block_size % 64 != 0)
      return fail(MOBA_ERR_UNSUPPORTED, "block_size is not a multiple of 64");
    const int64_t nb = (kv_len + block_size - 1) / block_size;  // last block may be partial
    if (nb > moba::kMaxBlocks || batch > 65535)
      return fail(MOBA_ERR_UNSUPPORTED, "too many blocks or sequences");
    if (kv_len >= ((int64_t)1 << 31)) return fail(MOBA_ERR_UNSUPPORTED, "kv_len >= 2^31");
    if (first_block < 0 || first_block >= nb)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "first_block %d outside [0, %lld)", first_block,
                  (long long)nb);
    Dims d;
    d.S = batch; d.L = kv_len; d.Hkv = n_kv_heads; d.D = head_dim; d.B = block_size;
    d.nb = (int)nb; d.bf16 = dtype == MOBA_DTYPE_BF16;
    Launch l{(hipStream_t)stream};
    const size_t pbytes = moba::block_mean_update_partial_floats(d, first_block) * 4;
    void* partial = nullptr;
    if (pbytes) {
      const hipError_t e = hipMallocAsync(&partial, pbytes, l.st);
      if (e != hipSuccess || !partial) {
        (void)hipGetLastError();
        return fail(MOBA_ERR_OUT_OF_MEMORY, "hipMallocAsync(%zu bytes) failed", pbytes);
      }
    }
    l.run(K_BLOCK_MEAN, [&] {
      return moba::launch_block_mean(k, k_block_mean, (float*)partial, d, l.st, false,
                                     first_block);
    });
    if (partial) (void)hipFreeAsync(partial, l.st);
    if (l.err != hipSuccess) return hip_fail(l);
    return MOBA_OK;
  });
}

moba_status moba_block_mean(const void* k, int32_t batch, int64_t kv_len, int32_t n_kv_heads,
                            int32_t head_dim, int32_t block_size, float* k_block_mean,
                            moba_dtype dtype, void* stream) {
  return block_mean_impl(k, batch, kv_len, n_kv_heads, head_dim, block_size, 0, k_block_mean,
                         dtype, stream);
}

moba_status moba_block_mean_update(const void* k, int32_t batch, int64_t kv_len,
                                   int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t first_block, float* k_block_mean, moba_dtype dtype,
                                   void* stream) {
  return block_mean_impl(k, batch, kv_len, n_kv_heads, head_dim, block_size, first_block,
                         k_block_mean, dtype, stream);
}

moba_status moba_route(const int32_t* sel, int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                       int64_t q_len, int64_t kv_len, int32_t block_size, int32_t topk,
                       uint32_t* bucket_off, uint32_t* list, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return guarded([&]() -> moba_status {
    if (!sel || !bucket_off || !list)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "sel, bucket_off and list must be non-NULL");
    if (((uintptr_t)sel | (uintptr_t)bucket_off | (uintptr_t)list) & 3)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "sel, bucket_off and list must be 4-byte aligned");
    if ((uintptr_t)workspace & 15)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    Plan p;
    moba_status st = plan_route(batch, n_heads, n_kv_heads, q_len, kv_len, block_size, topk, &p);
    if (st != MOBA_OK) return st;
    if (workspace && workspace_bytes < p.total)
      return fail(MOBA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu bytes",
                  workspace_bytes, p.total);
    Dims& d = p.d;
    moba_args wa;
    std::memset(&wa, 0, sizeof(wa));
    wa.workspace = workspace;
    wa.stream = stream;
    Workspace ws;
    st = get_workspace(&wa, p, &ws);
    if (st != MOBA_OK) return st;
    Launch l{(hipStream_t)stream};
    char* w = ws.base;   // (topk 1: the counts are all zero, every bucket empty)
    uint32_t* counts = (uint32_t*)(w + p.off_counts);
    uint32_t* btotal = (uint32_t*)(w + p.off_btotal);
    uint32_t* toff = (uint32_t*)(w + p.off_toff);
    l.run(K_RCOUNT, [&] { return moba::launch_route_count(sel, counts, d, l.st); });
    const bool small_scan = moba::route_scan_small_fits(d);
    if (small_scan) {
      l.run(K_RSCAN_SMALL,
            [&] { return moba::launch_route_scan_small(counts, bucket_off, toff, d, l.st); });
    } else {
      l.run(K_RSCAN_ROWS, [&] { return moba::launch_route_scan_rows(counts, btotal, d, l.st); });
      l.run(K_RSCAN_BUCKETS, [&] {
        return moba::launch_route_scan_buckets(btotal, bucket_off, toff, d, l.st);
      });
    }
    l.run(K_RSCATTER, [&] {
      return moba::launch_route_scatter(sel, counts, bucket_off, list, d, l.st, small_scan);
    });
    if (l.err != hipSuccess) return hip_fail(l);
    return MOBA_OK;
  });
}

size_t moba_route_workspace_size(int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                                 int64_t q_len, int64_t kv_len, int32_t block_size,
                                 int32_t topk) {
  size_t n = 0;
  (void)guarded([&]() -> moba_status {
    Plan p;
    const moba_status st =
        plan_route(batch, n_heads, n_kv_heads, q_len, kv_len, block_size, topk, &p);
    if (st == MOBA_OK) n = p.total;
    return st;
  });
  return n;
}

const char* moba_status_string(moba_status s) {
  switch (s) {
    case MOBA_OK: return "MOBA_OK";
    case MOBA_ERR_INVALID_ARGUMENT: return "MOBA_ERR_INVALID_ARGUMENT";
    case MOBA_ERR_UNSUPPORTED: return "MOBA_ERR_UNSUPPORTED";
    case MOBA_ERR_OUT_OF_MEMORY: return "MOBA_ERR_OUT_OF_MEMORY";
    case MOBA_ERR_HIP: return "MOBA_ERR_HIP";
  }
  return "MOBA_STATUS_UNKNOWN";
}

const char* moba_last_error(void) { return g_last_error.c_str(); }

int32_t moba_abi_version(void) { return MOBA_ABI_VERSION; }

moba_status moba_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> g(g_prof.mu);
  g_prof.on = on != 0;
  return MOBA_OK;
}

static void drain_locked() {
  for (const ProfRecord& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      g_prof.total_ms[r.id] += ms;
      g_prof.launches[r.id] += 1;
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.recs.clear();
}

moba_status moba_profile_reset(void) {
  std::lock_guard<std::mutex> g(g_prof.mu);
  drain_locked();
  for (int i = 0; i < K_COUNT; ++i) {
    g_prof.total_ms[i] = 0.0;
    g_prof.launches[i] = 0;
  }
  return MOBA_OK;
}

moba_status moba_profile_read(const char* name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches)
    return fail(MOBA_ERR_INVALID_ARGUMENT, "name, total_ms and launches must be non-NULL");
  int id = -1;
  for (int i = 0; i < K_COUNT; ++i)
    if (std::strcmp(name, kKernelNames[i]) == 0) id = i;
  if (id < 0) return fail(MOBA_ERR_INVALID_ARGUMENT, "unknown kernel name '%s'", name);
  std::lock_guard<std::mutex> g(g_prof.mu);
  drain_locked();
  *total_ms = g_prof.total_ms[id];
  *launches = g_prof.launches[id];
  return MOBA_OK;
}

}  // extern "C"
