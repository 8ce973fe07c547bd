// Host-side launch interface of the MoBA kernels (internal to libmoba.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

constexpr int kRouteChunkRows = 128;   // query rows per routing chunk (one head)
constexpr int kMaxBlocks = 8192;       // largest supported number of KV blocks
constexpr int kOwnSplitSteps = 8;      // own-block tiles longer than this (64-key tiles) split in two
constexpr int kFullChunkTiles = 64;    // key chunk (64-key tiles) of split full attention
constexpr int kFullMaxParts = 64;      // at most this many chunks per row
constexpr int kMaxTopk = 17;           // largest supported topk (16 routed blocks + own)
constexpr int kRoutedLdsRows = 4096;   // buckets whose offsets the routed kernel keeps in LDS
constexpr int kScanSmallMax = 16 * 1024;  // count-matrix entries route_scan_small handles
constexpr int kDecChunk = 512;         // keys per decode work item
constexpr int kMergeMaxItems = 8192;   // decode partials the merge lists per head, at most
constexpr int kMaxGridCacheDevices = 64;  // devices whose per-device pointers are kept
// Device scratch of moba_forward_noalloc (a static array per GPU).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;

// Problem dimensions shared by every launch of one call.
struct Dims {
  int S = 1;          // batch (sequences)
  int H = 1;          // query heads
  int Hkv = 1;        // KV heads
  int G = 1;          // H / Hkv
  int D = 128;        // head dim
  int B = 64;         // block size
  int topk = 1;       // blocks per query, own block included
  int kp = 0;         // topk - 1: routed (past) blocks per query at most
  int nb = 1;         // number of KV blocks, ceil(L / B); the last one may be partial
  int64_t Lq = 1;     // queries per sequence
  int64_t L = 1;      // keys per sequence
  int64_t Lv = 64;    // row stride of the transposed V: L rounded up to a multiple of 64
  int64_t q_off = 0;  // position of query row 0 (L - Lq)
  bool bf16 = true;   // element type of q, k, v, out
  // routing
  int nchunk_r = 1;   // routing chunks per (sequence, head)
  int ncols = 1;      // G * nchunk_r: columns of the per-bucket count rows
  int nrows = 1;      // S * Hkv * nb buckets
  int64_t slots = 0;  // S * H * Lq * kp routed slots
  int tile_m = 128;   // routed entries per attention tile (128 or 256)
  // routed pass: a forward may route one (sequence, KV head) at a time to
  // bound the partial outputs it holds.  The pass covers query heads
  // [ph0, ph0 + pH) of sequences [ps0, ps0 + pS) and the buckets
  // [prow0, prow0 + pnrows) (bucket row (s * Hkv + g) * nb + j); its routed
  // slots are numbered (((s - ps0) * pH + h - ph0) * Lq + r) * kp + t, pslots
  // of them.  Without passes: ps0 = 0, pS = S, ph0 = 0, pH = H, prow0 = 0,
  // pnrows = nrows, pslots = slots (see whole_pass).
  int ps0 = 0, pS = 1, ph0 = 0, pH = 1;
  int64_t prow0 = 0;
  int pnrows = 1;
  int64_t pslots = 0;
  // decode batches: per-sequence cache lengths (device int32 [S], nullable);
  // sequence s then attends keys [0, clamp(kv_lens[s], 1, L)) and L is the
  // cache's row count
  const int32_t* kv_lens = nullptr;
};

// Pass fields covering the whole problem.
inline void whole_pass(Dims& d) {
  d.ps0 = 0; d.pS = d.S; d.ph0 = 0; d.pH = d.H;
  d.prow0 = 0; d.pnrows = d.nrows; d.pslots = d.slots;
}
// Pass fields for KV heads [g, g + ng) of sequence s (their ng * G query
// heads).
inline void group_pass(Dims& d, int s, int g, int ng) {
  d.ps0 = s; d.pS = 1; d.ph0 = g * d.G; d.pH = ng * d.G;
  d.prow0 = ((int64_t)s * d.Hkv + g) * d.nb; d.pnrows = ng * d.nb;
  d.pslots = (int64_t)ng * d.G * d.Lq * d.kp;
}

// Device address of this device's scratch array (kNoAllocScratchBytes),
// looked up once per device with hipGetSymbolAddress.
hipError_t noalloc_scratch(void** out);

// Block means; `partial` holds block_mean_partial_floats(d) floats (may be
// NULL when that is 0).
// With defer_finalize the split sums stay in `partial` and the following
// launch_transpose_v (given the same partial / kbar) finishes the means.
// j0 > 0 computes only blocks j0 .. nb-1 (partial then holds
// block_mean_update_partial_floats(d, j0) floats; no defer_finalize).
int block_mean_splits(const Dims& d);
size_t block_mean_partial_floats(const Dims& d);
size_t block_mean_update_partial_floats(const Dims& d, int j0);
hipError_t launch_block_mean(const void* k, float* kbar, float* partial, const Dims& d,
                             hipStream_t st, bool defer_finalize = false, int j0 = 0);
// bf16: block pooling (sums per split, or means when there is one split) and
// the V transform in one launch; launch_block_mean_finalize then finishes the
// means (nothing to do with one split).
// ktail [S, 64, Hkv, D] (needed when L % 64 != 0, else may be NULL): the
// last, partial 64-key tile of K, zero padded, read by the query kernels.
hipError_t launch_pool_transpose(const void* k, const void* v, float* kbar, float* partial,
                                 void* vt, void* ktail, const Dims& d, hipStream_t st);
hipError_t launch_block_mean_finalize(float* kbar, const float* partial, const Dims& d,
                                      hipStream_t st);
hipError_t launch_transpose_v(const void* k, const void* v, void* vt, void* ktail,
                              const Dims& d, hipStream_t st, const float* bm_partial = nullptr,
                              float* kbar = nullptr);
// counts (nullable): when given, the bf16 gate also writes the routing
// histogram of its 128-row chunk (the route_count step), see route.hip.
hipError_t launch_gate_topk(const void* q, const float* kbar, int32_t* sel, const Dims& d,
                            hipStream_t st, uint32_t* counts = nullptr);
// True when launch_gate_topk can produce the routing counts itself (never
// when it runs the decode gate, see gate_uses_decode_kernel).
bool gate_writes_counts(const Dims& d);
bool gate_uses_decode_kernel(const Dims& d);
hipError_t launch_route_count(const int32_t* sel, uint32_t* counts, const Dims& d,
                              hipStream_t st);
hipError_t launch_route_scan_rows(uint32_t* counts, uint32_t* bucket_total, const Dims& d,
                                  hipStream_t st);
hipError_t launch_route_scan_buckets(const uint32_t* bucket_total, uint32_t* bucket_off,
                                     uint32_t* tile_off, const Dims& d, hipStream_t st);
// The scans, the scatter and the routed attention work on the pass's buckets
// (d.prow0 .. + d.pnrows): bucket_total, bucket_off and tile_off are indexed
// from the pass's first bucket, counts globally; list and the partials hold
// the pass's slots only.
// Small problems (nrows * ncols <= 16K): both scans in one workgroup; counts
// then hold list positions within the pass (scatter with counts_global).
bool route_scan_small_fits(const Dims& d);
hipError_t launch_route_scan_small(uint32_t* counts, uint32_t* bucket_off, uint32_t* tile_off,
                                   const Dims& d, hipStream_t st);
hipError_t launch_route_scatter(const int32_t* sel, const uint32_t* counts,
                                const uint32_t* bucket_off, uint32_t* list, const Dims& d,
                                hipStream_t st, bool counts_global);
// Upper bound of the number of routed tiles (grid size of the routed kernel).
int64_t routed_tile_bound(const Dims& d);
hipError_t launch_attn_routed_bf16(const void* q, const void* k, const void* vt,
                                   const uint32_t* list, const uint32_t* bucket_off,
                                   const uint32_t* tile_off, void* part_o, float* part_lse,
                                   const Dims& d, hipStream_t st);
hipError_t launch_attn_routed_f32(const void* q, const void* k, const void* v,
                                  const uint32_t* list, const uint32_t* bucket_off,
                                  const uint32_t* tile_off, void* part_o, float* part_lse,
                                  const Dims& d, hipStream_t st);
// mode 0: own block + merge of the routed partials; mode 1: full causal attention;
// mode 2 (bf16 only): own block written as a partial (o to part_o, log2-sum-exp
// to part_lse, indexed by query-head) for launch_merge_partials_bf16.
// The bf16 form reads V^T [S, Hkv, D, L]; the fp32 form reads V as given.
// mode 3: full causal attention in key chunks of kFullChunkTiles tiles, one
// partial per chunk ([nparts, S*H*Lq, D] and log2-sum-exp [nparts, S*H*Lq]).
// ktail: as written by launch_pool_transpose / launch_transpose_v (needed
// when L % 64 != 0).
// lse_out (nullable, mode 0): natural log-sum-exp [S, H, Lq] of each query's
// scaled logits over all its keys.
hipError_t launch_attn_query_bf16(const void* q, const void* k, const void* vt,
                                  const void* ktail, const void* part_o, const float* part_lse,
                                  void* out, int mode, const Dims& d, hipStream_t st,
                                  int nparts = 0, float* lse_out = nullptr);
// Chunks of split full attention for a bf16 problem too small to fill the
// chip with whole row tiles, else 0.
int full_split_parts(const Dims& d);
// Merge of nown key-range partials per query-head with its kp routed ones.
hipError_t launch_merge_partials_bf16(const void* own_o, const float* own_lse, int nown,
                                      const void* po, const float* plse, void* out,
                                      const Dims& d, hipStream_t st, float* lse_out = nullptr);
hipError_t launch_attn_query_f32(const void* q, const void* k, const void* v, const void* part_o,
                                 const float* part_lse, void* out, int mode, const Dims& d,
                                 hipStream_t st, float* lse_out = nullptr);

// Decode (q_len == 1): union of kept blocks per (sequence, KV head), split-K
// attention over 512-key chunks, log-sum-exp merge.
bool decode_supported(const Dims& d);   // q_len 1, G <= 8, block_size % 512 == 0
int decode_chunk();
int decode_umax(const Dims& d);
int decode_gm(const Dims& d);           // query heads per decode work item (1, 2, 4 or 8)
size_t decode_part_floats(const Dims& d);
hipError_t launch_decode_plan(const int32_t* sel, int32_t* ublk, uint32_t* umask,
                              int32_t* ucount, bool all_blocks, const Dims& d, hipStream_t st);
hipError_t launch_decode_attn(const void* q, const void* k, const void* v, const int32_t* ublk,
                              const uint32_t* umask, const int32_t* ucount, float* part,
                              const Dims& d, hipStream_t st);
hipError_t launch_decode_merge(const float* part, const int32_t* ublk, const uint32_t* umask,
                               const int32_t* ucount, void* out, const Dims& d, hipStream_t st,
                               float* lse_out = nullptr);

// Backward (bf16), see attn_bwd.hip.  dvec [S*H*Lq] fp32 in query-head order;
// ktail / vtail [S, 64, Hkv, D] when L % 64 != 0 (launch_bwd_tail does nothing
// otherwise); dqp one bf16 row per routed slot; lse is the forward's natural
// log-sum-exp.
hipError_t launch_bwd_dot(const void* out, const void* dout, const float* lse, float* dvec,
                          void* rowstat, const Dims& d, hipStream_t st);
hipError_t launch_bwd_tail(const void* k, const void* v, void* ktail, void* vtail, const Dims& d,
                          hipStream_t st);
hipError_t launch_bwd_dq_routed(const void* q, const void* dout, const void* k, const void* v,
                                const float* lse, const float* dvec,
                                const uint32_t* list, const uint32_t* bucket_off,
                                const uint32_t* tile_off, void* dqp, const Dims& d,
                                hipStream_t st);
hipError_t launch_bwd_dq_own(const void* q, const void* dout, const void* k, const void* v,
                             const void* ktail, const void* vtail,
                             const float* lse, const float* dvec, const void* dqp, void* dq,
                             const Dims& d, hipStream_t st);
// list / bucket_off NULL: no routed entries (top-k 1 or a single block).
// kvpart: bwd_dkdv_partial_floats(d) floats (small problems split every
// bucket into segments whose fp32 partials are added afterwards; else NULL).
int bwd_dkdv_waves(const Dims& d);
int bwd_dkdv_segments(const Dims& d);
size_t bwd_dkdv_partial_floats(const Dims& d);
// rowstat (bf16 dk/dv): float2 (lse log2(e), Dv) per query-head row in
// memory order [S, Lq, H], written by launch_bwd_dot when non-null.  ent: the
// row index (s*Lq + r)*H + h of every routed entry (uint32, routing order),
// written by launch_bwd_entry_rows from the routing list.
hipError_t launch_bwd_entry_rows(const uint32_t* list, const uint32_t* bucket_off, void* ent,
                                const Dims& d, hipStream_t st);
hipError_t launch_bwd_dkdv(const void* q, const void* dout, const void* k, const void* v,
                           const void* rowstat, const void* ent,
                           const uint32_t* bucket_off, void* dk, void* dv, float* kvpart,
                           const Dims& d, hipStream_t st);

// fp32 backward (see attn_bwd_f32.hip): no K^T; dqp one fp32 row per routed
// slot; list / bucket_off NULL when there are no routed entries.
hipError_t launch_bwd_dot_f32(const void* out, const void* dout, float* dvec, const Dims& d,
                              hipStream_t st);
hipError_t launch_bwd_dq_routed_f32(const void* q, const void* dout, const void* k,
                                    const void* v, const float* lse, const float* dvec,
                                    const uint32_t* list, const uint32_t* bucket_off,
                                    const uint32_t* tile_off, float* dqp, const Dims& d,
                                    hipStream_t st);
hipError_t launch_bwd_dq_own_f32(const void* q, const void* dout, const void* k, const void* v,
                                 const float* lse, const float* dvec, const float* dqp,
                                 void* dq, const Dims& d, hipStream_t st);
hipError_t launch_bwd_dkdv_f32(const void* q, const void* dout, const void* k, const void* v,
                               const float* lse, const float* dvec, const uint32_t* list,
                               const uint32_t* bucket_off, void* dk, void* dv, const Dims& d,
                               hipStream_t st);

// Mask-based form (see naive.hip): dense fp32 scores sc and bf16
// probabilities p, both [S, H, Lq, Lv]; vt as for the bf16 query kernels.
hipError_t launch_naive_scores(const void* q, const void* k, float* sc, const Dims& d,
                               hipStream_t st);
hipError_t launch_naive_softmax(const float* sc, const int32_t* sel, void* p, const Dims& d,
                                hipStream_t st);
hipError_t launch_naive_pv(const void* p, const void* vt, void* out, const Dims& d,
                           hipStream_t st);

}  // namespace moba
