/*
 * moba.h -- C ABI of the MI355X (gfx950) MoBA forward library (libmoba.so).
 *
 * MoBA (Mixture of Block Attention) splits the keys and values into blocks of
 * a fixed size, scores every query against every block with a parameter-less
 * gate, keeps the top-k blocks per query token and runs softmax attention over
 * the kept blocks only ("MoBA" project card, sourcepulse, "How It Works" and
 * "Highlighted Details": the two knobs "MoBA Block" and "MoBA Topk").  A query
 * never reads a future block and its own block is causally masked ("MoBA -
 * Moonshot AIが提案した新しいアテンションメカニズム", aiboss88, section
 * "MoBAの技術的原則", causality design).  The gate's affinity and the other
 * points the pages leave open are fixed as follows:
 *
 *   - score(query q, block j) = q . mean of the block's keys (unscaled);
 *   - the query's own block always counts as one of the k selected blocks;
 *     the other k-1 are its best past blocks, ties to the lower index;
 *   - the output is one softmax over the union of the selected keys, scale
 *     1/sqrt(head_dim), causal diagonal inclusive;
 *   - GQA: query head h reads KV head h / (n_heads / n_kv_heads); each query
 *     head gates on its own;
 *   - query row r of a sequence sits at position kv_len - q_len + r.
 *   - topk >= number of blocks is full causal attention.
 *   - kv_len need not be a multiple of block_size: there are
 *     nb = ceil(kv_len / block_size) blocks and the last one, when partial,
 *     holds (and is averaged over) the keys that exist.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, contiguous, 16-byte aligned.
 *     Layouts are row-major with head_dim innermost:
 *       q, out   [batch, q_len, n_heads, head_dim]
 *       k, v     [batch, kv_len, n_kv_heads, head_dim]
 *     (batch 1 with q_len == kv_len == seq_len for the plain calls.)
 *   - Element type is given by `dtype`; out has the input type (bf16 output
 *     is rounded to nearest even from fp32).  Accumulation is fp32.
 *   - The caller owns every buffer.  Inputs are read only; `out` (and
 *     `sel_out` when given) are fully overwritten.  The library keeps no
 *     pointer after the queued work completes.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns; there is no host synchronisation inside.
 *     Part of the work may run on an internal stream of the same device that
 *     is forked from and joined back into `stream` with events, so ordering
 *     with respect to `stream` is as if all of it ran on `stream`.
 *   - All argument checks run before anything is enqueued: a call that
 *     returns an error has enqueued nothing and written nothing.
 *     MOBA_ERR_INVALID_ARGUMENT: null required pointer, size < 1,
 *       n_heads % n_kv_heads != 0, q_len > kv_len, size overflow, workspace
 *       too small.
 *     MOBA_ERR_UNSUPPORTED: head_dim not 64 or 128, block_size not a multiple
 *       of 64, topk > 17, more than 8192 blocks, more than 2^32 routed slots,
 *       batch * n_heads > 65535, kv_len >= 2^31, kv_len * head_dim >= 2^31
 *       for bf16 with q_len > 1 (kv_len rounded up to 64), or 2^31 or more
 *       routing chunks (128 query rows of one head each).
 *     MOBA_ERR_OUT_OF_MEMORY: the internal workspace could not be allocated.
 *     MOBA_ERR_HIP: a HIP launch or runtime call failed.  Faults inside the
 *       kernels surface at the caller's next synchronisation.
 *   - moba_last_error() returns a thread-local text for the last failure.
 *   - Concurrent calls on different streams are safe (the internal stream
 *     is one per device, so the parts of concurrent calls that run on it
 *     queue behind each other); the profiling switch below is process-wide
 *     and not meant for concurrent use.
 */
#ifndef MOBA_H_
#define MOBA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: moba_args gained lse_out (a version-1 struct, without it, is still
 * accepted); moba_backward_ex, moba_block_mean_update and the packed
 * variable-length calls were added.
 * 3: moba_args gained kv_lens (per-sequence cache lengths for decode; the
 * version-1 and version-2 structs are still accepted); moba_naive_ex.
 * 4: moba_args gained routed_bytes_limit (earlier structs still accepted). */
#define MOBA_ABI_VERSION 4

typedef enum { MOBA_DTYPE_F32 = 0, MOBA_DTYPE_BF16 = 1 } moba_dtype;

typedef enum {
  MOBA_OK = 0,
  MOBA_ERR_INVALID_ARGUMENT = 1,
  MOBA_ERR_UNSUPPORTED = 2,
  MOBA_ERR_OUT_OF_MEMORY = 3,
  MOBA_ERR_HIP = 4
} moba_status;

/*
 * MoBA prefill forward for one sequence (batch 1, q_len == kv_len == seq_len):
 * out[i, h, :] = softmax over the selected keys of query i, head h.
 * Allocates its workspace stream-ordered (hipMallocAsync / hipFreeAsync).
 */
moba_status moba_forward(const void* q, const void* k, const void* v, int64_t seq_len,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t topk, void* out, moba_dtype dtype,
                         void* stream);

/*
 * Full causal attention (every key t <= position), the topk = all comparator
 * of the sparse/full switch.  Workspace (allocated stream-ordered): a
 * transposed copy of V for bf16 (plus the last K tile when kv_len is not a
 * multiple of 64); for bf16 problems too small to fill the GPU with whole
 * query rows, also one partial output per 4096-key chunk of every row
 * (merged at the end); with q_len 1, split-K partials over 512-key chunks.
 */
moba_status moba_full_attention(const void* q, const void* k, const void* v, int64_t seq_len,
                                int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                void* out, moba_dtype dtype, void* stream);

/* General form: batches, q_len <= kv_len (decode q_len = 1), precomputed block
 * means, the selection as an output, and a caller workspace. */
typedef struct moba_args {
  size_t struct_size;          /* = sizeof(moba_args) */
  const void* q;               /* [batch, q_len, n_heads, head_dim] */
  const void* k;               /* [batch, kv_len, n_kv_heads, head_dim] */
  const void* v;               /* [batch, kv_len, n_kv_heads, head_dim] */
  void* out;                   /* [batch, q_len, n_heads, head_dim] */
  const float* k_block_mean;   /* nullable: fp32 [batch, n_kv_heads, nb, head_dim]
                                  from moba_block_mean; computed when NULL */
  int32_t* sel_out;            /* nullable: int32 [batch, n_heads, q_len, topk];
                                  selected blocks ascending, -1 padded */
  int32_t batch;
  int32_t n_heads, n_kv_heads, head_dim, block_size, topk;
  int64_t q_len, kv_len;
  moba_dtype dtype;
  void* workspace;             /* nullable: device scratch of at least
                                  moba_workspace_size(args) bytes; when NULL the
                                  library allocates it stream-ordered */
  size_t workspace_bytes;
  void* stream;                /* hipStream_t, NULL = default stream */
  float* lse_out;              /* nullable: fp32 [batch, n_heads, q_len], the
                                  natural log of each query's softmax
                                  normaliser over its selected keys (scaled
                                  logits), kept for moba_backward_ex; ignored
                                  by the full-attention calls */
  const int32_t* kv_lens;      /* nullable: int32 [batch] on the device, the
                                  cache length of each sequence for a decode
                                  batch (q_len 1): sequence s attends keys
                                  [0, kv_lens[s]) of its cache rows and its
                                  query sits at position kv_lens[s] - 1;
                                  kv_len is then the cache's row count (the
                                  row stride of k and v), values are clamped
                                  to [1, kv_len].  Block means passed in may
                                  be those of the padded cache
                                  (moba_block_mean over kv_len rows): the gate
                                  reads only complete past blocks.  Supported
                                  where q_len 1 takes the decode kernels
                                  (block_size a multiple of 512, at most 8
                                  query heads per KV head), for
                                  moba_forward_ex and moba_full_attention_ex;
                                  else UNSUPPORTED */
  size_t routed_bytes_limit;   /* bytes of routed partial outputs (bf16 rows
                                  of head_dim values plus an fp32 log-sum-exp
                                  and a list entry each, one per (query,
                                  selected past block) pair) the bf16 forward
                                  may hold at once; 0 = 12 GiB.  Above it,
                                  problems with more than 2^20 query rows x
                                  heads and more than one (sequence, KV head)
                                  route in passes of as many KV heads of one
                                  sequence as fit the limit (at least one):
                                  the workspace then holds one pass, and the
                                  output is bitwise the same.  Ignored by the
                                  other calls */
} moba_args;
/* struct_size may also be that of the version-1 struct (up to and including
 * `stream`; lse_out and kv_lens are then NULL), of the version-2 struct (up
 * to and including `lse_out`; kv_lens is then NULL) or of the version-3 struct
 * (up to and including `kv_lens`; routed_bytes_limit is then 0). */

moba_status moba_forward_ex(const moba_args* a);

/*
 * moba_forward_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and the same output bits, with no allocation and no
 * internal stream or event.  Its workspace is a static device array of 64
 * MiB per GPU (kept until the process ends) instead of a.workspace (which is
 * ignored, as is workspace_bytes); a problem whose workspace
 * (moba_workspace_size) is larger is refused with MOBA_ERR_UNSUPPORTED
 * before anything is enqueued (a 32K-token single-head prefill needs about
 * 43 MB; a decode step with block means passed in, a few MB).  Every call on
 * one GPU shares that GPU's array, and nothing in it needs to start at zero:
 * calls that overlap on one GPU (concurrent streams, or threads) race and
 * must be serialised by the caller.
 */
moba_status moba_forward_noalloc(const moba_args* a);

/* Full attention in the general form; block_size, topk, k_block_mean and
 * sel_out are ignored. */
moba_status moba_full_attention_ex(const moba_args* a);

/*
 * Backward of moba_forward_ex for continued training (the pages require it:
 * "MoBA" project card, "Highlighted Details"; they give no backward pass).
 * Gradients of sum(out * dout) with respect to q, k and v with the forward's
 * selection held fixed: top-k is piecewise constant and passes no gradient,
 * so the gate and the block means get none.  For a query with key set T,
 * p = softmax(c K_T q), c = 1/sqrt(head_dim):
 *   dv_t += p_t dO,  ds_t = p_t (dO.v_t - dO.o),  dq = c sum_t ds_t k_t,
 *   dk_t += c ds_t q   (GQA: a KV head sums over its group's query heads).
 * bf16 (MFMA) or fp32 (VALU); the other limits are the forward's, and for
 * bf16 kv_len * head_dim (kv_len rounded up to 64) must stay below 2^31.
 * sel and lse are what moba_forward_ex wrote to sel_out and lse_out for the
 * same q, k, v.  dq, dk, dv are fully overwritten (keys no query attends get
 * zero gradients).  Workspace (stream-ordered when NULL): dO.o per
 * query-head, the routing tables rebuilt from sel, one dq partial per routed
 * slot (in the input dtype) and, for bf16, K^T.
 */
typedef struct moba_bwd_args {
  size_t struct_size;          /* = sizeof(moba_bwd_args) */
  const void* q;               /* [batch, q_len, n_heads, head_dim] */
  const void* k;               /* [batch, kv_len, n_kv_heads, head_dim] */
  const void* v;               /* [batch, kv_len, n_kv_heads, head_dim] */
  const void* out;             /* forward output, layout of q */
  const void* dout;            /* upstream gradient, layout of q */
  const float* lse;            /* [batch, n_heads, q_len] (lse_out of the forward) */
  const int32_t* sel;          /* [batch, n_heads, q_len, topk] (sel_out of the forward) */
  void* dq;                    /* layout of q */
  void* dk;                    /* layout of k */
  void* dv;                    /* layout of v */
  int32_t batch;
  int32_t n_heads, n_kv_heads, head_dim, block_size, topk;
  int64_t q_len, kv_len;
  moba_dtype dtype;
  void* workspace;             /* nullable, >= moba_backward_workspace_size bytes */
  size_t workspace_bytes;
  void* stream;                /* hipStream_t, NULL = default stream */
} moba_bwd_args;

moba_status moba_backward_ex(const moba_bwd_args* a);
size_t moba_backward_workspace_size(const moba_bwd_args* a);

/*
 * Packed variable-length batches: `batch` sequences laid one after the other
 * along the token axis, q and out [total_q, n_heads, head_dim], k and v
 * [total_k, n_kv_heads, head_dim]; sequence s owns query rows
 * cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and keys cu_seqlens_k[s] ..
 * cu_seqlens_k[s+1]-1 (HOST arrays of batch + 1 int64 entries starting at 0,
 * non-decreasing; a sequence's query count may not exceed its key count, and
 * its queries sit at the end of its keys, as in moba_forward_ex).  Lengths
 * may be anything, including zero (the sequence is skipped).  Each sequence
 * is computed as its own moba_forward_ex / moba_backward_ex call on the
 * caller's stream (no interaction between sequences); one workspace sized for
 * the largest sequence serves all of them.  sel_out / lse_out (and sel / lse
 * of the backward) hold per sequence a [n_heads, q_len_s, topk] /
 * [n_heads, q_len_s] block, the blocks one after the other in sequence order
 * (sequence s's block starts at element n_heads * cu_seqlens_q[s] * topk of
 * sel and n_heads * cu_seqlens_q[s] of lse).  Every sequence is checked
 * before anything is enqueued; a HIP failure part-way returns MOBA_ERR_HIP
 * with the earlier sequences' work already enqueued.  The backward writes
 * zero dk, dv for the keys of a sequence that has no queries.
 */
typedef struct moba_varlen_args {
  size_t struct_size;          /* = sizeof(moba_varlen_args) */
  const void* q;               /* [total_q, n_heads, head_dim] */
  const void* k;               /* [total_k, n_kv_heads, head_dim] */
  const void* v;
  void* out;                   /* forward: written; backward: the forward output (read) */
  const void* dout;            /* backward only: upstream gradient, layout of q */
  void* dq;                    /* backward only: layout of q */
  void* dk;                    /* backward only: layout of k */
  void* dv;                    /* backward only: layout of v */
  const int64_t* cu_seqlens_q; /* host, batch + 1 */
  const int64_t* cu_seqlens_k; /* host, batch + 1 */
  int32_t* sel;                /* forward: nullable output; backward: input (required) */
  float* lse;                  /* forward: nullable output; backward: input (required) */
  int32_t batch;
  int32_t n_heads, n_kv_heads, head_dim, block_size, topk;
  moba_dtype dtype;
  void* workspace;             /* nullable, >= moba_varlen_workspace_size bytes */
  size_t workspace_bytes;
  void* stream;                /* hipStream_t, NULL = default stream */
} moba_varlen_args;

moba_status moba_forward_varlen(const moba_varlen_args* a);
moba_status moba_backward_varlen(const moba_varlen_args* a);
/* backward = 0: workspace of moba_forward_varlen; 1: of moba_backward_varlen. */
size_t moba_varlen_workspace_size(const moba_varlen_args* a, int32_t backward);

/*
 * Mask-based MoBA, the "naive" form the pages set beside the efficient one
 * ("MoBA" project card, "Highlighted Details" and "Limitations & Caveats":
 * for understanding and visualising the masks; the baseline of the quoted
 * efficient-vs-naive speedup at 32K tokens, 1 head, block 2048, top-k 3).
 * Same arguments, gate and selection as moba_forward_ex, then ordinary
 * attention over the dense score matrix: s = c q.k for EVERY (query, key)
 * pair (c = 1/sqrt(head_dim)), keys outside the query's selected blocks or
 * after the query masked out, row softmax, P V.  The output equals
 * moba_forward_ex's up to rounding.  bf16 only (fp32 is UNSUPPORTED);
 * lse_out is ignored.  A comparison baseline, deliberately dense: the
 * workspace holds fp32 scores and bf16 probabilities for every pair,
 * 6 * batch * n_heads * q_len * kv_len bytes (kv_len rounded up to 64) on top
 * of the block means, the selection, V^T and the K tail tile;
 * batch * n_heads * q_len must stay below 2^31.  Workspace bytes from
 * moba_naive_workspace_size (0 for an invalid argument set).
 */
moba_status moba_naive_ex(const moba_args* a);
size_t moba_naive_workspace_size(const moba_args* a);

/* Workspace bytes moba_forward_ex / moba_full_attention_ex need for `a`
 * (0 for an invalid argument set; read moba_last_error()). */
size_t moba_workspace_size(const moba_args* a);
size_t moba_full_workspace_size(const moba_args* a);

/* Block-mean keys: k_block_mean[s, g, j, :] = mean of k[s, t, g, :] over the
 * keys of block j, j < ceil(kv_len / block_size) (a partial last block: over
 * the keys it holds; fp32 accumulation).  The decode path reuses it across
 * calls on the same cache. */
moba_status moba_block_mean(const void* k, int32_t batch, int64_t kv_len, int32_t n_kv_heads,
                            int32_t head_dim, int32_t block_size, float* k_block_mean,
                            moba_dtype dtype, void* stream);

/* Incremental form for a cache that grows (decode): recomputes the means of
 * blocks first_block .. ceil(kv_len / block_size) - 1 only, with the same
 * arithmetic (the same bits) as moba_block_mean, and leaves blocks before
 * first_block untouched.  The gate only scores complete past blocks, so after
 * appending tokens it suffices to pass the first block that was incomplete
 * before the append.  first_block outside [0, nb) is INVALID_ARGUMENT. */
moba_status moba_block_mean_update(const void* k, int32_t batch, int64_t kv_len,
                                   int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t first_block, float* k_block_mean, moba_dtype dtype,
                                   void* stream);

/*
 * The query -> KV-block dispatch of the forward on its own (the pages liken
 * the gate to an MoE router with the blocks as experts: "MoBA" project card,
 * "How It Works"; AiBoss MoBA article, "MoBAの主な機能"): from a selection
 * `sel` [batch, n_heads, q_len, topk] (sel_out of moba_forward_ex, device),
 * every routed entry -- query row r of head h in sequence s with its t-th
 * kept PAST block (t < topk - 1; the own block is not routed) -- is listed
 * in the bucket of (s, h / (n_heads / n_kv_heads), block), buckets in that
 * order:
 *   bucket_off [batch * n_kv_heads * nb + 1] (uint32, device): entry
 *     offsets, bucket_off[0] = 0 and the last one the number of entries;
 *   list [batch * n_heads * q_len * (topk - 1)] (uint32, device; only the
 *     first bucket_off[last] are written): slot ids
 *     ((s * n_heads + h) * q_len + r) * (topk - 1) + t, ascending inside
 *     each bucket (a stable counting sort: the same bits on every run).
 * nb = ceil(kv_len / block_size); query row r sits at position
 * kv_len - q_len + r; the limits and checks are moba_forward_ex's.  Entries
 * whose block is not a kept past block (-1 padding) are skipped.
 * Workspace: moba_route_workspace_size bytes (stream-ordered when NULL).
 */
moba_status moba_route(const int32_t* sel, int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                       int64_t q_len, int64_t kv_len, int32_t block_size, int32_t topk,
                       uint32_t* bucket_off, uint32_t* list, void* workspace,
                       size_t workspace_bytes, void* stream);
size_t moba_route_workspace_size(int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                                 int64_t q_len, int64_t kv_len, int32_t block_size,
                                 int32_t topk);

const char* moba_status_string(moba_status s);
const char* moba_last_error(void);
int32_t moba_abi_version(void);

/*
 * Per-kernel timing for measurement.  While enabled, every kernel the library
 * launches is bracketed by HIP events on the launch stream.  moba_profile_read
 * waits for the recorded events and returns, for the kernel named `name`, the
 * summed duration in milliseconds and the number of launches since the last
 * reset.  Names: "block_mean", "transpose_v", "gate_topk", "route_count",
 * "route_scan_rows", "route_scan_buckets", "route_scatter", "attn_routed",
 * "attn_own_merge", "attn_full", "decode_plan", "decode_attn",
 * "decode_merge", "merge_partials", "pool_transpose", "block_mean_finalize",
 * "route_scan_small", and for the backward "bwd_dot", "bwd_tail",
 * "bwd_dq_routed", "bwd_dq_own", "bwd_dkdv", "bwd_entries", and for moba_naive_ex
 * "naive_scores", "naive_softmax", "naive_pv".  Unknown names give
 * MOBA_ERR_INVALID_ARGUMENT.  (bf16 prefill runs the own-block attention,
 * "attn_own_merge", on an internal stream of the same device, forked from
 * and joined back into the caller's stream.)
 */
moba_status moba_profile_enable(int32_t on);
moba_status moba_profile_reset(void);
moba_status moba_profile_read(const char* name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H_ */
