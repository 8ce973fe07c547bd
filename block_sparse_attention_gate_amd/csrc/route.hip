// Query -> KV-block dispatch.
//
// The pages liken the gate to an MoE router with the blocks as experts
// ("MoBA" project card, "How It Works"; AiBoss MoBA article,
// "MoBAの主な機能": FlashAttention combined with MoE optimisation).  Here
// every (query, selected PAST block) pair is a routed entry and is regrouped
// into the bucket of (sequence, KV head, block), so that one attention tile
// reads one block's K/V for up to 128 or 256 routed queries.
//
// Entry slot id: ((s*H + h)*Lq + r)*kp + t for the t-th past block of query
// row r of head h (kp = topk - 1).  Buckets are ordered (s, g, j); inside a
// bucket entries are in ascending slot id (stable counting sort):
//   1. route_count: per routing chunk (one head, 128 query rows) an LDS
//      histogram over the blocks, written to counts[bucket][column] (the
//      gate kernel writes it itself when it can);
//   2. route_scan_rows: exclusive scan of each bucket's columns (LDS scan);
//   3. route_scan_buckets: exclusive scan over buckets -> bucket offsets and
//      attention-tile offsets;
//      (small problems: route_scan_small does 2 and 3 in one workgroup with
//      one flat scan over all counts, which leaves global list positions);
//   4. route_scatter: each chunk replays its entries in order; a wave ranks
//      equal buckets among its lanes with ballots and writes the slot ids.
#include "common.h"
#include "kernels.h"

namespace moba {

struct RouteArgs {
  int64_t Lq, q_off, prow0;
  int H, Hkv, G, B, nb, topk, kp, nchunk_r, ncols, nchunks, nbits;
  int ps0, ph0, pH;   // the pass's first sequence and head, heads per sequence
};

// pass = false: every chunk of the problem (route_count); else the chunks of
// the pass's heads (route_scatter).
static RouteArgs route_args(const Dims& d, bool pass) {
  RouteArgs a;
  a.Lq = d.Lq; a.q_off = d.q_off; a.H = d.H; a.Hkv = d.Hkv; a.G = d.G; a.B = d.B;
  a.nb = d.nb; a.topk = d.topk; a.kp = d.kp; a.nchunk_r = d.nchunk_r; a.ncols = d.ncols;
  a.ps0 = pass ? d.ps0 : 0;
  a.ph0 = pass ? d.ph0 : 0;
  a.pH = pass ? d.pH : d.H;
  a.prow0 = pass ? d.prow0 : 0;
  a.nchunks = (pass ? d.pS * d.pH : d.S * d.H) * d.nchunk_r;
  int bits = 0;
  while ((1 << bits) < d.nb) ++bits;
  a.nbits = bits;
  return a;
}

// Chunk ci -> (s, h, c); one wave per chunk, 4 waves per workgroup.
__device__ __forceinline__ void chunk_coords(const RouteArgs& a, int ci, int& s, int& h, int& c) {
  c = ci % a.nchunk_r;
  const int sh = ci / a.nchunk_r;
  h = a.ph0 + sh % a.pH;
  s = a.ps0 + sh / a.pH;
}

__global__ __launch_bounds__(256) void k_route_count(const int32_t* __restrict__ sel,
                                                     uint32_t* __restrict__ counts, RouteArgs a) {
  extern __shared__ uint32_t lds_hist[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ci = blockIdx.x * 4 + w;
  if (ci >= a.nchunks) return;
  uint32_t* hist = lds_hist + w * a.nb;
  for (int j = lane; j < a.nb; j += 64) hist[j] = 0;
  int s, h, c;
  chunk_coords(a, ci, s, h, c);
  const int64_t r0 = (int64_t)c * kRouteChunkRows;
  const int64_t rows = (a.Lq - r0 < kRouteChunkRows) ? a.Lq - r0 : kRouteChunkRows;
  const int total = (int)rows * a.kp;
  const int32_t* selh = sel + ((int64_t)s * a.H + h) * a.Lq * a.topk;
  for (int e = lane; e < total; e += 64) {
    const int64_t r = r0 + e / a.kp;
    const int t = e % a.kp;
    const int own = (int)((a.q_off + r) / a.B);
    if (t < own) {  // t < min(kp, own) since t < kp
      const int j = selh[r * a.topk + t];
      if (j >= 0 && j < own) atomicAdd(&hist[j], 1u);  // same predicate as the scatter
    }
  }
  const int g = h / a.G;
  const int col = (h - g * a.G) * a.nchunk_r + c;
  for (int j = lane; j < a.nb; j += 64) {
    const int64_t row = ((int64_t)s * a.Hkv + g) * a.nb + j;
    counts[row * a.ncols + col] = hist[j];
  }
}

// Workgroup-wide exclusive scan of one value per thread (256 threads).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return before + incl - v;
}

__global__ __launch_bounds__(256) void k_route_scan_rows(uint32_t* __restrict__ counts,
                                                         uint32_t* __restrict__ bucket_total,
                                                         int ncols) {
  __shared__ uint32_t wsum[4];
  uint32_t* p = counts + (int64_t)blockIdx.x * ncols;
  uint32_t carry = 0;
  for (int base = 0; base < ncols; base += 1024) {
    const int i0 = base + threadIdx.x * 4;
    uint32_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (i0 + e < ncols) ? p[i0 + e] : 0u;
    const uint32_t tsum = v[0] + v[1] + v[2] + v[3];
    uint32_t seg;
    const uint32_t ex = block_excl_scan(tsum, wsum, seg);
    uint32_t run = carry + ex;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e < ncols) p[i0 + e] = run;
      run += v[e];
    }
    carry += seg;
  }
  if (threadIdx.x == 0) bucket_total[blockIdx.x] = carry;
}

__global__ __launch_bounds__(256) void k_route_scan_buckets(const uint32_t* __restrict__ total,
                                                            uint32_t* __restrict__ bucket_off,
                                                            uint32_t* __restrict__ tile_off,
                                                            int nrows, int tile_m) {
  __shared__ uint32_t wsum[4];
  uint32_t carry_e = 0, carry_t = 0;
  for (int base = 0; base < nrows; base += 256) {
    const int i = base + threadIdx.x;
    const uint32_t e = i < nrows ? total[i] : 0u;
    const uint32_t t = (e + tile_m - 1) / tile_m;
    uint32_t seg_e, seg_t;
    const uint32_t ex_e = block_excl_scan(e, wsum, seg_e);
    const uint32_t ex_t = block_excl_scan(t, wsum, seg_t);
    if (i < nrows) {
      bucket_off[i] = carry_e + ex_e;
      tile_off[i] = carry_t + ex_t;
    }
    carry_e += seg_e;
    carry_t += seg_t;
  }
  if (threadIdx.x == 0) {
    bucket_off[nrows] = carry_e;
    tile_off[nrows] = carry_t;
  }
}

// counts_global: counts already hold global list positions (route_scan_small).
__global__ __launch_bounds__(256) void k_route_scatter(const int32_t* __restrict__ sel,
                                                       const uint32_t* __restrict__ counts,
                                                       const uint32_t* __restrict__ bucket_off,
                                                       uint32_t* __restrict__ list, RouteArgs a,
                                                       int counts_global) {
  extern __shared__ uint32_t lds_cur[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ci = blockIdx.x * 4 + w;
  if (ci >= a.nchunks) return;
  uint32_t* cur = lds_cur + w * a.nb;
  int s, h, c;
  chunk_coords(a, ci, s, h, c);
  const int g = h / a.G;
  const int col = (h - g * a.G) * a.nchunk_r + c;
  for (int j = lane; j < a.nb; j += 64) {
    const int64_t row = ((int64_t)s * a.Hkv + g) * a.nb + j;
    cur[j] = (counts_global ? 0u : bucket_off[row - a.prow0]) + counts[row * a.ncols + col];
  }
  const int64_t r0 = (int64_t)c * kRouteChunkRows;
  const int64_t rows = (a.Lq - r0 < kRouteChunkRows) ? a.Lq - r0 : kRouteChunkRows;
  const int total = (int)rows * a.kp;
  const int32_t* selh = sel + ((int64_t)s * a.H + h) * a.Lq * a.topk;
  // slot ids of the pass: (((s - ps0) * pH + h - ph0) * Lq + r) * kp + t
  const uint64_t slot_base =
      (((uint64_t)(s - a.ps0) * a.pH + (h - a.ph0)) * a.Lq + r0) * a.kp;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int base = 0; base < total; base += 64) {
    const int e = base + lane;
    bool valid = e < total;
    int j = 0;
    if (valid) {
      const int64_t r = r0 + e / a.kp;
      const int t = e % a.kp;
      const int own = (int)((a.q_off + r) / a.B);
      valid = t < own;
      if (valid) j = selh[r * a.topk + t];
      valid = valid && j >= 0 && j < own;  // same predicate as the count
      if (!valid) j = 0;
    }
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < a.nbits; ++bit) {
      const bool set = (j >> bit) & 1;
      const uint64_t bb = __ballot(valid && set);
      peers &= set ? bb : ~bb;
    }
    const uint32_t rank = (uint32_t)__popcll(peers & lt_mask);
    if (valid) list[cur[j] + rank] = (uint32_t)(slot_base + (uint64_t)e);
    __asm__ volatile("" ::: "memory");
    if (valid && rank == 0) cur[j] += (uint32_t)__popcll(peers);
    __asm__ volatile("" ::: "memory");
  }
}

hipError_t launch_route_count(const int32_t* sel, uint32_t* counts, const Dims& d,
                              hipStream_t st) {
  const RouteArgs a = route_args(d, false);
  const unsigned grid = (unsigned)((a.nchunks + 3) / 4);
  hipLaunchKernelGGL(k_route_count, dim3(grid), dim3(256), 4 * d.nb * sizeof(uint32_t), st, sel,
                     counts, a);
  return hipGetLastError();
}

hipError_t launch_route_scan_rows(uint32_t* counts, uint32_t* bucket_total, const Dims& d,
                                  hipStream_t st) {
  hipLaunchKernelGGL(k_route_scan_rows, dim3(d.nrows), dim3(256), 0, st, counts, bucket_total,
                     d.ncols);
  return hipGetLastError();
}

hipError_t launch_route_scan_buckets(const uint32_t* bucket_total, uint32_t* bucket_off,
                                     uint32_t* tile_off, const Dims& d, hipStream_t st) {
  hipLaunchKernelGGL(k_route_scan_buckets, dim3(1), dim3(256), 0, st, bucket_total + d.prow0,
                     bucket_off, tile_off, d.pnrows, d.tile_m);
  return hipGetLastError();
}

hipError_t launch_route_scatter(const int32_t* sel, const uint32_t* counts,
                                const uint32_t* bucket_off, uint32_t* list, const Dims& d,
                                hipStream_t st, bool counts_global) {
  const RouteArgs a = route_args(d, true);
  const unsigned grid = (unsigned)((a.nchunks + 3) / 4);
  hipLaunchKernelGGL(k_route_scatter, dim3(grid), dim3(256), 4 * d.nb * sizeof(uint32_t), st,
                     sel, counts, bucket_off, list, a, counts_global ? 1 : 0);
  return hipGetLastError();
}

// Small problems: one workgroup turns the whole count matrix [nrows][ncols]
// into global list positions with one flat exclusive scan (row-major order is
// bucket order, then column order), and derives the bucket and tile offsets
// from it.  Thread t scans the contiguous segment [t*seg, (t+1)*seg).
constexpr int kScanSmallThreads = 1024;

__global__ __launch_bounds__(kScanSmallThreads) void k_route_scan_small(
    uint32_t* __restrict__ counts, uint32_t* __restrict__ bucket_off,
    uint32_t* __restrict__ tile_off, int nrows, int ncols, int tile_m) {
  __shared__ uint32_t wsum[kScanSmallThreads / 64];
  __shared__ uint32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = kScanSmallThreads / 64;
  const int total = nrows * ncols;
  // segments of a multiple of 4 counts: 16-byte loads and stores (the count
  // matrix starts 256-byte aligned); the last segment may be ragged
  const int seg = ((total + kScanSmallThreads - 1) / kScanSmallThreads + 3) & ~3;
  const int b0 = tid * seg;
  const int b1 = b0 + seg < total ? b0 + seg : total;
  uint32_t v[kScanSmallMax / kScanSmallThreads];
  const int nv = b1 > b0 ? b1 - b0 : 0;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kScanSmallMax / kScanSmallThreads; i += 4) {
    if (i + 4 <= nv) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(counts + b0 + i);
      v[i] = x[0]; v[i + 1] = x[1]; v[i + 2] = x[2]; v[i + 3] = x[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i + e] = (i + e < nv) ? counts[b0 + i + e] : 0u;
    }
  }
#pragma unroll
  for (int i = 0; i < kScanSmallMax / kScanSmallThreads; ++i) mine += v[i];
  // workgroup exclusive scan of the segment sums
  uint32_t incl = mine;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  uint32_t run = before + incl - mine;
#pragma unroll
  for (int i = 0; i < kScanSmallMax / kScanSmallThreads; ++i) {
    const uint32_t c = v[i];
    v[i] = run;
    run += c;
  }
#pragma unroll
  for (int i = 0; i < kScanSmallMax / kScanSmallThreads; i += 4) {
    if (i + 4 <= nv) {
      *reinterpret_cast<u32x4*>(counts + b0 + i) = u32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < nv) counts[b0 + i + e] = v[i + e];
    }
  }
  uint32_t grand = 0;
  for (int i = 0; i < NW; ++i) grand += wsum[i];
  __syncthreads();  // every position written before rows read them back
  // bucket offsets and per-bucket tile counts; scan of the tile counts
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < nrows; base += kScanSmallThreads) {
    const int row = base + tid;
    uint32_t t = 0;
    if (row < nrows) {
      const uint32_t off = counts[(int64_t)row * ncols];
      const uint32_t end = row + 1 < nrows ? counts[(int64_t)(row + 1) * ncols] : grand;
      bucket_off[row] = off;
      t = (end - off + tile_m - 1) / tile_m;
    }
    uint32_t ti = t;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(ti, o);
      if (lane >= o) ti += y;
    }
    __syncthreads();
    if (lane == 63) wsum[w] = ti;
    __syncthreads();
    uint32_t tb = carry_s;
    for (int i = 0; i < w; ++i) tb += wsum[i];
    if (row < nrows) tile_off[row] = tb + ti - t;
    uint32_t seg_t = 0;
    for (int i = 0; i < NW; ++i) seg_t += wsum[i];
    __syncthreads();
    if (tid == 0) carry_s += seg_t;
    __syncthreads();
  }
  if (tid == 0) {
    bucket_off[nrows] = grand;
    tile_off[nrows] = carry_s;
  }
}

hipError_t launch_route_scan_small(uint32_t* counts, uint32_t* bucket_off, uint32_t* tile_off,
                                   const Dims& d, hipStream_t st) {
  hipLaunchKernelGGL(k_route_scan_small, dim3(1), dim3(kScanSmallThreads), 0, st,
                     counts + d.prow0 * d.ncols, bucket_off, tile_off, d.pnrows, d.ncols,
                     d.tile_m);
  return hipGetLastError();
}

}  // namespace moba
