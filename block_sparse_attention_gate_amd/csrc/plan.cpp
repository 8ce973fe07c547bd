// Host-side planning rules of the kernels: which kernel variant a problem
// takes and how large its scratch buffers are.  Plain C++ (no device code),
// shared by the launchers in the .hip sources and by the C ABI, so that a
// host-only build of the ABI layer (the sanitizer build of the tests) runs
// the same rules as the library.
#include "kernels.h"

namespace moba {

static int gcd_int(int a, int b) {
  while (b) { const int t = a % b; a = b; b = t; }
  return a;
}

// ---------------------------------------------------------------- pooling
int block_mean_splits(const Dims& d) {
  // enough workgroups to cover the chip (>= 1024), at least 64 rows each
  int splits = 1;
  const int64_t wgs = (int64_t)d.nb * d.S;
  while (wgs * splits < 1024 && d.B % (splits * 2) == 0 && d.B / (splits * 2) >= 64) splits *= 2;
  return splits;
}

size_t block_mean_partial_floats(const Dims& d) {
  const int sp = block_mean_splits(d);
  return sp > 1 ? (size_t)d.S * d.nb * sp * d.Hkv * d.D : 0;
}

// The split count is that of the whole problem also when only blocks j0..
// are computed, so that every block's sum is formed in the same order (the
// same bits) as by the full computation.
size_t block_mean_update_partial_floats(const Dims& d, int j0) {
  const int sp = block_mean_splits(d);
  return sp > 1 ? (size_t)d.S * (d.nb - j0) * sp * d.Hkv * d.D : 0;
}

// ------------------------------------------------------------------- gate
// bf16 with one query row per (sequence, head): the decode gate (one
// workgroup per query-head), whatever the group size.  It writes no routing
// histogram, so the route_count step must run after it when the call routes.
bool gate_uses_decode_kernel(const Dims& d) { return d.bf16 && d.Lq == 1; }

// The routing histogram comes from the same predicate as the gate's
// dispatch: only the 128-row bf16 gate writes it.
bool gate_writes_counts(const Dims& d) {
  return d.bf16 && !gate_uses_decode_kernel(d) && kRouteChunkRows == 128;
}

// ---------------------------------------------------------------- routing
bool route_scan_small_fits(const Dims& d) {
  return (int64_t)d.pnrows * d.ncols <= kScanSmallMax;
}

int64_t routed_tile_bound(const Dims& d) {
  return (d.pslots + d.tile_m - 1) / d.tile_m + d.pnrows;
}

// ------------------------------------------------------- full attention
int full_split_parts(const Dims& d) {
  if (!d.bf16) return 0;
  const int HW = gcd_int(d.G, 4);
  const int RW = 256 / HW;  // eight-wave workgroups
  const int64_t wgs = (d.Lq + RW - 1) / RW * (int64_t)(d.S * d.H / HW);
  if (wgs >= 1024) return 0;  // whole row tiles already fill the chip
  const int64_t tiles = (d.q_off + d.Lq + 63) / 64;  // key tiles of the longest row
  const int64_t p = (tiles + kFullChunkTiles - 1) / kFullChunkTiles;
  return p > 1 && p <= kFullMaxParts ? (int)p : 0;
}

// ----------------------------------------------------------------- decode
int decode_umax(const Dims& d) {
  const int u = d.G * d.topk;
  return u < d.nb ? u : d.nb;
}

int decode_chunk() { return kDecChunk; }

int decode_gm(const Dims& d) {
  return d.G <= 1 ? 1 : d.G <= 2 ? 2 : d.G <= 4 ? 4 : 8;
}

size_t decode_part_floats(const Dims& d) {
  return (size_t)d.S * d.Hkv * decode_umax(d) * (d.B / kDecChunk) * decode_gm(d) * (d.D + 2);
}

bool decode_supported(const Dims& d) {
  // the merge lists at most kMergeMaxItems partials per head
  return d.Lq == 1 && d.G <= 8 && d.B % kDecChunk == 0 &&
         (int64_t)decode_umax(d) * (d.B / kDecChunk) <= kMergeMaxItems;
}

// --------------------------------------------------------------- backward
int bwd_dkdv_waves(const Dims& d) { return d.B % 128 == 0 ? 4 : 2; }

int bwd_dkdv_segments(const Dims& d) {
  const int KC = 32 * bwd_dkdv_waves(d);
  const int64_t wgs = (int64_t)d.S * d.Hkv * d.nb * ((d.B + KC - 1) / KC);
  if (wgs >= 1024) return 1;
  const int64_t sgs = (1024 + wgs - 1) / wgs;
  return sgs > 8 ? 8 : (int)sgs;
}

size_t bwd_dkdv_partial_floats(const Dims& d) {
  const int nseg = bwd_dkdv_segments(d);
  return nseg > 1 ? (size_t)nseg * 2 * d.S * d.L * d.Hkv * d.D : 0;
}

}  // namespace moba
