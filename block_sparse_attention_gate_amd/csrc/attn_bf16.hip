// Flash-style attention on MFMA (bf16 inputs, fp32 accumulation).
//
// Two kernels share one inner step:
//   k_attn_routed: one tile = up to 32 * NW routed entries (128 or 256) of
//     one (sequence, KV head, block) bucket; the block is a selected PAST
//     block, so all of its keys are visible (no mask).  Writes, per entry, the normalised partial
//     output (bf16) and its log2-sum-exp (fp32) to the entry's slot.
//   k_attn_query: query-centric causal attention.  Mode 0 (own block): keys
//     from the start of the query's block up to and including the query
//     (causal mask inside the current block, AiBoss MoBA article,
//     "MoBAの技術的原則"), then merges the routed partials of that query by
//     their log-sum-exp, which gives one softmax over the union of the
//     selected keys.  Mode 1: full causal attention (the topk = all case of
//     the full/sparse switch, "MoBA" project card, "How It Works").  Mode 2:
//     the own block only, written as a partial (o, log-sum-exp) for
//     k_merge_partials, so that it can run concurrently with the routing;
//     workgroups with more than kOwnSplitSteps key tiles split their key
//     range in two halves, written to two partials (an empty half writes
//     log-sum-exp = -inf).  Mode 3: full causal attention split into key
//     chunks of chunk_tiles 64-key tiles, one partial per chunk, for problems
//     too small to fill the chip with whole row tiles (the merge follows).
//
// Wave tile: 32 queries (lane l owns query l%32) x 64 keys per step.
//   S^T = K Q^T on 32x32x16 MFMA (K rows in the kperm order, see common.h),
//   online softmax in fp32 (base-2, scale folded into one FMA),
//   O^T += V^T P^T on 32x32x16 MFMA; V^T rows come from the transposed V.
// Workgroup: NW = 4 or 8 waves sharing double-buffered LDS tiles of K [64][D]
// and V^T [D][64] (rows padded by 16 bytes against bank conflicts); all
// threads stage the next tile from HBM through registers while the current
// one is used.
#include "common.h"
#include "kernels.h"

namespace moba {

template <int D, int NW = 4>
struct Tiles {
  static constexpr int NT = 64 * NW;  // threads per workgroup
  static constexpr int KS = D + 8;   // K tile row stride (elements)
  static constexpr int VS = 64 + 8;  // V^T tile row stride (elements)
  static constexpr int KE = 64 * KS;
  static constexpr int VE = D * VS;
  static constexpr int BUF = KE + VE;
  static constexpr int KCH = 64 * (D / 8) / NT;  // 16-byte K chunks per thread
  static constexpr int VCH = D * 8 / NT;         // 16-byte V^T chunks per thread
};

// Global -> register staging of one 64-key tile (all threads).  The
// per-thread offsets inside a tile are fixed; only the tile base (uniform)
// moves, so the loop does no per-thread 64-bit address arithmetic.
template <int D, int NW>
struct TileRegs {
  using T = Tiles<D, NW>;
  u32x4 kr[T::KCH];
  u32x4 vr[T::VCH];
  int koff[T::KCH];   // element offsets inside a K tile (global)
  int voff[T::VCH];   // element offsets inside a V^T tile (global)
  int kls[T::KCH];    // LDS element offsets
  int vls[T::VCH];

  __device__ __forceinline__ void setup(int krow_stride, int Lv, int tid) {
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      const int c = tid + T::NT * i;
      const int row = c / (D / 8), cc = c % (D / 8);
      koff[i] = row * krow_stride + cc * 8;
      kls[i] = row * T::KS + cc * 8;
    }
#pragma unroll
    for (int i = 0; i < T::VCH; ++i) {
      const int c = tid + T::NT * i;
      const int dd = c / 8, kc = c % 8;
      voff[i] = dd * Lv + kc * 8;
      vls[i] = T::KE + dd * T::VS + kc * 8;
    }
  }
  // ktile / vttile: K row `key0` and V^T column `key0` of the tile (uniform).
  __device__ __forceinline__ void load(const bf16_t* ktile, const bf16_t* vttile) {
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) kr[i] = *reinterpret_cast<const u32x4*>(ktile + koff[i]);
#pragma unroll
    for (int i = 0; i < T::VCH; ++i) vr[i] = *reinterpret_cast<const u32x4*>(vttile + voff[i]);
  }
  __device__ __forceinline__ void store(bf16_t* buf) const {
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) *reinterpret_cast<u32x4*>(buf + kls[i]) = kr[i];
#pragma unroll
    for (int i = 0; i < T::VCH; ++i) *reinterpret_cast<u32x4*>(buf + vls[i]) = vr[i];
  }
};

// Largest base-2 gap between a row's logits and its running reference max
// before the accumulators are rescaled (probabilities stay <= 2^8, far from
// fp32 or bf16 overflow).
constexpr float kRescaleSlack = 8.0f;
constexpr float kProbBound = 256.0f;  // 2^kRescaleSlack

template <int D>
struct FlashAcc {
  f32x16 o[D / 32];
  float m;  // reference max of the scaled logits (base 2)
  float l;  // running sum of this lane half's probabilities
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
    m = -__builtin_inff();
    l = 0.f;
  }
};

// The 32 probabilities of one lane for one 64-key step against the reference
// -mneg (base 2), rounded to bf16 for the P.V product; returns their fp32 sum
// (two interleaved partial sums).
__device__ __forceinline__ float step_probs(const f32x16 (&s)[2], float sl2, float mneg,
                                            bf16x8 (&pb)[2][2]) {
  float sum[2] = {0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * c + r], sl2, mneg));
        sum[kt] += p;
        pb[kt][c][r] = static_cast<__bf16>(p);
      }
  return sum[0] + sum[1];
}

// One 64-key step of one wave.  MASK: drop keys outside [klo, qpos].
// VPRE (0..4): 16-key groups of V^T fragments read from LDS before the
// softmax, so that their latency passes under it (bounded by the kernel's
// register budget); the rest are read after it.
template <int D, bool MASK, int VPRE>
__device__ __forceinline__ void flash_step(const bf16_t* buf, const bf16x8 (&qf)[D / 16],
                                           FlashAcc<D>& acc, int n, int hh, float sl2,
                                           int key0, int klo, int qpos) {
  using T = Tiles<D>;
  // S^T = K Q^T for two 32-key subtiles; all K fragments are read first so
  // the LDS latency overlaps, and the two accumulation chains interleave.
  bf16x8 ka[D / 16], kb[D / 16];
  const bf16_t* krow0 = buf + kperm(n) * T::KS + 8 * hh;
  const bf16_t* krow1 = krow0 + 32 * T::KS;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) ka[t] = ld_bf16x8(krow0 + 16 * t);
#pragma unroll
  for (int t = 0; t < D / 16; ++t) kb[t] = ld_bf16x8(krow1 + 16 * t);
  f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    s[0] = mfma32(ka[t], qf[t], s[0]);
    s[1] = mfma32(kb[t], qf[t], s[1]);
  }
  const bf16_t* vbase = buf + T::KE + 8 * hh + n * T::VS;
  bf16x8 va[D / 32][4];
  if (VPRE > 0) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kc = 0; kc < VPRE; ++kc) va[dt][kc] = ld_bf16x8(vbase + 32 * dt * T::VS + 16 * kc);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (MASK) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) {
        const int key = key0 + 32 * kt + acc_key(reg, hh);
        if (key > qpos || key < klo) s[kt][reg] = -__builtin_inff();
      }
  }
  // Lazy rescale, checked through the probabilities: they are first taken
  // against the current reference max acc.m.  A lane sum <= 2^kRescaleSlack
  // bounds each of them, and the step needs no max.  Otherwise (a logit well
  // above the reference, or the first step, where the reference is -inf and
  // the sum is not finite) the wave computes the step max, moves the
  // reference of every row whose max passed it, rescales O and l, and takes
  // the probabilities again.  Exact up to rounding: l sums the same
  // probabilities against the same reference, and the output is divided by
  // it at the end.
  bf16x8 pb[2][2];
  float psum = step_probs(s, sl2, -acc.m, pb);
  if (__any(!(psum <= kProbBound))) {
    float mx = s[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) mx = fmaxf(mx, s[kt][reg]);
    mx = fmaxf(mx, half_swap(mx));
    const float mnew = fmaxf(acc.m, mx * sl2);
    const float mref = (mnew == -__builtin_inff()) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(acc.m - mref);
    acc.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) acc.o[dt][reg] *= alpha;
    acc.m = mnew;
    psum = step_probs(s, sl2, -mref, pb);
  }
  acc.l += psum;
  // O^T += V^T P^T: the D/32 accumulators are independent; interleave them.
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int kc = VPRE; kc < 4; ++kc) va[dt][kc] = ld_bf16x8(vbase + 32 * dt * T::VS + 16 * kc);
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      acc.o[dt] = mfma32(va[dt][kc], pb[kc >> 1][kc & 1], acc.o[dt]);
}

// V^T fragment groups read before the softmax (flash_step's VPRE) per kernel
// shape: as many as the register budget holds without spilling (two waves
// per SIMD: 256 registers).
template <int D, int NW, bool ROUTED>
constexpr int vpre_groups() {
  if (D == 64) return 4;
  if (NW == 8) return 2;
  return 0;
}

template <int D>
__device__ __forceinline__ void load_q(const bf16_t* qrow, bool valid, int hh,
                                       bf16x8 (&qf)[D / 16]) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    qf[t] = ld_bf16x8(qrow + 16 * t + 8 * hh);
    if (!valid) qf[t] = bf16x8{};
  }
}

// ---------------------------------------------------------------------------
// Routed tiles.  grid = upper bound of the tile count; workgroups past the
// device-side tile count exit.  The tile order is XCD-aware: workgroup b runs
// on XCD b % 8, and XCD x takes the contiguous tile range
// [x*per, (x+1)*per), so the tiles of one bucket (same K/V block) share an L2.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_attn_routed(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ vt,
    const uint32_t* __restrict__ list, const uint32_t* __restrict__ bucket_off,
    const uint32_t* __restrict__ tile_off, bf16_t* __restrict__ po, float* __restrict__ plse,
    int64_t Lq, int64_t L, int64_t Lv, int H, int Hkv, int kp, int B, int nb, int nrows,
    float sl2, uint32_t nslots, int64_t prow0, int ph0, int pH) {
  using T = Tiles<D, NW>;
  constexpr int VPRE = vpre_groups<D, NW, true>();
  constexpr int TM = 32 * NW;  // routed entries per tile
  // Eight-wave tiles (one workgroup per CU) copy the tile and bucket offsets
  // into LDS with parallel loads and search them there, instead of a chain of
  // dependent global loads before the first K/V tile can be requested.
  constexpr int RL = NW == 8 ? kRoutedLdsRows : 0;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * T::BUF];
  __shared__ uint32_t offs[RL > 0 ? 2 * (RL + 1) : 1];
  const int tid = threadIdx.x;
  const bool in_lds = RL > 0 && nrows <= RL;
  if (in_lds) {
    for (int i = tid; i <= nrows; i += T::NT) {
      offs[i] = tile_off[i];
      offs[RL + 1 + i] = bucket_off[i];
    }
    __syncthreads();
  }
  auto tile_at = [&](int i) { return in_lds ? offs[i] : tile_off[i]; };
  auto bucket_at = [&](int i) { return in_lds ? offs[RL + 1 + i] : bucket_off[i]; };
  const uint32_t ntiles = tile_at(nrows);
  const uint32_t per = (ntiles + 7) / 8;
  const uint32_t bid = blockIdx.x;
  if (bid / 8 >= per) return;
  const uint32_t tile = (bid % 8) * per + bid / 8;
  if (tile >= ntiles) return;
  int lo = 0, hi = nrows;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_at(mid) <= tile) lo = mid; else hi = mid;
  }
  const int row = lo;
  const uint32_t start = (tile - tile_at(row)) * TM;
  const uint32_t b0 = bucket_at(row);
  const uint32_t avail = bucket_at(row + 1) - b0 - start;
  const int cnt = avail < (uint32_t)TM ? (int)avail : TM;
  // bucket rows and slots are the pass's (prow0, ph0, pH: see Dims)
  const int64_t grow = prow0 + row;
  const int j = (int)(grow % nb);
  const int sg = (int)(grow / nb), g = sg % Hkv, s = sg / Hkv;

  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int e = 32 * w + n;
  const bool wave_on = 32 * w < cnt;
  const uint32_t slot_raw = (e < cnt) ? list[b0 + start + e] : 0u;
  const bool valid = e < cnt && slot_raw < nslots;  // never write outside the partials
  const uint32_t slot = valid ? slot_raw : 0u;
  const uint32_t qh = slot / (uint32_t)kp;
  const int64_t r = qh % Lq;
  const int h = ph0 + (int)((qh / Lq) % pH);
  bf16x8 qf[D / 16];
  load_q<D>(q + (((int64_t)s * Lq + r) * H + h) * D, valid, hh, qf);

  const bf16_t* kbase = k + ((int64_t)s * L * Hkv + g) * D;
  const bf16_t* vtbase = vt + ((int64_t)s * Hkv + g) * D * Lv;
  const int64_t kstart = (int64_t)j * B;
  const int nsteps = B / 64;  // a selected past block is always whole
  FlashAcc<D> acc;
  acc.init();
  TileRegs<D, NW> tr;
  tr.setup(Hkv * D, (int)Lv, tid);
  const int64_t ktile_step = (int64_t)64 * Hkv * D;
  const bf16_t* ktile = kbase + kstart * Hkv * D;
  const bf16_t* vttile = vtbase + kstart;
  tr.load(ktile, vttile);
  tr.store(lds);
  __syncthreads();
  // Every wave runs the same loads, stores and barriers; the waves holding
  // entries also compute (two loops keep the accumulators out of a branch).
  if (wave_on) {
    for (int it = 0; it < nsteps; ++it) {
      const bool more = it + 1 < nsteps;
      ktile += ktile_step;
      vttile += 64;
      if (more) tr.load(ktile, vttile);
      flash_step<D, false, VPRE>(lds + (it & 1) * T::BUF, qf, acc, n, hh, sl2, 0, 0, 0);
      if (more) tr.store(lds + ((it + 1) & 1) * T::BUF);
      __syncthreads();
    }
  } else {
    for (int it = 0; it < nsteps; ++it) {
      const bool more = it + 1 < nsteps;
      ktile += ktile_step;
      vttile += 64;
      if (more) tr.load(ktile, vttile);
      if (more) tr.store(lds + ((it + 1) & 1) * T::BUF);
      __syncthreads();
    }
  }
  if (!valid) return;
  const float ltot = acc.l + half_swap(acc.l);
  const float inv = 1.0f / ltot;
  bf16_t* orow = po + (int64_t)slot * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * dt + 8 * i + 4 * hh;
      const uint32_t w0 = (uint32_t)f32_to_bf16(acc.o[dt][4 * i] * inv) |
                          ((uint32_t)f32_to_bf16(acc.o[dt][4 * i + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(acc.o[dt][4 * i + 2] * inv) |
                          ((uint32_t)f32_to_bf16(acc.o[dt][4 * i + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + d0) = make_uint2(w0, w1);
    }
  if (hh == 0) plse[slot] = acc.m + __log2f(ltot);
}

// ---------------------------------------------------------------------------
// Query-centric causal attention (own block + merge, own-block partials,
// full, full in key chunks).
// A workgroup covers HW heads of one KV group x RW query rows (HW*RW = 32*NW);
// wave w takes head h0 + w % HW and rows [r0 + 32*(w / HW), +32).
// grid (ceil(Lq / RW) * P, S * H / HW), P = 2 in mode 2, nparts in mode 3,
// else 1.
// ---------------------------------------------------------------------------
template <int D, int MODE, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_attn_query(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ vt,
    const bf16_t* __restrict__ po, const float* __restrict__ plse, bf16_t* __restrict__ out,
    const bf16_t* __restrict__ ktail, float* __restrict__ lse_out, int Lq, int L, int Lv,
    int q_off, int H, int Hkv, int kp, int B, int HW, float sl2, int nparts, int chunk_tiles,
    int ps0, int ph0, int pH) {
  using T = Tiles<D, NW>;
  constexpr int VPRE = vpre_groups<D, NW, false>();
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * T::BUF];
  const int RW = 32 * NW / HW;
  // Modes 2 and 3: blockIdx.x = P * item + part (P key-range parts per item).
  const int P = MODE == 2 ? 2 : (MODE == 3 ? nparts : 1);
  const int item = (int)blockIdx.x / P;
  const int part = (int)blockIdx.x % P;
  const int nitems = (int)gridDim.x / P;
  // Longest work first.  Full attention: the last row tiles.  Own block (when
  // blocks hold whole row tiles): the tiles at the end of every block first.
  int rt;
  if (MODE == 1 || MODE == 3) {
    rt = nitems - 1 - item;
  } else if (q_off % B == 0 && B % RW == 0 && Lq % B == 0) {
    const int tpb = B / RW, nbq = Lq / B;
    const int rank = item / nbq, blk = item % nbq;
    rt = blk * tpb + (tpb - 1 - rank);
  } else {
    rt = item;
  }
  // blockIdx.y: (sequence, head group) of the pass's heads [ph0, ph0 + pH)
  // of sequences ps0.. (the whole problem without passes)
  const int hgroups = pH / HW;
  const int s = ps0 + (int)blockIdx.y / hgroups;
  const int h0 = ph0 + ((int)blockIdx.y % hgroups) * HW;
  const int g = h0 / (H / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int h = h0 + w % HW;
  const int rw0 = rt * RW;                 // first row of the workgroup
  const int r0 = rw0 + 32 * (w / HW);      // first row of this wave
  const int r = r0 + n;
  const bool valid = r < Lq;
  const bool wave_on = r0 < Lq;
  const int pos = q_off + r;
  // key windows [klo, khi)
  const int wlast = (r0 + 31 < Lq ? r0 + 31 : Lq - 1);
  const int klo_w = (MODE == 0 || MODE == 2) ? ((q_off + r0) / B) * B : 0;
  const int khi_w = wave_on ? q_off + wlast + 1 : 0;
  const int wglast = (rw0 + RW - 1 < Lq ? rw0 + RW - 1 : Lq - 1);
  const int klo_g = (MODE == 0 || MODE == 2) ? ((q_off + rw0) / B) * B : 0;
  const int khi_g = q_off + wglast + 1;
  int t0 = klo_g / 64, t1 = (khi_g + 63) / 64;
  if (MODE == 2 || MODE == 3) {
    if (MODE == 2) {
      const int nst = t1 - t0;
      const int ts = nst > kOwnSplitSteps ? t0 + nst / 2 : t1;
      if (part == 0) t1 = ts; else t0 = ts;
    } else {
      const int a0 = t0 + part * chunk_tiles, a1 = a0 + chunk_tiles;
      t0 = a0;
      t1 = a1 < t1 ? a1 : t1;
    }
    if (t0 >= t1) {
      // empty part: log-sum-exp -inf, which the merge skips
      if (valid && hh == 0) {
        const int64_t nqh = (int64_t)gridDim.y * HW * Lq;
        const_cast<float*>(plse)[part * nqh + ((int64_t)s * H + h) * Lq + r] = -__builtin_inff();
      }
      return;
    }
  }
  const int klo_l = (MODE == 0 || MODE == 2) ? (pos / B) * B : 0;

  bf16x8 qf[D / 16];
  load_q<D>(q + (((int64_t)s * Lq + (valid ? r : 0)) * H + h) * D, valid, hh, qf);
  const bf16_t* kbase = k + ((int64_t)s * L * Hkv + g) * D;
  const bf16_t* vtbase = vt + ((int64_t)s * Hkv + g) * D * Lv;
  const int pos_first = q_off + r0;        // smallest query position of the wave
  FlashAcc<D> acc;
  acc.init();
  TileRegs<D, NW> tr;
  tr.setup(Hkv * D, Lv, tid);
  const int64_t ktile_step = (int64_t)64 * Hkv * D;
  const bf16_t* ktile = kbase + (int64_t)t0 * ktile_step;
  const bf16_t* vttile = vtbase + (int64_t)t0 * 64;
  // The tile holding the end of a sequence whose length is not a multiple of
  // 64 reads its K rows from `ktail` ([S, 64, Hkv, D], the same row stride as
  // K, rows past L zero) so that no load passes the end of K; its keys past L
  // are never visible (every tile from the one holding the wave's first
  // query on runs under the causal mask).  A uniform pointer choice.
  const int ttail = (L % 64) ? L / 64 : -1;
  const bf16_t* ktail_sg = ttail >= 0 ? ktail + ((int64_t)s * 64 * Hkv + g) * D : kbase;
  auto load_tile = [&](int ti) { tr.load(ti == ttail ? ktail_sg : ktile, vttile); };
  load_tile(t0);
  tr.store(lds);
  __syncthreads();
  // Per wave the workgroup's tiles [t0, t1) split into: idle before the
  // wave's window, full tiles, tiles that need the mask (diagonal or the
  // block start), idle after.  Each phase is its own loop; every iteration of
  // every loop does the same loads, stores and one barrier.
  int ws_ = t1, wd_ = t1, we_ = t1;
  if (wave_on) {
    ws_ = klo_w / 64;                                  // first tile of the window
    we_ = (khi_w + 63) / 64;                           // one past the last
    // first tile that needs the mask: its last key passes the wave's first
    // query (key0 + 63 > pos_first)
    const int d_ = (pos_first + 1) / 64;
    wd_ = d_ < ws_ ? ws_ : (d_ > we_ ? we_ : d_);
    if (klo_w % 64 != 0) wd_ = ws_;                    // window start not tile-aligned
    // rows of the wave in two blocks (queries at an offset that is not a
    // multiple of 32): the lanes' windows start at different keys, so every
    // tile takes the per-lane mask
    if ((MODE == 0 || MODE == 2) && ((q_off + wlast) / B) * B != klo_w) wd_ = ws_;
    // restrict the phases to this workgroup's tiles [t0, t1)
    ws_ = ws_ < t0 ? t0 : (ws_ > t1 ? t1 : ws_);
    we_ = we_ < ws_ ? ws_ : (we_ > t1 ? t1 : we_);
    wd_ = wd_ < ws_ ? ws_ : (wd_ > we_ ? we_ : wd_);
  }
  int it = t0;
  auto advance = [&](int i) {
    const bool more = i + 1 < t1;
    ktile += ktile_step;
    vttile += 64;
    if (more) load_tile(i + 1);
    return more;
  };
  for (; it < ws_; ++it) {
    const bool more = advance(it);
    if (more) tr.store(lds + ((it + 1 - t0) & 1) * T::BUF);
    __syncthreads();
  }
  for (; it < wd_; ++it) {
    const bool more = advance(it);
    flash_step<D, false, VPRE>(lds + ((it - t0) & 1) * T::BUF, qf, acc, n, hh, sl2, 0, 0, 0);
    if (more) tr.store(lds + ((it + 1 - t0) & 1) * T::BUF);
    __syncthreads();
  }
  for (; it < we_; ++it) {
    const bool more = advance(it);
    flash_step<D, true, VPRE>(lds + ((it - t0) & 1) * T::BUF, qf, acc, n, hh, sl2, it * 64, klo_l,
                        pos);
    if (more) tr.store(lds + ((it + 1 - t0) & 1) * T::BUF);
    __syncthreads();
  }
  for (; it < t1; ++it) {
    const bool more = advance(it);
    if (more) tr.store(lds + ((it + 1 - t0) & 1) * T::BUF);
    __syncthreads();
  }
  if (!valid) return;
  const float ltot = acc.l + half_swap(acc.l);
  bf16_t* orow = out + (((int64_t)s * Lq + r) * H + h) * D;
  float inv = 1.0f / ltot;
  if (MODE == 2 || MODE == 3) {
    // partial (this part of the key range) of query-head qh: normalised o
    // (bf16) and log2-sum-exp; a row with no visible key here gets o = 0, -inf
    const int64_t nqh = (int64_t)gridDim.y * HW * Lq;
    const int64_t qh = ((int64_t)s * H + h) * Lq + r + part * nqh;
    orow = const_cast<bf16_t*>(po) + qh * D;
    if (!(ltot > 0.f)) inv = 0.f;
    if (hh == 0)
      const_cast<float*>(plse)[qh] = ltot > 0.f ? acc.m + __log2f(ltot) : -__builtin_inff();
  }
  // log2 of the softmax normaliser over all of the query's keys (scaled
  // logits), kept for the backward as a natural log (mode 0)
  float lse_all = acc.m + __log2f(ltot);
  if (MODE == 0 && kp > 0) {
    // Merge: out = sum_x 2^(lse_x - M) o_x / sum_x 2^(lse_x - M) over the own
    // partial and the routed partials of this query.
    const int own = pos / B;
    const int npast = kp < own ? kp : own;
    const float lse_own = acc.m + __log2f(ltot);
    float M = lse_own;
    const int64_t sbase = (((int64_t)(s - ps0) * pH + (h - ph0)) * Lq + r) * kp;
    // all routed log-sum-exps first (independent loads), then the partial
    // rows four at a time (four rows in flight per lane instead of one).  A
    // lane loads 16 bytes of a row, the half hh of each 32-byte group; the
    // two lanes of a query then exchange the middle 8 bytes
    // (v_permlane32_swap), which leaves each with its 4-element pieces of the
    // accumulator layout (elements 8i + 4hh + [0, 4) of each 32-row group).
    float lsv[kMaxTopk - 1];
#pragma unroll
    for (int t = 0; t < kMaxTopk - 1; ++t)
      lsv[t] = t < npast ? plse[sbase + t] : -__builtin_inff();
#pragma unroll
    for (int t = 0; t < kMaxTopk - 1; ++t) M = fmaxf(M, lsv[t]);
    const float w_own = __builtin_amdgcn_exp2f(lse_own - M);
    float wsum = w_own;
    const float sc = w_own / ltot;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int reg = 0; reg < 16; ++reg) acc.o[dt][reg] *= sc;
#pragma unroll
    for (int t0 = 0; t0 < kMaxTopk - 1; t0 += 4) {
      if (t0 < npast) {
        u32x4 raw[4][D / 32][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16_t* prow = po + (sbase + (t0 + u < npast ? t0 + u : t0)) * D;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int m = 0; m < 2; ++m)
              raw[u][dt][m] = *reinterpret_cast<const u32x4*>(prow + 32 * dt + 16 * m + 8 * hh);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // a slot past npast re-reads slot t0 with weight 0
          const float wt = t0 + u < npast ? __builtin_amdgcn_exp2f(lsv[t0 + u] - M) : 0.f;
          wsum += wt;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const u32x4 x = raw[u][dt][m];
              // [0]: pieces i = 2m, [1]: i = 2m + 1 (first and second dwords)
              const auto w0 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
              const auto w1 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const int i = 2 * m + e;
                const uint32_t a = w0[e], b = w1[e];
                acc.o[dt][4 * i] = fmaf(wt, __uint_as_float(a << 16), acc.o[dt][4 * i]);
                acc.o[dt][4 * i + 1] = fmaf(wt, __uint_as_float(a & 0xffff0000u), acc.o[dt][4 * i + 1]);
                acc.o[dt][4 * i + 2] = fmaf(wt, __uint_as_float(b << 16), acc.o[dt][4 * i + 2]);
                acc.o[dt][4 * i + 3] = fmaf(wt, __uint_as_float(b & 0xffff0000u), acc.o[dt][4 * i + 3]);
              }
            }
        }
      }
    }
    inv = 1.0f / wsum;
    lse_all = M + __log2f(wsum);
  }
  if (MODE == 0 && lse_out != nullptr && hh == 0)
    lse_out[((int64_t)s * H + h) * Lq + r] = lse_all * kLn2;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * dt + 8 * i + 4 * hh;
      const uint32_t w0 = (uint32_t)f32_to_bf16(acc.o[dt][4 * i] * inv) |
                          ((uint32_t)f32_to_bf16(acc.o[dt][4 * i + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(acc.o[dt][4 * i + 2] * inv) |
                          ((uint32_t)f32_to_bf16(acc.o[dt][4 * i + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + d0) = make_uint2(w0, w1);
    }
}

// Merge of the key-range partials (two halves of the own block, or the key
// chunks of split full attention; nown of them, one after the other in
// own_o / own_lse) with the routed partials of every query-head:
// out = sum_x 2^(lse_x - M) o_x / sum_x 2^(lse_x - M).  16 lanes
// per query-head, D/16 dims per lane.  grid ceil(nqh / 16), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void k_merge_partials(
    const bf16_t* __restrict__ own_o, const float* __restrict__ own_lse, int nown,
    const bf16_t* __restrict__ po, const float* __restrict__ plse, bf16_t* __restrict__ out,
    float* __restrict__ lse_out, int64_t nqh, int64_t Lq, int H, int64_t q_off, int B, int kp) {
  constexpr int EPL = D / 16;
  const int64_t qh = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
  if (qh >= nqh) return;
  const int sub = threadIdx.x % 16;
  const int64_t r = qh % Lq, sh = qh / Lq;
  const int h = (int)(sh % H);
  const int64_t s = sh / H;
  const int64_t own = (q_off + r) / B;
  const int npast = (int)(kp < own ? kp : own);
  // part 0 always holds keys (the first key of the range is visible)
  const float lse0 = own_lse[qh];
  float M = lse0;
  for (int p = 1; p < nown; ++p) M = fmaxf(M, own_lse[p * nqh + qh]);
  for (int t = 0; t < npast; ++t) M = fmaxf(M, plse[qh * kp + t]);
  float acc[EPL];
  auto load = [&](const bf16_t* p, float (&x)[EPL]) {
    if (EPL == 8) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(raw[i] << 16);
        x[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
      }
    } else {
      const uint2 raw = *reinterpret_cast<const uint2*>(p);
      x[0] = __uint_as_float(raw.x << 16);
      x[1] = __uint_as_float(raw.x & 0xffff0000u);
      x[2] = __uint_as_float(raw.y << 16);
      x[3] = __uint_as_float(raw.y & 0xffff0000u);
    }
  };
  float x[EPL];
  load(own_o + qh * D + sub * EPL, x);
  const float w0 = __builtin_amdgcn_exp2f(lse0 - M);
  float wsum = w0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = w0 * x[i];
  for (int p = 1; p < nown; ++p) {
    const float lp = own_lse[p * nqh + qh];
    if (!(lp > -__builtin_inff())) continue;  // empty part
    const float w1 = __builtin_amdgcn_exp2f(lp - M);
    wsum += w1;
    load(own_o + (p * nqh + qh) * D + sub * EPL, x);
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = fmaf(w1, x[i], acc[i]);
  }
  for (int t = 0; t < npast; ++t) {
    const float wt = __builtin_amdgcn_exp2f(plse[qh * kp + t] - M);
    wsum += wt;
    load(po + (qh * kp + t) * D + sub * EPL, x);
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = fmaf(wt, x[i], acc[i]);
  }
  const float inv = 1.0f / wsum;
  if (lse_out != nullptr && sub == 0) lse_out[qh] = (M + __log2f(wsum)) * kLn2;
  bf16_t* orow = out + ((s * Lq + r) * H + h) * D + sub * EPL;
  uint32_t wds[EPL / 2];
#pragma unroll
  for (int i = 0; i < EPL / 2; ++i)
    wds[i] = (uint32_t)f32_to_bf16(acc[2 * i] * inv) |
             ((uint32_t)f32_to_bf16(acc[2 * i + 1] * inv) << 16);
  if (EPL == 8)
    *reinterpret_cast<u32x4*>(orow) = u32x4{wds[0], wds[1], wds[EPL / 2 > 2 ? 2 : 0],
                                            wds[EPL / 2 > 3 ? 3 : 0]};
  else
    *reinterpret_cast<uint2*>(orow) = make_uint2(wds[0], wds[1]);
}

hipError_t launch_merge_partials_bf16(const void* own_o, const float* own_lse, int nown,
                                      const void* po, const float* plse, void* out,
                                      const Dims& d, hipStream_t st, float* lse_out) {
  const int64_t nqh = (int64_t)d.S * d.H * d.Lq;
  const unsigned grid = (unsigned)((nqh + 15) / 16);
#define MOBA_MERGE(DV)                                                                       \
  hipLaunchKernelGGL(k_merge_partials<DV>, dim3(grid), dim3(256), 0, st,                     \
                     static_cast<const bf16_t*>(own_o), own_lse, nown,                       \
                     static_cast<const bf16_t*>(po), plse, static_cast<bf16_t*>(out),        \
                     lse_out, nqh, d.Lq, d.H, d.q_off, d.B, d.kp)
  if (d.D == 128) MOBA_MERGE(128); else MOBA_MERGE(64);
#undef MOBA_MERGE
  return hipGetLastError();
}

static int gcd_int(int a, int b) {
  while (b) { const int t = a % b; a = b; b = t; }
  return a;
}

hipError_t launch_attn_routed_bf16(const void* q, const void* k, const void* vt,
                                   const uint32_t* list, const uint32_t* bucket_off,
                                   const uint32_t* tile_off, void* part_o, float* part_lse,
                                   const Dims& d, hipStream_t st) {
  const int64_t grid = routed_tile_bound(d);
  const float sl2 = kLog2e / sqrtf((float)d.D);
#define MOBA_ROUTED(DV, NWV)                                                                 \
  hipLaunchKernelGGL((k_attn_routed<DV, NWV>), dim3((unsigned)grid), dim3(64 * NWV), 0, st,  \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),           \
                     static_cast<const bf16_t*>(vt), list, bucket_off, tile_off,             \
                     static_cast<bf16_t*>(part_o), part_lse, d.Lq, d.L, d.Lv, d.H, d.Hkv,    \
                     d.kp, d.B, d.nb, d.pnrows, sl2, (uint32_t)d.pslots, d.prow0, d.ph0, d.pH)
  if (d.tile_m == 256) {
    if (d.D == 128) MOBA_ROUTED(128, 8); else MOBA_ROUTED(64, 8);
  } else {
    if (d.D == 128) MOBA_ROUTED(128, 4); else MOBA_ROUTED(64, 4);
  }
#undef MOBA_ROUTED
  return hipGetLastError();
}

// Workgroup shape of the query kernels: HW heads of one KV group per
// workgroup, NW waves; eight waves when that still gives >= 2048 workgroups.
static void query_shape(const Dims& d, int* HW, int* NW) {
  *HW = gcd_int(d.G, 4);
  const int64_t wgs8 = (d.Lq + 256 / *HW - 1) / (256 / *HW) * (int64_t)(d.S * d.H / *HW);
  *NW = wgs8 >= 2048 ? 8 : 4;
}

hipError_t launch_attn_query_bf16(const void* q, const void* k, const void* vt,
                                  const void* ktail, const void* part_o, const float* part_lse,
                                  void* out, int mode, const Dims& d, hipStream_t st,
                                  int nparts, float* lse_out) {
  if (d.L % 64 != 0 && ktail == nullptr) return hipErrorInvalidValue;
  int HW, NW;
  query_shape(d, &HW, &NW);
  if (mode == 3) NW = 8;
  const int RW = 32 * NW / HW;
  const int per = mode == 2 ? 2 : (mode == 3 ? nparts : 1);
  dim3 grid((unsigned)((d.Lq + RW - 1) / RW * per), d.pS * d.pH / HW);
  const float sl2 = kLog2e / sqrtf((float)d.D);
#define MOBA_QUERY(DV, MV, NWV)                                                              \
  hipLaunchKernelGGL((k_attn_query<DV, MV, NWV>), grid, dim3(64 * NWV), 0, st,               \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),           \
                     static_cast<const bf16_t*>(vt), static_cast<const bf16_t*>(part_o),     \
                     part_lse, static_cast<bf16_t*>(out), static_cast<const bf16_t*>(ktail), \
                     mode == 0 ? lse_out : nullptr, (int)d.Lq, (int)d.L, (int)d.Lv,            \
                     (int)d.q_off, d.H, d.Hkv, d.kp, d.B, HW, sl2, nparts, kFullChunkTiles, \
                     d.ps0, d.ph0, d.pH)
#define MOBA_QUERY_NW(DV, MV) \
  if (NW == 8) MOBA_QUERY(DV, MV, 8); else MOBA_QUERY(DV, MV, 4);
  if (d.D == 128) {
    if (mode == 0) { MOBA_QUERY_NW(128, 0) }
    else if (mode == 1) { MOBA_QUERY_NW(128, 1) }
    else if (mode == 2) { MOBA_QUERY_NW(128, 2) }
    else { MOBA_QUERY(128, 3, 8); }
  } else {
    if (mode == 0) { MOBA_QUERY_NW(64, 0) }
    else if (mode == 1) { MOBA_QUERY_NW(64, 1) }
    else if (mode == 2) { MOBA_QUERY_NW(64, 2) }
    else { MOBA_QUERY(64, 3, 8); }
  }
#undef MOBA_QUERY_NW
#undef MOBA_QUERY
  return hipGetLastError();
}

}  // namespace moba
