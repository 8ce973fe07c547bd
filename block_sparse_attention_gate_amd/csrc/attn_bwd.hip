// Backward of the MoBA attention (bf16 inputs, fp32 accumulation), for the
// continued training the pages require ("MoBA" project card, "Highlighted
// Details"; Dev Tutorial, step 1 note).  The forward's selection is held
// fixed: top-k passes no gradient, so the gate and the block means get none.
// For one query with key set T, scaled logits z_t = c k_t.q (c = 1/sqrt(D)),
// p = softmax(z) = 2^(z log2(e) - lse2) with the forward's log-sum-exp, and
// Dv = dO.o:
//   dv_t += p_t dO,   ds_t = p_t (dO.v_t - Dv),   dq = c sum_t ds_t k_t,
//   dk_t += c ds_t q.
// Kernels:
//   k_bwd_dot        Dv per query-head (and, for dk/dv, lse and Dv per row
//                    in memory order).
//   k_bwd_entry_rows the Q / dO row index of every routed entry.
//   k_bwd_tail       for a length that is not a multiple of 64, the last K
//                    and V tiles [S, 64, Hkv, D] zero padded (so that no tile
//                    load passes the end).
//   k_bwd_dq_routed  per routed tile (the forward's tile list): S^T = K Q^T
//                    and dP^T = V dO^T on MFMA, dS^T in registers, then
//                    dQ^T += K^T dS^T with K^T read transposed from the K
//                    tile; one bf16 dq partial per routed slot.
//   k_bwd_dq_own     per query: the own block (causal mask) the same way, plus
//                    the query's routed dq partials -> dq.
//   k_bwd_dkdv       per 32 * NW keys of one block (key-stationary, no
//                    atomics): loops over the block's routed entries and its
//                    own queries 64 at a time; S = Q K^T and dP = dO V^T with
//                    the wave's K and V rows as register B operands, then
//                    dV^T += dO^T P and dK^T += Q^T dS with the A operands
//                    read transposed (LDS transpose reads) from the same Q /
//                    dO tiles.
// Queries are loaded into the MFMA A rows in the kperm order (common.h), so
// the accumulator of a product over 32 queries is directly the B operand of
// the following product over those queries.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moba {

// ------------------------------------------------------------ Dv = dO . o
// One row per LPR = D/8 lanes (16 bytes of o and dO each); the row index is
// in memory order (s, r, h).  Dv is written in query-head order; with
// rowstat (bf16 dk/dv) also (lse log2(e), Dv) per row in memory order.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dot(const bf16_t* __restrict__ o,
                                                 const bf16_t* __restrict__ dout,
                                                 const float* __restrict__ lse,
                                                 float* __restrict__ dvec,
                                                 float2* __restrict__ rowstat, int64_t nrows,
                                                 int64_t Lq, int H) {
  constexpr int LPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + sub * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + row * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), acc);
      acc = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(b[e] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < nrows && sub == 0) {
    const int64_t h = row % H, sr = row / H, r = sr % Lq, s = sr / Lq;
    const int64_t qh = (s * H + h) * Lq + r;
    dvec[qh] = acc;
    if (rowstat) rowstat[row] = make_float2(lse[qh] * kLog2e, acc);
  }
}

// ------------------------------------------------------------ the last tiles
// For a length that is not a multiple of 64: the last K and V tiles of every
// (sequence, KV head), [S, 64, Hkv, D], zero past the end (so that no tile
// load passes the end).  grid (Hkv, S), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_tail(const bf16_t* __restrict__ k,
                                                  const bf16_t* __restrict__ v,
                                                  bf16_t* __restrict__ ktail,
                                                  bf16_t* __restrict__ vtail, int Hkv, int64_t L) {
  constexpr int CPR = D / 8;
  const int g = blockIdx.x, s = blockIdx.y;
  const int64_t key0 = L / 64 * 64;
  const int64_t nkey = L - key0;  // 1..63
  for (int c = threadIdx.x; c < 64 * CPR; c += 256) {
    const int row = c / CPR, cc = c % CPR;
    const int64_t src = (((int64_t)s * L + key0 + row) * Hkv + g) * D + cc * 8;
    const int64_t dst = (((int64_t)s * 64 + row) * Hkv + g) * D + cc * 8;
    u32x4 kv = u32x4{0u, 0u, 0u, 0u}, vv = u32x4{0u, 0u, 0u, 0u};
    if (row < nkey) {
      kv = *reinterpret_cast<const u32x4*>(k + src);
      vv = *reinterpret_cast<const u32x4*>(v + src);
    }
    *reinterpret_cast<u32x4*>(ktail + dst) = kv;
    *reinterpret_cast<u32x4*>(vtail + dst) = vv;
  }
}

// LDS tiles of 64 rows (keys or queries) of D bf16, unpadded, with the
// 16-byte chunks of row r permuted by XOR with kv_swz(r).  The pattern makes
// both reads of the tiles free of LDS bank conflicts: 16 consecutive rows at
// one chunk (MFMA A rows with the contraction over d), and 4 consecutive rows
// x 4 consecutive chunks (a 32-lane half of a transpose read, A rows d with
// the contraction over the tile's rows).
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int D>
__device__ __forceinline__ int kv_off(int r, int chunk) {
  return r * D + ((chunk ^ kv_swz<D>(r)) << 3);
}

// A operand of a product over the tile's rows (rows d = 32 dt + lane % 32,
// k-slots = tile rows 16 c2 + 8 (lane / 32) + [0, 8)) from a row-major
// [row][d] tile.
// The LDS transpose read (16-bit elements, 64 bits per lane) hands lane i of
// each 16-lane group element i % 4 of the values read by lanes i / 4 + 4e of
// its group, e = 0..3; so lane 4e + f of a group reads dims 4f.. of row e,
// and lane i receives dim i of four consecutive rows.  Two reads give the
// eight rows.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* tile, int dt, int c2, int lane) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const int grp = lane >> 4, e = (lane >> 2) & 3, f = lane & 3;
  const int col = 32 * dt + 16 * (grp & 1) + 4 * f;
  bf16x4 part[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = 16 * c2 + 8 * (grp >> 1) + 4 * half + e;
    const bf16_t* p = tile + kv_off<D>(r, col >> 3) + (col & 7);
    part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)const_cast<bf16_t*>(p));
  }
  return bf16x8{part[0][0], part[0][1], part[0][2], part[0][3],
                part[1][0], part[1][1], part[1][2], part[1][3]};
}

// 8 bf16 of a query-like row for lane half hh: fragments of the B operand
// (lane = query) of S^T = K Q^T and dP^T = V dO^T.
template <int D>
__device__ __forceinline__ void bwd_row_frags(const bf16_t* row, bool valid, int hh,
                                              bf16x8 (&f)[D / 16]) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    f[t] = ld_bf16x8(row + 16 * t + 8 * hh);
    if (!valid) f[t] = bf16x8{};
  }
}

// ============================================================== dq kernels
// K and V tiles of 64 keys, swizzled rows (kv_off); K^T for dQ^T += K^T dS^T
// is read from the K tile with transpose reads.
template <int D, int NW>
struct DqTiles {
  static constexpr int NT = 64 * NW;
  static constexpr int KE = 64 * D;
  static constexpr int BUF = 2 * KE;             // K, V (bf16 elements)
  static constexpr int RCH = 64 * (D / 8) / NT;  // 16-byte chunks per thread of K (and V)
};

// Global -> register staging of one 64-key tile of K and V (row stride
// Hkv*D); fixed per-thread offsets.
template <int D, int NW>
struct DqRegs {
  using T = DqTiles<D, NW>;
  u32x4 kr[T::RCH], vr[T::RCH];
  int roff[T::RCH], rls[T::RCH];
  __device__ __forceinline__ void setup(int krow_stride, int tid) {
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) {
      const int c = tid + T::NT * i;
      const int row = c / (D / 8), cc = c % (D / 8);
      roff[i] = row * krow_stride + cc * 8;
      rls[i] = kv_off<D>(row, cc);
    }
  }
  __device__ __forceinline__ void load(const bf16_t* ksrc, const bf16_t* vsrc) {
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) kr[i] = *reinterpret_cast<const u32x4*>(ksrc + roff[i]);
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) vr[i] = *reinterpret_cast<const u32x4*>(vsrc + roff[i]);
  }
  __device__ __forceinline__ void store(bf16_t* buf) const {
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) *reinterpret_cast<u32x4*>(buf + rls[i]) = kr[i];
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) *reinterpret_cast<u32x4*>(buf + T::KE + rls[i]) = vr[i];
  }
};

// One 64-key step of one wave (32 queries, lane n = query), as two 32-key
// halves: S^T = K Q^T and dP^T = V dO^T (K / V rows in the kperm order),
// dS^T in registers, then dQ^T += K^T dS^T.  MASK: drop keys outside
// [klo, qpos].
template <int D, bool MASK>
__device__ __forceinline__ void dq_step(const bf16_t* buf, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&df)[D / 16], f32x16 (&dq)[D / 32],
                                        int lane, float sl2, float lse2, float dv, int key0,
                                        int klo, int qpos) {
  constexpr int KE = 64 * D;
  const int n = lane & 31, hh = lane >> 5;
  const int ar = kperm(n);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const bf16_t* kr = buf + kv_off<D>(32 * kt + ar, 2 * t + hh);
      s = mfma32(ld_bf16x8(kr), qf[t], s);
      dp = mfma32(ld_bf16x8(kr + KE), df[t], dp);
    }
    // The first two K^T fragments of the dQ product are read before dS, so
    // that their LDS latency passes under it (more would not fit the register
    // budget of two waves per SIMD).
    bf16x8 kf0[D / 32];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) kf0[dt] = tr_frag<D>(buf, dt, 2 * kt, lane);
    __builtin_amdgcn_sched_barrier(0);
    // dS^T = P^T (dP^T - Dv), P^T = 2^(S^T sl2 - lse2); registers [8c, 8c+8)
    // hold keys 32 kt + 16 c + 8 hh + [0, 8): the B operand layout
    bf16x8 dsb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int reg = 8 * c + r;
        float p = __builtin_amdgcn_exp2f(fmaf(s[reg], sl2, -lse2));
        if (MASK) {
          const int key = key0 + 32 * kt + acc_key(reg, hh);
          if (key > qpos || key < klo) p = 0.f;
        }
        dsb[c][r] = static_cast<__bf16>(p * (dp[reg] - dv));
      }
#pragma unroll
    for (int dt = 2; dt < D / 32; ++dt) kf0[dt] = tr_frag<D>(buf, dt, 2 * kt, lane);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) dq[dt] = mfma32(kf0[dt], dsb[0], dq[dt]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      dq[dt] = mfma32(tr_frag<D>(buf, dt, 2 * kt + 1, lane), dsb[1], dq[dt]);
  }
}

// dq^T accumulator (lane = query, rows d) -> a bf16 row, scaled.
template <int D>
__device__ __forceinline__ void store_dq_row(bf16_t* row, const f32x16 (&dq)[D / 32], int hh,
                                             float scale) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * dt + 8 * i + 4 * hh;
      const uint32_t w0 = (uint32_t)f32_to_bf16(dq[dt][4 * i] * scale) |
                          ((uint32_t)f32_to_bf16(dq[dt][4 * i + 1] * scale) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(dq[dt][4 * i + 2] * scale) |
                          ((uint32_t)f32_to_bf16(dq[dt][4 * i + 3] * scale) << 16);
      *reinterpret_cast<uint2*>(row + d0) = make_uint2(w0, w1);
    }
}

// Routed tiles: same tile list and XCD-aware order as the forward's routed
// kernel (grid = upper bound of the tile count; surplus workgroups exit).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_bwd_dq_routed(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ dvec,
    const uint32_t* __restrict__ list, const uint32_t* __restrict__ bucket_off,
    const uint32_t* __restrict__ tile_off, bf16_t* __restrict__ dqp, int64_t Lq, int64_t L,
    int H, int Hkv, int kp, int B, int nb, int nrows, float sl2, float scale,
    uint32_t nslots) {
  using T = DqTiles<D, NW>;
  constexpr int TM = 32 * NW;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * T::BUF];
  const uint32_t ntiles = tile_off[nrows];
  const uint32_t per = (ntiles + 7) / 8;
  const uint32_t bid = blockIdx.x;
  if (bid / 8 >= per) return;
  const uint32_t tile = (bid % 8) * per + bid / 8;
  if (tile >= ntiles) return;
  int lo = 0, hi = nrows;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= tile) lo = mid; else hi = mid;
  }
  const int row = lo;
  const uint32_t start = (tile - tile_off[row]) * TM;
  const uint32_t avail = bucket_off[row + 1] - bucket_off[row] - start;
  const int cnt = avail < (uint32_t)TM ? (int)avail : TM;
  const int j = row % nb;
  const int sg = row / nb, g = sg % Hkv, s = sg / Hkv;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int e = 32 * w + n;
  const bool wave_on = 32 * w < cnt;
  const uint32_t slot_raw = (e < cnt) ? list[bucket_off[row] + start + e] : 0u;
  const bool valid = e < cnt && slot_raw < nslots;
  const uint32_t slot = valid ? slot_raw : 0u;
  const uint32_t qh = slot / (uint32_t)kp;
  const int64_t r = qh % Lq;
  const int h = (int)((qh / Lq) % H);
  const int64_t qrow = (((int64_t)s * Lq + r) * H + h) * D;
  bf16x8 qf[D / 16], df[D / 16];
  bwd_row_frags<D>(q + qrow, valid, hh, qf);
  bwd_row_frags<D>(dout + qrow, valid, hh, df);
  const float lse2 = valid ? lse[qh] * kLog2e : 0.f;
  const float dv = valid ? dvec[qh] : 0.f;

  const int64_t krs = (int64_t)Hkv * D;
  const bf16_t* ktile = k + ((int64_t)s * L * Hkv + g) * D + (int64_t)j * B * krs;
  const bf16_t* vtile = v + ((int64_t)s * L * Hkv + g) * D + (int64_t)j * B * krs;
  const int nsteps = B / 64;  // a selected past block is always whole
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  DqRegs<D, NW> tr;
  tr.setup((int)krs, tid);
  tr.load(ktile, vtile);
  tr.store(lds);
  __syncthreads();
  for (int it = 0; it < nsteps; ++it) {
    const bool more = it + 1 < nsteps;
    ktile += 64 * krs;
    vtile += 64 * krs;
    if (more) tr.load(ktile, vtile);
    if (wave_on)
      dq_step<D, false>(lds + (it & 1) * T::BUF, qf, df, acc, lane, sl2, lse2, dv, 0, 0, 0);
    if (more) tr.store(lds + ((it + 1) & 1) * T::BUF);
    __syncthreads();
  }
  if (!valid) return;
  store_dq_row<D>(dqp + (int64_t)slot * D, acc, hh, scale);
}

// Own block of every query (keys from the start of its block up to itself)
// plus the sum of its routed dq partials -> dq.  Workgroup: HW heads of one KV
// group x RW = 32*NW/HW query rows; wave w: head h0 + w % HW, rows
// [r0, r0 + 32).  grid (ceil(Lq / RW), S * H / HW).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_bwd_dq_own(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ ktail, const bf16_t* __restrict__ vtail,
    const float* __restrict__ lse, const float* __restrict__ dvec,
    const bf16_t* __restrict__ dqp, bf16_t* __restrict__ dq, int Lq, int L, int q_off,
    int H, int Hkv, int kp, int B, int HW, float sl2, float scale) {
  using T = DqTiles<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * T::BUF];
  const int RW = 32 * NW / HW;
  const int rt = blockIdx.x;
  const int hgroups = H / HW;
  const int s = blockIdx.y / hgroups;
  const int h0 = (blockIdx.y % hgroups) * HW;
  const int g = h0 / (H / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int h = h0 + w % HW;
  const int rw0 = rt * RW;
  const int r0 = rw0 + 32 * (w / HW);
  const int r = r0 + n;
  const bool valid = r < Lq;
  const bool wave_on = r0 < Lq;
  const int pos = q_off + r;
  const int wlast = (r0 + 31 < Lq ? r0 + 31 : Lq - 1);
  const int klo_w = ((q_off + r0) / B) * B;
  const int khi_w = wave_on ? q_off + wlast + 1 : 0;
  const int wglast = (rw0 + RW - 1 < Lq ? rw0 + RW - 1 : Lq - 1);
  const int klo_g = ((q_off + rw0) / B) * B;
  const int khi_g = q_off + wglast + 1;
  const int t0 = klo_g / 64, t1 = (khi_g + 63) / 64;
  const int klo_l = (pos / B) * B;

  const int64_t qh = ((int64_t)s * H + h) * Lq + (valid ? r : 0);
  const int64_t qrow = (((int64_t)s * Lq + (valid ? r : 0)) * H + h) * D;
  bf16x8 qf[D / 16], df[D / 16];
  bwd_row_frags<D>(q + qrow, valid, hh, qf);
  bwd_row_frags<D>(dout + qrow, valid, hh, df);
  const float lse2 = valid ? lse[qh] * kLog2e : 0.f;
  const float dv = valid ? dvec[qh] : 0.f;

  const int64_t krs = (int64_t)Hkv * D;
  const bf16_t* kbase = k + ((int64_t)s * L * Hkv + g) * D;
  const bf16_t* vbase = v + ((int64_t)s * L * Hkv + g) * D;
  // the tile holding the end of a length that is not a multiple of 64 reads
  // K and V from the zero-padded copies (uniform pointer choice)
  const int ttail = (L % 64) ? L / 64 : -1;
  const bf16_t* ktail_sg = ttail >= 0 ? ktail + ((int64_t)s * 64 * Hkv + g) * D : kbase;
  const bf16_t* vtail_sg = ttail >= 0 ? vtail + ((int64_t)s * 64 * Hkv + g) * D : vbase;
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  DqRegs<D, NW> tr;
  tr.setup((int)krs, tid);
  auto load_tile = [&](int ti) {
    const int64_t off = (int64_t)ti * 64 * krs;
    if (ti == ttail) tr.load(ktail_sg, vtail_sg);
    else tr.load(kbase + off, vbase + off);
  };
  load_tile(t0);
  tr.store(lds);
  __syncthreads();
  // phases per wave: idle, full tiles, masked tiles (diagonal), idle
  int ws_ = t1, wd_ = t1, we_ = t1;
  if (wave_on) {
    ws_ = klo_w / 64;
    we_ = (khi_w + 63) / 64;
    const int d_ = (q_off + r0 + 1) / 64;
    wd_ = d_ < ws_ ? ws_ : (d_ > we_ ? we_ : d_);
    // rows in two blocks: every tile takes the per-lane window
    if (((q_off + wlast) / B) * B != klo_w) wd_ = ws_;
    ws_ = ws_ < t0 ? t0 : (ws_ > t1 ? t1 : ws_);
    we_ = we_ < ws_ ? ws_ : (we_ > t1 ? t1 : we_);
    wd_ = wd_ < ws_ ? ws_ : (wd_ > we_ ? we_ : wd_);
  }
  for (int it = t0; it < t1; ++it) {
    const bool more = it + 1 < t1;
    if (more) load_tile(it + 1);
    bf16_t* cur = lds + ((it - t0) & 1) * T::BUF;
    if (it >= ws_ && it < wd_)
      dq_step<D, false>(cur, qf, df, acc, lane, sl2, lse2, dv, 0, 0, 0);
    else if (it >= wd_ && it < we_)
      dq_step<D, true>(cur, qf, df, acc, lane, sl2, lse2, dv, it * 64, klo_l, pos);
    if (more) tr.store(lds + ((it + 1 - t0) & 1) * T::BUF);
    __syncthreads();
  }
  if (!valid) return;
  // dq = c (own part) + the routed partials (already scaled)
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int reg = 0; reg < 16; ++reg) acc[dt][reg] *= scale;
  const int own = pos / B;
  const int npast = kp < own ? kp : own;
  for (int t = 0; t < npast; ++t) {
    const bf16_t* prow = dqp + (qh * kp + t) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 x = *reinterpret_cast<const uint2*>(prow + 32 * dt + 8 * i + 4 * hh);
        acc[dt][4 * i] += __uint_as_float(x.x << 16);
        acc[dt][4 * i + 1] += __uint_as_float(x.x & 0xffff0000u);
        acc[dt][4 * i + 2] += __uint_as_float(x.y << 16);
        acc[dt][4 * i + 3] += __uint_as_float(x.y & 0xffff0000u);
      }
  }
  store_dq_row<D>(dq + qrow, acc, hh, 1.0f);
}

// ============================================== routed entries -> query rows
// For the dk/dv kernel, which reads every routed entry of a bucket once per
// key chunk: per entry e (a slot id ((s*H + h)*Lq + r)*kp + t in routing
// order) the row index (s*Lq + r)*H + h of its Q / dO rows and of rowstat,
// so that the kernel's per-step gather needs no division.  grid
// ceil(slots / 256) (an upper bound of the entry count), 256 threads.
__global__ __launch_bounds__(256) void k_bwd_entry_rows(const uint32_t* __restrict__ list,
                                                        const uint32_t* __restrict__ total,
                                                        uint32_t* __restrict__ ent, int kp,
                                                        int Lq, int H) {
  const uint32_t e = blockIdx.x * 256u + threadIdx.x;
  if (e >= *total) return;
  const uint32_t qhh = list[e] / (uint32_t)kp;      // (s*H + h)*Lq + r
  const uint32_t sh = qhh / (uint32_t)Lq;
  const uint32_t r = qhh - sh * (uint32_t)Lq;
  const uint32_t sq = sh / (uint32_t)H, h = sh - sq * (uint32_t)H;
  ent[e] = (sq * (uint32_t)Lq + r) * (uint32_t)H + h;
}

// ============================================================ dk, dv kernel
// Q and dO tiles of QN = 64 queries, row-major in LDS.  The A operands of
// dV^T += dO^T P and dK^T += Q^T dS (rows d, contraction over queries) are
// read from the same row-major tiles with the LDS transpose read.
template <int D, int NW>
struct KvTiles {
  static constexpr int NT = 64 * NW;
  static constexpr int QN = 64;
  static constexpr int QE = QN * D;
  static constexpr int BUF = 2 * QE;            // Q, dO (bf16 elements)
  static constexpr int CH = D / 8 / NW;         // 16-byte chunks of a row per thread per tensor
};

// Calls f(std::integral_constant<int, K>) for K = B .. E-1 in order (a loop
// whose index is a compile-time constant in the body).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Key-stationary: workgroup (s, g, block j, chunk c, segment) owns keys
// [jB + c*32*NW, +32*NW) of the block (wave w the 32 from +32w) and loops over
// its segment of the block's routed entries, then of its own queries (one
// head at a time, 64 positions per step, causal mask).  With nseg = 1 it
// writes dk, dv; with more segments (small problems, whose few long buckets
// would leave the chip idle) each segment writes fp32 partials
// [nseg][2][S, L, Hkv, D] that k_bwd_reduce_kv adds in segment order.
// grid (S * Hkv * nb * ceil(B / (32 NW)) * nseg), 64*NW threads.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_bwd_dkdv(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float2* __restrict__ rowstat, const uint32_t* __restrict__ ent,
    const uint32_t* __restrict__ bucket_off, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv,
    float* __restrict__ kvpart, int Lq, int L, int q_off, int H, int Hkv, int B, int nb,
    int nchunk, int nseg, float sl2, float scale) {
  using T = KvTiles<D, NW>;
  constexpr int QN = T::QN;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * T::BUF];
  __shared__ __attribute__((aligned(16))) float stat[2][2][QN];  // [buffer][lse2, Dv][query]
  const int KC = 32 * NW;
  const int seg = (int)(blockIdx.x % nseg);
  const int item = (int)(blockIdx.x / nseg);
  const int c = item % nchunk;
  const int row = item / nchunk;          // bucket (s, g, j)
  const int j = row % nb;
  const int sg = row / nb, g = sg % Hkv, s = sg / Hkv;
  const int G = H / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int bstart = j * B;
  const int bend = (j + 1) * B < L ? (j + 1) * B : L;     // keys of the block: [bstart, bend)
  const int kc0 = bstart + c * KC;                         // first key of this workgroup
  const int key = kc0 + 32 * w + n;                        // this lane's key (B operand column)
  const bool key_ok = key < bend;
  const int64_t krs = (int64_t)Hkv * D;

  // the wave's K and V rows as B operands: lane (key n, half hh), k-step t:
  // dims 16 t + 8 hh + [0, 8)
  bf16x8 kb[D / 16], vb[D / 16];
  {
    const int64_t off = ((int64_t)s * L + (key_ok ? key : bstart)) * krs + (int64_t)g * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      kb[t] = ld_bf16x8(k + off + 16 * t + 8 * hh);
      vb[t] = ld_bf16x8(v + off + 16 * t + 8 * hh);
      if (!key_ok) {
        kb[t] = bf16x8{};
        vb[t] = bf16x8{};
      }
    }
  }
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dka[dt] = f32x16{};
    dva[dt] = f32x16{};
  }

  // steps: routed entries (QN per step), then own queries (head by head, QN
  // positions per step starting at the first position that sees a key here)
  const bool routed = bucket_off != nullptr;   // no routing tables: no past blocks
  const int nrt_all = routed ? (int)(bucket_off[row + 1] - bucket_off[row]) : 0;
  const int rlo = (int)((int64_t)nrt_all * seg / nseg);   // this segment's entries
  const int nrt = (int)((int64_t)nrt_all * (seg + 1) / nseg) - rlo;
  const uint32_t rbase = routed ? bucket_off[row] + (uint32_t)rlo : 0u;
  const int rsteps = (nrt + QN - 1) / QN;
  int p0 = kc0 > q_off ? kc0 : q_off;                      // first own query position
  const int pend = bend;                                   // one past the last
  const int npos = pend > p0 ? pend - p0 : 0;
  const int psteps_h = (npos + QN - 1) / QN;
  const int nown_all = G * psteps_h;                       // own steps of all segments
  const int olo = (int)((int64_t)nown_all * seg / nseg);   // this segment's own steps
  const int nsteps = rsteps + (int)((int64_t)nown_all * (seg + 1) / nseg) - olo;

  // Staging, three steps in flight: the row index of the entries of step
  // it+2 (routed steps read it from `ent`), the Q / dO rows and the two
  // statistics of step it+1 (requested at the start of step it), and the
  // LDS tiles of step it.  Lane l finds query l of a step; wave w loads the rows
  // of queries RPW w .. RPW (w + 1) - 1, RPI whole rows per load (CPR lanes
  // per row, the row index passed between lanes), so that a load touches RPI
  // rows rather than 64: the gather's cost is the number of rows a load
  // instruction touches, not its bytes.
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;       // rows per load instruction
  constexpr int RPW = QN / NW;        // rows per wave
  static_assert(RPW == RPI * T::CH, "one load per chunk slot");
  u32x4 qr[T::CH], dr[T::CH];
  int rok[T::CH];                     // the row of load i exists
  bool row_ok = false;               // query `lane` of step it+1 exists
  float2 st_ld = make_float2(0.f, 0.f);   // wave 0: lse2, Dv of query `lane` (step it+1)
  uint32_t ida = 0u;                 // row index of query `lane` of step it+1, then it+2
  // query `lane` of a step: its row index (s*Lq + r)*H + h, or false
  auto query_at = [&](int step, uint32_t id, int64_t& qr_idx) -> bool {
    if (step < rsteps) {
      if (step * QN + lane >= nrt) return false;
      qr_idx = id;
      return true;
    }
    const int st = step - rsteps + olo;
    const int hl = st / psteps_h, pc = st - hl * psteps_h;
    const int p = p0 + pc * QN + lane;
    if (p >= pend) return false;
    qr_idx = ((int64_t)s * Lq + (p - q_off)) * H + g * G + hl;
    return true;
  };
  // The loads below go to valid addresses whatever the query (row 0 and
  // the bucket's last entry stand in for invalid ones) and are not selected
  // on right away: a select on a loaded value would wait for the load there,
  // at the start of the step.  Invalid rows are zeroed when the tiles are
  // stored.
  auto fetch_id = [&](int step) {
    if (step >= rsteps) return;  // own steps need no ids (and rsteps > 0 means nrt > 0)
    const int e = step * QN + lane;
    ida = ent[rbase + (e < nrt ? e : nrt - 1)];   // entries past nrt: query_at rejects them
  };
  auto fetch_rows = [&](int step) {
    int64_t qr_idx = 0;
    row_ok = query_at(step, ida, qr_idx);
    if (!row_ok) qr_idx = 0;
    // row index < S*Lq*H, which is below 2^32 for any input that fits in
    // device memory
    const int myrow = (int)(uint32_t)qr_idx;
    const int myok = row_ok ? 1 : 0;
#pragma unroll
    for (int i = 0; i < T::CH; ++i) {
      const int src = RPW * w + RPI * i + lane / CPR;   // query of this lane's row
      const uint32_t ri = (uint32_t)__shfl(myrow, src);
      rok[i] = __shfl(myok, src);
      const int64_t off = (int64_t)ri * D + 8 * (lane % CPR);
      qr[i] = *reinterpret_cast<const u32x4*>(q + off);
      dr[i] = *reinterpret_cast<const u32x4*>(dout + off);
    }
    if (w == 0) st_ld = rowstat[qr_idx];
  };
  auto stage_chunk = [&](int buf, int i) {
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    const int o = kv_off<D>(RPW * w + RPI * i + lane / CPR, lane % CPR);
    *reinterpret_cast<u32x4*>(lds + buf * T::BUF + o) = rok[i] ? qr[i] : z;
    *reinterpret_cast<u32x4*>(lds + buf * T::BUF + T::QE + o) = rok[i] ? dr[i] : z;
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < T::CH; ++i) stage_chunk(buf, i);
  };
  // an invalid query gets lse2 = +inf, hence p = 0 (its rows are zero too)
  auto stage_stats = [&](int buf) {
    if (w == 0) {
      stat[buf][0][lane] = row_ok ? st_ld.x : __builtin_inff();
      stat[buf][1][lane] = row_ok ? st_ld.y : 0.f;
    }
  };

  // prologue: tiles of step 0, id of step 1
  if (nsteps > 0) {
    fetch_id(0);
    fetch_rows(0);
    stage_store(0);
    stage_stats(0);
    if (nsteps > 1) fetch_id(1);
  }
  __syncthreads();
  // One step is a fixed sequence of 4 NS MFMA slots (NS = D / 8), each with
  // its A fragment read from LDS kPre slots ahead:
  //   phase 0  S and dP of queries 0-31 (t = slot / 2; S on even slots)
  //   phase 1  S and dP of queries 32-63, with the softmax of queries 0-31
  //   phase 2  dV^T and dK^T over queries 0-31 (transpose reads), with the
  //            softmax of queries 32-63
  //   phase 3  dV^T and dK^T over queries 32-63, with the stores of the next
  //            step's tiles in its last slots
  // One wave runs per SIMD, so the softmax arithmetic and the LDS traffic
  // have to issue between the MFMAs of the same wave; scheduling barriers
  // keep each slot's instructions in place.  The products and their
  // accumulation order are those of the plain loop nest (dV^T / dK^T over
  // query groups 0..3 in order).
  constexpr int NS = D / 8;          // slots per phase
  constexpr int EPS = 16 / NS;       // softmax elements per slot
  constexpr int GS = 4 / EPS;        // slots per group of four elements
  constexpr int kPre = 6;
  const int arow = kperm(n);
  auto frag = [&](const bf16_t* b, int k) -> bf16x8 {
    if (k < 2 * NS) {
      const int qb = k / NS, t = (k % NS) >> 1, tensor = k & 1;
      return ld_bf16x8(b + tensor * T::QE + kv_off<D>(32 * qb + arow, 2 * t + hh));
    }
    const int qb = (k - 2 * NS) / NS, idx = (k - 2 * NS) % NS;
    const int dt = idx >> 2, c = (idx >> 1) & 1, tensor = idx & 1;   // 0: dO^T, 1: Q^T
    return tr_frag<D>(b + (tensor ? 0 : T::QE), dt, 2 * qb + c, lane);
  };
  // P and dS: register reg of a half's S / dP accumulator (lane half hh)
  // holds query 32 qb + acc_key(reg, hh); registers [8c, 8c + 8) are the
  // queries 32 qb + 16 c + 8 hh + [0, 8) in order, the B operand layout of P
  // and dS for the products over queries.  Queries at positions before the
  // key (own steps) get p = 0.
  auto soft = [&](int qb, int reg, bool mask, int pos0, float s, float dp, const f32x4& l4,
                  const f32x4& d4, bf16x8 (&pb)[2], bf16x8 (&dsb)[2]) {
    const int jj = reg & 3;
    const int qi = 32 * qb + acc_key(reg, hh);
    float p = __builtin_amdgcn_exp2f(fmaf(s, sl2, -l4[jj]));
    if (mask && pos0 + qi < key) p = 0.f;
    const float ds = p * (dp - d4[jj]);
    pb[reg >> 3][reg & 7] = static_cast<__bf16>(p);
    dsb[reg >> 3][reg & 7] = static_cast<__bf16>(ds);
  };

  f32x16 s0, d0, s1, d1;   // S and dP of the two query halves of a step
  // step `it`; MASK (own steps): the causal mask inside the block
  auto step = [&](int it, auto maskc) {
    constexpr bool MASK = decltype(maskc)::value;
    const int CB = it & 1;
    const bf16_t* b = lds + CB * T::BUF;
    const float* st = &stat[CB][0][0];
    int pos0 = 0;   // position of the step's first query (own steps)
    if constexpr (MASK) {
      const int sidx = it - rsteps + olo;
      pos0 = p0 + (sidx - (sidx / psteps_h) * psteps_h) * QN;
    }
    // the next step's rows (and the id of the one after) are requested
    // first; they are stored to the other buffer in the last slots
    if (it + 1 < nsteps) {
      fetch_rows(it + 1);
      if (it + 2 < nsteps) fetch_id(it + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    s0 = f32x16{}; d0 = f32x16{}; s1 = f32x16{}; d1 = f32x16{};
    bf16x8 pb0[2], dsb0[2], pb1[2], dsb1[2];
    f32x4 l4[2] = {f32x4{}, f32x4{}}, d4[2] = {f32x4{}, f32x4{}};
    bf16x8 fr[4 * NS];
    static_for<0, kPre>([&](auto kc) { fr[kc.value] = frag(b, kc.value); });
    static_for<0, 4 * NS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int ph = k / NS, ks = k % NS;
      // statistics of the four queries of softmax element group g (elements
      // 4g..4g+3 of the two halves' 32): read GS slots before their first
      // use (slot NS + g GS), after the last use of group g - 2 (the same
      // registers)
      if constexpr (k >= NS - GS && k < NS + 7 * GS && (k - NS + GS) % GS == 0) {
        constexpr int g = (k - NS + GS) / GS;
        const int qi0 = 32 * (g >> 2) + acc_key(4 * (g & 3), hh);
        l4[g & 1] = *reinterpret_cast<const f32x4*>(st + qi0);
        d4[g & 1] = *reinterpret_cast<const f32x4*>(st + QN + qi0);
      }
      if constexpr (ph == 0) {
        constexpr int t = ks >> 1;
        if constexpr (k & 1) d0 = mfma32(fr[k], vb[t], d0);
        else s0 = mfma32(fr[k], kb[t], s0);
      } else if constexpr (ph == 1) {
        constexpr int t = ks >> 1;
        if constexpr (k & 1) d1 = mfma32(fr[k], vb[t], d1);
        else s1 = mfma32(fr[k], kb[t], s1);
        static_for<0, EPS>([&](auto ec) {
          constexpr int reg = ks * EPS + decltype(ec)::value, g = reg >> 2;
          soft(0, reg, MASK, pos0, s0[reg], d0[reg], l4[g & 1], d4[g & 1], pb0, dsb0);
        });
      } else if constexpr (ph == 2) {
        constexpr int dt = ks >> 2, c = (ks >> 1) & 1;
        if constexpr (ks & 1) dka[dt] = mfma32(fr[k], dsb0[c], dka[dt]);
        else dva[dt] = mfma32(fr[k], pb0[c], dva[dt]);
        static_for<0, EPS>([&](auto ec) {
          constexpr int reg = ks * EPS + decltype(ec)::value, g = 4 + (reg >> 2);
          soft(1, reg, MASK, pos0, s1[reg], d1[reg], l4[g & 1], d4[g & 1], pb1, dsb1);
        });
      } else {
        constexpr int dt = ks >> 2, c = (ks >> 1) & 1;
        if constexpr (ks & 1) dka[dt] = mfma32(fr[k], dsb1[c], dka[dt]);
        else dva[dt] = mfma32(fr[k], pb1[c], dva[dt]);
        if constexpr (ks >= NS - 8) {
          constexpr int i = ks - (NS - 8);   // tile chunk stores of the next step
          if constexpr (i < T::CH) stage_chunk(CB ^ 1, i);
        }
      }
      if constexpr (k + kPre < 4 * NS) fr[k + kPre] = frag(b, k + kPre);
      __builtin_amdgcn_sched_barrier(0);
    });
    stage_stats(CB ^ 1);
    // every accumulator stays in the same accumulation registers across
    // steps: without this the register allocator rotates some of them
    // through other registers at the loop edge (~100 moves per step)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) asm volatile("" : "+a"(dka[dt]), "+a"(dva[dt]));
    asm volatile("" : "+a"(s0), "+a"(d0), "+a"(s1), "+a"(d1));
    __syncthreads();
  };
  // routed steps first (no mask), then the own steps
  for (int it = 0; it < rsteps; ++it) step(it, std::false_type{});
  for (int it = rsteps; it < nsteps; ++it) step(it, std::true_type{});
  if (!key_ok) return;
  // dK^T / dV^T accumulators: lane = key, register 4i + jj = dim
  // 32 dt + 8 i + 4 hh + jj
  const int64_t orow = ((int64_t)s * L + key) * krs + (int64_t)g * D;
  if (nseg > 1) {
    // one plane holds S*L*Hkv*D floats; gridDim.x = S*Hkv*nb*nchunk*nseg
    const int64_t nseq = (int64_t)gridDim.x / ((int64_t)nseg * nchunk * nb * Hkv);
    const int64_t plane = nseq * L * krs;
    float* pk = kvpart + (int64_t)(2 * seg) * plane + orow;
    float* pv = pk + plane;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 32 * dt + 8 * i + 4 * hh;
        *reinterpret_cast<f32x4*>(pk + d0) =
            f32x4{dka[dt][4 * i] * scale, dka[dt][4 * i + 1] * scale,
                  dka[dt][4 * i + 2] * scale, dka[dt][4 * i + 3] * scale};
        *reinterpret_cast<f32x4*>(pv + d0) =
            f32x4{dva[dt][4 * i], dva[dt][4 * i + 1], dva[dt][4 * i + 2], dva[dt][4 * i + 3]};
      }
    return;
  }
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * dt + 8 * i + 4 * hh;
      const uint32_t k0 = (uint32_t)f32_to_bf16(dka[dt][4 * i] * scale) |
                          ((uint32_t)f32_to_bf16(dka[dt][4 * i + 1] * scale) << 16);
      const uint32_t k1 = (uint32_t)f32_to_bf16(dka[dt][4 * i + 2] * scale) |
                          ((uint32_t)f32_to_bf16(dka[dt][4 * i + 3] * scale) << 16);
      const uint32_t v0 = (uint32_t)f32_to_bf16(dva[dt][4 * i]) |
                          ((uint32_t)f32_to_bf16(dva[dt][4 * i + 1]) << 16);
      const uint32_t v1 = (uint32_t)f32_to_bf16(dva[dt][4 * i + 2]) |
                          ((uint32_t)f32_to_bf16(dva[dt][4 * i + 3]) << 16);
      *reinterpret_cast<uint2*>(dk + orow + d0) = make_uint2(k0, k1);
      *reinterpret_cast<uint2*>(dv + orow + d0) = make_uint2(v0, v1);
    }
}

// Sum of the dk / dv segment partials in segment order (deterministic) ->
// bf16.  n = S*L*Hkv*D elements per plane, 4 per thread.
__global__ __launch_bounds__(256) void k_bwd_reduce_kv(const float* __restrict__ part,
                                                       bf16_t* __restrict__ dk,
                                                       bf16_t* __restrict__ dv, int64_t n,
                                                       int nseg) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sgi = 0; sgi < nseg; ++sgi) {
    ak += *reinterpret_cast<const f32x4*>(part + (int64_t)(2 * sgi) * n + i);
    av += *reinterpret_cast<const f32x4*>(part + (int64_t)(2 * sgi + 1) * n + i);
  }
  const uint32_t k0 = (uint32_t)f32_to_bf16(ak[0]) | ((uint32_t)f32_to_bf16(ak[1]) << 16);
  const uint32_t k1 = (uint32_t)f32_to_bf16(ak[2]) | ((uint32_t)f32_to_bf16(ak[3]) << 16);
  const uint32_t v0 = (uint32_t)f32_to_bf16(av[0]) | ((uint32_t)f32_to_bf16(av[1]) << 16);
  const uint32_t v1 = (uint32_t)f32_to_bf16(av[2]) | ((uint32_t)f32_to_bf16(av[3]) << 16);
  *reinterpret_cast<uint2*>(dk + i) = make_uint2(k0, k1);
  *reinterpret_cast<uint2*>(dv + i) = make_uint2(v0, v1);
}

// ================================================================ launchers
static int gcd_i(int a, int b) {
  while (b) { const int t = a % b; a = b; b = t; }
  return a;
}

hipError_t launch_bwd_dot(const void* out, const void* dout, const float* lse, float* dvec,
                          void* rowstat, const Dims& d, hipStream_t st) {
  const int64_t nrows = (int64_t)d.S * d.Lq * d.H;
  const int rpb = 256 / (d.D / 8);
  const unsigned grid = (unsigned)((nrows + rpb - 1) / rpb);
  if (d.D == 128)
    hipLaunchKernelGGL(k_bwd_dot<128>, dim3(grid), dim3(256), 0, st,
                       static_cast<const bf16_t*>(out), static_cast<const bf16_t*>(dout), lse,
                       dvec, static_cast<float2*>(rowstat), nrows, d.Lq, d.H);
  else
    hipLaunchKernelGGL(k_bwd_dot<64>, dim3(grid), dim3(256), 0, st,
                       static_cast<const bf16_t*>(out), static_cast<const bf16_t*>(dout), lse,
                       dvec, static_cast<float2*>(rowstat), nrows, d.Lq, d.H);
  return hipGetLastError();
}

hipError_t launch_bwd_tail(const void* k, const void* v, void* ktail, void* vtail, const Dims& d,
                          hipStream_t st) {
  if (d.L % 64 == 0) return hipSuccess;
  if (ktail == nullptr || vtail == nullptr) return hipErrorInvalidValue;
  const dim3 grid(d.Hkv, d.S);
#define MOBA_BT(DV)                                                                          \
  hipLaunchKernelGGL(k_bwd_tail<DV>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(k), \
                     static_cast<const bf16_t*>(v), static_cast<bf16_t*>(ktail),            \
                     static_cast<bf16_t*>(vtail), d.Hkv, d.L)
  if (d.D == 128) MOBA_BT(128); else MOBA_BT(64);
#undef MOBA_BT
  return hipGetLastError();
}

hipError_t launch_bwd_dq_routed(const void* q, const void* dout, const void* k, const void* v,
                                const float* lse, const float* dvec,
                                const uint32_t* list, const uint32_t* bucket_off,
                                const uint32_t* tile_off, void* dqp, const Dims& d,
                                hipStream_t st) {
  const int64_t grid = routed_tile_bound(d);
  const float sl2 = kLog2e / sqrtf((float)d.D);
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_BQR(DV, NWV)                                                                      \
  hipLaunchKernelGGL((k_bwd_dq_routed<DV, NWV>), dim3((unsigned)grid), dim3(64 * NWV), 0, st,  \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(dout),          \
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),             \
                     lse, dvec, list, bucket_off, tile_off,                                    \
                     static_cast<bf16_t*>(dqp), d.Lq, d.L, d.H, d.Hkv, d.kp, d.B, d.nb,        \
                     d.nrows, sl2, scale, (uint32_t)d.slots)
  // eight-wave tiles of 256 routed entries only (the four-wave form does not
  // fit two waves per SIMD)
  if (d.tile_m != 256) return hipErrorInvalidValue;
  if (d.D == 128) MOBA_BQR(128, 8); else MOBA_BQR(64, 8);
#undef MOBA_BQR
  return hipGetLastError();
}

hipError_t launch_bwd_dq_own(const void* q, const void* dout, const void* k, const void* v,
                             const void* ktail, const void* vtail,
                             const float* lse, const float* dvec, const void* dqp, void* dq,
                             const Dims& d, hipStream_t st) {
  if (d.L % 64 != 0 && (ktail == nullptr || vtail == nullptr)) return hipErrorInvalidValue;
  const int HW = gcd_i(d.G, 4);
  // eight-wave workgroups (two waves per SIMD) unless that leaves fewer than
  // two workgroups per CU; four-wave ones then (one wave per SIMD, more
  // workgroups)
  const int64_t hg = (int64_t)d.S * d.H / HW;
  const int NW = ((d.Lq + 256 / HW - 1) / (256 / HW)) * hg >= 512 ? 8 : 4;
  const int RW = 32 * NW / HW;
  const dim3 grid((unsigned)((d.Lq + RW - 1) / RW), (unsigned)hg);
  const float sl2 = kLog2e / sqrtf((float)d.D);
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_BQO(DV, NWV)                                                                       \
  hipLaunchKernelGGL((k_bwd_dq_own<DV, NWV>), grid, dim3(64 * NWV), 0, st,                      \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(dout),           \
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),              \
                     static_cast<const bf16_t*>(ktail), static_cast<const bf16_t*>(vtail),      \
                     lse, dvec, static_cast<const bf16_t*>(dqp), static_cast<bf16_t*>(dq),      \
                     (int)d.Lq, (int)d.L, (int)d.q_off, d.H, d.Hkv, d.kp, d.B, HW, sl2, scale)
  if (NW == 8) {
    if (d.D == 128) MOBA_BQO(128, 8); else MOBA_BQO(64, 8);
  } else {
    if (d.D == 128) MOBA_BQO(128, 4); else MOBA_BQO(64, 4);
  }
#undef MOBA_BQO
  return hipGetLastError();
}

hipError_t launch_bwd_entry_rows(const uint32_t* list, const uint32_t* bucket_off, void* ent,
                                const Dims& d, hipStream_t st) {
  if (d.slots <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_entry_rows, dim3((unsigned)((d.slots + 255) / 256)), dim3(256), 0, st,
                     list, bucket_off + d.nrows, static_cast<uint32_t*>(ent), d.kp, (int)d.Lq, d.H);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* dout, const void* k, const void* v,
                           const void* rowstat, const void* ent,
                           const uint32_t* bucket_off, void* dk, void* dv, float* kvpart,
                           const Dims& d, hipStream_t st) {
  const int NWv = bwd_dkdv_waves(d);
  const int KC = 32 * NWv;
  const int nchunk = (d.B + KC - 1) / KC;
  const int nseg = bwd_dkdv_segments(d);
  if (nseg > 1 && kvpart == nullptr) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)d.S * d.Hkv * d.nb * nchunk * nseg;
  const float sl2 = kLog2e / sqrtf((float)d.D);
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_BKV(DV, NWV)                                                                       \
  hipLaunchKernelGGL((k_bwd_dkdv<DV, NWV>), dim3((unsigned)grid), dim3(64 * NWV), 0, st, \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(dout),           \
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),              \
                     static_cast<const float2*>(rowstat), static_cast<const uint32_t*>(ent),    \
                     bucket_off, static_cast<bf16_t*>(dk),                                      \
                     static_cast<bf16_t*>(dv), kvpart, (int)d.Lq, (int)d.L, (int)d.q_off, d.H,  \
                     d.Hkv, d.B, d.nb, nchunk, nseg, sl2, scale)
  if (NWv == 4) {
    if (d.D == 128) MOBA_BKV(128, 4); else MOBA_BKV(64, 4);
  } else {
    if (d.D == 128) MOBA_BKV(128, 2); else MOBA_BKV(64, 2);
  }
#undef MOBA_BKV
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nseg == 1) return e;
  const int64_t n = (int64_t)d.S * d.L * d.Hkv * d.D;   // a multiple of 4 (D is)
  hipLaunchKernelGGL(k_bwd_reduce_kv, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st,
                     kvpart, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), n, nseg);
  return hipGetLastError();
}

}  // namespace moba
