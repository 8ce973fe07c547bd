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
//   k_bwd_dot        Dv per query-head.
//   k_bwd_transform  K^T [S, Hkv, D, Lv] (zero past L) and, for a length that
//                    is not a multiple of 64, the last K and V tiles [S, 64,
//                    Hkv, D] zero padded (so that no tile load passes the end).
//   k_bwd_dq_routed  per routed tile (the forward's tile list): S^T = K Q^T
//                    and dP^T = V dO^T on MFMA, dS^T in registers, then
//                    dQ^T += K^T dS^T; one bf16 dq partial per routed slot.
//   k_bwd_dq_own     per query: the own block (causal mask) the same way, plus
//                    the query's routed dq partials -> dq.
//   k_bwd_dkdv       per 32 * NW keys of one block (key-stationary, no
//                    atomics): loops over the block's routed entries and its
//                    own queries 32 at a time; S = Q K^T and dP = dO V^T with
//                    the wave's K and V rows as register B operands, then
//                    dV^T += dO^T P and dK^T += Q^T dS from transposed Q / dO
//                    tiles in LDS.
// Queries are loaded into the MFMA A rows in the kperm order (common.h), so
// the accumulator of a product over 32 queries is directly the B operand of
// the following product over those queries.
#include "common.h"
#include "kernels.h"

namespace moba {

// ------------------------------------------------------------ Dv = dO . o
// One row per LPR = D/8 lanes (16 bytes of o and dO each); the row index is
// in memory order (s, r, h) and Dv is written in query-head order.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dot(const bf16_t* __restrict__ o,
                                                 const bf16_t* __restrict__ dout,
                                                 float* __restrict__ dvec, int64_t nrows,
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
    dvec[(s * H + h) * Lq + r] = acc;
  }
}

// --------------------------------------------------- K^T and the last tiles
// grid (Lv / 64, Hkv, S), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_transform(const bf16_t* __restrict__ k,
                                                       const bf16_t* __restrict__ v,
                                                       bf16_t* __restrict__ kt,
                                                       bf16_t* __restrict__ ktail,
                                                       bf16_t* __restrict__ vtail, int Hkv,
                                                       int64_t L, int64_t Lv) {
  constexpr int LD = D + 8, CPR = D / 8;
  __shared__ bf16_t tile[64 * LD];
  const int g = blockIdx.y, s = blockIdx.z;
  const int64_t key0 = (int64_t)blockIdx.x * 64;
  const int64_t nkey = L - key0;  // >= 1
  for (int c = threadIdx.x; c < 64 * CPR; c += 256) {
    const int row = c / CPR, cc = c % CPR;
    const int64_t src = (((int64_t)s * L + key0 + row) * Hkv + g) * D + cc * 8;
    u32x4 kv = u32x4{0u, 0u, 0u, 0u};
    if (row < nkey) kv = *reinterpret_cast<const u32x4*>(k + src);
    *reinterpret_cast<u32x4*>(&tile[row * LD + cc * 8]) = kv;
    if (nkey < 64) {
      const int64_t dst = (((int64_t)s * 64 + row) * Hkv + g) * D + cc * 8;
      u32x4 vv = u32x4{0u, 0u, 0u, 0u};
      if (row < nkey) vv = *reinterpret_cast<const u32x4*>(v + src);
      *reinterpret_cast<u32x4*>(ktail + dst) = kv;
      *reinterpret_cast<u32x4*>(vtail + dst) = vv;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D * 8; c += 256) {
    const int dd = c / 8, kc = c % 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[(kc * 8 + 2 * e) * LD + dd];
      const uint32_t hi = tile[(kc * 8 + 2 * e + 1) * LD + dd];
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(kt + (((int64_t)s * Hkv + g) * D + dd) * Lv + key0 + kc * 8) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Unsigned 32-bit division by a divisor fixed for the launch, with a multiply
// and shifts (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994: the round-up multiplier of ceil(log2 d) + 32 bits).
struct FastDiv {
  uint32_t d, m, s1, s2;
};

static FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv& f) {
  const uint32_t t = __umulhi(f.m, x);
  return (t + ((x - t) >> f.s1)) >> f.s2;
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
template <int D, int NW>
struct DqTiles {
  static constexpr int NT = 64 * NW;
  static constexpr int KS = D + 8;              // K and V tile row stride
  static constexpr int TS = 64 + 8;             // K^T tile row stride
  static constexpr int KE = 64 * KS;
  static constexpr int BUF = 2 * KE + D * TS;   // K [64][KS], V [64][KS], K^T [D][TS]
  static constexpr int RCH = 64 * (D / 8) / NT;  // 16-byte chunks per thread of K (and V)
  static constexpr int TCH = D * 8 / NT;         // of K^T
};

// Global -> register staging of one 64-key tile of K, V (row-major, row
// stride Hkv*D) and K^T (row stride Lv); fixed per-thread offsets.
template <int D, int NW>
struct DqRegs {
  using T = DqTiles<D, NW>;
  u32x4 kr[T::RCH], vr[T::RCH], tr[T::TCH];
  int roff[T::RCH], rls[T::RCH], toff[T::TCH], tls[T::TCH];
  __device__ __forceinline__ void setup(int krow_stride, int Lv, int tid) {
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) {
      const int c = tid + T::NT * i;
      const int row = c / (D / 8), cc = c % (D / 8);
      roff[i] = row * krow_stride + cc * 8;
      rls[i] = row * T::KS + cc * 8;
    }
#pragma unroll
    for (int i = 0; i < T::TCH; ++i) {
      const int c = tid + T::NT * i;
      const int dd = c / 8, kc = c % 8;
      toff[i] = dd * Lv + kc * 8;
      tls[i] = 2 * T::KE + dd * T::TS + kc * 8;
    }
  }
  __device__ __forceinline__ void load(const bf16_t* kt, const bf16_t* vt, const bf16_t* ktt) {
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) kr[i] = *reinterpret_cast<const u32x4*>(kt + roff[i]);
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) vr[i] = *reinterpret_cast<const u32x4*>(vt + roff[i]);
#pragma unroll
    for (int i = 0; i < T::TCH; ++i) tr[i] = *reinterpret_cast<const u32x4*>(ktt + toff[i]);
  }
  __device__ __forceinline__ void store(bf16_t* buf) const {
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) *reinterpret_cast<u32x4*>(buf + rls[i]) = kr[i];
#pragma unroll
    for (int i = 0; i < T::RCH; ++i) *reinterpret_cast<u32x4*>(buf + T::KE + rls[i]) = vr[i];
#pragma unroll
    for (int i = 0; i < T::TCH; ++i) *reinterpret_cast<u32x4*>(buf + tls[i]) = tr[i];
  }
};

// One 64-key step of one wave (32 queries, lane n = query).  MASK: drop keys
// outside [klo, qpos].
template <int D, bool MASK>
__device__ __forceinline__ void dq_step(const bf16_t* buf, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&df)[D / 16], f32x16 (&dq)[D / 32],
                                        int n, int hh, float sl2, float lse2, float dv,
                                        int key0, int klo, int qpos) {
  using T = DqTiles<D, 4>;
  f32x16 s[2] = {f32x16{}, f32x16{}};
  f32x16 dp[2] = {f32x16{}, f32x16{}};
  {
    const bf16_t* r0 = buf + kperm(n) * T::KS + 8 * hh;
    const bf16_t* r1 = r0 + 32 * T::KS;
    bf16x8 a0[D / 16], a1[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) a0[t] = ld_bf16x8(r0 + 16 * t);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) a1[t] = ld_bf16x8(r1 + 16 * t);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      s[0] = mfma32(a0[t], qf[t], s[0]);
      s[1] = mfma32(a1[t], qf[t], s[1]);
    }
  }
  {
    const bf16_t* r0 = buf + T::KE + kperm(n) * T::KS + 8 * hh;
    const bf16_t* r1 = r0 + 32 * T::KS;
    bf16x8 a0[D / 16], a1[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) a0[t] = ld_bf16x8(r0 + 16 * t);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) a1[t] = ld_bf16x8(r1 + 16 * t);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      dp[0] = mfma32(a0[t], df[t], dp[0]);
      dp[1] = mfma32(a1[t], df[t], dp[1]);
    }
  }
  // dS^T = P^T (dP^T - Dv), P^T = 2^(S^T sl2 - lse2); registers [8c, 8c+8) of
  // subtile kt hold keys 32 kt + 16 c + 8 hh + [0, 8): the B operand layout.
  bf16x8 dsb[2][2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int reg = 8 * c + r;
        float p = __builtin_amdgcn_exp2f(fmaf(s[kt][reg], sl2, -lse2));
        if (MASK) {
          const int key = key0 + 32 * kt + acc_key(reg, hh);
          if (key > qpos || key < klo) p = 0.f;
        }
        dsb[kt][c][r] = static_cast<__bf16>(p * (dp[kt][reg] - dv));
      }
  // dQ^T += K^T dS^T
  const bf16_t* tbase = buf + 2 * T::KE + 8 * hh + n * T::TS;
  bf16x8 ta[D / 32][4];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) ta[dt][kc] = ld_bf16x8(tbase + 32 * dt * T::TS + 16 * kc);
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) dq[dt] = mfma32(ta[dt][kc], dsb[kc >> 1][kc & 1], dq[dt]);
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
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ kt,
    const float* __restrict__ lse, const float* __restrict__ dvec,
    const uint32_t* __restrict__ list, const uint32_t* __restrict__ bucket_off,
    const uint32_t* __restrict__ tile_off, bf16_t* __restrict__ dqp, int64_t Lq, int64_t L,
    int64_t Lv, int H, int Hkv, int kp, int B, int nb, int nrows, float sl2, float scale,
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
  const bf16_t* tt = kt + ((int64_t)s * Hkv + g) * D * Lv + (int64_t)j * B;
  const int nsteps = B / 64;  // a selected past block is always whole
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  DqRegs<D, NW> tr;
  tr.setup((int)krs, (int)Lv, tid);
  tr.load(ktile, vtile, tt);
  tr.store(lds);
  __syncthreads();
  for (int it = 0; it < nsteps; ++it) {
    const bool more = it + 1 < nsteps;
    ktile += 64 * krs;
    vtile += 64 * krs;
    tt += 64;
    if (more) tr.load(ktile, vtile, tt);
    if (wave_on)
      dq_step<D, false>(lds + (it & 1) * T::BUF, qf, df, acc, n, hh, sl2, lse2, dv, 0, 0, 0);
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
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_bwd_dq_own(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const bf16_t* __restrict__ kt,
    const bf16_t* __restrict__ ktail, const bf16_t* __restrict__ vtail,
    const float* __restrict__ lse, const float* __restrict__ dvec,
    const bf16_t* __restrict__ dqp, bf16_t* __restrict__ dq, int Lq, int L, int Lv, int q_off,
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
  const bf16_t* tbase = kt + ((int64_t)s * Hkv + g) * D * Lv;
  // the tile holding the end of a length that is not a multiple of 64 reads
  // K and V from the zero-padded copies (uniform pointer choice)
  const int ttail = (L % 64) ? L / 64 : -1;
  const bf16_t* ktail_sg = ttail >= 0 ? ktail + ((int64_t)s * 64 * Hkv + g) * D : kbase;
  const bf16_t* vtail_sg = ttail >= 0 ? vtail + ((int64_t)s * 64 * Hkv + g) * D : vbase;
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  DqRegs<D, NW> tr;
  tr.setup((int)krs, Lv, tid);
  auto load_tile = [&](int ti) {
    const int64_t off = (int64_t)ti * 64 * krs;
    if (ti == ttail) tr.load(ktail_sg, vtail_sg, tbase + (int64_t)ti * 64);
    else tr.load(kbase + off, vbase + off, tbase + (int64_t)ti * 64);
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
      dq_step<D, false>(cur, qf, df, acc, n, hh, sl2, lse2, dv, 0, 0, 0);
    else if (it >= wd_ && it < we_)
      dq_step<D, true>(cur, qf, df, acc, n, hh, sl2, lse2, dv, it * 64, klo_l, pos);
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

// ============================================================ dk, dv kernel
// QN = 32 NQ queries per step.
template <int D, int NW, int NQ>
struct KvTiles {
  static constexpr int NT = 64 * NW;
  static constexpr int QN = 32 * NQ;
  static constexpr int QS = D + 8;              // Q / dO tile row stride (QN rows)
  static constexpr int TS = QN + 8;             // Q^T / dO^T tile row stride (D rows)
  static constexpr int QE = QN * QS;
  static constexpr int TE = D * TS;
  static constexpr int BUF = 2 * QE + 2 * TE;   // Q, dO, Q^T, dO^T (bf16 elements)
  static constexpr int CH = QN * (D / 8) / NT;  // 16-byte chunks per thread per tensor
};

// Key-stationary: workgroup (s, g, block j, chunk c, segment) owns keys
// [jB + c*32*NW, +32*NW) of the block (wave w the 32 from +32w) and loops over
// its segment of the block's routed entries, then of its own queries (one
// head at a time, QN positions per step, causal mask), QN = 32 NQ queries per
// step.  With nseg = 1 it writes dk, dv; with more segments (small problems,
// whose few long buckets would leave the chip idle) each segment writes fp32
// partials [nseg][2][S, L, Hkv, D] that k_bwd_reduce_kv adds in segment order.
// grid (S * Hkv * nb * ceil(B / (32 NW)) * nseg), 64*NW threads.
template <int D, int NW, int NQ>
__global__ __launch_bounds__(64 * NW, 1) void k_bwd_dkdv(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, const float* __restrict__ lse,
    const float* __restrict__ dvec, const uint32_t* __restrict__ list,
    const uint32_t* __restrict__ bucket_off, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv,
    float* __restrict__ kvpart, int Lq, int L, int q_off, int H, int Hkv, int kp, int B, int nb,
    int nchunk, int nseg, FastDiv fd_kp, FastDiv fd_lq, float sl2, float scale) {
  using T = KvTiles<D, NW, NQ>;
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

  // Staging, three steps in flight: the entry ids of step it+2 (routed steps
  // read them from the list), the Q / dO rows and the two statistics of step
  // it+1 (requested once step it's first products are issued), and the LDS
  // tiles of step it.
  // Thread chunk i covers query qi = (tid + NT i) % QN, dims cc*8.. with
  // cc = (tid + NT i) / QN: the lanes of a transposed store then write
  // different queries of one row.
  u32x4 qr[T::CH], dr[T::CH];
  float st_l = 0.f, st_d = 0.f;      // threads < QN: lse2, Dv of query tid (step it+1)
  uint32_t ida[T::CH];               // entry ids of step it+1, then it+2
  uint32_t sida = 0u;                // threads < QN: the id of query tid
  // query (row offset, query-head index) of query qi of a step, or false
  auto query_at = [&](int step, int qi, uint32_t id, int64_t& qrow, int64_t& qhi) -> bool {
    int r, h;
    if (step < rsteps) {
      if (step * QN + qi >= nrt) return false;
      const uint32_t qhh = fdiv(id, fd_kp);             // (s*H + h)*Lq + r
      const uint32_t sh = fdiv(qhh, fd_lq);             // s*H + h
      r = (int)(qhh - sh * fd_lq.d);
      h = (int)(sh - (uint32_t)s * H);
      if (r < 0 || r >= Lq || h < 0 || h >= H) return false;  // never for a routed slot
    } else {
      const int st = step - rsteps + olo;
      const int hl = st / psteps_h, pc = st - hl * psteps_h;
      const int p = p0 + pc * QN + qi;
      if (p >= pend) return false;
      r = p - q_off;
      h = g * G + hl;
    }
    qrow = (((int64_t)s * Lq + r) * H + h) * D;
    qhi = ((int64_t)s * H + h) * Lq + r;
    return true;
  };
  auto fetch_ids = [&](int step) {
    if (step >= rsteps) return;  // own steps need no ids
#pragma unroll
    for (int i = 0; i < T::CH; ++i) {
      const int e = step * QN + (tid + T::NT * i) % QN;
      ida[i] = e < nrt ? list[rbase + e] : 0u;
    }
    if (tid < QN) {
      const int e = step * QN + tid;
      sida = e < nrt ? list[rbase + e] : 0u;
    }
  };
  auto fetch_rows = [&](int step) {
#pragma unroll
    for (int i = 0; i < T::CH; ++i) {
      const int cidx = tid + T::NT * i;
      const int qi = cidx % QN, cc = cidx / QN;
      int64_t qrow = 0, qhi = 0;
      const bool ok = query_at(step, qi, ida[i], qrow, qhi);
      qr[i] = ok ? *reinterpret_cast<const u32x4*>(q + qrow + cc * 8) : u32x4{0u, 0u, 0u, 0u};
      dr[i] = ok ? *reinterpret_cast<const u32x4*>(dout + qrow + cc * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < QN) {
      int64_t qrow = 0, qhi = 0;
      const bool ok = query_at(step, tid, sida, qrow, qhi);
      // an invalid query gets lse2 = +inf, hence p = 0 (its rows are zero)
      st_l = ok ? lse[qhi] * kLog2e : __builtin_inff();
      st_d = ok ? dvec[qhi] : 0.f;
    }
  };
  auto stage_store = [&](int buf) {
    bf16_t* b = lds + buf * T::BUF;
#pragma unroll
    for (int i = 0; i < T::CH; ++i) {
      const int cidx = tid + T::NT * i;
      const int qi = cidx % QN, cc = cidx / QN;
      *reinterpret_cast<u32x4*>(b + qi * T::QS + cc * 8) = qr[i];
      *reinterpret_cast<u32x4*>(b + T::QE + qi * T::QS + cc * 8) = dr[i];
      const bf16_t* qe = reinterpret_cast<const bf16_t*>(&qr[i]);
      const bf16_t* de = reinterpret_cast<const bf16_t*>(&dr[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        b[2 * T::QE + (cc * 8 + e) * T::TS + qi] = qe[e];
        b[2 * T::QE + T::TE + (cc * 8 + e) * T::TS + qi] = de[e];
      }
    }
    if (tid < QN) {
      stat[buf][0][tid] = st_l;
      stat[buf][1][tid] = st_d;
    }
  };

  // prologue: tiles of step 0, ids of step 1
  if (nsteps > 0) {
    fetch_ids(0);
    fetch_rows(0);
    stage_store(0);
    if (nsteps > 1) fetch_ids(1);
  }
  __syncthreads();
  for (int it = 0; it < nsteps; ++it) {
    const int cb = it & 1;
    const bool more = it + 1 < nsteps;
    const bf16_t* b = lds + cb * T::BUF;
    const bool own_step = it >= rsteps;
    // S = Q K^T and dP = dO V^T (32 queries per block x the wave's 32 keys);
    // A rows in the kperm order
    f32x16 sacc[NQ], dpacc[NQ];
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      sacc[qb] = f32x16{};
      dpacc[qb] = f32x16{};
    }
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      const bf16_t* qa = b + (32 * qb + kperm(n)) * T::QS + 8 * hh;
      const bf16_t* da = b + T::QE + (32 * qb + kperm(n)) * T::QS + 8 * hh;
      bf16x8 fa[D / 16], fd[D / 16];
#pragma unroll
      for (int t = 0; t < D / 16; ++t) fa[t] = ld_bf16x8(qa + 16 * t);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) fd[t] = ld_bf16x8(da + 16 * t);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        sacc[qb] = mfma32(fa[t], kb[t], sacc[qb]);
        dpacc[qb] = mfma32(fd[t], vb[t], dpacc[qb]);
      }
    }
    // the next step's rows are requested while this step's math runs
    if (more) {
      fetch_rows(it + 1);
      if (it + 2 < nsteps) fetch_ids(it + 2);
    }
    // register 4i + jj of half hh of query block qb holds query
    // 32 qb + acc_key(4i + jj, hh): four consecutive queries per i
    int ppos0 = 0;
    if (own_step) {
      const int st = it - rsteps + olo;
      const int hl = st / psteps_h;
      ppos0 = p0 + (st - hl * psteps_h) * QN;
    }
    bf16x8 pb[2 * NQ], dsb[2 * NQ];
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi0 = 32 * qb + acc_key(4 * i, hh);
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&stat[cb][0][qi0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&stat[cb][1][qi0]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int reg = 4 * i + jj;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[qb][reg], sl2, -l4[jj]));
          if (own_step && ppos0 + qi0 + jj < key) p = 0.f;   // causal: query before the key
          const float ds = p * (dpacc[qb][reg] - d4[jj]);
          pb[2 * qb + (reg >> 3)][reg & 7] = static_cast<__bf16>(p);
          dsb[2 * qb + (reg >> 3)][reg & 7] = static_cast<__bf16>(ds);
        }
      }
    // dV^T += dO^T P, dK^T += Q^T dS: A = the transposed tiles (rows d,
    // k-slots queries 16 c2 + 8 hh + [0, 8)), B = P / dS
    {
      const bf16_t* qt = b + 2 * T::QE + n * T::TS + 8 * hh;
      const bf16_t* dtp = b + 2 * T::QE + T::TE + n * T::TS + 8 * hh;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int c2 = 0; c2 < 2 * NQ; ++c2) {
          const bf16x8 ad = ld_bf16x8(dtp + 32 * dt * T::TS + 16 * c2);
          const bf16x8 aq = ld_bf16x8(qt + 32 * dt * T::TS + 16 * c2);
          dva[dt] = mfma32(ad, pb[c2], dva[dt]);
          dka[dt] = mfma32(aq, dsb[c2], dka[dt]);
        }
    }
    if (more) stage_store(cb ^ 1);
    __syncthreads();
  }
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

hipError_t launch_bwd_dot(const void* out, const void* dout, float* dvec, const Dims& d,
                          hipStream_t st) {
  const int64_t nrows = (int64_t)d.S * d.Lq * d.H;
  const int rpb = 256 / (d.D / 8);
  const unsigned grid = (unsigned)((nrows + rpb - 1) / rpb);
  if (d.D == 128)
    hipLaunchKernelGGL(k_bwd_dot<128>, dim3(grid), dim3(256), 0, st,
                       static_cast<const bf16_t*>(out), static_cast<const bf16_t*>(dout), dvec,
                       nrows, d.Lq, d.H);
  else
    hipLaunchKernelGGL(k_bwd_dot<64>, dim3(grid), dim3(256), 0, st,
                       static_cast<const bf16_t*>(out), static_cast<const bf16_t*>(dout), dvec,
                       nrows, d.Lq, d.H);
  return hipGetLastError();
}

hipError_t launch_bwd_transform(const void* k, const void* v, void* kt, void* ktail, void* vtail,
                                const Dims& d, hipStream_t st) {
  if (d.L % 64 != 0 && (ktail == nullptr || vtail == nullptr)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(d.Lv / 64), d.Hkv, d.S);
#define MOBA_BT(DV)                                                                             \
  hipLaunchKernelGGL(k_bwd_transform<DV>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(k), \
                     static_cast<const bf16_t*>(v), static_cast<bf16_t*>(kt),                   \
                     static_cast<bf16_t*>(ktail), static_cast<bf16_t*>(vtail), d.Hkv, d.L, d.Lv)
  if (d.D == 128) MOBA_BT(128); else MOBA_BT(64);
#undef MOBA_BT
  return hipGetLastError();
}

hipError_t launch_bwd_dq_routed(const void* q, const void* dout, const void* k, const void* v,
                                const void* kt, const float* lse, const float* dvec,
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
                     static_cast<const bf16_t*>(kt), lse, dvec, list, bucket_off, tile_off,    \
                     static_cast<bf16_t*>(dqp), d.Lq, d.L, d.Lv, d.H, d.Hkv, d.kp, d.B, d.nb,  \
                     d.nrows, sl2, scale, (uint32_t)d.slots)
  if (d.tile_m == 256) {
    if (d.D == 128) MOBA_BQR(128, 8); else MOBA_BQR(64, 8);
  } else {
    if (d.D == 128) MOBA_BQR(128, 4); else MOBA_BQR(64, 4);
  }
#undef MOBA_BQR
  return hipGetLastError();
}

hipError_t launch_bwd_dq_own(const void* q, const void* dout, const void* k, const void* v,
                             const void* kt, const void* ktail, const void* vtail,
                             const float* lse, const float* dvec, const void* dqp, void* dq,
                             const Dims& d, hipStream_t st) {
  if (d.L % 64 != 0 && (ktail == nullptr || vtail == nullptr)) return hipErrorInvalidValue;
  const int HW = gcd_i(d.G, 4);
  constexpr int NW = 4;
  const int RW = 32 * NW / HW;
  const dim3 grid((unsigned)((d.Lq + RW - 1) / RW), d.S * d.H / HW);
  const float sl2 = kLog2e / sqrtf((float)d.D);
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_BQO(DV)                                                                            \
  hipLaunchKernelGGL((k_bwd_dq_own<DV, NW>), grid, dim3(64 * NW), 0, st,                        \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(dout),           \
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),              \
                     static_cast<const bf16_t*>(kt), static_cast<const bf16_t*>(ktail),         \
                     static_cast<const bf16_t*>(vtail), lse, dvec,                              \
                     static_cast<const bf16_t*>(dqp), static_cast<bf16_t*>(dq), (int)d.Lq,      \
                     (int)d.L, (int)d.Lv, (int)d.q_off, d.H, d.Hkv, d.kp, d.B, HW, sl2, scale)
  if (d.D == 128) MOBA_BQO(128); else MOBA_BQO(64);
#undef MOBA_BQO
  return hipGetLastError();
}

int bwd_dkdv_waves(const Dims& d) { return d.B % 128 == 0 ? 4 : 2; }
constexpr int kDkdvNQ = 2;   // 64 queries per step

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

hipError_t launch_bwd_dkdv(const void* q, const void* dout, const void* k, const void* v,
                           const float* lse, const float* dvec, const uint32_t* list,
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
  const FastDiv fkp = make_fastdiv((uint32_t)(d.kp > 0 ? d.kp : 1));
  const FastDiv flq = make_fastdiv((uint32_t)d.Lq);
#define MOBA_BKV(DV, NWV)                                                                       \
  hipLaunchKernelGGL((k_bwd_dkdv<DV, NWV, kDkdvNQ>), dim3((unsigned)grid), dim3(64 * NWV), 0, st, \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(dout),           \
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), lse, dvec,   \
                     list, bucket_off, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv),      \
                     kvpart, (int)d.Lq, (int)d.L, (int)d.q_off, d.H, d.Hkv, d.kp, d.B, d.nb,    \
                     nchunk, nseg, fkp, flq, sl2, scale)
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
