// fp32 backward (VALU), the fp32 counterpart of attn_bwd.hip.
//
// Same quantities, with the forward's selection held fixed and its natural
// log-sum-exp lse: for a query with key set T and c = 1/sqrt(D),
//   p_t = exp(c q.k_t - lse),  dv_t += p_t dO,  ds_t = p_t (dO.v_t - dO.o),
//   dq = c sum_t ds_t k_t,     dk_t += c ds_t q
// (GQA: a KV head sums over its group's query heads).  Decomposition:
//   k_bwd_dot_f32        dO.o per query-head;
//   k_bwd_dq_routed_f32  per routed tile of the forward's tile list: the
//                        block's keys staged through LDS 32 at a time, one
//                        fp32 dq partial per routed slot;
//   k_bwd_dq_own_f32     per query: the own block (causal mask), plus the
//                        query's routed dq partials -> dq;
//   k_bwd_dkdv_f32       per 64 keys of one block (key-stationary, four lanes
//                        per key, D/4 dims each): the bucket's routed entries,
//                        then the block's own queries of every head of the KV
//                        group, staged 32 at a time in LDS.
// One query per LPE = D/64 lanes (64 dims each) in the dq kernels, 128 per
// workgroup, as in the fp32 forward.
#include "common.h"
#include "kernels.h"

namespace moba {

template <int D>
struct BwdF32 {
  static constexpr int LPE = D / 64;
  static constexpr int NT = 128 * LPE;       // threads of a dq workgroup
  static constexpr int CH = 32 * D / 4 / NT;  // float4 chunks per thread per staged tile
};

// dvec[(s*H + h)*Lq + r] = dO . o of row (s, r, h): D/4 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dot_f32(const float* __restrict__ o,
                                                     const float* __restrict__ dout,
                                                     float* __restrict__ dvec, int64_t nrows,
                                                     int64_t Lq, int H) {
  constexpr int LPR = D / 4;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < nrows) {
    const float4 a = *reinterpret_cast<const float4*>(o + row * D + sub * 4);
    const float4 b = *reinterpret_cast<const float4*>(dout + row * D + sub * 4);
    acc = fmaf(a.x, b.x, fmaf(a.y, b.y, fmaf(a.z, b.z, a.w * b.w)));
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < nrows && sub == 0) {
    const int64_t h = row % H, sr = row / H, r = sr % Lq, s = sr / Lq;
    dvec[(s * H + h) * Lq + r] = acc;
  }
}

// Stages keys [key0, key0 + 32) of K and V; rows at or past L repeat row
// L - 1 (their keys lie past every query and are masked).
template <int D>
__device__ __forceinline__ void bwd_f32_load_tile(float* ks, float* vs, const float* kbase,
                                                  const float* vbase, int64_t stride,
                                                  int64_t key0, int64_t L, int tid) {
  using T = BwdF32<D>;
#pragma unroll
  for (int i = 0; i < T::CH; ++i) {
    const int c = tid + T::NT * i;
    const int row = c / (D / 4), cc = c % (D / 4);
    const int64_t key = key0 + row < L ? key0 + row : L - 1;
    const int64_t off = key * stride + cc * 4;
    reinterpret_cast<float4*>(ks)[c] = *reinterpret_cast<const float4*>(kbase + off);
    reinterpret_cast<float4*>(vs)[c] = *reinterpret_cast<const float4*>(vbase + off);
  }
}

__device__ __forceinline__ void load64(const float* p, float (&r)[64]) {
#pragma unroll
  for (int dd = 0; dd < 64; dd += 4) {
    const float4 x = *reinterpret_cast<const float4*>(p + dd);
    r[dd] = x.x; r[dd + 1] = x.y; r[dd + 2] = x.z; r[dd + 3] = x.w;
  }
}

// One 32-key tile for one lane (64 dims at dbase): dq += c * sum ds_t k_t.
// MASK: keys outside [klo, qpos] get p = 0.
template <int D, bool MASK>
__device__ __forceinline__ void bwd_f32_dq_step(const float* ks, const float* vs,
                                                const float (&qr)[64], const float (&dor)[64],
                                                float (&dq)[64], int dbase, float scale,
                                                float lse, float dvq, int64_t key0, int64_t klo,
                                                int64_t qpos) {
#pragma unroll 2
  for (int kk = 0; kk < 32; ++kk) {
    const float* kr = ks + kk * D + dbase;
    const float* vr = vs + kk * D + dbase;
    float sdot = 0.f, pdot = 0.f;
#pragma unroll
    for (int dd = 0; dd < 64; dd += 4) {
      const float4 x = *reinterpret_cast<const float4*>(kr + dd);
      const float4 y = *reinterpret_cast<const float4*>(vr + dd);
      sdot = fmaf(qr[dd], x.x, sdot);
      sdot = fmaf(qr[dd + 1], x.y, sdot);
      sdot = fmaf(qr[dd + 2], x.z, sdot);
      sdot = fmaf(qr[dd + 3], x.w, sdot);
      pdot = fmaf(dor[dd], y.x, pdot);
      pdot = fmaf(dor[dd + 1], y.y, pdot);
      pdot = fmaf(dor[dd + 2], y.z, pdot);
      pdot = fmaf(dor[dd + 3], y.w, pdot);
    }
    if (D == 128) {
      sdot += __shfl_xor(sdot, 1);
      pdot += __shfl_xor(pdot, 1);
    }
    float p = expf(sdot * scale - lse);
    if (MASK) {
      const int64_t key = key0 + kk;
      if (key > qpos || key < klo) p = 0.f;
    }
    const float ds = p * (pdot - dvq) * scale;
#pragma unroll
    for (int dd = 0; dd < 64; dd += 4) {
      const float4 x = *reinterpret_cast<const float4*>(kr + dd);
      dq[dd] = fmaf(ds, x.x, dq[dd]);
      dq[dd + 1] = fmaf(ds, x.y, dq[dd + 1]);
      dq[dd + 2] = fmaf(ds, x.z, dq[dd + 2]);
      dq[dd + 3] = fmaf(ds, x.w, dq[dd + 3]);
    }
  }
}

// Routed tiles (the forward's tile list and tile size): one fp32 dq partial
// per routed slot.
template <int D>
__global__ __launch_bounds__(BwdF32<D>::NT) void k_bwd_dq_routed_f32(
    const float* __restrict__ q, const float* __restrict__ dout, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ lse, const float* __restrict__ dvec,
    const uint32_t* __restrict__ list, const uint32_t* __restrict__ bucket_off,
    const uint32_t* __restrict__ tile_off, float* __restrict__ dqp, int64_t Lq, int64_t L,
    int H, int Hkv, int kp, int B, int nb, int nrows, float scale, uint32_t nslots,
    int tile_m) {
  using T = BwdF32<D>;
  __shared__ __attribute__((aligned(16))) float ks[32 * D];
  __shared__ __attribute__((aligned(16))) float vs[32 * D];
  const uint32_t ntiles = tile_off[nrows];
  const uint32_t tile = blockIdx.x;
  if (tile >= ntiles) return;
  int lo = 0, hi = nrows;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= tile) lo = mid; else hi = mid;
  }
  const int row = lo;
  const uint32_t start = (tile - tile_off[row]) * tile_m;
  const uint32_t avail = bucket_off[row + 1] - bucket_off[row] - start;
  const int cnt = avail < (uint32_t)tile_m ? (int)avail : tile_m;
  const int j = row % nb;
  const int sg = row / nb, g = sg % Hkv, s = sg / Hkv;
  const int tid = threadIdx.x;
  const int e = tid / T::LPE, dbase = (tid % T::LPE) * 64;
  const uint32_t slot_raw = (e < cnt) ? list[bucket_off[row] + start + e] : 0u;
  const bool valid = e < cnt && slot_raw < nslots;
  const uint32_t slot = valid ? slot_raw : 0u;
  const uint32_t qh = slot / (uint32_t)kp;  // (s*H + h)*Lq + r
  const int64_t r = qh % Lq;
  const int h = (int)((qh / Lq) % H);
  const int64_t qrow = (((int64_t)s * Lq + r) * H + h) * D + dbase;
  float qr[64], dor[64], dq[64];
  load64(q + qrow, qr);
  load64(dout + qrow, dor);
#pragma unroll
  for (int dd = 0; dd < 64; ++dd) dq[dd] = 0.f;
  const float lq = lse[qh], dvq = dvec[qh];
  const int64_t stride = (int64_t)Hkv * D;
  const float* kbase = k + ((int64_t)s * L * Hkv + g) * D;
  const float* vbase = v + ((int64_t)s * L * Hkv + g) * D;
  for (int64_t key0 = (int64_t)j * B; key0 < (int64_t)(j + 1) * B; key0 += 32) {
    __syncthreads();
    bwd_f32_load_tile<D>(ks, vs, kbase, vbase, stride, key0, L, tid);
    __syncthreads();
    bwd_f32_dq_step<D, false>(ks, vs, qr, dor, dq, dbase, scale, lq, dvq, key0, 0, 0);
  }
  if (!valid) return;
  float* prow = dqp + (int64_t)slot * D + dbase;
#pragma unroll
  for (int dd = 0; dd < 64; dd += 4)
    *reinterpret_cast<float4*>(prow + dd) = make_float4(dq[dd], dq[dd + 1], dq[dd + 2], dq[dd + 3]);
}

// Query-centric own block (keys from the start of the query's block up to the
// query) plus the routed partials.  grid (ceil(Lq / 128), S * H).
template <int D>
__global__ __launch_bounds__(BwdF32<D>::NT) void k_bwd_dq_own_f32(
    const float* __restrict__ q, const float* __restrict__ dout, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ lse, const float* __restrict__ dvec,
    const float* __restrict__ dqp, float* __restrict__ dq_out, int64_t Lq, int64_t L,
    int64_t q_off, int H, int Hkv, int kp, int B, float scale) {
  using T = BwdF32<D>;
  __shared__ __attribute__((aligned(16))) float ks[32 * D];
  __shared__ __attribute__((aligned(16))) float vs[32 * D];
  const int s = blockIdx.y / H, h = blockIdx.y % H, g = h / (H / Hkv);
  const int tid = threadIdx.x;
  const int e = tid / T::LPE, dbase = (tid % T::LPE) * 64;
  const int64_t rw0 = (int64_t)blockIdx.x * 128;
  const int64_t r = rw0 + e;
  const bool valid = r < Lq;
  const int64_t rr = valid ? r : Lq - 1;
  const int64_t pos = q_off + rr;
  const int64_t klo_l = (pos / B) * B;
  const int64_t wglast = (rw0 + 127 < Lq ? rw0 + 127 : Lq - 1);
  const int64_t klo_g = ((q_off + rw0) / B) * B;
  const int64_t khi_g = q_off + wglast + 1;
  const int64_t qh = ((int64_t)s * H + h) * Lq + rr;
  const int64_t qrow = (((int64_t)s * Lq + rr) * H + h) * D + dbase;
  float qr[64], dor[64], dq[64];
  load64(q + qrow, qr);
  load64(dout + qrow, dor);
#pragma unroll
  for (int dd = 0; dd < 64; ++dd) dq[dd] = 0.f;
  const float lq = lse[qh], dvq = dvec[qh];
  const int64_t stride = (int64_t)Hkv * D;
  const float* kbase = k + ((int64_t)s * L * Hkv + g) * D;
  const float* vbase = v + ((int64_t)s * L * Hkv + g) * D;
  for (int64_t key0 = (klo_g / 32) * 32; key0 < khi_g; key0 += 32) {
    __syncthreads();
    bwd_f32_load_tile<D>(ks, vs, kbase, vbase, stride, key0, L, tid);
    __syncthreads();
    if (key0 + 31 <= pos && key0 >= klo_l)
      bwd_f32_dq_step<D, false>(ks, vs, qr, dor, dq, dbase, scale, lq, dvq, key0, 0, 0);
    else if (key0 <= pos && key0 + 32 > klo_l)
      bwd_f32_dq_step<D, true>(ks, vs, qr, dor, dq, dbase, scale, lq, dvq, key0, klo_l, pos);
  }
  if (!valid) return;
  // the query's routed partials: slots qh*kp + t for its t < min(kp, own) past blocks
  const int own = (int)(pos / B);
  const int npast = kp < own ? kp : own;
  for (int t = 0; t < npast; ++t) {
    const float* prow = dqp + (qh * kp + t) * D + dbase;
#pragma unroll
    for (int dd = 0; dd < 64; dd += 4) {
      const float4 x = *reinterpret_cast<const float4*>(prow + dd);
      dq[dd] += x.x; dq[dd + 1] += x.y; dq[dd + 2] += x.z; dq[dd + 3] += x.w;
    }
  }
  float* orow = dq_out + qrow;
#pragma unroll
  for (int dd = 0; dd < 64; dd += 4)
    *reinterpret_cast<float4*>(orow + dd) = make_float4(dq[dd], dq[dd + 1], dq[dd + 2], dq[dd + 3]);
}

// Key-stationary dk / dv: workgroup = 64 keys of block j of (s, g) (grid
// S*Hkv*nb * ceil(B / 64), bucket row fastest-varying last); lane group of
// four per key, lane `sub` owning dims [sub*D/4, +D/4).  Queries: the bucket's
// routed entries (every key of a past block is visible), then the queries of
// block j of every head of the group (visible keys: up to the query).
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dkdv_f32(
    const float* __restrict__ q, const float* __restrict__ dout, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ lse, const float* __restrict__ dvec,
    const uint32_t* __restrict__ list, const uint32_t* __restrict__ bucket_off,
    float* __restrict__ dk, float* __restrict__ dv, int64_t Lq, int64_t L, int64_t q_off, int H,
    int Hkv, int kp, int B, int nb, float scale) {
  constexpr int DL = D / 4;
  constexpr int QC = D / 4;  // float4 chunks of a staged query row
  __shared__ __attribute__((aligned(16))) float qs[32 * D];
  __shared__ __attribute__((aligned(16))) float dos[32 * D];
  __shared__ float ls[32], dvs[32];
  __shared__ int64_t ps[32];
  const int cpb = (B + 63) / 64;
  const int c = (int)(blockIdx.x % cpb);
  const int64_t row = blockIdx.x / cpb;
  const int j = (int)(row % nb);
  const int64_t sg = row / nb;
  const int g = (int)(sg % Hkv), s = (int)(sg / Hkv);
  const int G = H / Hkv;
  const int tid = threadIdx.x, kl = tid / 4, sub = tid % 4;
  const int dbase = sub * DL;
  const int64_t key = (int64_t)j * B + 64 * c + kl;
  const bool kvalid = 64 * c + kl < B && key < L;
  const int64_t kidx = (((int64_t)s * L + (kvalid ? key : L - 1)) * Hkv + g) * D + dbase;
  float kr[DL], vr[DL], dka[DL], dva[DL];
#pragma unroll
  for (int dd = 0; dd < DL; dd += 4) {
    const float4 x = *reinterpret_cast<const float4*>(k + kidx + dd);
    const float4 y = *reinterpret_cast<const float4*>(v + kidx + dd);
    kr[dd] = x.x; kr[dd + 1] = x.y; kr[dd + 2] = x.z; kr[dd + 3] = x.w;
    vr[dd] = y.x; vr[dd + 1] = y.y; vr[dd + 2] = y.z; vr[dd + 3] = y.w;
    dka[dd] = dka[dd + 1] = dka[dd + 2] = dka[dd + 3] = 0.f;
    dva[dd] = dva[dd + 1] = dva[dd + 2] = dva[dd + 3] = 0.f;
  }
  const int64_t rbeg = list != nullptr ? bucket_off[row] : 0;
  const int64_t nrouted = list != nullptr ? bucket_off[row + 1] - rbeg : 0;
  // own queries: positions [p0, p1) of block j that are query rows
  const int64_t bstart = (int64_t)j * B;
  const int64_t p0 = bstart > q_off ? bstart : q_off;
  const int64_t bend = bstart + B < L ? bstart + B : L;
  const int64_t p1 = bend < q_off + Lq ? bend : q_off + Lq;
  const int64_t nrows_own = p1 > p0 ? p1 - p0 : 0;
  const int64_t total = nrouted + (int64_t)G * nrows_own;
  for (int64_t base = 0; base < total; base += 32) {
    __syncthreads();  // the previous 32 queries are no longer read
    for (int i = tid; i < 32 * QC; i += 256) {
      const int qi = i / QC, cc = i % QC;
      const int64_t e = base + qi;
      if (e >= total) continue;
      int64_t qh, pos, r;
      int h;
      if (e < nrouted) {
        const uint32_t slot = list[rbeg + e];
        qh = slot / (uint32_t)kp;
        r = qh % Lq;
        h = (int)((qh / Lq) % H);
        pos = INT64_MAX;  // a past block: every key is visible
      } else {
        const int64_t o = e - nrouted;
        h = g * G + (int)(o / nrows_own);
        pos = p0 + o % nrows_own;
        r = pos - q_off;
        qh = ((int64_t)s * H + h) * Lq + r;
      }
      const int64_t qrow = (((int64_t)s * Lq + r) * H + h) * D + cc * 4;
      reinterpret_cast<float4*>(qs)[qi * QC + cc] = *reinterpret_cast<const float4*>(q + qrow);
      reinterpret_cast<float4*>(dos)[qi * QC + cc] =
          *reinterpret_cast<const float4*>(dout + qrow);
      if (cc == 0) {
        ls[qi] = lse[qh];
        dvs[qi] = dvec[qh];
        ps[qi] = pos;
      }
    }
    __syncthreads();
    const int nq = total - base < 32 ? (int)(total - base) : 32;
    for (int qi = 0; qi < nq; ++qi) {
      const float* qrw = qs + qi * D + dbase;
      const float* drw = dos + qi * D + dbase;
      float sdot = 0.f, pdot = 0.f;
#pragma unroll
      for (int dd = 0; dd < DL; dd += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qrw + dd);
        const float4 y = *reinterpret_cast<const float4*>(drw + dd);
        sdot = fmaf(x.x, kr[dd], sdot);
        sdot = fmaf(x.y, kr[dd + 1], sdot);
        sdot = fmaf(x.z, kr[dd + 2], sdot);
        sdot = fmaf(x.w, kr[dd + 3], sdot);
        pdot = fmaf(y.x, vr[dd], pdot);
        pdot = fmaf(y.y, vr[dd + 1], pdot);
        pdot = fmaf(y.z, vr[dd + 2], pdot);
        pdot = fmaf(y.w, vr[dd + 3], pdot);
      }
      sdot += __shfl_xor(sdot, 1);
      sdot += __shfl_xor(sdot, 2);
      pdot += __shfl_xor(pdot, 1);
      pdot += __shfl_xor(pdot, 2);
      float p = expf(sdot * scale - ls[qi]);
      if (key > ps[qi]) p = 0.f;
      const float ds = p * (pdot - dvs[qi]) * scale;
#pragma unroll
      for (int dd = 0; dd < DL; dd += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qrw + dd);
        const float4 y = *reinterpret_cast<const float4*>(drw + dd);
        dva[dd] = fmaf(p, y.x, dva[dd]);
        dva[dd + 1] = fmaf(p, y.y, dva[dd + 1]);
        dva[dd + 2] = fmaf(p, y.z, dva[dd + 2]);
        dva[dd + 3] = fmaf(p, y.w, dva[dd + 3]);
        dka[dd] = fmaf(ds, x.x, dka[dd]);
        dka[dd + 1] = fmaf(ds, x.y, dka[dd + 1]);
        dka[dd + 2] = fmaf(ds, x.z, dka[dd + 2]);
        dka[dd + 3] = fmaf(ds, x.w, dka[dd + 3]);
      }
    }
  }
  if (!kvalid) return;
#pragma unroll
  for (int dd = 0; dd < DL; dd += 4) {
    *reinterpret_cast<float4*>(dk + kidx + dd) =
        make_float4(dka[dd], dka[dd + 1], dka[dd + 2], dka[dd + 3]);
    *reinterpret_cast<float4*>(dv + kidx + dd) =
        make_float4(dva[dd], dva[dd + 1], dva[dd + 2], dva[dd + 3]);
  }
}

hipError_t launch_bwd_dot_f32(const void* out, const void* dout, float* dvec, const Dims& d,
                              hipStream_t st) {
  const int64_t nrows = (int64_t)d.S * d.Lq * d.H;
  const int rpb = 256 / (d.D / 4);
  const unsigned grid = (unsigned)((nrows + rpb - 1) / rpb);
#define MOBA_BD(DV)                                                                            \
  hipLaunchKernelGGL(k_bwd_dot_f32<DV>, dim3(grid), dim3(256), 0, st,                          \
                     static_cast<const float*>(out), static_cast<const float*>(dout), dvec, \
                     nrows, d.Lq, d.H)
  if (d.D == 128) MOBA_BD(128); else MOBA_BD(64);
#undef MOBA_BD
  return hipGetLastError();
}

hipError_t launch_bwd_dq_routed_f32(const void* q, const void* dout, const void* k,
                                    const void* v, const float* lse, const float* dvec,
                                    const uint32_t* list, const uint32_t* bucket_off,
                                    const uint32_t* tile_off, float* dqp, const Dims& d,
                                    hipStream_t st) {
  const int64_t grid = routed_tile_bound(d);
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_DQR(DV)                                                                          \
  hipLaunchKernelGGL(k_bwd_dq_routed_f32<DV>, dim3((unsigned)grid), dim3(BwdF32<DV>::NT), 0, \
                     st, static_cast<const float*>(q), static_cast<const float*>(dout),      \
                     static_cast<const float*>(k), static_cast<const float*>(v), lse, dvec,  \
                     list, bucket_off, tile_off, dqp, d.Lq, d.L, d.H, d.Hkv, d.kp, d.B,     \
                     d.nb, d.nrows, scale, (uint32_t)d.slots, d.tile_m)
  if (d.D == 128) MOBA_DQR(128); else MOBA_DQR(64);
#undef MOBA_DQR
  return hipGetLastError();
}

hipError_t launch_bwd_dq_own_f32(const void* q, const void* dout, const void* k, const void* v,
                                 const float* lse, const float* dvec, const float* dqp,
                                 void* dq, const Dims& d, hipStream_t st) {
  const dim3 grid((unsigned)((d.Lq + 127) / 128), (unsigned)(d.S * d.H));
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_DQO(DV)                                                                          \
  hipLaunchKernelGGL(k_bwd_dq_own_f32<DV>, grid, dim3(BwdF32<DV>::NT), 0, st,                \
                     static_cast<const float*>(q), static_cast<const float*>(dout),          \
                     static_cast<const float*>(k), static_cast<const float*>(v), lse, dvec,  \
                     dqp, static_cast<float*>(dq), d.Lq, d.L, d.q_off, d.H, d.Hkv, d.kp,    \
                     d.B, scale)
  if (d.D == 128) MOBA_DQO(128); else MOBA_DQO(64);
#undef MOBA_DQO
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const void* q, const void* dout, const void* k, const void* v,
                               const float* lse, const float* dvec, const uint32_t* list,
                               const uint32_t* bucket_off, void* dk, void* dv, const Dims& d,
                               hipStream_t st) {
  const int64_t grid = (int64_t)d.nrows * ((d.B + 63) / 64);
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_DKV(DV)                                                                          \
  hipLaunchKernelGGL(k_bwd_dkdv_f32<DV>, dim3((unsigned)grid), dim3(256), 0, st,             \
                     static_cast<const float*>(q), static_cast<const float*>(dout),          \
                     static_cast<const float*>(k), static_cast<const float*>(v), lse, dvec,  \
                     list, bucket_off, static_cast<float*>(dk), static_cast<float*>(dv),     \
                     d.Lq, d.L, d.q_off, d.H, d.Hkv, d.kp, d.B, d.nb, scale)
  if (d.D == 128) MOBA_DKV(128); else MOBA_DKV(64);
#undef MOBA_DKV
  return hipGetLastError();
}

}  // namespace moba
