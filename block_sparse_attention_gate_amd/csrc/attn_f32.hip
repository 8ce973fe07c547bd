// fp32 attention kernels (VALU), the fp32 counterpart of attn_bf16.hip.
//
// Same decomposition as the bf16 path -- routed partials per selected past
// block, then the own block under its causal mask merged with the partials
// by log-sum-exp, or full causal attention -- computed with fp32 FMA.  One
// query (or routed entry) per LPE = D/64 lanes, each lane owning 64 of the D
// dimensions; 128 queries or entries per workgroup; K and V staged through
// LDS 32 keys at a time.
#include "common.h"
#include "kernels.h"

namespace moba {

template <int D>
struct F32Tile {
  static constexpr int LPE = D / 64;
  static constexpr int NT = 128 * LPE;       // threads per workgroup
  static constexpr int KEYS = 32;
  static constexpr int CH = KEYS * D / 4 / NT;  // float4 chunks per thread per tensor
};

// Stages keys [key0, key0 + 32); rows at or past L (the end of a sequence
// whose length is not a multiple of 32) repeat row L - 1.  Those keys lie
// past every query position, so the causal mask drops them.
template <int D>
__device__ __forceinline__ void f32_load_tile(float* ks, float* vs, const float* kbase,
                                              const float* vbase, int64_t stride, int64_t key0,
                                              int64_t L, int tid) {
  using T = F32Tile<D>;
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

struct F32Acc {
  float o[64];
  float m, l;
};

// One 32-key step for one lane (64 dims at dbase).  Natural-base softmax.
template <int D, bool MASK>
__device__ __forceinline__ void f32_step(const float* ks, const float* vs, const float (&qr)[64],
                                         F32Acc& a, int dbase, float scale, int64_t key0,
                                         int64_t klo, int64_t qpos) {
  float sc[32];
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) {
    const float* kr = ks + kk * D + dbase;
    float dot = 0.f;
#pragma unroll
    for (int dd = 0; dd < 64; dd += 4) {
      const float4 x = *reinterpret_cast<const float4*>(kr + dd);
      dot = fmaf(qr[dd], x.x, dot);
      dot = fmaf(qr[dd + 1], x.y, dot);
      dot = fmaf(qr[dd + 2], x.z, dot);
      dot = fmaf(qr[dd + 3], x.w, dot);
    }
    if (D == 128) dot += __shfl_xor(dot, 1);
    sc[kk] = dot * scale;
    if (MASK) {
      const int64_t key = key0 + kk;
      if (key > qpos || key < klo) sc[kk] = -__builtin_inff();
    }
  }
  float mx = sc[0];
#pragma unroll
  for (int kk = 1; kk < 32; ++kk) mx = fmaxf(mx, sc[kk]);
  const float mnew = fmaxf(a.m, mx);
  const float mref = (mnew == -__builtin_inff()) ? 0.f : mnew;
  const float alpha = expf(a.m - mref);
  float ps = 0.f;
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) {
    sc[kk] = expf(sc[kk] - mref);
    ps += sc[kk];
  }
  a.l = a.l * alpha + ps;
  a.m = mnew;
#pragma unroll
  for (int dd = 0; dd < 64; ++dd) a.o[dd] *= alpha;
#pragma unroll 4
  for (int kk = 0; kk < 32; ++kk) {
    const float* vr = vs + kk * D + dbase;
    const float p = sc[kk];
#pragma unroll
    for (int dd = 0; dd < 64; dd += 4) {
      const float4 x = *reinterpret_cast<const float4*>(vr + dd);
      a.o[dd] = fmaf(p, x.x, a.o[dd]);
      a.o[dd + 1] = fmaf(p, x.y, a.o[dd + 1]);
      a.o[dd + 2] = fmaf(p, x.z, a.o[dd + 2]);
      a.o[dd + 3] = fmaf(p, x.w, a.o[dd + 3]);
    }
  }
}

template <int D>
__device__ __forceinline__ void f32_load_q(const float* qrow, int dbase, float (&qr)[64]) {
#pragma unroll
  for (int dd = 0; dd < 64; dd += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qrow + dbase + dd);
    qr[dd] = x.x; qr[dd + 1] = x.y; qr[dd + 2] = x.z; qr[dd + 3] = x.w;
  }
}

// Routed tiles (same tile list as the bf16 path, no XCD remap needed here).
template <int D>
__global__ __launch_bounds__(F32Tile<D>::NT) void k_attn_routed_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const uint32_t* __restrict__ list, const uint32_t* __restrict__ bucket_off,
    const uint32_t* __restrict__ tile_off, float* __restrict__ po, float* __restrict__ plse,
    int64_t Lq, int64_t L, int H, int Hkv, int kp, int B, int nb, int nrows, float scale,
    uint32_t nslots, int tile_m) {
  using T = F32Tile<D>;
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
  const bool valid = e < cnt && slot_raw < nslots;  // never write outside the partials
  const uint32_t slot = valid ? slot_raw : 0u;
  const uint32_t qh = slot / (uint32_t)kp;
  const int64_t r = qh % Lq;
  const int h = (int)((qh / Lq) % H);
  float qr[64];
  f32_load_q<D>(q + (((int64_t)s * Lq + r) * H + h) * D, dbase, qr);
  F32Acc a;
#pragma unroll
  for (int dd = 0; dd < 64; ++dd) a.o[dd] = 0.f;
  a.m = -__builtin_inff();
  a.l = 0.f;
  const int64_t stride = (int64_t)Hkv * D;
  const float* kbase = k + ((int64_t)s * L * Hkv + g) * D;
  const float* vbase = v + ((int64_t)s * L * Hkv + g) * D;
  for (int64_t key0 = (int64_t)j * B; key0 < (int64_t)(j + 1) * B; key0 += 32) {
    __syncthreads();
    f32_load_tile<D>(ks, vs, kbase, vbase, stride, key0, L, tid);
    __syncthreads();
    f32_step<D, false>(ks, vs, qr, a, dbase, scale, key0, 0, 0);
  }
  if (!valid) return;
  const float inv = 1.0f / a.l;
  float* orow = po + (int64_t)slot * D + dbase;
#pragma unroll
  for (int dd = 0; dd < 64; dd += 4)
    *reinterpret_cast<float4*>(orow + dd) =
        make_float4(a.o[dd] * inv, a.o[dd + 1] * inv, a.o[dd + 2] * inv, a.o[dd + 3] * inv);
  if (dbase == 0) plse[slot] = a.m + logf(a.l);
}

// Query-centric: MODE 0 own block + merge, MODE 1 full causal.
// grid (ceil(Lq / 128), S * H).
template <int D, int MODE>
__global__ __launch_bounds__(F32Tile<D>::NT) void k_attn_query_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ po, const float* __restrict__ plse, float* __restrict__ out,
    float* __restrict__ lse_out, int64_t Lq, int64_t L, int64_t q_off, int H, int Hkv, int kp,
    int B, float scale) {
  using T = F32Tile<D>;
  __shared__ __attribute__((aligned(16))) float ks[32 * D];
  __shared__ __attribute__((aligned(16))) float vs[32 * D];
  const int rt = (MODE == 1) ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int s = blockIdx.y / H, h = blockIdx.y % H, g = h / (H / Hkv);
  const int tid = threadIdx.x;
  const int e = tid / T::LPE, dbase = (tid % T::LPE) * 64;
  const int64_t rw0 = (int64_t)rt * 128;
  const int64_t r = rw0 + e;
  const bool valid = r < Lq;
  const int64_t pos = q_off + (valid ? r : Lq - 1);
  const int64_t klo_l = (MODE == 0) ? (pos / B) * B : 0;
  const int64_t wglast = (rw0 + 127 < Lq ? rw0 + 127 : Lq - 1);
  const int64_t klo_g = (MODE == 0) ? ((q_off + rw0) / B) * B : 0;
  const int64_t khi_g = q_off + wglast + 1;
  float qr[64];
  f32_load_q<D>(q + (((int64_t)s * Lq + (valid ? r : 0)) * H + h) * D, dbase, qr);
  F32Acc a;
#pragma unroll
  for (int dd = 0; dd < 64; ++dd) a.o[dd] = 0.f;
  a.m = -__builtin_inff();
  a.l = 0.f;
  const int64_t stride = (int64_t)Hkv * D;
  const float* kbase = k + ((int64_t)s * L * Hkv + g) * D;
  const float* vbase = v + ((int64_t)s * L * Hkv + g) * D;
  for (int64_t key0 = (klo_g / 32) * 32; key0 < khi_g; key0 += 32) {
    __syncthreads();
    f32_load_tile<D>(ks, vs, kbase, vbase, stride, key0, L, tid);
    __syncthreads();
    if (key0 + 31 <= pos && key0 >= klo_l)
      f32_step<D, false>(ks, vs, qr, a, dbase, scale, key0, 0, 0);
    else if (key0 <= pos && key0 + 32 > klo_l)
      f32_step<D, true>(ks, vs, qr, a, dbase, scale, key0, klo_l, pos);
  }
  if (!valid) return;
  float* orow = out + (((int64_t)s * Lq + r) * H + h) * D + dbase;
  if (MODE == 0 && kp > 0) {
    const int own = (int)(pos / B);
    const int npast = kp < own ? kp : own;
    const float lse_own = a.m + logf(a.l);
    const int64_t sbase = (((int64_t)s * H + h) * Lq + r) * kp;
    float M = lse_own;
    for (int t = 0; t < npast; ++t) M = fmaxf(M, plse[sbase + t]);
    const float w_own = expf(lse_own - M);
    float wsum = w_own;
#pragma unroll
    for (int dd = 0; dd < 64; ++dd) a.o[dd] *= w_own / a.l;
    for (int t = 0; t < npast; ++t) {
      const float wt = expf(plse[sbase + t] - M);
      wsum += wt;
      const float* prow = po + (sbase + t) * D + dbase;
#pragma unroll
      for (int dd = 0; dd < 64; dd += 4) {
        const float4 x = *reinterpret_cast<const float4*>(prow + dd);
        a.o[dd] = fmaf(wt, x.x, a.o[dd]);
        a.o[dd + 1] = fmaf(wt, x.y, a.o[dd + 1]);
        a.o[dd + 2] = fmaf(wt, x.z, a.o[dd + 2]);
        a.o[dd + 3] = fmaf(wt, x.w, a.o[dd + 3]);
      }
    }
    const float inv = 1.0f / wsum;
    if (lse_out != nullptr && dbase == 0) lse_out[((int64_t)s * H + h) * Lq + r] = M + logf(wsum);
#pragma unroll
    for (int dd = 0; dd < 64; dd += 4)
      *reinterpret_cast<float4*>(orow + dd) =
          make_float4(a.o[dd] * inv, a.o[dd + 1] * inv, a.o[dd + 2] * inv, a.o[dd + 3] * inv);
    return;
  }
  if (MODE == 0 && lse_out != nullptr && dbase == 0)
    lse_out[((int64_t)s * H + h) * Lq + r] = a.m + logf(a.l);
  const float inv = 1.0f / a.l;
#pragma unroll
  for (int dd = 0; dd < 64; dd += 4)
    *reinterpret_cast<float4*>(orow + dd) =
        make_float4(a.o[dd] * inv, a.o[dd + 1] * inv, a.o[dd + 2] * inv, a.o[dd + 3] * inv);
}

hipError_t launch_attn_routed_f32(const void* q, const void* k, const void* v,
                                  const uint32_t* list, const uint32_t* bucket_off,
                                  const uint32_t* tile_off, void* part_o, float* part_lse,
                                  const Dims& d, hipStream_t st) {
  const int64_t grid = routed_tile_bound(d);
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_RF32(DV)                                                                       \
  hipLaunchKernelGGL(k_attn_routed_f32<DV>, dim3((unsigned)grid), dim3(F32Tile<DV>::NT), 0, \
                     st, static_cast<const float*>(q), static_cast<const float*>(k),        \
                     static_cast<const float*>(v), list, bucket_off, tile_off,              \
                     static_cast<float*>(part_o), part_lse, d.Lq, d.L, d.H, d.Hkv, d.kp,    \
                     d.B, d.nb, d.nrows, scale, (uint32_t)d.slots, d.tile_m)
  if (d.D == 128) MOBA_RF32(128); else MOBA_RF32(64);
#undef MOBA_RF32
  return hipGetLastError();
}

hipError_t launch_attn_query_f32(const void* q, const void* k, const void* v, const void* part_o,
                                 const float* part_lse, void* out, int mode, const Dims& d,
                                 hipStream_t st, float* lse_out) {
  dim3 grid((unsigned)((d.Lq + 127) / 128), d.S * d.H);
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_QF32(DV, MV)                                                                    \
  hipLaunchKernelGGL((k_attn_query_f32<DV, MV>), grid, dim3(F32Tile<DV>::NT), 0, st,         \
                     static_cast<const float*>(q), static_cast<const float*>(k),             \
                     static_cast<const float*>(v), static_cast<const float*>(part_o),        \
                     part_lse, static_cast<float*>(out), mode == 0 ? lse_out : nullptr,      \
                     d.Lq, d.L, d.q_off, d.H, d.Hkv, d.kp, d.B, scale)
  if (d.D == 128) {
    if (mode == 0) MOBA_QF32(128, 0); else MOBA_QF32(128, 1);
  } else {
    if (mode == 0) MOBA_QF32(64, 0); else MOBA_QF32(64, 1);
  }
#undef MOBA_QF32
  return hipGetLastError();
}

}  // namespace moba
