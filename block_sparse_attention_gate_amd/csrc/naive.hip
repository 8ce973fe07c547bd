// Mask-based MoBA: the selection applied as a mask to ordinary attention
// over the dense score matrix.  This is the "naive" form the pages set beside
// the efficient one (MoBA project card, "Highlighted Details" and
// "Limitations & Caveats": for understanding and visualising the masks, the
// baseline of the quoted efficient-vs-naive speedup at 32K tokens; the
// tutorial's step 1 applies the gate's choice as a mask to regular attention).
// It is kept as a comparison baseline: every (query, key) score is computed
// and stored, then masked.
//   k_naive_scores:  S = c Q K^T for every query row and key (fp32, HBM).
//   k_naive_softmax: per query row, keys outside the row's selected blocks or
//                    after the query get probability 0; softmax of the rest
//                    (bf16 P, HBM).
//   k_naive_pv:      out = P V over every key (MFMA, P and V^T from HBM).
#include "common.h"
#include "kernels.h"

namespace moba {

// grid (ceil(Lq / 32), S * H), 256 threads: the workgroup's 32 query rows
// against every key; wave w takes the 32-key tiles w, w + 4, ...  Keys at or
// past L read row L - 1 (the softmax masks them).  Row stride of sc: Lp.
template <int D>
__global__ __launch_bounds__(256) void k_naive_scores(const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ k,
                                                      float* __restrict__ sc, int64_t Lq,
                                                      int64_t L, int64_t Lp, int H, int Hkv,
                                                      float scale) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, n = lane & 31, hh = lane >> 5;
  const int sh = blockIdx.y, s = sh / H, h = sh % H, g = h / (H / Hkv);
  const int64_t r0 = (int64_t)blockIdx.x * 32;
  const int64_t r = r0 + n;
  const bool valid = r < Lq;
  // A operand: query row n, dims [16t + 8hh, +8)
  bf16x8 qf[D / 16];
  const bf16_t* qrow = q + (((int64_t)s * Lq + (valid ? r : 0)) * H + h) * D + 8 * hh;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) qf[t] = valid ? ld_bf16x8(qrow + 16 * t) : bf16x8{};
  float* sbase = sc + ((int64_t)sh * Lq + r0) * Lp;
  for (int64_t key0 = 32 * w; key0 < Lp; key0 += 128) {
    // B operand: key column n, the same dims
    const int64_t key = key0 + n < L ? key0 + n : L - 1;
    const bf16_t* krow = k + (((int64_t)s * L + key) * Hkv + g) * D + 8 * hh;
    f32x16 c = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 16; ++t) c = mfma32(qf[t], ld_bf16x8(krow + 16 * t), c);
    // lane: key column key0 + n; register 4i + j: query row 8i + 4hh + j
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 8 * i + 4 * hh + j;
        if (r0 + row < Lq) sbase[row * Lp + key0 + n] = c[4 * i + j] * scale;
      }
  }
}

__device__ __forceinline__ float block_reduce(float x, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  __syncthreads();  // red may still be read by a previous reduction
  if (lane == 0) red[w] = x;
  __syncthreads();
  x = red[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) x = is_max ? fmaxf(x, red[i]) : x + red[i];
  return x;
}

// One workgroup (256 threads) per query row ((s * H + h) * Lq + r): a bit per
// KV block for the row's selected blocks, then the max, the sum and the
// probabilities over the keys that are selected and not after the query
// (natural exp; masked keys and keys past L get 0).
__global__ __launch_bounds__(256) void k_naive_softmax(const float* __restrict__ sc,
                                                       const int32_t* __restrict__ sel,
                                                       bf16_t* __restrict__ p, int64_t Lq,
                                                       int64_t L, int64_t Lp, int64_t q_off,
                                                       int B, int nb, int topk) {
  __shared__ uint32_t bits[kMaxBlocks / 32];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t pos = q_off + row % Lq;
  for (int i = tid; i < (nb + 31) / 32; i += 256) bits[i] = 0u;
  __syncthreads();
  if (tid < topk) {
    const int j = sel[row * topk + tid];
    if (j >= 0 && j < nb) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  const int64_t kend = pos + 1 < L ? pos + 1 : L;  // keys [0, kend) may be visible
  auto visible = [&](int64_t t) {
    const int j = (int)(t / B);
    return t < kend && ((bits[j >> 5] >> (j & 31)) & 1u);
  };
  const float* srow = sc + row * Lp;
  float m = -__builtin_inff();
  for (int64_t t = tid; t < kend; t += 256)
    if (visible(t)) m = fmaxf(m, srow[t]);
  m = block_reduce(m, red, true);
  float l = 0.f;
  for (int64_t t = tid; t < kend; t += 256)
    if (visible(t)) l += __expf(srow[t] - m);
  l = block_reduce(l, red, false);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  bf16_t* prow = p + row * Lp;
  for (int64_t t = tid; t < Lp; t += 256)
    prow[t] = f32_to_bf16(visible(t) ? __expf(srow[t] - m) * inv : 0.f);
}

// grid (ceil(Lq / 32), S * H), one wave: 32 query rows x all D dims, summed
// over every key (16 per MFMA).  A operand: P row n, keys [16c + 8hh, +8);
// B operand: V^T row (dim) 32dt + n, the same keys.  (Four waves per
// workgroup over quarters of the key range, or 128 rows sharing V^T chunks
// staged in LDS, measured slower at 32K tokens: the P reads bound it.)
template <int D>
__global__ __launch_bounds__(64) void k_naive_pv(const bf16_t* __restrict__ p,
                                                 const bf16_t* __restrict__ vt,
                                                 bf16_t* __restrict__ out, int64_t Lq,
                                                 int64_t Lp, int H, int Hkv) {
  const int lane = threadIdx.x, n = lane & 31, hh = lane >> 5;
  const int sh = blockIdx.y, s = sh / H, h = sh % H, g = h / (H / Hkv);
  const int64_t r0 = (int64_t)blockIdx.x * 32;
  const int64_t r = r0 + n < Lq ? r0 + n : Lq - 1;
  const bf16_t* prow = p + ((int64_t)sh * Lq + r) * Lp + 8 * hh;
  const bf16_t* vrow = vt + ((int64_t)s * Hkv + g) * D * Lp + (int64_t)n * Lp + 8 * hh;
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
#pragma unroll 4
  for (int64_t c = 0; c < Lp; c += 16) {
    const bf16x8 a = ld_bf16x8(prow + c);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      acc[dt] = mfma32(a, ld_bf16x8(vrow + (int64_t)32 * dt * Lp + c), acc[dt]);
  }
  // lane: dim column 32dt + n; register 4i + j: query row 8i + 4hh + j
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t row = r0 + 8 * i + 4 * hh + j;
        if (row < Lq)
          out[(((int64_t)s * Lq + row) * H + h) * D + 32 * dt + n] =
              f32_to_bf16(acc[dt][4 * i + j]);
      }
}

hipError_t launch_naive_scores(const void* q, const void* k, float* sc, const Dims& d,
                               hipStream_t st) {
  const dim3 grid((unsigned)((d.Lq + 31) / 32), (unsigned)(d.S * d.H));
  const float scale = 1.0f / sqrtf((float)d.D);
#define MOBA_NS(DV)                                                                           \
  hipLaunchKernelGGL((k_naive_scores<DV>), grid, dim3(256), 0, st,                            \
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), sc, d.Lq, \
                     d.L, d.Lv, d.H, d.Hkv, scale)
  if (d.D == 128) MOBA_NS(128); else MOBA_NS(64);
#undef MOBA_NS
  return hipGetLastError();
}

hipError_t launch_naive_softmax(const float* sc, const int32_t* sel, void* p, const Dims& d,
                                hipStream_t st) {
  const int64_t rows = (int64_t)d.S * d.H * d.Lq;
  hipLaunchKernelGGL(k_naive_softmax, dim3((unsigned)rows), dim3(256), 0, st, sc, sel,
                     static_cast<bf16_t*>(p), d.Lq, d.L, d.Lv, d.q_off, d.B, d.nb, d.topk);
  return hipGetLastError();
}

hipError_t launch_naive_pv(const void* p, const void* vt, void* out, const Dims& d,
                           hipStream_t st) {
  const dim3 grid((unsigned)((d.Lq + 31) / 32), (unsigned)(d.S * d.H));
#define MOBA_NPV(DV)                                                                          \
  hipLaunchKernelGGL((k_naive_pv<DV>), grid, dim3(64), 0, st, static_cast<const bf16_t*>(p), \
                     static_cast<const bf16_t*>(vt), static_cast<bf16_t*>(out), d.Lq, d.Lv,  \
                     d.H, d.Hkv)
  if (d.D == 128) MOBA_NPV(128); else MOBA_NPV(64);
#undef MOBA_NPV
  return hipGetLastError();
}

}  // namespace moba
