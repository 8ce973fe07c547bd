// Decode: one new query per sequence against a long K/V cache.
//
// Same method as the prefill (gate on block means, top-k with the own block,
// one softmax over the kept keys), but the work is dominated by reading the
// kept K/V blocks from HBM, so the kernels are organised around reading each
// kept block once:
//   k_decode_plan:  per (sequence, KV head): the union of the blocks kept by
//                   the group's query heads, each with the mask of heads that
//                   kept it (a block kept by several heads is read once).
//   k_decode_attn:  per (union block, key chunk): scores of the chunk for the
//                   heads in the mask, a chunk-local softmax and P.V, written
//                   as an unnormalised partial (max, sum, o).
//   k_decode_merge: per (sequence, head): log-sum-exp merge of the partials
//                   of the head's kept blocks -> out.
// With q_len = 1 the query sits at the last cache position, so every kept
// block is visible up to the end of the cache: past blocks whole, the own
// block up to the query (a chunk past the end holds no key and writes an
// empty partial).
#include "common.h"
#include "kernels.h"

namespace moba {


// grid S*Hkv, 64 threads.
// all_blocks = 1 selects every block for every head (split-K full attention).
__global__ __launch_bounds__(64) void k_decode_plan(const int32_t* __restrict__ sel,
                                                    int32_t* __restrict__ ublk,
                                                    uint32_t* __restrict__ umask,
                                                    int32_t* __restrict__ ucount, int H,
                                                    int Hkv, int nb, int topk, int umax,
                                                    int all_blocks) {
  extern __shared__ uint32_t lds_mask[];  // [nb]
  const int sg = blockIdx.x, s = sg / Hkv, g = sg % Hkv, G = H / Hkv;
  const int lane = threadIdx.x;
  const uint32_t all = (G >= 32) ? 0xffffffffu : ((1u << G) - 1u);
  for (int j = lane; j < nb; j += 64) lds_mask[j] = all_blocks ? all : 0u;
  __syncthreads();
  for (int e = lane; !all_blocks && e < G * topk; e += 64) {
    const int hl = e / topk, t = e % topk;
    const int j = sel[((int64_t)s * H + g * G + hl) * topk + t];  // q_len = 1
    if (j >= 0 && j < nb) atomicOr(&lds_mask[j], 1u << hl);
  }
  __syncthreads();
  int base = 0;
  const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  for (int j0 = 0; j0 < nb; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t m = j < nb ? lds_mask[j] : 0u;
    const uint64_t bal = __ballot(m != 0u);
    if (m != 0u) {
      const int idx = base + __popcll(bal & lt);
      if (idx < umax) {
        ublk[(int64_t)sg * umax + idx] = j;
        umask[(int64_t)sg * umax + idx] = m;
      }
    }
    base += __popcll(bal);
  }
  if (lane == 0) ucount[sg] = base < umax ? base : umax;
}

// 1-D grid over (sequence * KV head) x union slot x chunk with the (sequence,
// KV head) index fastest: neighbouring workgroups read different KV heads,
// whose rows interleave in HBM, instead of piling onto one head's rows.
// 256 threads.  GM = max heads per group.
template <typename T, int D, int GM>
__global__ __launch_bounds__(256) void k_decode_attn(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ ublk, const uint32_t* __restrict__ umask,
    const int32_t* __restrict__ ucount, float* __restrict__ part, int64_t L, int H, int Hkv,
    int B, int umax, float scale_log2, int nsg, const int32_t* __restrict__ kv_lens) {
  constexpr int DG = D / 8;             // d-groups of 8 (score and P.V phases)
  constexpr int KG = 256 / DG;          // key groups
  __shared__ float qs[GM][D];
  __shared__ float ps[GM][kDecChunk];
  __shared__ float red[KG][D];
  __shared__ float stat[GM][2];
  __shared__ float wred[4];

  const int cpb = B / kDecChunk;
  const int sg = (int)(blockIdx.x % nsg);
  const int rest = (int)(blockIdx.x / nsg);
  const int u = rest % umax, c = rest / umax;
  if (u >= ucount[sg] || c >= cpb) return;
  const int s = sg / Hkv, g = sg % Hkv, G = H / Hkv;
  const int j = ublk[(int64_t)sg * umax + u];
  const uint32_t mask = umask[(int64_t)sg * umax + u];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t key0 = (int64_t)j * B + (int64_t)c * kDecChunk;
  const int64_t item = ((int64_t)sg * umax + u) * (B / kDecChunk) + c;
  // keys of this chunk that exist: a chunk of a partial last block may hold
  // fewer than kDecChunk, or none (then its partial is empty: max -inf).
  // With kv_lens the sequence's cache ends at its own length (clamped to
  // [1, L]); L stays the row count of the cache.
  int64_t Ls = L;
  if (kv_lens != nullptr) {
    const int64_t x = kv_lens[s];
    Ls = x < 1 ? 1 : (x > L ? L : x);
  }
  const int nkey = Ls - key0 >= kDecChunk ? kDecChunk : (Ls > key0 ? (int)(Ls - key0) : 0);
  if (nkey == 0) {
    for (int hl = 0; hl < G && hl < GM; ++hl) {
      if (!((mask >> hl) & 1u)) continue;
      float* prow = part + (item * GM + hl) * (D + 2);
      for (int dd = tid; dd < D + 2; dd += 256) prow[dd] = dd == 0 ? -__builtin_inff() : 0.f;
    }
    return;
  }

  for (int e = tid; e < G * D; e += 256) {
    const int hl = e / D, dd = e % D;
    qs[hl][dd] = load_as_f32(q + ((int64_t)s * H + g * G + hl) * D + dd) * scale_log2;
  }
  __syncthreads();

  // scores (base 2, scale folded into q).  Thread (key group kg, dim group
  // dg): the DG lanes of a key group read one key row's D elements
  // contiguously (16 bytes each; a wave load covers whole rows), multiply
  // their 8 dims with the query slices, and add the partial dots across the
  // group with butterfly shuffles.
  constexpr int SU = 4;                   // keys in flight per thread
  constexpr int LPRS = sizeof(T) == 2 ? 1 : 2;   // 16-byte loads per 8 elements
  {
    const int dgs = tid % DG, kgs = tid / DG;
    const T* kb = k + (((int64_t)s * L + key0) * Hkv + g) * D + dgs * 8;
    float qv[GM][8];
#pragma unroll
    for (int hl = 0; hl < GM; ++hl)
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[hl][i] = hl < G ? qs[hl][dgs * 8 + i] : 0.f;
    for (int kb0 = kgs; kb0 < kDecChunk; kb0 += KG * SU) {
      u32x4 raw[SU][LPRS];
#pragma unroll
      for (int uu = 0; uu < SU; ++uu) {
        const int kk = kb0 + uu * KG;     // a key past the end re-reads the last row (masked)
        const T* krow = kb + (int64_t)(kk < nkey ? kk : nkey - 1) * Hkv * D;
#pragma unroll
        for (int l2 = 0; l2 < LPRS; ++l2)
          raw[uu][l2] = *reinterpret_cast<const u32x4*>(krow + l2 * (8 / LPRS));
      }
#pragma unroll
      for (int uu = 0; uu < SU; ++uu) {
        const int kk = kb0 + uu * KG;
        float x[8];
#pragma unroll
        for (int l2 = 0; l2 < LPRS; ++l2) {
          const T* e = reinterpret_cast<const T*>(&raw[uu][l2]);
#pragma unroll
          for (int i = 0; i < 8 / LPRS; ++i) x[l2 * (8 / LPRS) + i] = load_as_f32(e + i);
        }
#pragma unroll
        for (int hl = 0; hl < GM; ++hl) {
          if (!(hl < G && ((mask >> hl) & 1u))) continue;   // uniform
          float part = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) part = fmaf(x[i], qv[hl][i], part);
#pragma unroll
          for (int o = DG / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
          if (dgs == 0) ps[hl][kk] = kk < nkey ? part : -__builtin_inff();
        }
      }
    }
  }
  __syncthreads();

  // chunk-local softmax statistics per selected head
  for (int hl = 0; hl < G && hl < GM; ++hl) {
    if (!((mask >> hl) & 1u)) continue;
    float mx = -__builtin_inff();
    for (int key = tid; key < kDecChunk; key += 256) mx = fmaxf(mx, ps[hl][key]);
    mx = wave_max(mx);
    if (lane == 0) wred[w] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
    __syncthreads();
    float sum = 0.f;
    for (int key = tid; key < kDecChunk; key += 256) {
      const float p = __builtin_amdgcn_exp2f(ps[hl][key] - mx);
      ps[hl][key] = p;
      sum += p;
    }
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) wred[w] = sum;
    __syncthreads();
    if (tid == 0) {
      stat[hl][0] = mx;
      stat[hl][1] = wred[0] + wred[1] + wred[2] + wred[3];
    }
    __syncthreads();
  }

  // P.V: thread (key group kg, d group dg)
  const int dg = tid % DG, kg = tid / DG;
  const T* vb = v + (((int64_t)s * L + key0) * Hkv + g) * D + dg * 8;
  float o[GM][8];
#pragma unroll
  for (int hl = 0; hl < GM; ++hl)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[hl][i] = 0.f;
  constexpr int VU = 8;                 // keys whose V rows are in flight together
  constexpr int LPR = sizeof(T) == 2 ? 1 : 2;   // 16-byte loads per 8 elements
  for (int key0 = kg; key0 < kDecChunk; key0 += KG * VU) {
    u32x4 raw[VU][LPR];
#pragma unroll
    for (int uu = 0; uu < VU; ++uu) {
      const int kv = key0 + uu * KG;  // past the end: the last row, with p = 0
      const T* vrow = vb + (int64_t)(kv < nkey ? kv : nkey - 1) * Hkv * D;
#pragma unroll
      for (int l2 = 0; l2 < LPR; ++l2)
        raw[uu][l2] = *reinterpret_cast<const u32x4*>(vrow + l2 * (8 / LPR));
    }
#pragma unroll
    for (int uu = 0; uu < VU; ++uu) {
      const int key = key0 + uu * KG;
      float x[8];
#pragma unroll
      for (int l2 = 0; l2 < LPR; ++l2) {
        const T* e = reinterpret_cast<const T*>(&raw[uu][l2]);
#pragma unroll
        for (int i = 0; i < 8 / LPR; ++i) x[l2 * (8 / LPR) + i] = load_as_f32(e + i);
      }
#pragma unroll
      for (int hl = 0; hl < GM; ++hl) {
        if (hl < G && ((mask >> hl) & 1u)) {
          const float p = ps[hl][key];
#pragma unroll
          for (int i = 0; i < 8; ++i) o[hl][i] = fmaf(p, x[i], o[hl][i]);
        }
      }
    }
  }
  // reduce over key groups, one head at a time; write (max, sum, o)
#pragma unroll
  for (int hl = 0; hl < GM; ++hl) {
    if (!(hl < G && ((mask >> hl) & 1u))) continue;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) red[kg][dg * 8 + i] = o[hl][i];
    __syncthreads();
    float* prow = part + (item * GM + hl) * (D + 2);
    for (int dd = tid; dd < D; dd += 256) {
      float acc = 0.f;
      for (int r = 0; r < KG; ++r) acc += red[r][dd];
      prow[2 + dd] = acc;
    }
    if (tid == 0) {
      prow[0] = stat[hl][0];
      prow[1] = stat[hl][1];
    }
  }
}

// grid S*H, D threads.  Wave 0 lists this head's partials in a fixed order
// (union slot, then chunk); the max, the weights and the sum of the partials
// are then workgroup reductions, and the weighted sum of the partial rows
// keeps eight loads in flight (fixed order: deterministic).
template <typename T, int D, int GM>
__global__ __launch_bounds__(D) void k_decode_merge(const float* __restrict__ part,
                                                    const int32_t* __restrict__ ublk,
                                                    const uint32_t* __restrict__ umask,
                                                    const int32_t* __restrict__ ucount,
                                                    T* __restrict__ out,
                                                    float* __restrict__ lse_out, int H, int Hkv,
                                                    int B, int umax) {
  __shared__ int items[kMergeMaxItems];
  __shared__ float wts[kMergeMaxItems];
  __shared__ int nitems_s;
  __shared__ float red_s[D / 64];
  const int sh = blockIdx.x, s = sh / H, h = sh % H, G = H / Hkv, g = h / G, hl = h % G;
  const int sg = s * Hkv + g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int cpb = B / kDecChunk;
  const int n = ucount[sg];
  if (tid < 64) {
    int base = 0;
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    for (int i0 = 0; i0 < n * cpb; i0 += 64) {
      const int i = i0 + lane;
      const bool ok = i < n * cpb && ((umask[(int64_t)sg * umax + i / cpb] >> hl) & 1u);
      const uint64_t bal = __ballot(ok);
      const int idx = base + __popcll(bal & lt);
      if (ok && idx < kMergeMaxItems) items[idx] = (int)(((int64_t)sg * umax + i / cpb) * cpb + i % cpb);
      base += __popcll(bal);
    }
    if (lane == 0) nitems_s = base < kMergeMaxItems ? base : kMergeMaxItems;
  }
  __syncthreads();
  const int ni = nitems_s;
  constexpr int NWV = D / 64;  // waves in the workgroup
  // max of the partial maxima, then the weights and the weighted sum of the
  // partial sums: one item per thread per pass, reduced across the workgroup
  float M = -__builtin_inff();
  for (int t = tid; t < ni; t += D) M = fmaxf(M, part[((int64_t)items[t] * GM + hl) * (D + 2)]);
  M = wave_max(M);
  if (lane == 0) red_s[tid >> 6] = M;
  __syncthreads();
  M = red_s[0];
#pragma unroll
  for (int i = 1; i < NWV; ++i) M = fmaxf(M, red_s[i]);
  float lp = 0.f;
  for (int t = tid; t < ni; t += D) {
    const float* prow = part + ((int64_t)items[t] * GM + hl) * (D + 2);
    const float wv = __builtin_amdgcn_exp2f(prow[0] - M);
    wts[t] = wv;
    lp = fmaf(wv, prow[1], lp);
  }
  for (int o = 32; o >= 1; o >>= 1) lp += __shfl_xor(lp, o);
  __syncthreads();  // M read by every thread before red_s is reused; wts complete
  if (lane == 0) red_s[tid >> 6] = lp;
  __syncthreads();
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < NWV; ++i) lsum += red_s[i];
  // o: eight partial rows in flight, eight accumulators, fixed order
  float acc8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc8[e] = 0.f;
  int t = 0;
  for (; t + 8 <= ni; t += 8) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = part[((int64_t)items[t + e] * GM + hl) * (D + 2) + 2 + tid];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc8[e] = fmaf(wts[t + e], x[e], acc8[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (t + e < ni)
      acc8[e] = fmaf(wts[t + e], part[((int64_t)items[t + e] * GM + hl) * (D + 2) + 2 + tid],
                     acc8[e]);
  const float acc = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) +
                    ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
  const float r = acc / lsum;
  if (lse_out != nullptr && tid == 0) lse_out[sh] = (M + __log2f(lsum)) * kLn2;
  T* orow = out + ((int64_t)s * H + h) * D;
  if (sizeof(T) == 2)
    reinterpret_cast<bf16_t*>(orow)[tid] = f32_to_bf16(r);
  else
    reinterpret_cast<float*>(orow)[tid] = r;
}

hipError_t launch_decode_plan(const int32_t* sel, int32_t* ublk, uint32_t* umask,
                              int32_t* ucount, bool all_blocks, const Dims& d, hipStream_t st) {
  hipLaunchKernelGGL(k_decode_plan, dim3(d.S * d.Hkv), dim3(64), d.nb * sizeof(uint32_t), st, sel,
                     ublk, umask, ucount, d.H, d.Hkv, d.nb, d.topk, decode_umax(d),
                     all_blocks ? 1 : 0);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t decode_attn_gm(const void* q, const void* k, const void* v,
                                 const int32_t* ublk, const uint32_t* umask,
                                 const int32_t* ucount, float* part, const Dims& d,
                                 hipStream_t st) {
  const int umax = decode_umax(d);
  const int nsg = d.S * d.Hkv;
  const int64_t nwg = (int64_t)nsg * umax * (d.B / kDecChunk);
  const float sl2 = kLog2e / sqrtf((float)d.D);
#define MOBA_DEC(GMV)                                                                      \
  hipLaunchKernelGGL((k_decode_attn<T, D, GMV>), dim3((unsigned)nwg), dim3(256), 0, st,    \
                     static_cast<const T*>(q), static_cast<const T*>(k),                   \
                     static_cast<const T*>(v), ublk, umask, ucount, part, d.L, d.H, d.Hkv, \
                     d.B, umax, sl2, nsg, d.kv_lens)
  switch (decode_gm(d)) {
    case 1: MOBA_DEC(1); break;
    case 2: MOBA_DEC(2); break;
    case 4: MOBA_DEC(4); break;
    default: MOBA_DEC(8); break;
  }
#undef MOBA_DEC
  return hipGetLastError();
}

hipError_t launch_decode_attn(const void* q, const void* k, const void* v, const int32_t* ublk,
                              const uint32_t* umask, const int32_t* ucount, float* part,
                              const Dims& d, hipStream_t st) {
  if (d.bf16) {
    if (d.D == 128) return decode_attn_gm<bf16_t, 128>(q, k, v, ublk, umask, ucount, part, d, st);
    return decode_attn_gm<bf16_t, 64>(q, k, v, ublk, umask, ucount, part, d, st);
  }
  if (d.D == 128) return decode_attn_gm<float, 128>(q, k, v, ublk, umask, ucount, part, d, st);
  return decode_attn_gm<float, 64>(q, k, v, ublk, umask, ucount, part, d, st);
}

template <typename T, int D>
static hipError_t decode_merge_gm(const float* part, const int32_t* ublk, const uint32_t* umask,
                                  const int32_t* ucount, void* out, const Dims& d,
                                  hipStream_t st, float* lse_out) {
  const int umax = decode_umax(d);
#define MOBA_DM(GMV)                                                                         \
  hipLaunchKernelGGL((k_decode_merge<T, D, GMV>), dim3(d.S * d.H), dim3(D), 0, st, part, ublk, \
                     umask, ucount, static_cast<T*>(out), lse_out, d.H, d.Hkv, d.B, umax)
  switch (decode_gm(d)) {
    case 1: MOBA_DM(1); break;
    case 2: MOBA_DM(2); break;
    case 4: MOBA_DM(4); break;
    default: MOBA_DM(8); break;
  }
#undef MOBA_DM
  return hipGetLastError();
}

hipError_t launch_decode_merge(const float* part, const int32_t* ublk, const uint32_t* umask,
                               const int32_t* ucount, void* out, const Dims& d,
                               hipStream_t st, float* lse_out) {
  if (d.bf16) {
    if (d.D == 128)
      return decode_merge_gm<bf16_t, 128>(part, ublk, umask, ucount, out, d, st, lse_out);
    return decode_merge_gm<bf16_t, 64>(part, ublk, umask, ucount, out, d, st, lse_out);
  }
  if (d.D == 128)
    return decode_merge_gm<float, 128>(part, ublk, umask, ucount, out, d, st, lse_out);
  return decode_merge_gm<float, 64>(part, ublk, umask, ucount, out, d, st, lse_out);
}

}  // namespace moba
