// Gate and top-k selection.
//
// For every query token the gate scores each PAST block by the dot product
// of the query with the block's mean key; it is parameter-less and picks the
// best blocks per query token ("MoBA" project card, "How It Works").  A query
// never selects a future block and always keeps its own block, which is then
// causally masked (AiBoss MoBA article, "MoBAの技術的原則", causality design).
// The own block counts as one of the k; the best k-1 past blocks are kept,
// ties going to the lower block index.  Output: sel[s, h, r, 0..k) ascending,
// -1 padded.
#include "common.h"
#include "kernels.h"

namespace moba {

// bf16 queries: scores on MFMA.  S^T[block][query] = kbar . q with kbar split
// into three bf16 terms (hi + mid + lo reproduce the fp32 mean exactly up to
// fp32 rounding), so the scores carry fp32 accuracy.  Lane l owns query
// column l%32 and sees 16 of every 32 blocks; the two lane halves keep their
// own top list and merge at the end.  grid (ceil(Lq/128), S*H), 256 threads.
// With `counts` the workgroup (128 rows of one head = one routing chunk) also
// writes the routing histogram of its kept past blocks: counts[bucket][col]
// with col = (h - g*G) * nchunk_r + chunk (see route.hip).
template <int D, int KM, bool STAGE>
__global__ __launch_bounds__(256) void k_gate_topk_bf16(
    const bf16_t* __restrict__ q, const float* __restrict__ kbar, int32_t* __restrict__ sel,
    int64_t Lq, int64_t q_off, int H, int Hkv, int B, int nb, int topk,
    uint32_t* __restrict__ counts, int nchunk_r, int ncols) {
  extern __shared__ uint32_t ghist[];  // [nb] when counts != nullptr
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int sh = blockIdx.y, s = sh / H, h = sh % H, G = H / Hkv, g = h / G;
  if (counts) {
    for (int j = threadIdx.x; j < nb; j += 256) ghist[j] = 0u;
    __syncthreads();
  }
  const int64_t rbase = (int64_t)blockIdx.x * 128 + w * 32;
  const bool wave_on = rbase < Lq;
  const int64_t r = rbase + n;
  const bool valid = r < Lq;
  const int b = valid ? (int)((q_off + r) / B) : 0;
  const int kp = topk - 1;
  const int nkeep = kp < b ? kp : b;
  TopList<KM> top;
  top.init();
  const int tid = threadIdx.x;
  const int64_t rw0 = (int64_t)blockIdx.x * 128;
  const int64_t rwl = rw0 + 127 < Lq ? rw0 + 127 : Lq - 1;
  const int ntile = kp > 0 ? ((int)((q_off + rwl) / B) + 31) / 32 : 0;
  const int64_t rlast = wave_on ? (rbase + 31 < Lq ? rbase + 31 : Lq - 1) : 0;
  const int bmax = wave_on ? (int)((q_off + rlast) / B) : 0;
  const float* kb = kbar + ((int64_t)s * Hkv + g) * nb * D;
  bf16x8 qf[D / 16];
  {
    const bf16_t* qrow = q + (((int64_t)s * Lq + (valid ? r : 0)) * H + h) * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qf[t] = ld_bf16x8(qrow + 16 * t + 8 * hh);
      if (!valid) qf[t] = bf16x8{};
    }
  }
  // Many blocks (STAGE): the workgroup stages each 32-block tile of the block
  // means once, split into the three bf16 terms (hi, mid, lo: x = hi + mid +
  // lo exactly to within the last term's rounding), in LDS; the four waves
  // read their MFMA A operands from there instead of each re-reading and
  // re-splitting the fp32 rows.  Tiles run up to the workgroup's last query
  // block; a wave computes only the tiles below its own last query block.
  if constexpr (STAGE) {
    constexpr int KS = D + 8;                     // padded LDS row (elements)
    constexpr int CH = 32 * D / 4 / 256;          // float4 chunks per thread per tile
    __shared__ __attribute__((aligned(16))) bf16_t ktile[3][32 * KS];
    float4 xr[CH];
    auto fetch = [&](int jt) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + 256 * i, row = c / (D / 4), cc = c % (D / 4);
        const int jrow = jt * 32 + row < nb ? jt * 32 + row : nb - 1;
        xr[i] = *reinterpret_cast<const float4*>(kb + (int64_t)jrow * D + cc * 4);
      }
    };
    auto split_store = [&]() {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + 256 * i, row = c / (D / 4), cc = c % (D / 4);
        const float xs[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
        uint16_t p0[4], p1[4], p2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 hi = static_cast<__bf16>(xs[e]);
          const float r1 = xs[e] - static_cast<float>(hi);
          const __bf16 mid = static_cast<__bf16>(r1);
          const float r2 = r1 - static_cast<float>(mid);
          const __bf16 lo = static_cast<__bf16>(r2);
          p0[e] = __builtin_bit_cast(uint16_t, hi);
          p1[e] = __builtin_bit_cast(uint16_t, mid);
          p2[e] = __builtin_bit_cast(uint16_t, lo);
        }
        const int off = row * KS + cc * 4;
        *reinterpret_cast<uint2*>(&ktile[0][off]) =
            make_uint2(p0[0] | ((uint32_t)p0[1] << 16), p0[2] | ((uint32_t)p0[3] << 16));
        *reinterpret_cast<uint2*>(&ktile[1][off]) =
            make_uint2(p1[0] | ((uint32_t)p1[1] << 16), p1[2] | ((uint32_t)p1[3] << 16));
        *reinterpret_cast<uint2*>(&ktile[2][off]) =
            make_uint2(p2[0] | ((uint32_t)p2[1] << 16), p2[2] | ((uint32_t)p2[3] << 16));
      }
    };
    if (ntile > 0) fetch(0);
    for (int jt = 0; jt < ntile; ++jt) {
      __syncthreads();  // the previous tile is no longer read
      split_store();
      __syncthreads();
      if (jt + 1 < ntile) fetch(jt + 1);
      if (wave_on && jt * 32 < bmax) {
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const int off = n * KS + 16 * t + 8 * hh;
          acc = mfma32(ld_bf16x8(&ktile[0][off]), qf[t], acc);
          acc = mfma32(ld_bf16x8(&ktile[1][off]), qf[t], acc);
          acc = mfma32(ld_bf16x8(&ktile[2][off]), qf[t], acc);
        }
        // A candidate at or below a lane's last list entry leaves its list
        // unchanged, so the insertion (a compare-and-shift over the whole
        // list) is skipped when no lane of the wave has a better one: exact,
        // and once the lists fill (long contexts) most candidates skip.
#pragma unroll
        for (int reg = 0; reg < 16; ++reg) {
          const int j = jt * 32 + 8 * (reg >> 2) + 4 * hh + (reg & 3);
          const bool better = j < b && acc[reg] > top.s[KM - 1];
          if (__any(better)) {
            if (j < b) top.insert_ascending(acc[reg], j);
          }
        }
      }
    }
  } else {
    // few blocks (at most two tiles of 32): each wave reads and splits the
    // fp32 rows itself, and the kernel holds no LDS tile (it then shares CUs
    // with concurrent kernels more readily)
    if (wave_on && kp > 0) {
      for (int jt = 0; jt * 32 < bmax; ++jt) {
        const int jrow = (jt * 32 + n < nb) ? jt * 32 + n : nb - 1;
        const float* arow = kb + (int64_t)jrow * D + 8 * hh;
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const float4 x0 = *reinterpret_cast<const float4*>(arow + 16 * t);
          const float4 x1 = *reinterpret_cast<const float4*>(arow + 16 * t + 4);
          const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          bf16x8 a0, a1, a2;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 hi = static_cast<__bf16>(xs[e]);
            const float r1 = xs[e] - static_cast<float>(hi);
            const __bf16 mid = static_cast<__bf16>(r1);
            const float r2 = r1 - static_cast<float>(mid);
            a0[e] = hi;
            a1[e] = mid;
            a2[e] = static_cast<__bf16>(r2);
          }
          acc = mfma32(a0, qf[t], acc);
          acc = mfma32(a1, qf[t], acc);
          acc = mfma32(a2, qf[t], acc);
        }
#pragma unroll
        for (int reg = 0; reg < 16; ++reg) {
          const int j = jt * 32 + 8 * (reg >> 2) + 4 * hh + (reg & 3);
          const bool better = j < b && acc[reg] > top.s[KM - 1];
          if (__any(better)) {
            if (j < b) top.insert_ascending(acc[reg], j);
          }
        }
      }
    }
  }
  if (wave_on) {
    if (kp > 0) {
      // Merge the other lane half's list: snapshot it first, since both halves
      // rewrite their own lists while merging.
      float os[KM];
      int oi[KM];
#pragma unroll
      for (int t = 0; t < KM; ++t) {
        os[t] = half_swap(top.s[t]);
        oi[t] = __shfl_xor(top.i[t], 32);
      }
#pragma unroll
      for (int t = 0; t < KM; ++t) top.insert_any(os[t], oi[t]);
      top.truncate(kp);
      top.sort_indices();
    }
    if (valid && hh == 0) {
      int32_t* out = sel + (((int64_t)s * H + h) * Lq + r) * topk;
#pragma unroll
      for (int t = 0; t < KM + 1; ++t) {
        if (t < topk) {
          const int kept = (t < KM) ? top.i[t < KM ? t : 0] : 0;
          out[t] = t < nkeep ? kept : (t == nkeep ? b : -1);
          if (counts && t < nkeep) atomicAdd(&ghist[kept], 1u);
        }
      }
      for (int t = KM + 1; t < topk; ++t) out[t] = -1;
    }
  }
  if (counts) {
    __syncthreads();
    const int col = (h - g * G) * nchunk_r + blockIdx.x;
    for (int j = threadIdx.x; j < nb; j += 256)
      counts[(((int64_t)s * Hkv + g) * nb + j) * ncols + col] = ghist[j];
  }
}

// Wave-wide best (score, index) pair: larger score first, lower index on
// ties.  Butterfly over DPP lane moves (quad permutes, half-row and row
// mirrors) and the gfx950 16- and 32-lane swaps; every level combines each
// lane with a partner from the other half of its current group, so after six
// levels every lane holds the wave's best pair.
__device__ __forceinline__ void best_pair_step(float& s, int& i, float os, int oi) {
  if (os > s || (os == s && oi < i)) {
    s = os;
    i = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ void best_pair_dpp(float& s, int& i) {
  const float os = __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(s), CTRL, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xf, 0xf, false);
  best_pair_step(s, i, os, oi);
}
__device__ __forceinline__ void wave_best_pair(float& s, int& i) {
  best_pair_dpp<0xB1>(s, i);   // quad_perm [1,0,3,2]
  best_pair_dpp<0x4E>(s, i);   // quad_perm [2,3,0,1]
  best_pair_dpp<0x141>(s, i);  // row_half_mirror: lane l <-> 7 - l in each 8
  best_pair_dpp<0x140>(s, i);  // row_mirror: lane l <-> 15 - l in each 16
  {
    const auto rs = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s),
                                                     false, false);
    const auto ri = __builtin_amdgcn_permlane16_swap((uint32_t)i, (uint32_t)i, false, false);
    // each lane now sees its own pair and the one 16 lanes away, in some order
    float s0 = __uint_as_float(rs[0]);
    int i0 = (int)ri[0];
    best_pair_step(s0, i0, __uint_as_float(rs[1]), (int)ri[1]);
    s = s0;
    i = i0;
  }
  {
    const auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s),
                                                     false, false);
    const auto ri = __builtin_amdgcn_permlane32_swap((uint32_t)i, (uint32_t)i, false, false);
    float s0 = __uint_as_float(rs[0]);
    int i0 = (int)ri[0];
    best_pair_step(s0, i0, __uint_as_float(rs[1]), (int)ri[1]);
    s = s0;
    i = i0;
  }
}

// Decode (one query per head, bf16): one workgroup of four waves per
// (sequence, head).  Lane l of wave w scores the past blocks
// j = 64 w + l, + 256, ... with fp32 dot products (the block mean in fp32,
// the query widened from bf16) and keeps its own top list; each wave takes
// the k-1 best of its 64 lists one at a time (wave_best_pair on the list
// heads, after which the winning lane drops its head), and wave 0 takes the
// k-1 best of the four waves' candidates the same way.  The order is total
// (score descending, block index ascending), so the result is that of one
// list over all blocks.  grid S*H, 256 threads.
template <int D, int KM>
__global__ __launch_bounds__(256) void k_gate_topk_decode_bf16(
    const bf16_t* __restrict__ q, const float* __restrict__ kbar, int32_t* __restrict__ sel,
    int64_t L, int H, int Hkv, int B, int nb, int topk, const int32_t* __restrict__ kv_lens) {
  __shared__ float cand_s[4][KM];
  __shared__ int cand_i[4][KM];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sh = blockIdx.x;
  const int s = sh / H, h = sh % H, g = h / (H / Hkv);
  // the sequence's cache length (kv_lens: per sequence, clamped to [1, L])
  int64_t Ls = L;
  if (kv_lens != nullptr) {
    const int64_t x = kv_lens[s];
    Ls = x < 1 ? 1 : (x > L ? L : x);
  }
  const int b = (int)((Ls - 1) / B);  // own block of the query at the last position
  const int kp = topk - 1;
  const int nkeep = kp < b ? kp : b;
  // the k-1 best of the wave's lane lists, best first, into (bs, bi)[t]
  auto wave_take = [&](TopList<KM>& top, float (&bs)[KM], int (&bi)[KM]) {
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      bs[t] = -__builtin_inff();
      bi[t] = 0x7fffffff;
      if (t < nkeep) {
        float xs = top.s[0];
        int xi = top.i[0];
        wave_best_pair(xs, xi);
        bs[t] = xs;
        bi[t] = xi;
        if (top.i[0] == xi) {  // exactly one lane holds block xi
#pragma unroll
          for (int u = 0; u + 1 < KM; ++u) {
            top.s[u] = top.s[u + 1];
            top.i[u] = top.i[u + 1];
          }
          top.s[KM - 1] = -__builtin_inff();
          top.i[KM - 1] = 0x7fffffff;
        }
      }
    }
  };
  if (nkeep > 0) {
    float qr[D];
    const bf16_t* qrow = q + ((int64_t)s * H + h) * D;
#pragma unroll
    for (int dd = 0; dd < D; dd += 8) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + dd);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qr[dd + 2 * e] = __uint_as_float(raw[e] << 16);
        qr[dd + 2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
      }
    }
    TopList<KM> top;
    top.init();
    const float* kb = kbar + ((int64_t)s * Hkv + g) * nb * D;
    for (int j = 64 * w + lane; j < b; j += 256) {
      const float* kr = kb + (int64_t)j * D;
      float a = 0.f;
#pragma unroll
      for (int dd = 0; dd < D; dd += 4) {
        const float4 x = *reinterpret_cast<const float4*>(kr + dd);
        a = fmaf(qr[dd], x.x, a);
        a = fmaf(qr[dd + 1], x.y, a);
        a = fmaf(qr[dd + 2], x.z, a);
        a = fmaf(qr[dd + 3], x.w, a);
      }
      top.insert_ascending(a, j);
    }
    float bs[KM];
    int bi[KM];
    wave_take(top, bs, bi);
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < KM; ++t) {
        cand_s[w][t] = bs[t];
        cand_i[w][t] = bi[t];
      }
    }
  }
  __syncthreads();
  if (w != 0) return;
  int kept[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) kept[t] = 0x7fffffff;
  if (nkeep > 0) {
    // one candidate per lane (4 * KM <= 64), then the same extraction
    TopList<KM> top;
    top.init();
    if (lane < 4 * KM) {
      top.s[0] = cand_s[lane / KM][lane % KM];
      top.i[0] = cand_i[lane / KM][lane % KM];
    }
    float bs[KM];
    wave_take(top, bs, kept);
  }
  if (lane != 0) return;
  // ascending order (unused slots hold INT_MAX and stay last)
#pragma unroll
  for (int pass = 0; pass < KM; ++pass)
#pragma unroll
    for (int t = (pass & 1); t + 1 < KM; t += 2) {
      const int x = kept[t], y = kept[t + 1];
      kept[t] = x < y ? x : y;
      kept[t + 1] = x < y ? y : x;
    }
  int32_t* out = sel + ((int64_t)s * H + h) * topk;
#pragma unroll
  for (int t = 0; t < KM + 1; ++t) {
    if (t < topk) {
      const int kv = (t < KM) ? kept[t < KM ? t : 0] : 0;
      out[t] = t < nkeep ? kv : (t == nkeep ? b : -1);
    }
  }
  for (int t = KM + 1; t < topk; ++t) out[t] = -1;
}

// fp32 queries: one thread per query, fp32 FMA dot products.
// grid (ceil(Lq/256), S*H), 256 threads.
template <int D, int KM>
__global__ __launch_bounds__(256) void k_gate_topk_f32(
    const float* __restrict__ q, const float* __restrict__ kbar, int32_t* __restrict__ sel,
    int64_t Lq, int64_t q_off, int H, int Hkv, int B, int nb, int topk,
    const int32_t* __restrict__ kv_lens) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= Lq) return;
  const int sh = blockIdx.y, s = sh / H, h = sh % H, g = h / (H / Hkv);
  // kv_lens (decode batches, q_len 1): the query sits at the sequence's last
  // cache position, clamped to [0, kv_len)
  int64_t pos = q_off + r;
  if (kv_lens != nullptr) {
    const int64_t x = kv_lens[s];
    pos = (x < 1 ? 1 : (x > q_off + Lq ? q_off + Lq : x)) - 1;
  }
  const int b = (int)(pos / B);
  const int kp = topk - 1;
  const int nkeep = kp < b ? kp : b;
  TopList<KM> top;
  top.init();
  if (kp > 0) {
    const float* qrow = q + (((int64_t)s * Lq + r) * H + h) * D;
    float qr[D];
#pragma unroll
    for (int dd = 0; dd < D; dd += 4) {
      const float4 x = *reinterpret_cast<const float4*>(qrow + dd);
      qr[dd] = x.x; qr[dd + 1] = x.y; qr[dd + 2] = x.z; qr[dd + 3] = x.w;
    }
    const float* kb = kbar + ((int64_t)s * Hkv + g) * nb * D;
    for (int j = 0; j < b; ++j) {
      const float* kr = kb + (int64_t)j * D;
      float acc = 0.f;
#pragma unroll
      for (int dd = 0; dd < D; dd += 4) {
        const float4 x = *reinterpret_cast<const float4*>(kr + dd);
        acc = fmaf(qr[dd], x.x, acc);
        acc = fmaf(qr[dd + 1], x.y, acc);
        acc = fmaf(qr[dd + 2], x.z, acc);
        acc = fmaf(qr[dd + 3], x.w, acc);
      }
      top.insert_ascending(acc, j);
    }
    top.truncate(kp);
    top.sort_indices();
  }
  int32_t* out = sel + (((int64_t)s * H + h) * Lq + r) * topk;
#pragma unroll
  for (int t = 0; t < KM + 1; ++t) {
    if (t < topk) {
      const int kept = (t < KM) ? top.i[t < KM ? t : 0] : 0;
      out[t] = t < nkeep ? kept : (t == nkeep ? b : -1);
    }
  }
  for (int t = KM + 1; t < topk; ++t) out[t] = -1;
}

template <int D>
static hipError_t gate_dispatch_d(const void* q, const float* kbar, int32_t* sel, const Dims& d,
                                  hipStream_t st, uint32_t* counts) {
  const int kp = d.topk - 1;
#define MOBA_GATE_CASE(KMV)                                                                  \
  if (kp <= KMV) {                                                                           \
    if (gate_uses_decode_kernel(d)) {                                                        \
      hipLaunchKernelGGL((k_gate_topk_decode_bf16<D, KMV>), dim3(d.S * d.H), dim3(256), 0,  \
                         st, static_cast<const bf16_t*>(q), kbar, sel, d.L, d.H, d.Hkv, d.B,  \
                         d.nb, d.topk, d.kv_lens);                                           \
    } else if (d.bf16) {                                                                     \
      dim3 grid((unsigned)((d.Lq + 127) / 128), d.S * d.H);                                  \
      if (d.nb > 64)                                                                         \
        hipLaunchKernelGGL((k_gate_topk_bf16<D, KMV, true>), grid, dim3(256),                \
                           counts ? d.nb * sizeof(uint32_t) : 0, st,                         \
                           static_cast<const bf16_t*>(q), kbar, sel, d.Lq, d.q_off, d.H,     \
                           d.Hkv, d.B, d.nb, d.topk, counts, d.nchunk_r, d.ncols);           \
      else                                                                                   \
        hipLaunchKernelGGL((k_gate_topk_bf16<D, KMV, false>), grid, dim3(256),               \
                           counts ? d.nb * sizeof(uint32_t) : 0, st,                         \
                           static_cast<const bf16_t*>(q), kbar, sel, d.Lq, d.q_off, d.H,     \
                           d.Hkv, d.B, d.nb, d.topk, counts, d.nchunk_r, d.ncols);           \
    } else {                                                                                 \
      dim3 grid((unsigned)((d.Lq + 255) / 256), d.S * d.H);                                  \
      hipLaunchKernelGGL((k_gate_topk_f32<D, KMV>), grid, dim3(256), 0, st,                  \
                         static_cast<const float*>(q), kbar, sel, d.Lq, d.q_off, d.H, d.Hkv,  \
                         d.B, d.nb, d.topk, d.kv_lens);                                      \
    }                                                                                        \
    return hipGetLastError();                                                                \
  }
  MOBA_GATE_CASE(1)
  MOBA_GATE_CASE(2)
  MOBA_GATE_CASE(4)
  MOBA_GATE_CASE(8)
  MOBA_GATE_CASE(12)
  MOBA_GATE_CASE(16)
#undef MOBA_GATE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gate_topk(const void* q, const float* kbar, int32_t* sel, const Dims& d,
                            hipStream_t st, uint32_t* counts) {
  if (counts && !gate_writes_counts(d)) return hipErrorInvalidValue;
  if (d.D == 128) return gate_dispatch_d<128>(q, kbar, sel, d, st, counts);
  return gate_dispatch_d<64>(q, kbar, sel, d, st, counts);
}

}  // namespace moba
