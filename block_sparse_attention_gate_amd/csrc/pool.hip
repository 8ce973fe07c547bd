// Block-mean pooling of K and the V layout transform.
//
// Block means feed the gate: the MoBA pages divide the context into blocks
// and gate every query against every block ("MoBA" project card, "How It
// Works"); the affinity is read here as the dot product with the block's
// mean key.  A last block that holds fewer than block_size keys is averaged
// over the keys it holds.  The V transform writes V^T [batch, Hkv, D, Lv]
// (Lv = L rounded up to a multiple of 64, the columns past L zero) so that
// the P.V product of the attention kernels reads 8 consecutive keys per lane
// and whole 64-key tiles.
#include "common.h"
#include "kernels.h"

namespace moba {

// Keys of block j: B, or what is left of L for a partial last block.
__device__ __forceinline__ int block_keys(int64_t L, int B, int j) {
  const int64_t left = L - (int64_t)j * B;
  return left < B ? (int)left : B;
}

// grid ((nb - j0) * splits, S, column groups); 256 threads: blocks j0 .. nb-1.
// Workgroup (j, split) accumulates VEC columns over rows
// [split*rows, (split+1)*rows) of block j in fp32; the row slices inside the
// workgroup are summed in a fixed order.  splits == 1 writes the mean
// directly; otherwise the per-split sums go to `partial`
// [S, nb - j0, splits, Hkv*D] and k_block_mean_finalize adds them in split
// order (deterministic, no atomics).
template <typename T>
__device__ __forceinline__ void block_mean_body(const T* __restrict__ k, float* __restrict__ kbar,
                                                float* __restrict__ partial, int Hkv, int D,
                                                int64_t L, int B, int nb, int j0, int splits,
                                                int bx, int s, int bz, float* red) {
  constexpr int VEC = 16 / sizeof(T);
  const int cols = Hkv * D;
  const int tpr = cols / VEC;
  const int cw = tpr < 256 ? tpr : 256;  // threads across columns
  const int RS = 256 / cw;               // row slices
  const int tid = threadIdx.x;
  const int ct = tid % cw, rs = tid / cw;
  const int jl = bx / splits, sp = bx % splits;
  const int j = j0 + jl, nbl = nb - j0;
  const int rows = B / splits;
  // rows of this split that exist (a partial last block has fewer)
  const int64_t first = (int64_t)j * B + (int64_t)sp * rows;
  const int nrow = L - first >= rows ? rows : (L > first ? (int)(L - first) : 0);
  const int col = (bz * cw + ct) * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  if (rs < RS && col < cols) {
    const T* base = k + ((int64_t)s * L + first) * cols + col;
    for (int r = rs; r < nrow; r += RS) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(base + (int64_t)r * cols);
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] += load_as_f32(e + v);
    }
  }
  const int width = cw * VEC;
  if (rs < RS) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[rs * width + ct * VEC + v] = acc[v];
  }
  __syncthreads();
  const float inv = 1.0f / (float)block_keys(L, B, j);
  for (int e = tid; e < width; e += 256) {
    const int c = bz * width + e;
    if (c >= cols) continue;
    float sum = 0.f;
    for (int r = 0; r < RS; ++r) sum += red[r * width + e];
    if (splits == 1) {
      const int g = c / D, dd = c % D;
      kbar[(((int64_t)s * Hkv + g) * nb + j) * D + dd] = sum * inv;
    } else {
      partial[(((int64_t)s * nbl + jl) * splits + sp) * cols + c] = sum;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_block_mean(const T* __restrict__ k,
                                                    float* __restrict__ kbar,
                                                    float* __restrict__ partial, int Hkv, int D,
                                                    int64_t L, int B, int nb, int j0,
                                                    int splits) {
  __shared__ float red[256 * (16 / sizeof(T))];
  block_mean_body<T>(k, kbar, partial, Hkv, D, L, B, nb, j0, splits, blockIdx.x, blockIdx.y,
                     blockIdx.z, red);
}

// Sum of the split partials of one column in split order (fixed order: the
// result does not depend on scheduling); loads are issued 8 at a time.
__device__ __forceinline__ float sum_splits(const float* __restrict__ p, int splits,
                                            int64_t stride) {
  float sum = 0.f;
  int sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(sp + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; sp < splits; ++sp) sum += p[(int64_t)sp * stride];
  return sum;
}

// grid (nb - j0, S); 256 threads.
__global__ __launch_bounds__(256) void k_block_mean_finalize(const float* __restrict__ partial,
                                                             float* __restrict__ kbar, int Hkv,
                                                             int D, int64_t L, int B, int nb,
                                                             int j0, int splits) {
  const int s = blockIdx.y, jl = blockIdx.x, j = j0 + jl, nbl = nb - j0, cols = Hkv * D;
  const float inv = 1.0f / (float)block_keys(L, B, j);
  for (int c = threadIdx.x; c < cols; c += 256) {
    const float sum =
        sum_splits(partial + ((int64_t)s * nbl + jl) * splits * cols + c, splits, cols);
    const int g = c / D, dd = c % D;
    kbar[(((int64_t)s * Hkv + g) * nb + j) * D + dd] = sum * inv;
  }
}

hipError_t launch_block_mean(const void* k, float* kbar, float* partial, const Dims& d,
                             hipStream_t st, bool defer_finalize, int j0) {
  if (j0 < 0 || j0 >= d.nb || (defer_finalize && j0 != 0)) return hipErrorInvalidValue;
  const int nbl = d.nb - j0;
  const int cols = d.Hkv * d.D;
  const int vec = d.bf16 ? 8 : 4;
  const int tpr = cols / vec;
  const int splits = block_mean_splits(d);
  dim3 grid(nbl * splits, d.S, (tpr + 255) / 256);
  if (d.bf16)
    hipLaunchKernelGGL(k_block_mean<bf16_t>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(k), kbar, partial, d.Hkv, d.D, d.L, d.B, d.nb,
                       j0, splits);
  else
    hipLaunchKernelGGL(k_block_mean<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(k), kbar, partial, d.Hkv, d.D, d.L, d.B, d.nb,
                       j0, splits);
  if (splits > 1 && !defer_finalize)
    hipLaunchKernelGGL(k_block_mean_finalize, dim3(nbl, d.S), dim3(256), 0, st, partial, kbar,
                       d.Hkv, d.D, d.L, d.B, d.nb, j0, splits);
  return hipGetLastError();
}

// V [S, L, Hkv, D] -> V^T [S, Hkv, D, Lv] (bf16), 64 keys of one KV head;
// keys past L (the tail of the last tile) are written as zeros.  The last
// tile of a sequence whose length is not a multiple of 64 also copies its K
// rows of head g to ktail [S, 64, Hkv, D] (rows past L zero), which the
// query kernels read instead of K for that tile.
template <int D>
__device__ __forceinline__ void transpose_body(const bf16_t* __restrict__ k,
                                               const bf16_t* __restrict__ v,
                                               bf16_t* __restrict__ vt,
                                               bf16_t* __restrict__ ktail, int Hkv, int64_t L,
                                               int64_t Lv, int64_t key0, int g, int s,
                                               bf16_t* tile) {
  constexpr int LD = D + 8;
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;  // 16-byte chunks per key row
  const int64_t nkey = L - key0;  // keys of this tile that exist (>= 1)
  if (nkey < 64) {
    for (int c = tid; c < 64 * CPR; c += 256) {
      const int row = c / CPR, cc = c % CPR;
      u32x4 val = u32x4{0u, 0u, 0u, 0u};
      if (row < nkey)
        val = *reinterpret_cast<const u32x4*>(
            k + (((int64_t)s * L + key0 + row) * Hkv + g) * D + cc * 8);
      *reinterpret_cast<u32x4*>(ktail + (((int64_t)s * 64 + row) * Hkv + g) * D + cc * 8) = val;
    }
  }
  for (int c = tid; c < 64 * CPR; c += 256) {
    const int row = c / CPR, cc = c % CPR;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (row < nkey)
      val = *reinterpret_cast<const u32x4*>(
          v + (((int64_t)s * L + key0 + row) * Hkv + g) * D + cc * 8);
    *reinterpret_cast<u32x4*>(&tile[row * LD + cc * 8]) = val;
  }
  __syncthreads();
  for (int c = tid; c < D * 8; c += 256) {
    const int dd = c / 8, kc = c % 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[(kc * 8 + 2 * e) * LD + dd];
      const uint32_t hi = tile[(kc * 8 + 2 * e + 1) * LD + dd];
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(vt + (((int64_t)s * Hkv + g) * D + dd) * Lv + key0 + kc * 8) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
}

// grid (Lv/64, Hkv, S).  When bm_partial is given, workgroups (j < nb, g = 0)
// of sequence s also finish the block mean of block j from the split sums.
template <int D>
__global__ __launch_bounds__(256) void k_transpose_v(const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v,
                                                     bf16_t* __restrict__ vt,
                                                     bf16_t* __restrict__ ktail, int Hkv,
                                                     int64_t L, int64_t Lv,
                                                     const float* __restrict__ bm_partial,
                                                     float* __restrict__ kbar, int B, int nb,
                                                     int splits) {
  __shared__ bf16_t tile[64 * (D + 8)];
  const int g = blockIdx.y, s = blockIdx.z;
  if (bm_partial && g == 0 && (int)blockIdx.x < nb) {
    const int j = blockIdx.x, cols = Hkv * D;
    const float inv = 1.0f / (float)block_keys(L, B, j);
    for (int c = threadIdx.x; c < cols; c += 256) {
      const float sum =
          sum_splits(bm_partial + ((int64_t)s * nb + j) * splits * cols + c, splits, cols);
      kbar[(((int64_t)s * Hkv + c / D) * nb + j) * D + c % D] = sum * inv;
    }
  }
  transpose_body<D>(k, v, vt, ktail, Hkv, L, Lv, (int64_t)blockIdx.x * 64, g, s, tile);
}

// One launch for the K pooling (block sums or means) and the V transform:
// flat grid, the first npool workgroups pool (block_mean grid order), the rest
// transpose (transpose grid order).
template <int D>
__global__ __launch_bounds__(256) void k_pool_transpose(const bf16_t* __restrict__ k,
                                                        const bf16_t* __restrict__ v,
                                                        float* __restrict__ kbar,
                                                        float* __restrict__ partial,
                                                        bf16_t* __restrict__ vt,
                                                        bf16_t* __restrict__ ktail, int Hkv,
                                                        int64_t L, int64_t Lv, int B, int nb,
                                                        int splits, int pool_x, int pool_y,
                                                        int pool_z) {
  __shared__ __attribute__((aligned(16))) float lds[64 * (D + 8) / 2 > 256 * 8 ? 64 * (D + 8) / 2 : 256 * 8];
  const int npool = pool_x * pool_y * pool_z;
  const int b = blockIdx.x;
  if (b < npool) {
    const int bx = b % pool_x, by = (b / pool_x) % pool_y, bz = b / (pool_x * pool_y);
    block_mean_body<bf16_t>(k, kbar, partial, Hkv, D, L, B, nb, 0, splits, bx, by, bz, lds);
  } else {
    const int t = b - npool;
    const int ntile = (int)(Lv / 64);
    const int x = t % ntile, g = (t / ntile) % Hkv, s = t / (ntile * Hkv);
    transpose_body<D>(k, v, vt, ktail, Hkv, L, Lv, (int64_t)x * 64, g, s,
                      reinterpret_cast<bf16_t*>(lds));
  }
}

hipError_t launch_transpose_v(const void* k, const void* v, void* vt, void* ktail,
                              const Dims& d, hipStream_t st, const float* bm_partial,
                              float* kbar) {
  if (d.L % 64 != 0 && ktail == nullptr) return hipErrorInvalidValue;
  dim3 grid((unsigned)(d.Lv / 64), d.Hkv, d.S);
  const int splits = bm_partial ? block_mean_splits(d) : 1;
  if (d.D == 128)
    hipLaunchKernelGGL(k_transpose_v<128>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                       static_cast<bf16_t*>(vt), static_cast<bf16_t*>(ktail), d.Hkv, d.L,
                       d.Lv, bm_partial, kbar, d.B, d.nb, splits);
  else
    hipLaunchKernelGGL(k_transpose_v<64>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                       static_cast<bf16_t*>(vt), static_cast<bf16_t*>(ktail), d.Hkv, d.L,
                       d.Lv, bm_partial, kbar, d.B, d.nb, splits);
  return hipGetLastError();
}

hipError_t launch_pool_transpose(const void* k, const void* v, float* kbar, float* partial,
                                 void* vt, void* ktail, const Dims& d, hipStream_t st) {
  if (d.L % 64 != 0 && ktail == nullptr) return hipErrorInvalidValue;
  const int cols = d.Hkv * d.D;
  const int tpr = cols / 8;
  const int splits = block_mean_splits(d);
  const int px = d.nb * splits, py = d.S, pz = (tpr + 255) / 256;
  const int64_t ntr = (d.Lv / 64) * d.Hkv * d.S;
  const dim3 grid((unsigned)((int64_t)px * py * pz + ntr));
  if (d.D == 128)
    hipLaunchKernelGGL(k_pool_transpose<128>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), kbar,
                       partial, static_cast<bf16_t*>(vt), static_cast<bf16_t*>(ktail), d.Hkv,
                       d.L, d.Lv, d.B, d.nb, splits, px, py, pz);
  else
    hipLaunchKernelGGL(k_pool_transpose<64>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), kbar,
                       partial, static_cast<bf16_t*>(vt), static_cast<bf16_t*>(ktail), d.Hkv,
                       d.L, d.Lv, d.B, d.nb, splits, px, py, pz);
  return hipGetLastError();
}

hipError_t launch_block_mean_finalize(float* kbar, const float* partial, const Dims& d,
                                      hipStream_t st) {
  const int splits = block_mean_splits(d);
  if (splits > 1)
    hipLaunchKernelGGL(k_block_mean_finalize, dim3(d.nb, d.S), dim3(256), 0, st, partial, kbar,
                       d.Hkv, d.D, d.L, d.B, d.nb, 0, splits);
  return hipGetLastError();
}

}  // namespace moba
