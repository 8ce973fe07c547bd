// Device-side helpers shared by the MoBA HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

typedef uint16_t bf16_t;  // storage type of bfloat16 values in HBM
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
// Native 16-byte vector for raw loads/stores (HIP's uint4 struct can keep
// values out of registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, b);
}

__device__ __forceinline__ float load_as_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_as_f32(const bf16_t* p) { return bf16_to_f32(*p); }

// 32x32x16 bf16 MFMA, fp32 accumulate.
//   A (32 x 16): lane l holds row l%32 and 8 contraction slots for half l/32.
//   B (16 x 32): lane l holds column l%32 and the same 8 slots.
//   C (32 x 32): lane l holds column l%32; register 4i+j is row 8i+4(l/32)+j.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Key order used when K is the A operand of S^T = K Q^T: A row m carries key
// kperm(m), which swaps bits 2 and 3 of m.  Then accumulator registers
// [8c, 8c+8) of lane half h hold keys 16c + 8h + [0, 8) in order, which is the
// B-operand layout of P^T for the following P.V product.
__device__ __forceinline__ int kperm(int m) {
  return (m & 0x13) | ((m & 0x8) >> 1) | ((m & 0x4) << 1);
}

// Key (0..31 inside a 32-key subtile) held by accumulator register `reg` of
// lane half `h` under the kperm order.
__device__ __forceinline__ int acc_key(int reg, int h) {
  const int i = reg >> 2, j = reg & 3;
  return 16 * (i >> 1) + 8 * h + 4 * (i & 1) + j;
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float half_swap(float x) { return __shfl_xor(x, 32); }

// ---------------------------------------------------------------------------
// Register top-K list of (score, block) pairs, best first.  Order: larger
// score first; equal scores keep the lower block index first.
// ---------------------------------------------------------------------------
template <int KM>
struct TopList {
  float s[KM];
  int i[KM];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      s[t] = -__builtin_inff();
      i[t] = 0x7fffffff;
    }
  }
  // Insert a candidate whose block index is larger than every index already
  // in the list: strict '>' then implements the lower-index tie-break.
  __device__ __forceinline__ void insert_ascending(float x, int j) {
#pragma unroll
    for (int t = KM - 1; t >= 0; --t) {
      const bool gt = x > s[t];
      const bool gtp = (t == 0) ? false : (x > s[t > 0 ? t - 1 : 0]);
      const float ps = s[t > 0 ? t - 1 : 0];
      const int pi = i[t > 0 ? t - 1 : 0];
      s[t] = gt ? (gtp ? ps : x) : s[t];
      i[t] = gt ? (gtp ? pi : j) : i[t];
    }
  }
  // Insert a candidate in any index order (full tie-break compare).
  __device__ __forceinline__ static bool before(float x, int xi, float y, int yi) {
    return x > y || (x == y && xi < yi);
  }
  __device__ __forceinline__ void insert_any(float x, int j) {
#pragma unroll
    for (int t = KM - 1; t >= 0; --t) {
      const int tp = t > 0 ? t - 1 : 0;
      const bool gt = before(x, j, s[t], i[t]);
      const bool gtp = (t == 0) ? false : before(x, j, s[tp], i[tp]);
      const float ps = s[tp];
      const int pi = i[tp];
      s[t] = gt ? (gtp ? ps : x) : s[t];
      i[t] = gt ? (gtp ? pi : j) : i[t];
    }
  }
  // Keep only the first `keep` entries (the list may have more slots than
  // the number of blocks to keep).
  __device__ __forceinline__ void truncate(int keep) {
#pragma unroll
    for (int t = 0; t < KM; ++t) {
      if (t >= keep) {
        s[t] = -__builtin_inff();
        i[t] = 0x7fffffff;
      }
    }
  }
  // Sort the block indices ascending (invalid entries hold INT_MAX and end up last).
  __device__ __forceinline__ void sort_indices() {
#pragma unroll
    for (int pass = 0; pass < KM; ++pass) {
#pragma unroll
      for (int t = (pass & 1); t + 1 < KM; t += 2) {
        const int a = i[t], b = i[t + 1];
        i[t] = a < b ? a : b;
        i[t + 1] = a < b ? b : a;
      }
    }
  }
};

}  // namespace moba
