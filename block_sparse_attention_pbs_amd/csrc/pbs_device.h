// Device-side building blocks shared by the PBS-Attn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bf16 pair (RNE), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_bits(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving map of a float32 onto uint32 for sorting by value DESCENDING with ties to
// the lower index: the returned 64-bit key sorts ascending.  -0 and +0 map to the same key;
// NaN maps below every number (sorts last).
__device__ __forceinline__ uint64_t desc_sort_key(float f, uint32_t index) {
  uint32_t u = __float_as_uint(f);
  uint32_t ord;
  if (f != f) {
    ord = 0u;
  } else {
    if ((u & 0x7fffffffu) == 0u) u = 0u;
    ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return (static_cast<uint64_t>(~ord) << 32) | index;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// In-LDS bitonic sort, ascending, of n2 (power of two) 64-bit keys by the whole block.
__device__ __forceinline__ void bitonic_sort_lds(uint64_t* keys, int n2) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int t = tid; t < (n2 >> 1); t += nt) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const uint64_t a = keys[lo], b = keys[hi];
        if ((a > b) == up) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
    }
  }
  __syncthreads();
}

// Sequence of token p in a packed batch row of T tokens: [lo, hi) with lo <= p < hi.  `cu` holds
// the n + 1 sequence starts (cu[0] = 0, cu[n] = T); without it the whole row is one sequence.  A
// binary search over cu (every lane of a wave looks up the same p, so the loads are uniform);
// malformed boundaries are clamped so that every derived index stays inside the row.
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int n, int T, int p, int& lo,
                                           int& hi) {
  if (cu == nullptr) {
    lo = 0;
    hi = T;
    return;
  }
  int a = 0, b = n;   // the last s in [0, n) with cu[s] <= p
  while (b - a > 1) {
    const int m = (a + b) >> 1;
    if (cu[m] <= p) a = m;
    else b = m;
  }
  lo = min(max(cu[a], 0), p);
  hi = max(min(cu[a + 1], T), p + 1);
}

}  // namespace pbs
