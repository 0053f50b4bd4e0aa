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

// v from lane (lane ^ M) of the wave.  M = 1, 2 and 8 are DPP moves on the vector ALU (quad
// permutations, and a rotation by 8 inside each row of 16 lanes, which is lane ^ 8); M = 4 and 16
// are LDS swizzles (xor masks inside each half-wave); M = 32 goes through ds_bpermute.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int x = static_cast<int>(v);
  if constexpr (M == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  } else if constexpr (M == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  } else if constexpr (M == 8) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
  } else if constexpr (M == 4 || M == 16) {
    return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(x, (M << 10) | 0x1F));
  } else {
    return static_cast<uint32_t>(__shfl_xor(x, M));
  }
}

// x from lane (lane ^ M) of the wave, for a 64-bit value.
template <int M>
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x) {
  const uint32_t lo = xor_lane<M>(static_cast<uint32_t>(x));
  const uint32_t hi = xor_lane<M>(static_cast<uint32_t>(x >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One compare-exchange step (merge size 2^LS, partner distance 2^LT) of bitonic_sort_regs, then
// the steps after it: the whole network is unrolled at compile time.
template <int E, int W, int LOGN, int LS, int LT>
__device__ __forceinline__ void bitonic_steps(uint64_t (&x)[E], int lane, int e0, uint64_t* lds) {
  constexpr int size = 1 << LS, stride = 1 << LT;
  if constexpr (stride < E) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
      if (r & stride) continue;
      const int r2 = r | stride;
      const bool up = (size < E) ? ((r & size) == 0) : ((e0 & size) == 0);
      const uint64_t u = x[r], v = x[r2];
      const bool sw = (u > v) == up;
      x[r] = sw ? v : u;
      x[r2] = sw ? u : v;
    }
  } else if constexpr (stride < 64 * E) {
    constexpr int LX = stride / E;
    const bool take_min = ((lane & LX) == 0) == ((e0 & size) == 0);
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const uint64_t y = shfl_xor64<LX>(x[r]);
      x[r] = ((x[r] < y) == take_min) ? x[r] : y;
    }
  } else {
    static_assert(W > 1, "a partner in another wave needs W > 1");
    const bool take_min = ((e0 & stride) == 0) == ((e0 & size) == 0);
    __syncthreads();   // the previous readers of lds are done
#pragma unroll
    for (int r = 0; r < E; ++r) lds[e0 + r] = x[r];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const uint64_t y = lds[(e0 + r) ^ stride];
      x[r] = ((x[r] < y) == take_min) ? x[r] : y;
    }
  }
  if constexpr (LT > 0) {
    bitonic_steps<E, W, LOGN, LS, LT - 1>(x, lane, e0, lds);
  } else if constexpr (LS < LOGN) {
    bitonic_steps<E, W, LOGN, LS + 1, LS>(x, lane, e0, lds);
  }
}

// Bitonic sort (ascending) of W*64*E 64-bit keys held in registers by the W waves of a
// workgroup: wave w, lane l holds element w*64*E + l*E + r in x[r].  Compare-exchange partners
// closer than E elements sit in the same lane, those closer than 64*E a lane xor away (exchanged
// by DPP moves, swizzles or ds_bpermute), the rest in another wave: those steps go through `lds`
// (W*64*E keys; two workgroup barriers per step).  With W = 1 no LDS and no barrier is used.
// Keys are distinct apart from equal padding, so the result is the unique ascending order.
template <int E, int W>
__device__ __forceinline__ void bitonic_sort_regs(uint64_t (&x)[E], int lane, int wave,
                                                  uint64_t* lds) {
  constexpr int LE = E == 1 ? 0 : E == 2 ? 1 : E == 4 ? 2 : E == 8 ? 3 : 4;
  static_assert((1 << LE) == E, "E must be 1, 2, 4, 8 or 16");
  constexpr int LW = W == 1 ? 0 : W == 2 ? 1 : W == 4 ? 2 : W == 8 ? 3 : 4;
  static_assert((1 << LW) == W, "W must be 1, 2, 4, 8 or 16");
  constexpr int LOGN = 6 + LE + LW;
  bitonic_steps<E, W, LOGN, 1, 0>(x, lane, (wave * 64 + lane) * E, lds);
  if constexpr (W > 1) __syncthreads();   // lds is free again
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
