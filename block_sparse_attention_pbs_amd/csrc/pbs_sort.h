// Register-resident bitonic sorting network and lane exchanges shared by the segment sort
// (pbs_permute) and the coverage ranking (pbs_block_select), gfx950 / CDNA4, wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbs {

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
    // The partner of element t*E + r (thread t) is element (t ^ stride/E)*E + r.  The keys go
    // through LDS register-major (slot r*T + t for T = 64*W threads), so the 64 lanes of a wave
    // touch 64 consecutive slots on both sides of the exchange (no bank conflicts).
    static_assert(W > 1, "a partner in another wave needs W > 1");
    constexpr int T = 64 * W;
    const int t = e0 / E;
    const bool take_min = ((e0 & stride) == 0) == ((e0 & size) == 0);
    __syncthreads();   // the previous readers of lds are done
#pragma unroll
    for (int r = 0; r < E; ++r) lds[r * T + t] = x[r];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const uint64_t y = lds[r * T + (t ^ (stride / E))];
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
// (W*64*E keys, laid out register-major; two workgroup barriers per step).  With W = 1 no LDS
// and no barrier is used.
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

}  // namespace pbs
