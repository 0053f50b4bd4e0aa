// pbs_permute: segmented argsort of the key scores and gather of the permuted K / V (gfx950).
//
// What it computes (arXiv 2510.21270; gist.science summary, Methodik 2: permutation only inside
// contiguous, non-overlapping segments of size S; Methodik 3 "Sortierung": keys in descending
// order of importance inside each segment; sciencestack.ai page, Lemma 3.1: keys and values
// move together): perm[p] = original position of the key at slot p; k_perm / v_perm are bit
// copies of the rows in that order.
//
// Kernels:
//  * seg_sort: one workgroup per (batch, KV head, segment).  The segment's scores become 64-bit
//    keys (order-preserving float bits, inverted for descending order, with the in-segment
//    position in the low word so equal scores keep their original order) and are sorted by a
//    bitonic network: held in registers by the workgroup's 16 waves, with only the steps between
//    waves going through LDS, when next_pow2(S) >= 1024; wholly in LDS for smaller segments
//    (S <= 16384 keys = 128 KiB).  The same pass writes the inverse
//    permutation (the slot of every original position), which the attention kernel walks to
//    read a query block's visible own-segment keys without searching the segment.
//  * gather: one workgroup per (batch, KV head, block of Bs slots).  16-byte lanes read whole
//    source rows (a row of K is contiguous, so every group of D/8 lanes issues one coalesced
//    row read) and write the permuted rows contiguously; the same pass produces the float32
//    mean of the block's keys (reduced through LDS) and the block's smallest original position.
#include "pbs_device.h"
#include "pbs_internal.h"
#include "pbs_sort.h"

namespace pbs {
namespace {

struct SortArgs {
  const float* scores;
  int32_t* perm;
  int32_t* inv;   // may be null
  int N, S, n2;
};

// Segments of 1024 <= next_pow2(S) = 1024*E <= 16384 keys: the 16 waves hold the keys in
// registers (E per lane) and sort them with bitonic_sort_regs, which needs the LDS only for the
// compare-exchange steps between waves (10 of the 91 steps at S = 8192).
template <int E>
__device__ __forceinline__ void seg_sort_regs(const SortArgs& a, uint64_t* lds, size_t base,
                                              int s0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e0 = tid * E;
  uint64_t x[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int p = e0 + r;
    x[r] = (p < a.S) ? desc_sort_key(a.scores[base + p], static_cast<uint32_t>(p)) : ~0ull;
  }
  bitonic_sort_regs<E, 16>(x, lane, wave, lds);
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int p = e0 + r;
    if (p < a.S) {
      const int32_t src = static_cast<int32_t>(x[r] & 0xffffffffull);   // position in segment
      a.perm[base + p] = s0 + src;
      if (a.inv) a.inv[base + src] = s0 + p;
    }
  }
}

__global__ __launch_bounds__(1024) void seg_sort_kernel(SortArgs a) {
  extern __shared__ uint64_t keys[];
  const int sigma = blockIdx.x;
  const size_t base = static_cast<size_t>(blockIdx.y) * a.N + static_cast<size_t>(sigma) * a.S;
  const int s0 = sigma * a.S;
  if (a.n2 >= 1024 && blockDim.x == 1024) {   // uniform: the launch picks the path
    switch (a.n2 >> 10) {
      case 1: seg_sort_regs<1>(a, keys, base, s0); return;
      case 2: seg_sort_regs<2>(a, keys, base, s0); return;
      case 4: seg_sort_regs<4>(a, keys, base, s0); return;
      case 8: seg_sort_regs<8>(a, keys, base, s0); return;
      default: seg_sort_regs<16>(a, keys, base, s0); return;
    }
  }
  for (int p = threadIdx.x; p < a.n2; p += blockDim.x)
    keys[p] = (p < a.S) ? desc_sort_key(a.scores[base + p], static_cast<uint32_t>(p)) : ~0ull;
  bitonic_sort_lds(keys, a.n2);
  for (int p = threadIdx.x; p < a.S; p += blockDim.x) {
    const int32_t src = static_cast<int32_t>(keys[p] & 0xffffffffull);   // position in segment
    a.perm[base + p] = s0 + src;
    if (a.inv) a.inv[base + src] = s0 + p;
  }
}

struct GatherArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm;
  uint16_t* k_perm;
  uint16_t* v_perm;
  float* k_pool;
  int32_t* minpos;
  int N, nb, Hkv;
  RowMap km;      // row addressing of k, v, k_perm and v_perm (either layout)
};

template <int D, int BS>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int RP = 256 / CH;     // rows per pass
  __shared__ float red[RP * D];
  __shared__ int32_t mins[256];
  const int tid = threadIdx.x;
  const int c = tid % CH, rg = tid / CH;
  const int j = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const size_t head = static_cast<size_t>(bh) * a.N;   // perm is [B, Hkv, N]
  float sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.f;
  int mn = 0x7fffffff;
#pragma unroll 4
  for (int r = rg; r < BS; r += RP) {
    const int pos = j * BS + r;
    const int src = a.perm[head + pos];
    mn = min(mn, src);
    const size_t so = a.km.off(b, h, src) + c * 8, po = a.km.off(b, h, pos) + c * 8;
    // non-temporal loads and stores: every source row is read once, every output row written once
    const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.k + so));
    const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v + so));
    __builtin_nontemporal_store(kv, reinterpret_cast<u32x4*>(a.k_perm + po));
    __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(a.v_perm + po));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sum[2 * e] += __uint_as_float(kv[e] << 16);
      sum[2 * e + 1] += __uint_as_float(kv[e] & 0xffff0000u);
    }
  }
  if (a.k_pool) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg * D + c * 8 + e] = sum[e];
  }
  mins[tid] = mn;
  __syncthreads();
  if (a.k_pool) {
    for (int dd = tid; dd < D; dd += 256) {
      float tot = 0.f;
      for (int q = 0; q < RP; ++q) tot += red[q * D + dd];
      a.k_pool[(static_cast<size_t>(bh) * a.nb + j) * D + dd] = tot / static_cast<float>(BS);
    }
  }
  if (a.minpos) {
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) mins[tid] = min(mins[tid], mins[tid + s]);
      __syncthreads();
    }
    if (tid == 0) a.minpos[static_cast<size_t>(bh) * a.nb + j] = mins[0];
  }
}

template <int D, int BS>
hipError_t launch_gather_t(const Dims& d, const GatherArgs& a, hipStream_t stream) {
  return launch(gather_kernel<D, BS>, dim3(d.nb, d.B * d.Hkv), dim3(256), 0, stream, a);
}

struct QGatherArgs {
  const uint16_t* q;
  const int32_t* perm;
  uint16_t* q_perm;
  int N, Hq, Hkv, G;
  RowMap qm;      // row addressing of q and q_perm (either layout)
};

// Queries moved with their tokens (the query-permutation variant): row p of query head g takes
// the query row perm[b, g / G, p] (sciencestack.ai page, Lemma 3.2; gist.science summary,
// Methodik 1, query permutation equivariance).  One workgroup per (batch * query head, 64 rows);
// D/8 lanes per row, each moving 16 bytes, so every row read and write is one coalesced run.
template <int D>
__global__ __launch_bounds__(256) void qgather_kernel(QGatherArgs a) {
  constexpr int CH = D / 8;
  constexpr int ROWS = 64;
  const int bg = blockIdx.y;                       // b * Hq + g
  const int b = bg / a.Hq, g = bg - b * a.Hq;
  const size_t phead = (static_cast<size_t>(b) * a.Hkv + g / a.G) * a.N;
  const int c = threadIdx.x % CH;
  for (int r = threadIdx.x / CH; r < ROWS; r += 256 / CH) {
    const int p = blockIdx.x * ROWS + r;
    if (p >= a.N) break;
    const int src = min(max(a.perm[phead + p], 0), a.N - 1);
    const u32x4 x =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.q + a.qm.off(b, g, src) + c * 8));
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(a.q_perm + a.qm.off(b, g, p) + c * 8));
  }
}

}  // namespace

hipError_t launch_permute_queries(const Dims& d, const int32_t* perm, const uint16_t* q,
                                  uint16_t* q_perm, hipStream_t stream) {
  QGatherArgs qa;
  qa.q = q; qa.perm = perm; qa.q_perm = q_perm;
  qa.N = d.N; qa.Hq = d.Hq; qa.Hkv = d.Hkv; qa.G = d.G;
  qa.qm = q_rows(d);
  const dim3 grid((d.N + 63) / 64, d.B * d.Hq);
  if (d.d == 128) return launch(qgather_kernel<128>, grid, dim3(256), 0, stream, qa);
  return launch(qgather_kernel<64>, grid, dim3(256), 0, stream, qa);
}

hipError_t launch_permute(const Dims& d, const float* scores, const uint16_t* k,
                          const uint16_t* v, int32_t* perm, uint16_t* k_perm, uint16_t* v_perm,
                          float* k_pool, int32_t* blk_minpos, int32_t* perm_inv,
                          hipStream_t stream) {
  SortArgs sa;
  sa.scores = scores; sa.perm = perm; sa.inv = perm_inv; sa.N = d.N; sa.S = d.S;
  int n2 = 1;
  while (n2 < d.S) n2 <<= 1;
  sa.n2 = n2;
  const size_t shmem = static_cast<size_t>(n2) * sizeof(uint64_t);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(seg_sort_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(shmem));
  if (e != hipSuccess) return e;
  const int threads = n2 >= 1024 ? 1024 : (n2 >= 64 ? n2 : 64);
  e = launch(seg_sort_kernel, dim3(d.nseg, d.B * d.Hkv), dim3(threads), shmem, stream, sa);
  if (e != hipSuccess) return e;
  GatherArgs ga;
  ga.k = k; ga.v = v; ga.perm = perm; ga.k_perm = k_perm; ga.v_perm = v_perm;
  ga.k_pool = k_pool; ga.minpos = blk_minpos; ga.N = d.N; ga.nb = d.nb; ga.Hkv = d.Hkv;
  ga.km = kv_rows(d);
  if (d.d == 128 && d.Bs == 128) return launch_gather_t<128, 128>(d, ga, stream);
  if (d.d == 128 && d.Bs == 64) return launch_gather_t<128, 64>(d, ga, stream);
  if (d.d == 64 && d.Bs == 128) return launch_gather_t<64, 128>(d, ga, stream);
  return launch_gather_t<64, 64>(d, ga, stream);
}

}  // namespace pbs
