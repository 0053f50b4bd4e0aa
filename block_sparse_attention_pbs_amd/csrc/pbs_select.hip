// pbs_block_select: per query block, which earlier-segment key blocks to compute (gfx950).
//
// What it computes (arXiv 2510.21270; gist.science summary, Methodik 4 "Block-Auswahl": block
// importance estimated by mean pooling on the permuted keys; sciencestack.ai page, Fig. 1 caption:
// own-segment blocks are always computed, inter-segment blocks may be skipped, and Fig. 2
// caption: coverage is the attention mass of the selected blocks; skillmd.com page,
// Implementation Steps: the active-block count max(1, int(num_blocks * keep))):
//   P[i, j] = softmax over candidates j < seg(i)*bps of scale * <qbar_i, kbar_j>,
// ranked by P descending (ties to the lower j); keep ratio r keeps max(1, floor(r*n)) of them,
// coverage tau keeps the shortest prefix whose sequential float32 sum reaches tau.  Optionally key
// block 0 (the block of the first tokens, where the attention sink lands) is ranked ahead of
// every other candidate; the pages name a first-token mask in the authors' code without defining
// it (codewithpapers.app record), and this is its plainest reading.  With several sequences
// packed along N, the candidates are the earlier-segment blocks of the query block's own
// sequence (block 0 above is then the sequence's first block).
//
// Kernels:
//  * pool: float32 mean of every block of Bs key rows, when the caller has no pooled keys from
//    pbs_permute.  HBM-bound, one workgroup per (head, block).
//  * select: one workgroup per (query block, up to 4 query heads of one KV head), one wave per
//    head.  The workgroup first pools its query blocks (the query rows are read from HBM while the
//    other workgroups of the CU rank their rows).  Logits are plain fp32 dot products (n <= 8192
//    candidates x d) computed by the whole workgroup, so each pooled key is read once for the
//    group; after one barrier every row is
//    its wave's own: softmax with wave reductions; keep ratio: the top-k set from a radix select
//    over the ranking keys with a per-row histogram in LDS (no sort); coverage: a bitonic sort
//    of next_pow2(n) 64-bit keys (in registers for 64 <= next_pow2(n) <= 1024, else in LDS) and
//    one strictly sequential fp32 coverage sum (so it is bit-identical to any other sequential
//    fp32 sum of the same values); the kept blocks are compacted in ascending order with a wave
//    scan.  No workgroup barrier after the logits.
#include <algorithm>
#include <cmath>

#include "pbs_device.h"
#include "pbs_internal.h"
#include "pbs_sort.h"

namespace pbs {
namespace {

struct PoolArgs {
  const uint16_t* x;
  float* out;
  int N, nb, H;
  RowMap xm;      // row addressing of x (either layout)
};

template <int D, int BS>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  constexpr int CH = D / 8;
  constexpr int RP = 256 / CH;
  __shared__ float red[RP * D];
  const int tid = threadIdx.x;
  const int c = tid % CH, rg = tid / CH;
  const int j = blockIdx.x;
  const int b = blockIdx.y / a.H, h = blockIdx.y - b * a.H;
  const size_t rs = static_cast<size_t>(a.xm.stride());
  const uint16_t* x0 = a.x + a.xm.off(b, h, j * BS) + c * 8;
  float sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.f;
  // every row load of the thread in flight at once (BS / RP of them); non-temporal: the rows are
  // read once here, and the whole tensor is far larger than L2 and MALL
  u32x4 rows[BS / RP];
#pragma unroll
  for (int q = 0; q < BS / RP; ++q)
    rows[q] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(x0 + static_cast<size_t>(rg + q * RP) * rs));
#pragma unroll
  for (int q = 0; q < BS / RP; ++q) {
    const u32x4 xv = rows[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sum[2 * e] += __uint_as_float(xv[e] << 16);
      sum[2 * e + 1] += __uint_as_float(xv[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * D + c * 8 + e] = sum[e];
  __syncthreads();
  for (int dd = tid; dd < D; dd += 256) {
    float tot = 0.f;
    for (int q = 0; q < RP; ++q) tot += red[q * D + dd];
    a.out[(static_cast<size_t>(blockIdx.y) * a.nb + j) * D + dd] = tot / static_cast<float>(BS);
  }
}

struct SelArgs {
  const uint16_t* q;   // the queries (pooled here, block by block)
  RowMap qm;           // row addressing of q (either layout)
  const float* kbar;   // [B*Hkv, nb, D]
  float* P;            // [B*Hq, nb, nb] or null
  int32_t* counts;     // [B*Hq, nb]
  int32_t* idx;        // [B*Hq, nb, max_off]
  int Hq, Hkv, G, hpw, nb, bps, max_off, n2max;
  int mode;            // 0 keep ratio, 1 coverage
  int p_in;            // read P instead of computing it
  int keep_first;      // rank key block 0 ahead of every other candidate
  double param;
  const int32_t* cu;   // packed sequences: nseq + 1 starts along N, or null (one sequence)
  int nseq, N, bs;
  float tau_f;         // least float f with (double)f >= param (coverage)
  float scale;
};

// Synchronisation of the lanes of one wave around its LDS work: the LDS executes a wave's
// instructions in order, so only the compiler has to be kept from moving memory operations across
// this point (no hardware barrier is involved).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP moves: a Hillis-Steele scan inside
// each row of 16 lanes (shifts by 1, 2, 4, 8; lanes shifted in from before the row read 0), then
// the last lane of row 0 / row 2 added to rows 1 / 3 and lane 31 added to rows 2 and 3.
__device__ __forceinline__ int wave_scan_incl(int x, int /*lane*/) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15, rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31, rows 2, 3
  return x;
}

// One level of the logits' transposing butterfly (half-width HW, then the narrower levels): the
// lanes of a group exchange half of their partial sums with the lane HW away.
template <int HW, int TPC>
__device__ __forceinline__ void butterfly_levels(float (&part)[4][TPC], int sl) {
  const bool upper = (sl & HW) != 0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < HW; ++c) {
      const float send = upper ? part[r][c] : part[r][c + HW];
      const float keep = upper ? part[r][c + HW] : part[r][c];
      part[r][c] = keep + __uint_as_float(xor_lane<HW>(__float_as_uint(send)));
    }
  if constexpr (HW > 1) butterfly_levels<HW / 2, TPC>(part, sl);
}

// One chunk of the coverage sum: c runs through the chunk's 64 ranked values (staged in LDS by
// lane) one float32 addition at a time, strictly sequentially, every lane doing the same uniform
// work; returns the position (0..63) of the first value at which the running sum reaches tf, or
// -1, and leaves c at the sum after all 64 (values past the end of the row are +0).
__device__ __forceinline__ int seq_sum64(float& c, float pv, float* stage, int lane, float tf) {
  stage[lane] = pv;
  wave_sync();
  int first = -1;
#pragma unroll
  for (int e4 = 0; e4 < 16; ++e4) {
    const float4 v = reinterpret_cast<const float4*>(stage)[e4];
    c = __fadd_rn(c, v.x);
    first = (first < 0 && c >= tf) ? 4 * e4 : first;
    c = __fadd_rn(c, v.y);
    first = (first < 0 && c >= tf) ? 4 * e4 + 1 : first;
    c = __fadd_rn(c, v.z);
    first = (first < 0 && c >= tf) ? 4 * e4 + 2 : first;
    c = __fadd_rn(c, v.w);
    first = (first < 0 && c >= tf) ? 4 * e4 + 3 : first;
  }
  wave_sync();   // the stage is refilled by the next chunk
  return first;
}

// Per-row LDS of the select kernel (one wave per row), carved from the dynamic LDS: the ranking
// keys (64-bit for the coverage sort, their 32-bit top words for the keep-ratio select), the
// probabilities, the kept flags and a 256-bin histogram.
struct RowLds {
  uint64_t* keys;   // n2max entries (coverage) / n2max 32-bit words (keep ratio)
  float* P;         // n2max
  uint8_t* flag;    // n2max
  int32_t* hist;    // 256
};

__host__ __device__ inline size_t row_lds_bytes(int n2max, int mode) {
  const size_t key_bytes = (mode == 0 ? 4u : 8u) * static_cast<size_t>(n2max);
  return (key_bytes + 4u * n2max + n2max + 256u * 4u + 15u) & ~static_cast<size_t>(15);
}

__device__ __forceinline__ RowLds row_lds(unsigned char* base, int n2max, int mode, int r) {
  unsigned char* p = base + static_cast<size_t>(r) * row_lds_bytes(n2max, mode);
  RowLds L;
  L.keys = reinterpret_cast<uint64_t*>(p);
  p += (mode == 0 ? 4u : 8u) * static_cast<size_t>(n2max);
  L.hist = reinterpret_cast<int32_t*>(p);
  p += 256u * 4u;
  L.P = reinterpret_cast<float*>(p);
  p += 4u * n2max;
  L.flag = p;
  return L;
}

// The float32 mean of the Bs rows of query block i of query head g into dst[0, D) (LDS), with
// the same summation order as pool_kernel for 256 threads: thread t of the nt takes dims
// (t % CH)*8 .. +8 of rows t / CH, + RP, + 2 RP, ... (RP = nt / CH), added in row order, then the
// RP partial sums are added in order and divided by Bs.  red holds RP * D floats.  Every thread of
// the workgroup takes part (two workgroup barriers).
template <int D>
__device__ __forceinline__ void pool_query_block(const SelArgs& a, int b, int g, int i, float* red,
                                                 float* dst, int tid, int nt) {
  constexpr int CH = D / 8;
  const int RP = nt / CH;
  const int c = tid % CH, rg = tid / CH;
  const size_t rs = static_cast<size_t>(a.qm.stride());
  const uint16_t* x0 = a.q + a.qm.off(b, g, i * a.bs) + c * 8;
  float sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.f;
  for (int r0 = rg; r0 < a.bs; r0 += 8 * RP) {
    // up to 8 row loads in flight; non-temporal: the query rows are read once here
    u32x4 rows[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * RP;
      rows[u] = r < a.bs ? __builtin_nontemporal_load(
                               reinterpret_cast<const u32x4*>(x0 + static_cast<size_t>(r) * rs))
                         : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r0 + u * RP < a.bs) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[2 * e] += __uint_as_float(rows[u][e] << 16);
          sum[2 * e + 1] += __uint_as_float(rows[u][e] & 0xffff0000u);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * D + c * 8 + e] = sum[e];
  __syncthreads();
  for (int dd = tid; dd < D; dd += nt) {
    float tot = 0.f;
    for (int q = 0; q < RP; ++q) tot += red[q * D + dd];
    dst[dd] = tot / static_cast<float>(a.bs);
  }
  __syncthreads();   // dst is complete, and red may be refilled
}

// Coverage ranking of one row of n <= 64*E candidates (n2 = next_pow2(n) = 64*E) in registers:
// the ranking keys sorted by bitonic_sort_regs, the probabilities staged in LDS in ranking order,
// then the running float32 sum.  The sum is the same strictly sequential chain as seq_sum64, 64 values
// at a time; a chunk is first added without tracking where it crosses tf and, only if it ends at
// or past tf (or a value is negative or NaN, where the running sum need not grow), added again
// from its start with the tracking.  Sets the kept flags; returns the kept count.
template <int E>
__device__ __forceinline__ int coverage_regs(const RowLds& L, int n, int lane, bool keep_first,
                                             float tf) {
  uint64_t x[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int p = lane * E + r;
    x[r] = (p < n) ? ((keep_first && p == 0) ? 0ull : desc_sort_key(L.P[p], static_cast<uint32_t>(p)))
                   : ~0ull;
  }
  bitonic_sort_regs<E, 1>(x, lane, 0, nullptr);
  float* stage = reinterpret_cast<float*>(L.keys);
  bool odd = false;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int m = lane * E + r;
    const float pv = (m < n) ? L.P[static_cast<uint32_t>(x[r])] : 0.f;
    odd |= !(pv >= 0.f);
    stage[m] = pv;
  }
  const bool plain = __builtin_amdgcn_ballot_w64(odd) == 0;
  wave_sync();
  int kk = n;
  float c = 0.f;
  for (int m0 = 0; m0 < n; m0 += 64) {
    const float4* s4 = reinterpret_cast<const float4*>(stage + m0);
    if (plain) {
      const float c0 = c;
#pragma unroll
      for (int e4 = 0; e4 < 16; ++e4) {
        const float4 v = s4[e4];
        c = __fadd_rn(c, v.x);
        c = __fadd_rn(c, v.y);
        c = __fadd_rn(c, v.z);
        c = __fadd_rn(c, v.w);
      }
      if (c < tf) continue;
      c = c0;
    }
    int first = -1;
#pragma unroll
    for (int e4 = 0; e4 < 16; ++e4) {
      const float4 v = s4[e4];
      c = __fadd_rn(c, v.x);
      first = (first < 0 && c >= tf) ? 4 * e4 : first;
      c = __fadd_rn(c, v.y);
      first = (first < 0 && c >= tf) ? 4 * e4 + 1 : first;
      c = __fadd_rn(c, v.z);
      first = (first < 0 && c >= tf) ? 4 * e4 + 2 : first;
      c = __fadd_rn(c, v.w);
      first = (first < 0 && c >= tf) ? 4 * e4 + 3 : first;
    }
    if (first >= 0 && m0 + first < n) {
      kk = m0 + first + 1;
      break;
    }
  }
  for (int j = lane; j < n; j += 64) L.flag[j] = 0;
  wave_sync();
#pragma unroll
  for (int r = 0; r < E; ++r)
    if (lane * E + r < kk) L.flag[static_cast<uint32_t>(x[r])] = 1;
  wave_sync();
  return kk;
}

// One workgroup per (query block, group of hpw query heads sharing a KV head), one wave per head
// (row).  The heads of a group have the same candidates, so their logits are computed together
// (each pooled key is read once per workgroup); everything after that is the wave's own work on
// its row: softmax, ranking and compaction with wave reductions and scans, with no workgroup
// barrier.
template <int D, int MODE>
__global__ __launch_bounds__(256) void select_kernel(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int sub = tid >> 6, lane = tid & 63;   // row of the workgroup, lane of its wave
  const int i = blockIdx.x;
  const int groups = a.Hq / a.hpw;
  const int b = blockIdx.y / groups;
  const int g0 = (blockIdx.y - b * groups) * a.hpw;
  const int g = g0 + sub;                      // this row's query head
  const int h = g / a.G;
  // candidates: the blocks of earlier segments of the query block's own sequence
  const int seg_first = (i / a.bps) * a.bps;
  int seq_lo, seq_hi;
  seq_bounds(a.cu, a.nseq, a.N, i * a.bs, seq_lo, seq_hi);
  const int first = min(seq_lo / a.bs, seg_first);   // the sequence's first block
  const int n = seg_first - first;                    // candidates first .. seg_first - 1
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  const RowLds L = row_lds(smem, a.n2max, MODE, sub);
  const size_t row = (static_cast<size_t>(b) * a.Hq + g) * a.nb + i;
  float* prow = a.P ? a.P + row * a.nb : nullptr;

  if (n == 0) {   // the whole workgroup takes this branch (n depends on the query block only)
    if (lane == 0) a.counts[row] = 0;
    if (prow && !a.p_in)
      for (int j = lane; j < a.nb; j += 64) prow[j] = 0.f;
    return;
  }

  if (a.p_in) {
    for (int j = lane; j < n; j += 64) L.P[j] = prow[first + j];
    wave_sync();
  } else {
    // Logits of all hpw rows.  A group of TPC lanes holds the rows' pooled queries in 8-wide
    // slices of the head dimension and takes TPC candidates at a time: every lane forms the
    // partial dot products of its slice with each candidate (each candidate row is read by the
    // group as one contiguous run), then a transposing butterfly over the group sums them so that
    // lane sl ends with the full logits of candidate sl (one exchange per dot product instead of
    // log2(TPC)).
    constexpr int TPC = D / 8;
    const int nt = 64 * a.hpw;
    const int sl = tid % TPC, grp = tid / TPC;
    // The rows' pooled queries, pooled here from Q (the first LDS bytes, which the rows' areas
    // reuse once the pooled queries are in registers): the query rows are read while other
    // workgroups on the CU rank theirs.
    float* qlds = reinterpret_cast<float*>(smem);
    for (int r = 0; r < a.hpw; ++r)
      pool_query_block<D>(a, b, g0 + r, i, qlds + a.hpw * D, qlds + r * D, tid, nt);
    float qv[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < a.hpw) {
        const float4* qp = reinterpret_cast<const float4*>(qlds + r * D + sl * 8);
        const float4 x0 = qp[0], x1 = qp[1];
        qv[r][0] = x0.x; qv[r][1] = x0.y; qv[r][2] = x0.z; qv[r][3] = x0.w;
        qv[r][4] = x1.x; qv[r][5] = x1.y; qv[r][6] = x1.z; qv[r][7] = x1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[r][e] = 0.f;
      }
    }
    __syncthreads();   // every thread holds its pooled queries; the LDS goes to the rows
    const float* kb = a.kbar + ((static_cast<size_t>(b) * a.Hkv + h) * a.nb + first) * D;
    for (int j0 = grp * TPC; j0 < n; j0 += nt) {
      float part[4][TPC];
#pragma unroll
      for (int c = 0; c < TPC; ++c) {
        const int j = min(j0 + c, n - 1);
        const float4* kp = reinterpret_cast<const float4*>(kb + static_cast<size_t>(j) * D + sl * 8);
        const float4 k0 = kp[0], k1 = kp[1];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          part[r][c] = qv[r][0] * k0.x + qv[r][1] * k0.y + qv[r][2] * k0.z + qv[r][3] * k0.w +
                       qv[r][4] * k1.x + qv[r][5] * k1.y + qv[r][6] * k1.z + qv[r][7] * k1.w;
      }
      butterfly_levels<TPC / 2, TPC>(part, sl);
      const int j = j0 + sl;
      if (j < n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < a.hpw) row_lds(smem, a.n2max, MODE, r).P[j] = part[r][0] * a.scale;
    }
    __syncthreads();   // the only workgroup barrier: every row's logits are in place
    // softmax of this row (wave reductions)
    float lmax = -INFINITY;
    for (int j = lane; j < n; j += 64) lmax = fmaxf(lmax, L.P[j]);
    const float mx = wave_max(lmax);
    float lsum = 0.f;
    for (int j = lane; j < n; j += 64) {
      const float e = __expf(L.P[j] - mx);
      L.P[j] = e;
      lsum += e;
    }
    const float inv = 1.f / wave_sum(lsum);
    for (int j = lane; j < n; j += 64) {
      const float p = L.P[j] * inv;
      L.P[j] = p;
      if (prow) prow[first + j] = p;
    }
    if (prow)
      for (int j = lane; j < a.nb; j += 64)
        if (j < first || j >= seg_first) prow[j] = 0.f;
    wave_sync();
  }

  // Ranking keys: (descending P, ascending block) as one ascending 64-bit key whose top word is
  // the complemented orderable value of P and whose low word is the block; with keep_first,
  // block 0 gets key 0, below every real key (whose top word is never 0).
  int kk;
  if constexpr (MODE == 0) {
    // Keep ratio: the kk lowest keys, found without sorting.  A radix select over the top words
    // (4 passes of 8 bits, a 256-bin histogram per row in LDS) finds the kk-th lowest top word H
    // and how many keys with top word H belong to the kept set; those are the lowest blocks among
    // the keys equal to H (the low word is the block), taken by a scan in block order.  The kept
    // set is exactly the first kk of the full ranking.
    uint32_t* hi = reinterpret_cast<uint32_t*>(L.keys);
    for (int p = lane; p < n; p += 64)
      hi[p] = (a.keep_first && p == 0) ? 0u : static_cast<uint32_t>(desc_sort_key(L.P[p], 0u) >> 32);
    kk = max(1, min(static_cast<int>(floor(a.param * static_cast<double>(n))), n));
    uint32_t prefix = 0, pmask = 0;
    int need = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      L.hist[4 * lane] = 0;
      L.hist[4 * lane + 1] = 0;
      L.hist[4 * lane + 2] = 0;
      L.hist[4 * lane + 3] = 0;
      wave_sync();
      for (int p = lane; p < n; p += 64) {
        const uint32_t x = hi[p];
        if ((x & pmask) == prefix) atomicAdd(&L.hist[(x >> shift) & 255u], 1);
      }
      wave_sync();
      const int c0 = L.hist[4 * lane], c1 = L.hist[4 * lane + 1], c2 = L.hist[4 * lane + 2],
                c3 = L.hist[4 * lane + 3];
      const int mine = c0 + c1 + c2 + c3;
      const int incl = wave_scan_incl(mine, lane);
      const int excl = incl - mine;
      // the lane whose four bins hold the need-th key: its digit and the count below it
      int dgt = 4 * lane, below = excl;
      if (below + c0 < need) { below += c0; ++dgt;
        if (below + c1 < need) { below += c1; ++dgt;
          if (below + c2 < need) { below += c2; ++dgt; } } }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(excl < need && need <= incl);
      const int src = __builtin_ctzll(bal);
      dgt = __builtin_amdgcn_readlane(dgt, src);
      below = __builtin_amdgcn_readlane(below, src);
      prefix |= static_cast<uint32_t>(dgt) << shift;
      pmask |= 0xffu << shift;
      need -= below;
      wave_sync();   // the histogram is reset by the next pass
    }
    // keep every key below H and the first `need` keys equal to H in block order
    const uint32_t H = prefix;
    const int per = (n + 63) / 64;
    const int lo = min(lane * per, n), hend = min(lo + per, n);
    int eq = 0;
    for (int j = lo; j < hend; ++j) eq += (hi[j] == H);
    int rank = wave_scan_incl(eq, lane) - eq;
    for (int j = lo; j < hend; ++j) {
      const uint32_t x = hi[j];
      L.flag[j] = (x < H || (x == H && rank++ < need)) ? 1 : 0;
    }
    wave_sync();
  } else {
    // Coverage: the ranking as a bitonic sort of next_pow2(n) 64-bit keys in LDS by the row's
    // wave, then the shortest prefix whose running float32 sum reaches tau.  The sum is strictly
    // sequential (one rounding per element, in ranking order), 64 ranked values at a time.
    // (double)c >= tau is tested as c >= tf, tf the least float with (double)tf >= tau.
    const float tf = a.tau_f;
    float c = 0.f;
    kk = n;
    if (n2 >= 64 && n2 <= 1024) {   // n2 is uniform over the workgroup
      switch (n2 >> 6) {
        case 1: kk = coverage_regs<1>(L, n, lane, a.keep_first, tf); break;
        case 2: kk = coverage_regs<2>(L, n, lane, a.keep_first, tf); break;
        case 4: kk = coverage_regs<4>(L, n, lane, a.keep_first, tf); break;
        case 8: kk = coverage_regs<8>(L, n, lane, a.keep_first, tf); break;
        default: kk = coverage_regs<16>(L, n, lane, a.keep_first, tf); break;
      }
    } else {
    for (int p = lane; p < n2; p += 64)
      L.keys[p] = (p < n) ? ((a.keep_first && p == 0) ? 0ull : desc_sort_key(L.P[p], static_cast<uint32_t>(p)))
                          : ~0ull;
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        wave_sync();
        for (int t = lane; t < (n2 >> 1); t += 64) {
          const int lo = 2 * t - (t & (stride - 1));
          const int hi = lo + stride;
          const bool up = ((lo & size) == 0);
          const uint64_t x = L.keys[lo], y = L.keys[hi];
          if ((x > y) == up) {
            L.keys[lo] = y;
            L.keys[hi] = x;
          }
        }
      }
    }
    wave_sync();
    for (int m0 = 0; m0 < n; m0 += 64) {
      const int m = m0 + lane;
      const float pv = (m < n) ? L.P[static_cast<int>(L.keys[m] & 0xffffffffull)] : 0.f;
      const int hit = seq_sum64(c, pv, reinterpret_cast<float*>(L.hist), lane, tf);
      if (hit >= 0 && m0 + hit < n) {
        kk = m0 + hit + 1;
        break;
      }
    }
    for (int j = lane; j < n; j += 64) L.flag[j] = 0;
    wave_sync();
    for (int m = lane; m < kk; m += 64) L.flag[static_cast<int>(L.keys[m] & 0xffffffffull)] = 1;
    wave_sync();
    }
  }

  // ascending compaction: lane l of the row owns candidates [l*per, (l+1)*per)
  const int per = (n + 63) / 64;
  const int lo = min(lane * per, n), hend = min(lo + per, n);
  int cnt = 0;
  for (int j = lo; j < hend; ++j) cnt += L.flag[j];
  int pos = wave_scan_incl(cnt, lane) - cnt;
  int32_t* out = a.idx + row * a.max_off;
  for (int j = lo; j < hend; ++j)
    if (L.flag[j]) out[pos++] = first + j;
  if (lane == 0) a.counts[row] = kk;
}

template <int D, int BS>
hipError_t launch_pool_t(const uint16_t* x, float* out, int heads, const Dims& d,
                         hipStream_t stream) {
  PoolArgs pa;
  pa.x = x; pa.out = out; pa.N = d.N; pa.nb = d.nb; pa.H = heads;
  pa.xm = RowMap{d.layout, heads, d.N, d.d};
  return launch(pool_kernel<D, BS>, dim3(d.nb, d.B * heads), dim3(256), 0, stream, pa);
}

hipError_t launch_pool(const uint16_t* x, float* out, int heads, const Dims& d,
                       hipStream_t stream) {
  if (d.d == 128 && d.Bs == 128) return launch_pool_t<128, 128>(x, out, heads, d, stream);
  if (d.d == 128 && d.Bs == 64) return launch_pool_t<128, 64>(x, out, heads, d, stream);
  if (d.d == 64 && d.Bs == 128) return launch_pool_t<64, 128>(x, out, heads, d, stream);
  return launch_pool_t<64, 64>(x, out, heads, d, stream);
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t select_workspace_bytes(const Dims& d) {
  const size_t kbar = static_cast<size_t>(d.B) * d.Hkv * d.nb * d.d * sizeof(float);
  return align256(kbar);
}

hipError_t launch_block_select(const Dims& d, const uint16_t* q, const uint16_t* k_perm,
                               const float* k_pool, float scale, int mode, double param,
                               float* blk_scores, bool scores_in, bool keep_first, int32_t* counts,
                               int32_t* idx, void* ws, const int32_t* cu, int nseq,
                               hipStream_t stream) {
  float* kbar_ws = static_cast<float*>(ws);
  hipError_t e;
  const float* kbar = k_pool;
  if (!scores_in && !kbar) {   // pooled keys (the queries are pooled inside the select kernel)
    e = launch_pool(k_perm, kbar_ws, d.Hkv, d, stream);
    if (e != hipSuccess) return e;
    kbar = kbar_ws;
  }
  SelArgs sa;
  sa.q = q; sa.qm = q_rows(d); sa.kbar = kbar; sa.P = blk_scores; sa.counts = counts; sa.idx = idx;
  sa.Hq = d.Hq; sa.Hkv = d.Hkv; sa.G = d.G; sa.nb = d.nb; sa.bps = d.bps; sa.max_off = d.max_off;
  int n2 = 1;
  while (n2 < d.max_off) n2 <<= 1;
  sa.n2max = n2;
  // Heads per workgroup (one wave each): the largest of 4, 2, 1 that divides the group size and
  // keeps the workgroup's LDS within 64 KiB (at least two workgroups per CU).
  const size_t per_row = row_lds_bytes(n2, mode);
  int hpw = 4;
  while (hpw > 1 && (d.G % hpw != 0 || hpw * per_row > 65536)) hpw >>= 1;
  sa.hpw = hpw;
  sa.mode = mode; sa.p_in = scores_in ? 1 : 0; sa.param = param; sa.scale = scale;
  sa.keep_first = keep_first ? 1 : 0;
  sa.cu = cu; sa.nseq = nseq; sa.N = d.N; sa.bs = d.Bs;
  sa.tau_f = static_cast<float>(param);
  if (static_cast<double>(sa.tau_f) < param) sa.tau_f = std::nextafter(sa.tau_f, INFINITY);
  // the rows' areas; before them, the same bytes hold the pooled queries and the pooling sums
  const size_t pool_bytes =
      scores_in ? 0 : static_cast<size_t>(hpw + 64 * hpw / (d.d / 8)) * d.d * sizeof(float);
  const size_t shmem = std::max(hpw * per_row, pool_bytes);
  auto kern = d.d == 128 ? (mode == 0 ? select_kernel<128, 0> : select_kernel<128, 1>)
                         : (mode == 0 ? select_kernel<64, 0> : select_kernel<64, 1>);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shmem));
  if (e != hipSuccess) return e;
  return launch(kern, dim3(d.nb, d.B * (d.Hq / hpw)), dim3(64 * hpw), shmem, stream, sa);
}

}  // namespace pbs
