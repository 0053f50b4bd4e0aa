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
//  * pool: float32 mean of every block of Bs rows (queries; keys too when the caller has no
//    pooled keys from pbs_permute).  HBM-bound, one workgroup per (head, block).
//  * select: one workgroup per (query block, up to 4 query heads of one KV head), 256 threads per
//    head.  Logits are plain fp32 dot products (n <= 8192 candidates x d), the softmax uses
//    per-row reductions.  Keep ratio: the top-k set comes from a radix select over the ranking
//    keys (no sort).  Coverage: the ranking is a bitonic sort of next_pow2(n) 64-bit keys in LDS
//    and the coverage prefix is one strictly sequential fp32 sum (so it is bit-identical to any
//    other sequential fp32 sum of the same values).  The kept blocks are compacted in ascending
//    order with a per-row prefix scan.
#include <cmath>

#include "pbs_device.h"
#include "pbs_internal.h"

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
#pragma unroll 4
  for (int r = rg; r < BS; r += RP) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x0 + static_cast<size_t>(r) * rs);
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
  const float* qbar;   // [B*Hq, nb, D]
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

constexpr int kSub = 256;   // threads per row (one row = one query head of the workgroup)
static_assert(kSub == 256, "the radix select keeps one 8-bit histogram bin per thread of a row");

// Sum / max over the kSub threads of one row (sub = the row's index in the workgroup).  Every thread
// of the workgroup calls these together.
__device__ __forceinline__ float row_reduce_max(float v, float* red, int sub, int st) {
  v = wave_max(v);
  __syncthreads();
  if ((st & 63) == 0) red[sub * 4 + (st >> 6)] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[sub * 4], red[sub * 4 + 1]), fmaxf(red[sub * 4 + 2], red[sub * 4 + 3]));
}
__device__ __forceinline__ float row_reduce_sum(float v, float* red, int sub, int st) {
  v = wave_sum(v);
  __syncthreads();
  if ((st & 63) == 0) red[sub * 4 + (st >> 6)] = v;
  __syncthreads();
  return (red[sub * 4] + red[sub * 4 + 1]) + (red[sub * 4 + 2] + red[sub * 4 + 3]);
}

// Ascending bitonic sort of n2 (power of two) 64-bit keys by the kSub threads of one row; every
// thread of the workgroup takes part in the barriers.
__device__ __forceinline__ void bitonic_sort_row(uint64_t* keys, int n2, int st) {
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int t = st; t < (n2 >> 1); t += kSub) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const uint64_t x = keys[lo], y = keys[hi];
        if ((x > y) == up) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
    }
  }
  __syncthreads();
}

// One workgroup per (query block, group of hpw query heads sharing a KV head); kSub threads per
// head.  The heads of a group have the same candidates, so their logits read each pooled key once
// (through the cache) and their sorts run side by side.
template <int D>
__global__ __launch_bounds__(1024) void select_kernel(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ float red[4 * 4];
  __shared__ int32_t scan[4 * kSub];
  __shared__ int32_t kept[4];

  const int tid = threadIdx.x;
  const int sub = tid / kSub, st = tid - sub * kSub;
  const int i = blockIdx.x;
  const int groups = a.Hq / a.hpw;
  const int b = blockIdx.y / groups;
  const int g = (blockIdx.y - b * groups) * a.hpw + sub;   // this row's query head
  const int h = g / a.G;
  // candidates: the blocks of earlier segments of the query block's own sequence
  const int seg_first = (i / a.bps) * a.bps;
  int seq_lo, seq_hi;
  seq_bounds(a.cu, a.nseq, a.N, i * a.bs, seq_lo, seq_hi);
  const int first = min(seq_lo / a.bs, seg_first);   // the sequence's first block
  const int n = seg_first - first;                    // candidates first .. seg_first - 1
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem) + static_cast<size_t>(sub) * a.n2max;
  float* Ps = reinterpret_cast<float*>(reinterpret_cast<uint64_t*>(smem) + static_cast<size_t>(a.hpw) * a.n2max) +
              static_cast<size_t>(sub) * a.n2max;
  int32_t* flag = reinterpret_cast<int32_t*>(Ps + static_cast<size_t>(a.hpw - sub) * a.n2max) +
                  static_cast<size_t>(sub) * a.n2max;
  const size_t row = (static_cast<size_t>(b) * a.Hq + g) * a.nb + i;
  float* prow = a.P ? a.P + row * a.nb : nullptr;

  if (n == 0) {   // the whole workgroup takes this branch (n depends on the query block only)
    if (st == 0) a.counts[row] = 0;
    if (prow && !a.p_in)
      for (int j = st; j < a.nb; j += kSub) prow[j] = 0.f;
    return;
  }

  if (a.p_in) {
    for (int j = st; j < n; j += kSub) Ps[j] = prow[first + j];
    __syncthreads();
  } else {
    // Logits of all hpw rows: TPC threads per candidate, each with an 8-wide slice of the head
    // dimension (the rows' pooled queries in registers), so a wave reads whole pooled-key rows
    // contiguously; the slices are summed across the TPC lanes.
    constexpr int TPC = D / 8;
    const int nt = kSub * a.hpw;
    const int cpi = nt / TPC;                   // candidates per sweep
    const int sl = tid % TPC, cj = tid / TPC;
    const size_t row0 = (static_cast<size_t>(b) * a.Hq + (g - sub)) * a.nb + i;   // first row
    float qv[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < a.hpw) {
        const float4* qp = reinterpret_cast<const float4*>(a.qbar + (row0 + static_cast<size_t>(r) * a.nb) * D + sl * 8);
        const float4 x0 = qp[0], x1 = qp[1];
        qv[r][0] = x0.x; qv[r][1] = x0.y; qv[r][2] = x0.z; qv[r][3] = x0.w;
        qv[r][4] = x1.x; qv[r][5] = x1.y; qv[r][6] = x1.z; qv[r][7] = x1.w;
      }
    }
    const float* kb = a.kbar + ((static_cast<size_t>(b) * a.Hkv + h) * a.nb + first) * D;
    float* Pall = reinterpret_cast<float*>(reinterpret_cast<uint64_t*>(smem) + static_cast<size_t>(a.hpw) * a.n2max);
#pragma unroll 2
    for (int j0 = 0; j0 < n; j0 += cpi) {
      const int j = j0 + cj;
      float4 k0 = make_float4(0.f, 0.f, 0.f, 0.f), k1 = k0;
      if (j < n) {
        const float4* kp = reinterpret_cast<const float4*>(kb + static_cast<size_t>(j) * D + sl * 8);
        k0 = kp[0];
        k1 = kp[1];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < a.hpw) {
          float acc = qv[r][0] * k0.x + qv[r][1] * k0.y + qv[r][2] * k0.z + qv[r][3] * k0.w +
                      qv[r][4] * k1.x + qv[r][5] * k1.y + qv[r][6] * k1.z + qv[r][7] * k1.w;
#pragma unroll
          for (int o = 1; o < TPC; o <<= 1) acc += __shfl_xor(acc, o);
          if (sl == 0 && j < n) Pall[static_cast<size_t>(r) * a.n2max + j] = acc * a.scale;
        }
      }
    }
    __syncthreads();
    float lmax = -INFINITY;
    for (int j = st; j < n; j += kSub) lmax = fmaxf(lmax, Ps[j]);
    const float mx = row_reduce_max(lmax, red, sub, st);
    float lsum = 0.f;
    for (int j = st; j < n; j += kSub) {
      const float e = __expf(Ps[j] - mx);
      Ps[j] = e;
      lsum += e;
    }
    const float tot = row_reduce_sum(lsum, red, sub, st);
    const float inv = 1.f / tot;
    for (int j = st; j < n; j += kSub) {
      const float p = Ps[j] * inv;
      Ps[j] = p;
      if (prow) prow[first + j] = p;
    }
    if (prow)
      for (int j = st; j < a.nb; j += kSub)
        if (j < first || j >= seg_first) prow[j] = 0.f;
    __syncthreads();
  }

  // Rank keys: (descending P, ascending block) as one ascending 64-bit key whose top word is the
  // complemented orderable value of P and whose low word is the block; with keep_first, block 0
  // gets key 0, below every real key (whose top word is never 0).
  if (a.mode == 0) {
    // Keep ratio: the kk lowest keys, found without sorting.  A radix select over the top words
    // (4 passes of 8 bits, per-row histograms in LDS) finds the kk-th lowest top word H and how
    // many keys with top word H belong to the kept set; those are the lowest blocks among the keys
    // equal to H (the low word is the block), taken by an exclusive scan in block order.  The kept
    // set is exactly the first kk of the full ranking.
    uint32_t* hi = reinterpret_cast<uint32_t*>(keys);
    for (int p = st; p < n; p += kSub)
      hi[p] = (a.keep_first && p == 0) ? 0u
                                       : static_cast<uint32_t>(desc_sort_key(Ps[p], 0u) >> 32);
    const int kk = max(1, min(static_cast<int>(floor(a.param * static_cast<double>(n))), n));
    int32_t* hist = scan + sub * kSub;      // 256 bins per row (kSub == 256)
    uint32_t prefix = 0, pmask = 0;
    int need = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[st] = 0;
      __syncthreads();
      for (int p = st; p < n; p += kSub) {
        const uint32_t x = hi[p];
        if ((x & pmask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1);
      }
      __syncthreads();
      if (st < 64) {   // the row's first wave finds the digit where the running count reaches need
        const int c0 = hist[4 * st], c1 = hist[4 * st + 1], c2 = hist[4 * st + 2], c3 = hist[4 * st + 3];
        const int mine = c0 + c1 + c2 + c3;
        int incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o);
          if (st >= o) incl += y;
        }
        const int excl = incl - mine;
        if (excl < need && need <= incl) {   // exactly one lane
          int dgt = 4 * st, below = excl;
          if (below + c0 < need) { below += c0; ++dgt;
            if (below + c1 < need) { below += c1; ++dgt;
              if (below + c2 < need) { below += c2; ++dgt; } } }
          red[sub * 4] = __int_as_float(dgt);
          red[sub * 4 + 1] = __int_as_float(need - below);
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(__float_as_int(red[sub * 4])) << shift;
      pmask |= 0xffu << shift;
      need = __float_as_int(red[sub * 4 + 1]);
      __syncthreads();
    }
    // keep every key below H and the first `need` keys equal to H in block order
    const uint32_t H = prefix;
    const int per = (n + kSub - 1) / kSub;
    const int lo = min(st * per, n), hi_end = min(lo + per, n);
    int eq = 0;
    for (int j = lo; j < hi_end; ++j) eq += (hi[j] == H);
    hist[st] = eq;
    __syncthreads();
    for (int off = 1; off < kSub; off <<= 1) {
      const int vv = (st >= off) ? hist[st - off] : 0;
      __syncthreads();
      hist[st] += vv;
      __syncthreads();
    }
    int rank = hist[st] - eq;
    for (int j = lo; j < hi_end; ++j) {
      const uint32_t x = hi[j];
      flag[j] = (x < H || (x == H && rank++ < need)) ? 1 : 0;
    }
    if (st == 0) kept[sub] = kk;
    __syncthreads();
  } else {
    for (int p = st; p < n2; p += kSub)
      keys[p] = (p < n) ? ((a.keep_first && p == 0) ? 0ull : desc_sort_key(Ps[p], static_cast<uint32_t>(p)))
                        : ~0ull;
    bitonic_sort_row(keys, n2, st);
  }

  if (a.mode == 0) {
    // flags are set
  } else if (st < 64) {
    // Shortest prefix of the ranking whose running float32 sum reaches tau: the sum is strictly
    // sequential (one rounding per element, in ranking order); the first wave of the row gathers
    // 64 ranked values at a time and adds them one by one from the lanes.  (double)c >= tau is
    // tested as c >= tf, tf the least float with (double)tf >= tau.
    const float tf = a.tau_f;
    float c = 0.f;
    int kk = n;
    for (int m0 = 0; m0 < n; m0 += 64) {
      const int m = m0 + st;
      const float pv = (m < n) ? Ps[static_cast<int>(keys[m] & 0xffffffffull)] : 0.f;
      const int cnt = min(64, n - m0);
      int e = 0;
      for (; e < cnt; ++e) {
        c = __fadd_rn(c, __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pv), e)));
        if (c >= tf) break;
      }
      if (e < cnt) {
        kk = m0 + e + 1;
        break;
      }
    }
    if (st == 0) kept[sub] = kk;
  }
  if (a.mode != 0) {
    for (int j = st; j < n; j += kSub) flag[j] = 0;
    __syncthreads();   // also publishes kept[sub] from the coverage scan
    const int kc = kept[sub];
    for (int m = st; m < kc; m += kSub) flag[static_cast<int>(keys[m] & 0xffffffffull)] = 1;
    __syncthreads();
  }
  const int kk = kept[sub];

  // ascending compaction: thread st of the row owns candidates [st*per, (st+1)*per)
  const int per = (n + kSub - 1) / kSub;
  const int lo = min(st * per, n), hi = min(lo + per, n);
  int cnt = 0;
  for (int j = lo; j < hi; ++j) cnt += flag[j];
  int32_t* sc = scan + sub * kSub;
  sc[st] = cnt;
  __syncthreads();
  for (int off = 1; off < kSub; off <<= 1) {
    const int v = (st >= off) ? sc[st - off] : 0;
    __syncthreads();
    sc[st] += v;
    __syncthreads();
  }
  int pos = sc[st] - cnt;
  int32_t* out = a.idx + row * a.max_off;
  for (int j = lo; j < hi; ++j)
    if (flag[j]) out[pos++] = first + j;
  if (st == 0) a.counts[row] = kk;
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
  const size_t qbar = static_cast<size_t>(d.B) * d.Hq * d.nb * d.d * sizeof(float);
  const size_t kbar = static_cast<size_t>(d.B) * d.Hkv * d.nb * d.d * sizeof(float);
  return align256(qbar) + align256(kbar);
}

hipError_t launch_block_select(const Dims& d, const uint16_t* q, const uint16_t* k_perm,
                               const float* k_pool, float scale, int mode, double param,
                               float* blk_scores, bool scores_in, bool keep_first, int32_t* counts,
                               int32_t* idx, void* ws, const int32_t* cu, int nseq,
                               hipStream_t stream) {
  float* qbar = static_cast<float*>(ws);
  float* kbar_ws = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                            align256(static_cast<size_t>(d.B) * d.Hq * d.nb * d.d * sizeof(float)));
  hipError_t e;
  const float* kbar = k_pool;
  if (!scores_in) {
    e = launch_pool(q, qbar, d.Hq, d, stream);
    if (e != hipSuccess) return e;
    if (!kbar) {
      e = launch_pool(k_perm, kbar_ws, d.Hkv, d, stream);
      if (e != hipSuccess) return e;
      kbar = kbar_ws;
    }
  }
  SelArgs sa;
  sa.qbar = qbar; sa.kbar = kbar; sa.P = blk_scores; sa.counts = counts; sa.idx = idx;
  sa.Hq = d.Hq; sa.Hkv = d.Hkv; sa.G = d.G; sa.nb = d.nb; sa.bps = d.bps; sa.max_off = d.max_off;
  int n2 = 1;
  while (n2 < d.max_off) n2 <<= 1;
  sa.n2max = n2;
  // Heads per workgroup: the largest of 4, 2, 1 that divides the group size and keeps the
  // workgroup's LDS within 64 KiB (two workgroups per CU).
  const size_t per_row = static_cast<size_t>(n2) * (sizeof(uint64_t) + sizeof(float) + sizeof(int32_t));
  int hpw = 4;
  while (hpw > 1 && (d.G % hpw != 0 || hpw * per_row > 65536)) hpw >>= 1;
  sa.hpw = hpw;
  sa.mode = mode; sa.p_in = scores_in ? 1 : 0; sa.param = param; sa.scale = scale;
  sa.keep_first = keep_first ? 1 : 0;
  sa.cu = cu; sa.nseq = nseq; sa.N = d.N; sa.bs = d.Bs;
  sa.tau_f = static_cast<float>(param);
  if (static_cast<double>(sa.tau_f) < param) sa.tau_f = std::nextafter(sa.tau_f, INFINITY);
  const size_t shmem = hpw * per_row;
  auto kern = d.d == 128 ? select_kernel<128> : select_kernel<64>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shmem));
  if (e != hipSuccess) return e;
  return launch(kern, dim3(d.nb, d.B * (d.Hq / hpw)), dim3(kSub * hpw), shmem, stream, sa);
}

}  // namespace pbs
