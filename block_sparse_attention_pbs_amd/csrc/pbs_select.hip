// pbs_block_select: per query block, which earlier-segment key blocks to compute (gfx950).
//
// What it computes (arXiv 2510.21270; gist.science summary, Methodik 4 "Block-Auswahl": block
// importance estimated by mean pooling on the permuted keys; sciencestack.ai page, Fig. 1 caption:
// own-segment blocks are always computed, inter-segment blocks may be skipped, and Fig. 2
// caption: coverage is the attention mass of the selected blocks; skillmd.com page,
// Implementation Steps: the active-block count max(1, int(num_blocks * keep))):
//   P[i, j] = softmax over candidates j < seg(i)*bps of scale * <qbar_i, kbar_j>,
// ranked by P descending (ties to the lower j); keep ratio r keeps max(1, floor(r*n)) of them,
// coverage tau keeps the shortest prefix whose sequential float32 sum reaches tau.
//
// Kernels:
//  * pool: float32 mean of every block of Bs rows (queries; keys too when the caller has no
//    pooled keys from pbs_permute).  HBM-bound, one workgroup per (head, block).
//  * select: one workgroup per (query head, query block).  Logits are plain fp32 dot products
//    (n <= 8192 candidates x d), the softmax uses block-wide reductions, the ranking is a
//    bitonic sort of 64-bit keys in LDS, the coverage prefix is one strictly sequential fp32
//    sum (so it is bit-identical to any other sequential fp32 sum of the same values), and the
//    kept blocks are compacted in ascending order with a workgroup prefix scan.
#include "pbs_device.h"
#include "pbs_internal.h"

namespace pbs {
namespace {

struct PoolArgs {
  const uint16_t* x;
  float* out;
  int N, nb;
};

template <int D, int BS>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  constexpr int CH = D / 8;
  constexpr int RP = 256 / CH;
  __shared__ float red[RP * D];
  const int tid = threadIdx.x;
  const int c = tid % CH, rg = tid / CH;
  const int j = blockIdx.x;
  const size_t head = static_cast<size_t>(blockIdx.y) * a.N;
  float sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.f;
#pragma unroll 4
  for (int r = rg; r < BS; r += RP) {
    const u32x4 xv =
        *reinterpret_cast<const u32x4*>(a.x + (head + static_cast<size_t>(j) * BS + r) * D + c * 8);
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
  int Hq, Hkv, G, nb, bps, max_off, n2;
  int mode;            // 0 keep ratio, 1 coverage
  int p_in;            // read P instead of computing it
  double param;
  float scale;
};

constexpr int kSelThreads = 256;

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kSelThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < kSelThreads / 64; ++i) r += red[i];
  return r;
}

template <int D>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);                 // n2
  float* Ps = reinterpret_cast<float*>(keys + a.n2);                   // n2
  int32_t* flag = reinterpret_cast<int32_t*>(Ps + a.n2);               // n2
  __shared__ float qs[D];
  __shared__ float red[kSelThreads / 64];
  __shared__ int32_t scan[kSelThreads];
  __shared__ int32_t kept;

  const int tid = threadIdx.x;
  const int i = blockIdx.x;
  const int bg = blockIdx.y;                  // b * Hq + g
  const int b = bg / a.Hq, g = bg - b * a.Hq;
  const int h = g / a.G;
  const int n = (i / a.bps) * a.bps;          // candidates: blocks of earlier segments
  const size_t row = static_cast<size_t>(bg) * a.nb + i;
  float* prow = a.P ? a.P + row * a.nb : nullptr;

  if (n == 0) {
    if (tid == 0) a.counts[row] = 0;
    if (prow && !a.p_in)
      for (int j = tid; j < a.nb; j += kSelThreads) prow[j] = 0.f;
    return;
  }

  if (a.p_in) {
    for (int j = tid; j < n; j += kSelThreads) Ps[j] = prow[j];
    __syncthreads();
  } else {
    for (int dd = tid; dd < D; dd += kSelThreads) qs[dd] = a.qbar[row * D + dd];
    __syncthreads();
    const float* kb = a.kbar + (static_cast<size_t>(b) * a.Hkv + h) * a.nb * D;
    float lmax = -INFINITY;
    for (int j = tid; j < n; j += kSelThreads) {
      const float4* kr = reinterpret_cast<const float4*>(kb + static_cast<size_t>(j) * D);
      float acc = 0.f;
#pragma unroll 8
      for (int q4 = 0; q4 < D / 4; ++q4) {
        const float4 kv = kr[q4];
        acc += qs[4 * q4] * kv.x + qs[4 * q4 + 1] * kv.y + qs[4 * q4 + 2] * kv.z + qs[4 * q4 + 3] * kv.w;
      }
      const float lg = acc * a.scale;
      Ps[j] = lg;
      lmax = fmaxf(lmax, lg);
    }
    const float mx = block_reduce_max(lmax, red);
    float lsum = 0.f;
    for (int j = tid; j < n; j += kSelThreads) {
      const float e = __expf(Ps[j] - mx);
      Ps[j] = e;
      lsum += e;
    }
    const float tot = block_reduce_sum(lsum, red);
    const float inv = 1.f / tot;
    for (int j = tid; j < n; j += kSelThreads) {
      const float p = Ps[j] * inv;
      Ps[j] = p;
      if (prow) prow[j] = p;
    }
    if (prow)
      for (int j = n + tid; j < a.nb; j += kSelThreads) prow[j] = 0.f;
    __syncthreads();
  }

  for (int p = tid; p < a.n2; p += kSelThreads)
    keys[p] = (p < n) ? desc_sort_key(Ps[p], static_cast<uint32_t>(p)) : ~0ull;
  bitonic_sort_lds(keys, a.n2);

  if (tid == 0) {
    int kk;
    if (a.mode == 0) {
      kk = static_cast<int>(floor(a.param * static_cast<double>(n)));
      kk = max(1, min(kk, n));
    } else {
      kk = n;
      float c = 0.f;
      for (int m = 0; m < n; ++m) {
        c = __fadd_rn(c, Ps[static_cast<int>(keys[m] & 0xffffffffull)]);
        if (static_cast<double>(c) >= a.param) {
          kk = m + 1;
          break;
        }
      }
    }
    kept = kk;
  }
  for (int j = tid; j < n; j += kSelThreads) flag[j] = 0;
  __syncthreads();
  const int kk = kept;
  for (int m = tid; m < kk; m += kSelThreads) flag[static_cast<int>(keys[m] & 0xffffffffull)] = 1;
  __syncthreads();

  // ascending compaction: thread tid owns candidates [tid*per, (tid+1)*per)
  const int per = (n + kSelThreads - 1) / kSelThreads;
  const int lo = min(tid * per, n), hi = min(lo + per, n);
  int cnt = 0;
  for (int j = lo; j < hi; ++j) cnt += flag[j];
  scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const int v = (tid >= off) ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int pos = scan[tid] - cnt;
  int32_t* out = a.idx + row * a.max_off;
  for (int j = lo; j < hi; ++j)
    if (flag[j]) out[pos++] = j;
  if (tid == 0) a.counts[row] = kk;
}

template <int D, int BS>
hipError_t launch_pool_t(const uint16_t* x, float* out, int heads, const Dims& d,
                         hipStream_t stream) {
  PoolArgs pa;
  pa.x = x; pa.out = out; pa.N = d.N; pa.nb = d.nb;
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
                               float* blk_scores, bool scores_in, int32_t* counts, int32_t* idx,
                               void* ws, hipStream_t stream) {
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
  sa.n2 = n2;
  sa.mode = mode; sa.p_in = scores_in ? 1 : 0; sa.param = param; sa.scale = scale;
  const size_t shmem = static_cast<size_t>(n2) * (sizeof(uint64_t) + sizeof(float) + sizeof(int32_t));
  auto kern = d.d == 128 ? select_kernel<128> : select_kernel<64>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shmem));
  if (e != hipSuccess) return e;
  return launch(kern, dim3(d.nb, d.B * d.Hq), dim3(kSelThreads), shmem, stream, sa);
}

}  // namespace pbs
