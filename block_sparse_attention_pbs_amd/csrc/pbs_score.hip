// pbs_score: query-aware key importance from the last query block (gfx950).
//
// What it computes (arXiv 2510.21270; gist.science summary, Methodik 3 "Proxy-Bewertung": the
// importance of the keys is estimated from the last block of queries by mean pooling of their
// attention scores; Methodik 2: no query sees a later segment): for each KV head, each of the
// R = G*Bs scoring rows (every query head of the group, rows [N-Bs, N)) takes a softmax over the
// keys of one segment that it may see (causal), and every key's probabilities are averaged over
// the rows.
//
// Two passes, both on v_mfma_f32_32x32x16_bf16 with S^T = K Q^T (a lane owns one scoring row):
//  1. stats:  per (segment, row) the softmax max m (log2 units) and sum l, streaming the
//             segment's keys through LDS;
//  2. reduce: per key, sum over all rows of exp2(z - m) / l.  A wave owns 32 keys for the
//             whole pass (its K fragments stay in registers); the rows stream through LDS in
//             chunks of 32; each lane accumulates its 16 keys over its rows in fp32 and a final
//             butterfly over the 32 lanes of each half-wave (wavefront reduction) gives the
//             per-key sum, scaled by 1/R.
#include "pbs_device.h"
#include "pbs_internal.h"

namespace pbs {
namespace {

struct ScoreArgs {
  const uint16_t* q;
  const uint16_t* k;
  float* scores;
  float2* stats;  // [B, Hkv, nseg, R] (m, l)
  int Hq, Hkv, G, N, S, nseg, R, Bs;
  float c;        // scale * log2(e)
};

// Scoring row r of a KV group -> (query head offset inside the group, query position).
__device__ __forceinline__ void score_row(const ScoreArgs& a, int r, int& g_local, int& t) {
  g_local = r / a.Bs;
  t = a.N - a.Bs + (r - g_local * a.Bs);
}

constexpr int kStatKeys = 64;  // keys per LDS tile in the stats pass

template <int D>
__global__ __launch_bounds__(256) void score_stats_kernel(ScoreArgs a) {
  constexpr int STR = D + 8;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kStatKeys * STR];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, c32 = lane & 31;
  const int sigma = blockIdx.x;
  const int bh = blockIdx.z;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int r = blockIdx.y * 128 + w * 32 + c32;
  const bool active = (blockIdx.y * 128 + w * 32) < a.R;  // wave-uniform (R % 32 == 0)
  int g_local = 0, t = 0;
  bf16x8 qf[NKS];
  if (active) {
    score_row(a, r, g_local, t);
    const int g = h * a.G + g_local;
    const uint16_t* qrow = a.q + ((static_cast<size_t>(b) * a.Hq + g) * a.N + t) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  }
  const size_t kv_head = (static_cast<size_t>(b) * a.Hkv + h) * a.N;
  const int s0 = sigma * a.S;
  float m = -INFINITY, l = 0.f;
  for (int k0 = s0; k0 < s0 + a.S; k0 += kStatKeys) {
    __syncthreads();
    {
      const uint16_t* kb = a.k + (kv_head + k0) * D;
      constexpr int CH = D / 8;
      for (int c = tid; c < kStatKeys * CH; c += 256) {
        const int rr = c / CH, col = (c % CH) * 8;
        *reinterpret_cast<u32x4*>(&Ks[rr * STR + col]) =
            *reinterpret_cast<const u32x4*>(kb + static_cast<size_t>(rr) * D + col);
      }
    }
    __syncthreads();
    if (!active) continue;
#pragma unroll
    for (int kt = 0; kt < kStatKeys / 32; ++kt) {
      f32x16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
      const uint16_t* krow = &Ks[(kt * 32 + c32) * STR + hl * 8];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(krow + ks * 16),
                                                     qf[ks], s, 0, 0, 0);
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + kt * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
        const float z = (key <= t) ? s[e] * a.c : -INFINITY;
        s[e] = z;
        mx = fmaxf(mx, z);
      }
      const float m_new = fmaxf(m, mx);
      if (m_new == -INFINITY) continue;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc += fast_exp2(s[e] - m_new);
      l = l * fast_exp2(m - m_new) + acc;
      m = m_new;
    }
  }
  if (!active) return;
  // merge the two half-waves (same row, different keys)
  const float m2 = __shfl_xor(m, 32);
  const float l2 = __shfl_xor(l, 32);
  const float mt = fmaxf(m, m2);
  const float lt = (mt == -INFINITY) ? 0.f
                                     : l * fast_exp2(m - mt) + l2 * fast_exp2(m2 - mt);
  if (hl == 0) a.stats[(static_cast<size_t>(bh) * a.nseg + sigma) * a.R + r] = make_float2(mt, lt);
}

template <int D>
__global__ __launch_bounds__(256) void score_reduce_kernel(ScoreArgs a) {
  constexpr int STR = D + 8;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[32 * STR];
  __shared__ float2 St[32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, c32 = lane & 31;
  const int bh = blockIdx.y;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int key0 = (blockIdx.x * 4 + w) * 32;
  const bool active = key0 < a.N;  // wave-uniform
  const int sigma = active ? key0 / a.S : 0;
  const size_t kv_head = (static_cast<size_t>(b) * a.Hkv + h) * a.N;
  // Every wave of the workgroup lies in one segment only if 128 | S; the stats rows are read
  // per wave, so waves of different segments are fine.
  bf16x8 kf[NKS];
  if (active) {
    const uint16_t* krow = a.k + (kv_head + key0 + c32) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(krow + ks * 16);
  }
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  const float2* st_seg = a.stats + (static_cast<size_t>(bh) * a.nseg + sigma) * a.R;
  for (int rc = 0; rc < a.R; rc += 32) {
    __syncthreads();
    {
      constexpr int CH = D / 8;
      for (int c = tid; c < 32 * CH; c += 256) {
        const int rr = c / CH, col = (c % CH) * 8;
        int gl, tt;
        score_row(a, rc + rr, gl, tt);
        const uint16_t* src =
            a.q + ((static_cast<size_t>(b) * a.Hq + h * a.G + gl) * a.N + tt) * D + col;
        *reinterpret_cast<u32x4*>(&Qs[rr * STR + col]) = *reinterpret_cast<const u32x4*>(src);
      }
    }
    __syncthreads();
    if (!active) continue;
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    const uint16_t* qrow = &Qs[c32 * STR + hl * 8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], *reinterpret_cast<const bf16x8*>(qrow + ks * 16),
                                                   s, 0, 0, 0);
    // lane column = scoring row rc + c32; lane value e = key key0 + (e/4)*8 + hl*4 + e%4
    int gl, tt;
    score_row(a, rc + c32, gl, tt);
    const float2 st = st_seg[rc + c32];
    const float inv_l = 1.f / st.y;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = key0 + (e >> 2) * 8 + hl * 4 + (e & 3);
      if (key <= tt) acc[e] += fast_exp2(s[e] * a.c - st.x) * inv_l;
    }
  }
  if (!active) return;
  const float inv_r = 1.f / static_cast<float>(a.R);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float v = acc[e];
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o);
    acc[e] = v;
  }
  if (c32 == 0) {
    float* out = a.scores + kv_head + key0;
#pragma unroll
    for (int e = 0; e < 16; ++e) out[(e >> 2) * 8 + hl * 4 + (e & 3)] = acc[e] * inv_r;
  }
}

template <int D>
hipError_t launch_score_t(const Dims& d, const ScoreArgs& a, hipStream_t stream) {
  dim3 g1(d.nseg, (a.R + 127) / 128, d.B * d.Hkv);
  hipError_t e = launch(score_stats_kernel<D>, g1, dim3(256), 0, stream, a);
  if (e != hipSuccess) return e;
  dim3 g2((d.N + 127) / 128, d.B * d.Hkv);
  return launch(score_reduce_kernel<D>, g2, dim3(256), 0, stream, a);
}

}  // namespace

size_t score_workspace_bytes(const Dims& d) {
  return static_cast<size_t>(d.B) * d.Hkv * d.nseg * d.G * d.Bs * sizeof(float2);
}

hipError_t launch_score(const Dims& d, const uint16_t* q, const uint16_t* k, float scale,
                        float* scores, void* ws, hipStream_t stream) {
  ScoreArgs a;
  a.q = q; a.k = k; a.scores = scores; a.stats = static_cast<float2*>(ws);
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.N = d.N; a.S = d.S; a.nseg = d.nseg;
  a.R = d.G * d.Bs; a.Bs = d.Bs;
  a.c = scale * kLog2e;
  return d.d == 128 ? launch_score_t<128>(d, a, stream) : launch_score_t<64>(d, a, stream);
}

}  // namespace pbs
