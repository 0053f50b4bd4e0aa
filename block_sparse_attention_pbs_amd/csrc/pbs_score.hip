// pbs_score: query-aware key importance from the last query block (gfx950).
//
// What it computes (arXiv 2510.21270; gist.science summary, Methodik 3 "Proxy-Bewertung": the
// importance of the keys is estimated from the last block of queries by mean pooling of their
// attention scores; Methodik 2: no query sees a later segment): for each KV head, each of the
// R = G*Bs scoring rows (every query head of the group, rows [N-Bs, N)) takes a softmax over the
// keys of one segment that it may see (causal), and every key's probabilities are averaged over
// the rows.  With several sequences packed along N, each sequence is scored on its own: the rows
// are the last Bs of the sequence that holds the segment.
//
// Three kernels, the matrix work on v_mfma_f32_32x32x16_bf16 with S^T = K Q^T (a lane owns one
// scoring row in the first, one key column in the last):
//  1. stats:   per (segment, chunk of keys, row) a reference m (log2 units) and the sum l of
//              exp2(z - m) over the chunk, streaming its keys through LDS in tiles of 128 keys
//              (64 where 128 does not divide the chunk), the next tile loaded into registers
//              while the current one is computed.  Segments are split into chunks of at most
//              1024 keys so that enough workgroups run to hide the loads' latency;
//  2. combine: per (segment, row) the chunks' (m, l) merged into one log2-normaliser
//              L = m + log2(l);
//  3. reduce:  per key, the sum over all rows of exp2(z - L).  A wave owns 32 keys for the whole
//              pass (its K fragments stay in registers); the rows stream through LDS in chunks
//              of 64 (the next chunk loaded into registers while the current one is computed,
//              32 rows per MFMA chain); each lane accumulates its 16 keys over its rows in
//              fp32, in row order, and a final butterfly over the 32 lanes of each half-wave
//              (wavefront reduction) gives the per-key sum, scaled by 1/R.
// A key can be after a scoring row only in the last Bs positions of the sequence, so only tiles
// that reach them apply the causal test.  Both passes run eight waves per workgroup: a stats
// workgroup streams each K tile once for 256 scoring rows, a reduce workgroup stages each chunk
// of rows once for 256 keys.
#include <mutex>
#include <type_traits>

#include "pbs_device.h"
#include "pbs_internal.h"

namespace pbs {
namespace {

struct ScoreArgs {
  const uint16_t* q;
  const uint16_t* k;
  float* scores;
  float2* part;   // [B, Hkv, nseg, nchunk, R] (m, l) of each key chunk
  float* lse2;    // [B, Hkv, nseg, R] log2-normaliser of each (segment, row)
  int Hq, Hkv, G, N, S, nseg, R, Bs;
  int bs_log2;    // Bs = 1 << bs_log2 (64 or 128)
  int chunk, nchunk;  // keys per chunk, chunks per segment
  float c;        // scale * log2(e)
  RowMap qm, km;  // row addressing of q and k (either layout)
  const int32_t* cu;  // packed sequences: nseq + 1 starts along N, or null (one sequence)
  int nseq;
};

// End of the sequence that holds segment sigma (N without packed sequences).
__device__ __forceinline__ int seq_end(const ScoreArgs& a, int sigma) {
  int lo, hi;
  seq_bounds(a.cu, a.nseq, a.N, sigma * a.S, lo, hi);
  return hi;
}

// Scoring row r of a KV group -> (query head offset inside the group, query position): the last
// Bs positions of the sequence, which ends at `end`.
__device__ __forceinline__ void score_row(const ScoreArgs& a, int r, int end, int& g_local,
                                          int& t) {
  g_local = r >> a.bs_log2;
  t = min(max(end - a.Bs + (r & (a.Bs - 1)), 0), a.N - 1);
}

constexpr int kStatKeys = 64;   // stats chunks are multiples of this LDS tile; 128-key tiles where they divide
#ifndef PBS_SCORE_STAT_WAVES
#define PBS_SCORE_STAT_WAVES 8
#endif
#ifndef PBS_SCORE_RED_WAVES
#define PBS_SCORE_RED_WAVES 8
#endif
constexpr int kStatWaves = PBS_SCORE_STAT_WAVES;  // waves (32 scoring rows each) per stats workgroup
constexpr int kRedWaves = PBS_SCORE_RED_WAVES;    // waves (32 keys each) per reduce workgroup

template <int D, int TK>   // TK: keys per LDS tile (64 or 128; divides the chunk)
__global__ __launch_bounds__(64 * kStatWaves) void score_stats_kernel(ScoreArgs a) {
  constexpr int STR = D + 8;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TK * STR];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, c32 = lane & 31;
  const int sigma = blockIdx.x / a.nchunk, ch = blockIdx.x - sigma * a.nchunk;
  const int bh = blockIdx.z;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int r = blockIdx.y * (32 * kStatWaves) + w * 32 + c32;
  const bool active = static_cast<int>(blockIdx.y) * (32 * kStatWaves) + w * 32 < a.R;  // wave-uniform
  const int end = seq_end(a, sigma);
  int g_local = 0, t = 0;
  bf16x8 qf[NKS];
  if (active) {
    score_row(a, r, end, g_local, t);
    const int g = h * a.G + g_local;
    const uint16_t* qrow = a.q + a.qm.off(b, g, t) + hl * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  }
  const size_t krs = static_cast<size_t>(a.km.stride());
  const int kbeg = sigma * a.S + ch * a.chunk;
  const int first_row = end - a.Bs;   // every scoring row is >= first_row
  // (m, l): the lane's reference (log2 units) and its sum of exp2(z - m) over the chunk.  The
  // reference is fixed at the max of the first 32 keys this lane's row sees, so later keys need
  // no max and no rescaling; the chunk's sum then holds terms up to exp2(max - m).  If a sum leaves
  // [0, 2^100] (a later key far above the reference), the workgroup runs the chunk again with a
  // running max, rescaling at every 32 keys (ONLINE).
  float m = -INFINITY, l = 0.f;
  auto chunk_pass = [&](auto online_tag) {
    constexpr bool ONLINE = decltype(online_tag)::value;
    m = -INFINITY;
    l = 0.f;
    // Staging: thread tid copies 16-byte pieces tid, tid + 64*waves, ... of each K tile; the next
    // tile's pieces are loaded into registers before the current tile is computed.
    constexpr int CH = D / 8;
    constexpr int NPT = TK * CH / (64 * kStatWaves);
    static_assert(NPT * 64 * kStatWaves == TK * CH, "whole 16-byte pieces per thread");
    u32x4 kv[NPT];
    auto load_tile = [&](int k0) {
      const uint16_t* kb = a.k + a.km.off(b, h, k0);
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int c = tid + i * 64 * kStatWaves, rr = c / CH, col = (c % CH) * 8;
        kv[i] = *reinterpret_cast<const u32x4*>(kb + static_cast<size_t>(rr) * krs + col);
      }
    };
    load_tile(kbeg);
    for (int k0 = kbeg; k0 < kbeg + a.chunk; k0 += TK) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int c = tid + i * 64 * kStatWaves, rr = c / CH, col = (c % CH) * 8;
        *reinterpret_cast<u32x4*>(&Ks[rr * STR + col]) = kv[i];
      }
      __syncthreads();
      if (k0 + TK < kbeg + a.chunk) load_tile(k0 + TK);
      if (!active) continue;
      const bool causal = k0 + TK - 1 > first_row;   // uniform: a key may follow a row
#pragma unroll
      for (int kt = 0; kt < TK / 32; ++kt) {
        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
        const uint16_t* krow = &Ks[(kt * 32 + c32) * STR + hl * 8];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(krow + ks * 16),
                                                       qf[ks], s, 0, 0, 0);
        if (causal) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = k0 + kt * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
            if (key > t) s[e] = -INFINITY;
          }
        }
        if (ONLINE || m == -INFINITY) {   // a.c > 0: the max commutes with the scaling
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
          const float m_new = fmaxf(m, mx * a.c);
          if (m_new == -INFINITY) continue;   // no key of the row yet
          if (ONLINE) l *= fast_exp2(m - m_new);
          m = m_new;
        }
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc += fast_exp2(fmaf(s[e], a.c, -m));
        l += acc;
      }
    }
  };
  chunk_pass(std::false_type{});
  if (__syncthreads_or((active && !(l <= 0x1p100f)) ? 1 : 0)) chunk_pass(std::true_type{});
  if (!active) return;
  // merge the two half-waves (same row, different keys)
  const float m2 = __shfl_xor(m, 32);
  const float l2 = __shfl_xor(l, 32);
  const float mt = fmaxf(m, m2);
  const float lt = (mt == -INFINITY) ? 0.f
                                     : l * fast_exp2(m - mt) + l2 * fast_exp2(m2 - mt);
  if (hl == 0)
    a.part[((static_cast<size_t>(bh) * a.nseg + sigma) * a.nchunk + ch) * a.R + r] = make_float2(mt, lt);
}

// Per (segment, row): the chunks' (m, l) merged into L = m + log2(l).  Every row sees at least one
// key of every segment (itself, or the whole segment when it lies before the row).
__global__ __launch_bounds__(256) void score_combine_kernel(ScoreArgs a) {
  const int local = blockIdx.x * 256 + threadIdx.x;       // sigma * R + r within one KV head
  if (local >= a.nseg * a.R) return;
  const int sigma = local / a.R, r = local - sigma * a.R;
  const size_t seg = static_cast<size_t>(blockIdx.y) * a.nseg + sigma;   // bh * nseg + sigma
  const float2* p = a.part + seg * a.nchunk * a.R + r;
  float m = -INFINITY;
  for (int c = 0; c < a.nchunk; ++c) m = fmaxf(m, p[static_cast<size_t>(c) * a.R].x);
  float l = 0.f;
  for (int c = 0; c < a.nchunk; ++c) {
    const float2 v = p[static_cast<size_t>(c) * a.R];
    if (v.x != -INFINITY) l += v.y * fast_exp2(v.x - m);
  }
  a.lse2[seg * a.R + r] = (l > 0.f) ? m + __log2f(l) : INFINITY;
}

template <int D>
__global__ __launch_bounds__(64 * kRedWaves) void score_reduce_kernel(ScoreArgs a) {
  constexpr int STR = D + 8;
  constexpr int NKS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[64 * STR];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, so the chunk loop is scalar
  const int hl = lane >> 5, c32 = lane & 31;
  const int bh = blockIdx.y;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  // One workgroup covers up to 32 * kRedWaves keys of ONE segment (every wave reads the same
  // scoring rows, which belong to the segment's sequence); a segment takes
  // ceil(S / (32 * kRedWaves)) workgroups and waves past its end idle.
  const int wps = (a.S + 32 * kRedWaves - 1) / (32 * kRedWaves);
  const int sigma = blockIdx.x / wps;
  const int off = ((blockIdx.x - sigma * wps) * kRedWaves + w) * 32;
  const bool active = off < a.S;  // wave-uniform
  const int key0 = sigma * a.S + (active ? off : 0);
  bf16x8 kf[NKS];
  if (active) {
    const uint16_t* krow = a.k + a.km.off(b, h, key0 + c32) + hl * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(krow + ks * 16);
  }
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  const float* st_seg = a.lse2 + (static_cast<size_t>(bh) * a.nseg + sigma) * a.R;
  const int end = seq_end(a, sigma);
  const bool causal = active && key0 + 31 > end - a.Bs;   // uniform: a key may follow a row
  // Rows are staged RC at a time (RC divides Bs, so a staged chunk is one query head's
  // consecutive positions t0 ... t0 + RC - 1, clamped at 0 for a sequence shorter than Bs) and
  // computed 32 at a time.  Thread tid copies the 16-byte pieces tid, tid + 64*waves, ... (piece c:
  // row c / (D/8), column chunk c % (D/8)); the next chunk's pieces and log2-normalisers are
  // loaded into registers before the current chunk is computed.
  constexpr int RC = 64, NSUB = RC / 32;
  constexpr int CH = D / 8, NPIECE = RC * CH;
  constexpr int NPT = (NPIECE + 64 * kRedWaves - 1) / (64 * kRedWaves);
  const size_t qstride = static_cast<size_t>(a.qm.stride());
  auto load_chunk = [&](int rc, u32x4 (&qv)[NPT]) {
    const int t0 = end - a.Bs + (rc & (a.Bs - 1));
    const uint16_t* head = a.q + a.qm.off(b, h * a.G + (rc >> a.bs_log2), 0);
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + i * 64 * kRedWaves;
      if (NPIECE % (64 * kRedWaves) == 0 || c < NPIECE)
        qv[i] = *reinterpret_cast<const u32x4*>(
            head + static_cast<size_t>(max(t0 + c / CH, 0)) * qstride + (c % CH) * 8);
    }
  };
  u32x4 qv[NPT];
  load_chunk(0, qv);
  float l2c[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) l2c[j] = active ? st_seg[j * 32 + c32] : 0.f;
  for (int rc = 0; rc < a.R; rc += RC) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int c = tid + i * 64 * kRedWaves;
      if (NPIECE % (64 * kRedWaves) == 0 || c < NPIECE)
        *reinterpret_cast<u32x4*>(&Qs[(c / CH) * STR + (c % CH) * 8]) = qv[i];
    }
    __syncthreads();
    const int rn = __builtin_amdgcn_readfirstlane(rc + RC);
    if (rn < a.R) load_chunk(rn, qv);
    if (!active) continue;
    float nl[NSUB];
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      nl[j] = -l2c[j];
      l2c[j] = st_seg[min(rn, a.R - RC) + j * 32 + c32];
    }
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      f32x16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
      const uint16_t* qrow = &Qs[(j * 32 + c32) * STR + hl * 8];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], *reinterpret_cast<const bf16x8*>(qrow + ks * 16),
                                                     s, 0, 0, 0);
      // lane column = scoring row rc + 32j + c32; lane value e = key key0 + (e/4)*8 + hl*4 + e%4
      if (causal) {
        int gl, tt;
        score_row(a, rc + j * 32 + c32, end, gl, tt);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + (e >> 2) * 8 + hl * 4 + (e & 3);
          if (key <= tt) acc[e] += fast_exp2(fmaf(s[e], a.c, nl[j]));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] += fast_exp2(fmaf(s[e], a.c, nl[j]));
      }
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
    float* out = a.scores + static_cast<size_t>(bh) * a.N + key0;
#pragma unroll
    for (int e = 0; e < 16; ++e) out[(e >> 2) * 8 + hl * 4 + (e & 3)] = acc[e] * inv_r;
  }
}

template <int D>
hipError_t launch_score_t(const Dims& d, const ScoreArgs& a, hipStream_t stream) {
  dim3 g1(d.nseg * a.nchunk, (a.R + 32 * kStatWaves - 1) / (32 * kStatWaves), d.B * d.Hkv);
  hipError_t e = (a.chunk % 128 == 0)
                    ? launch(score_stats_kernel<D, 128>, g1, dim3(64 * kStatWaves), 0, stream, a)
                    : launch(score_stats_kernel<D, 64>, g1, dim3(64 * kStatWaves), 0, stream, a);
  if (e != hipSuccess) return e;
  dim3 gc((d.nseg * a.R + 255) / 256, d.B * d.Hkv);
  e = launch(score_combine_kernel, gc, dim3(256), 0, stream, a);
  if (e != hipSuccess) return e;
  dim3 g2(d.nseg * ((d.S + 32 * kRedWaves - 1) / (32 * kRedWaves)), d.B * d.Hkv);
  return launch(score_reduce_kernel<D>, g2, dim3(64 * kRedWaves), 0, stream, a);
}

}  // namespace

// Keys per stats chunk: the segment split into at most 1024-key pieces (S and the chunk are
// multiples of the 64-key tile).
static int score_chunk(const Dims& d) {
  int c = d.S;
  while (c > 1024 && c % 2 == 0 && (c / 2) % kStatKeys == 0) c /= 2;
  return c;
}

// Scratch of pbs_score_noalloc: the score partials live in this array instead of a caller's
// workspace.  Every GPU the library runs on holds its own copy until the process ends; its device
// address is looked up once per device (the array's name is only a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t score_noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t score_workspace_bytes(const Dims& d) {
  const size_t rows = static_cast<size_t>(d.B) * d.Hkv * d.nseg * d.G * d.Bs;
  const size_t nchunk = static_cast<size_t>(d.S / score_chunk(d));
  const size_t part = (rows * nchunk * sizeof(float2) + 255) & ~static_cast<size_t>(255);
  return part + rows * sizeof(float);
}

hipError_t launch_score(const Dims& d, const uint16_t* q, const uint16_t* k, float scale,
                        float* scores, void* ws, const int32_t* cu, int nseq,
                        hipStream_t stream) {
  ScoreArgs a;
  a.q = q; a.k = k; a.scores = scores;
  a.cu = cu; a.nseq = nseq;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.N = d.N; a.S = d.S; a.nseg = d.nseg;
  a.R = d.G * d.Bs; a.Bs = d.Bs;
  a.bs_log2 = 0;
  while ((1 << a.bs_log2) < d.Bs) ++a.bs_log2;
  a.chunk = score_chunk(d);
  a.nchunk = d.S / a.chunk;
  const size_t rows = static_cast<size_t>(d.B) * d.Hkv * d.nseg * a.R;
  const size_t part = (rows * a.nchunk * sizeof(float2) + 255) & ~static_cast<size_t>(255);
  a.part = static_cast<float2*>(ws);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + part);
  a.c = scale * kLog2e;
  a.qm = q_rows(d);
  a.km = kv_rows(d);
  return d.d == 128 ? launch_score_t<128>(d, a, stream) : launch_score_t<64>(d, a, stream);
}

}  // namespace pbs
