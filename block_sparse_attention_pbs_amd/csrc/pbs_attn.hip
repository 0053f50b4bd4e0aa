// pbs_attn_fwd: block-sparse flash-attention forward with permuted keys (gfx950).
//
// What it computes (arXiv 2510.21270; sciencestack.ai page, Fig. 1 caption and Lemma 3.1;
// gist.science summary, Methodik 3 "Handling von Queries" and Methodik 4 "Kernel"): every query
// row t of query block i, segment s, attends to the keys of the kept earlier-segment blocks of
// its row (whole blocks) and to every key of its own segment whose ORIGINAL position is <= t.
// The own segment is walked in the order of the given key tensor (permuted copies), the causal
// test going through the stored original positions.  Queries are never permuted, so the output
// is written in original token order.
//
// Design (CDNA4, wave64):
//  * one workgroup per (query block, query head); BS/32 waves, 32 query rows per wave;
//  * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16 (A = K rows from
//    LDS, B = the wave's Q rows kept in registers), so each lane owns ONE query row: the online
//    softmax max / sum stay in the lane, with a single cross-half exchange per key block;
//  * the output is accumulated transposed, O^T += V^T P^T: P leaves the score accumulators as
//    the bf16 B operand without touching LDS (the key order inside a 16-key step is a
//    relabelling shared by both operands), and V^T is read from the row-major V tile with the
//    gfx950 transposing LDS load ds_read_b64_tr_b16;
//  * exp2 with scale*log2(e) folded into one multiply; fp32 accumulators; bf16 output (RNE).
#include "pbs_device.h"
#include "pbs_internal.h"

namespace pbs {
namespace {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm;
  const int32_t* minpos;
  const int32_t* counts;
  const int32_t* idx;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, G, N, nb, bps, max_off;
  int mode;      // 0 dense causal, 1 permuted PBS, 2 identity-order PBS
  float c;       // scale * log2(e)
};

template <int D, int BS>
struct AttnCfg {
  static constexpr int NW = BS / 32;     // waves per workgroup, 32 query rows each
  static constexpr int NT = NW * kWave;
  static constexpr int STR = D + 8;      // LDS row stride of the K / V tiles (bf16 elements)
  static constexpr int NKT = BS / 32;    // 32-key sub-tiles per key block
  static constexpr int NKS = D / 16;     // 16-wide k-steps over the head dim
  static constexpr int NMT = D / 32;     // 32-row tiles of O^T over the head dim
};

__device__ __forceinline__ i16x4 ds_read_tr(const uint16_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(lds_ptr));
}

template <int D, int BS>
__global__ __launch_bounds__(BS / 32 * 64) void attn_fwd_kernel(AttnArgs a) {
  using C = AttnCfg<D, BS>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BS * C::STR];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BS * C::STR];
  __shared__ int32_t Pos[BS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane >> 5;      // which half of the wave
  const int c32 = lane & 31;     // query row inside the wave
  const int i = gridDim.x - 1 - blockIdx.x;  // later query blocks carry more work: start them first
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int h = g / a.G;
  const size_t q_head = (static_cast<size_t>(b) * a.Hq + g) * a.N;
  const size_t kv_head = (static_cast<size_t>(b) * a.Hkv + h) * a.N;
  const int t = i * BS + w * 32 + c32;

  bf16x8 qf[C::NKS];
  {
    const uint16_t* qrow = a.q + (q_head + t) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  }
  f32x16 oacc[C::NMT];
#pragma unroll
  for (int mt = 0; mt < C::NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[mt][r] = 0.f;
  float m_i = -INFINITY;
  float l_i = 0.f;

  const int seg = i / a.bps;
  const int seg_first = seg * a.bps;
  int n_off = 0;
  const int32_t* list = nullptr;
  if (a.mode != 0) {
    const size_t row = (static_cast<size_t>(b) * a.Hq + g) * a.nb + i;
    n_off = min(max(a.counts[row], 0), seg_first);
    list = a.idx + row * a.max_off;
  }
  const int n_total = (a.mode == 0) ? (i + 1) : (n_off + a.bps);
  const int last_row = i * BS + BS - 1;
  const int32_t* minpos = a.minpos ? a.minpos + kv_head / BS : nullptr;

  for (int n = 0; n < n_total; ++n) {
    int j;
    bool masked;
    if (a.mode == 0) {
      j = n;
      masked = (j == i);
    } else if (n < n_off) {
      j = min(max(list[n], 0), seg_first - 1);
      masked = false;
    } else {
      j = seg_first + (n - n_off);
      if (a.mode == 2) {
        if (j > i) break;  // identity order: blocks past the diagonal hold only future keys
        masked = (j == i);
      } else {
        if (minpos && minpos[j] > last_row) continue;  // no key of this block is visible
        masked = true;
      }
    }

    __syncthreads();  // the previous tile is no longer read
    {
      const uint16_t* kb = a.k + (kv_head + static_cast<size_t>(j) * BS) * D;
      const uint16_t* vb = a.v + (kv_head + static_cast<size_t>(j) * BS) * D;
      constexpr int CH = D / 8;
#pragma unroll
      for (int c = tid; c < BS * CH; c += C::NT) {
        const int r = c / CH, col = (c % CH) * 8;
        *reinterpret_cast<u32x4*>(&Ks[r * C::STR + col]) =
            *reinterpret_cast<const u32x4*>(kb + static_cast<size_t>(r) * D + col);
        *reinterpret_cast<u32x4*>(&Vs[r * C::STR + col]) =
            *reinterpret_cast<const u32x4*>(vb + static_cast<size_t>(r) * D + col);
      }
      if (masked) {
        for (int r = tid; r < BS; r += C::NT)
          Pos[r] = (a.mode == 1) ? a.perm[kv_head + static_cast<size_t>(j) * BS + r] : j * BS + r;
      }
    }
    __syncthreads();

    // S^T (keys x query rows) for the whole key block.
    f32x16 s[C::NKT];
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
      const uint16_t* krow = &Ks[(kt * 32 + c32) * C::STR + hl * 8];
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + ks * 16);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kt], 0, 0, 0);
      }
    }

    // Online softmax: lane value r of sub-tile kt is key kt*32 + (r/4)*8 + hl*4 + r%4.
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float z = s[kt][r] * a.c;
        if (masked) {
          const int key = kt * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
          if (Pos[key] > t) z = -INFINITY;
        }
        s[kt][r] = z;
        mx = fmaxf(mx, z);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_i - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[kt][r] - m_use);
        s[kt][r] = p;
        rs += p;
      }
    }
    rs += __shfl_xor(rs, 32);
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int mt = 0; mt < C::NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[mt][r] *= alpha;

    // O^T += V^T P^T, 16 keys per MFMA.
    const int gp = lane >> 4, li = lane & 15;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[kt][8 * s2 + e]);
        const int key0 = kt * 32 + 16 * s2 + 4 * (gp >> 1) + (li >> 2);
#pragma unroll
        for (int mt = 0; mt < C::NMT; ++mt) {
          const int dv = mt * 32 + (gp & 1) * 16 + 4 * (li & 3);
          // Whole-vector casts only: extracting single elements of the transposing load's
          // result is lowered to a broadcast of element 0 by this compiler.
          const u32x2 lo = __builtin_bit_cast(u32x2, ds_read_tr(&Vs[key0 * C::STR + dv]));
          const u32x2 hi = __builtin_bit_cast(u32x2, ds_read_tr(&Vs[(key0 + 8) * C::STR + dv]));
          const u32x4 w4 = {lo[0], lo[1], hi[0], hi[1]};
          const bf16x8 va = __builtin_bit_cast(bf16x8, w4);
          oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[mt], 0, 0, 0);
        }
      }
    }
  }

  // O^T lane value r of tile mt is head-dim index mt*32 + (r/4)*8 + hl*4 + r%4 of row t.
  const float inv_l = (l_i > 0.f) ? 1.f / l_i : 0.f;
  uint16_t* orow = a.o + (q_head + t) * D;
#pragma unroll
  for (int mt = 0; mt < C::NMT; ++mt) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      u32x2 pk;
      pk[0] = pack_bf16x2(oacc[mt][rb * 4 + 0] * inv_l, oacc[mt][rb * 4 + 1] * inv_l);
      pk[1] = pack_bf16x2(oacc[mt][rb * 4 + 2] * inv_l, oacc[mt][rb * 4 + 3] * inv_l);
      *reinterpret_cast<u32x2*>(orow + mt * 32 + rb * 8 + hl * 4) = pk;
    }
  }
  if (a.lse && hl == 0) a.lse[q_head + t] = (m_i + __log2f(l_i)) * kLn2;
}

template <int D, int BS>
hipError_t launch_attn_t(const Dims& d, const AttnArgs& a, hipStream_t stream) {
  dim3 grid(d.nb, d.Hq, d.B);
  return launch(attn_fwd_kernel<D, BS>, grid, dim3(AttnCfg<D, BS>::NT), 0, stream, a);
}

}  // namespace

hipError_t launch_attn(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* perm, const int32_t* blk_minpos, const int32_t* counts,
                       const int32_t* idx, int mode, float scale, uint16_t* o, float* lse,
                       hipStream_t stream) {
  AttnArgs a;
  a.q = q; a.k = k; a.v = v;
  a.perm = perm; a.minpos = blk_minpos; a.counts = counts; a.idx = idx;
  a.o = o; a.lse = lse;
  a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.N = d.N; a.nb = d.nb; a.bps = d.bps;
  a.max_off = d.max_off > 0 ? d.max_off : 1;
  a.mode = mode;
  a.c = scale * kLog2e;
  if (d.d == 128 && d.Bs == 128) return launch_attn_t<128, 128>(d, a, stream);
  if (d.d == 128 && d.Bs == 64) return launch_attn_t<128, 64>(d, a, stream);
  if (d.d == 64 && d.Bs == 128) return launch_attn_t<64, 128>(d, a, stream);
  return launch_attn_t<64, 64>(d, a, stream);
}

}  // namespace pbs
