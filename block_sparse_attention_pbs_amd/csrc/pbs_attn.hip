// pbs_attn_fwd: block-sparse flash-attention forward with permuted keys (gfx950).
//
// What it computes (arXiv 2510.21270; sciencestack.ai page, Fig. 1 caption and Lemma 3.1;
// gist.science summary, Methodik 3 "Handling von Queries" and Methodik 4 "Kernel"): every query
// row t of query block i, segment s, attends to the keys of the kept earlier-segment blocks of
// its row (whole blocks) and to every key of its own segment whose ORIGINAL position is <= t.
// The own segment is read from the given key tensor (the permuted copies), the causal test
// going through the stored original positions; only its slots whose original position is at or
// before the query block's last row are loaded (any other key adds exactly zero to every row).
// Queries are never permuted, so the output is written in original token order.
//
// Design (CDNA4, wave64):
//  * one workgroup of Bs/32 waves per (query block, query head); wave w owns 32 query rows and
//    sees every key of every visited block, so no cross-wave reduction is needed;
//  * keys stream through LDS in stages of 32 keys, double-buffered and filled by asynchronous
//    direct buffer->LDS loads (buffer_load_dwordx4 ... lds, bounds-checked) one stage ahead of
//    the compute; a wave issues its share of the next stage's loads one by one between the
//    MFMAs of the current stage's score chain, where their issue costs no MFMA time, and reads
//    the first K fragments of a stage right after the barrier that lands it.  A workgroup
//    needs at most ~44 KiB of LDS and 168 VGPRs per lane, so three workgroups share a CU (three
//    waves per SIMD): while one waits or runs its softmax, the others keep the matrix cores
//    busy;
//  * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16 (A = K rows from
//    LDS, B = the wave's Q rows held in registers), so each lane owns one query row and the
//    softmax statistics need one cross-half exchange.  The accumulators live in VGPRs (built
//    with the VGPR form of the MFMAs), so scores feed the softmax without register moves;
//  * the output is accumulated transposed, O^T += V^T P^T: P leaves the score accumulators as the
//    bf16 B operand without touching LDS (the key order inside a 16-key step is a relabelling
//    shared by both operands); V^T comes from the row-major V tile through the transposing LDS
//    load ds_read_b64_tr_b16;
//  * K rows are padded by 16 bytes and V rows by 64 bytes in LDS, which makes both the K fragment
//    reads (16 rows x 16 B) and the transposing V reads (4 rows x 64 B) free of bank conflicts and
//    keeps every LDS address a per-lane base plus an immediate;
//  * exp2 with scale*log2(e) folded into one FMA per element, and a fixed per-row reference max
//    (the first finite block max of the row): the accumulator is never rescaled inside the loop.
//    A later max more than 2^64 above the reference only sets a flag, and the workgroup then
//    recomputes with the exact row max (never seen on realistic inputs, but it keeps every value
//    in range on any input);
//  * the own segment of the permuted-key path is a stream of its visible keys, taken in the order
//    of their original positions: the inverse permutation (from pbs_permute) names the slot of
//    every position, so the keys of positions seg_start .. the block's last row are exactly the
//    slots perm_inv[seg_start ..], 32 per stage, read two stages ahead into a small LDS ring;
//    each stream stage gathers its 32 rows from the permuted copies, the stages of positions
//    before the block's first row unmasked, the last Bs keys masked through the stored
//    positions perm[slot];
//  * work order: heaviest query blocks first, and consecutive workgroups of one XCD (the
//    hardware deals workgroups round-robin over the 8 XCDs) walk one KV head, so the K/V tiles a
//    head's query blocks share stay in that XCD's L2.
#include <type_traits>

#include "pbs_device.h"
#include "pbs_internal.h"

namespace pbs {
namespace {

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm;
  const int32_t* inv;   // mode 1: slot of every original position (the inverse permutation)
  const int32_t* minpos;
  const int32_t* counts;
  const int32_t* idx;
  const uint16_t* k2;   // mode 3: the original (unpermuted) keys and values, read for the own
  const uint16_t* v2;   //         segment in natural order
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, G, N, nb, bps, max_off;
  int mode;      // 0 dense causal, 1 permuted PBS, 2 identity-order PBS, 3 permuted off-diagonal
                 // blocks with the own segment in natural order, 4 permuted PBS with permuted
                 // queries (output rows written back at their original positions)
  int xcd_map;   // 0: launch order; 1: each XCD runs whole KV heads; 2: each KV head is split
                 // over xcd_split XCDs, query blocks dealt round-robin among them
  int xcd_split;
  float c;       // scale * log2(e)
  RowMap qm, km; // row addressing of q / o and of every key and value tensor (either layout)
  int kv_rs;     // elements between consecutive rows of one K/V head (km.stride())
  // Element offsets of the K/V stage tiles in LDS.  Passed at run time on purpose: the compiler
  // then keeps one (tile base + lane) address per tile and folds every in-tile offset into the
  // DS instruction, instead of materialising one register per (stage, offset) pair.
  int tile_off[4];
};

#ifndef PBS_ATTN_STAGE_KEYS
#define PBS_ATTN_STAGE_KEYS 32
#endif
#ifndef PBS_ATTN_MIN_WAVES
#define PBS_ATTN_MIN_WAVES 3
#endif
constexpr int kStageKeys = PBS_ATTN_STAGE_KEYS;  // keys per LDS stage
constexpr int kOffWindow = 1792; // off-diagonal list entries held in LDS at a time
constexpr int kOwnMax = 256;     // own-segment blocks (S / Bs <= 16384 / 64)
constexpr int kRing = 4;         // key-stream stages whose slots are held in LDS (mode 1)

template <int D, int BS>
struct Cfg {
  static constexpr int NW = BS / 32;       // waves: 32 query rows each
  static constexpr int NT = NW * 64;
  static constexpr int SK = kStageKeys;    // keys per stage
  static constexpr int HALVES = BS / SK;   // stages per key block
  static constexpr int NKT = SK / 32;      // 32-key sub-tiles per stage
  static constexpr int NKS = D / 16;       // 16-wide k-steps over the head dim
  static constexpr int NMT = D / 32;       // 32-row tiles of O^T over the head dim
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int KPAD = 1;           // spare 16-byte chunks per K row
  static constexpr int VPAD = 4;           // spare 16-byte chunks per V row
  static constexpr int KTILE = SK * (D + 8 * KPAD);   // bf16 elements of a K stage in LDS
  static constexpr int VTILE = SK * (D + 8 * VPAD);   // bf16 elements of a V stage in LDS
  static constexpr int KCH = SK * (CPR + KPAD);      // 16-byte chunks of a K stage in LDS
  static constexpr int VCH = SK * (CPR + VPAD);      // 16-byte chunks of a V stage in LDS
  static constexpr int NLDK = (KCH + 63) / 64;       // direct loads (64 lanes) per K stage
  static constexpr int NLDV = (VCH + 63) / 64;       // direct loads (64 lanes) per V stage
  // Key-stream (gathered) loads: every load starts on a row, so lane l always fetches chunk
  // l % ROW of row l / ROW of that load's rows; the lanes past the last whole row run into the
  // next row (the next load writes the same bytes there) and, after the last load, into spare
  // rows behind the tile.
  static constexpr int KROW = CPR + KPAD, VROW = CPR + VPAD;    // 16-byte chunks per LDS row
  static constexpr int RK = 64 / KROW, RV = 64 / VROW;          // whole rows per load
  static constexpr int NGK = (SK + RK - 1) / RK, NGV = (SK + RV - 1) / RV;   // loads per stage
  static constexpr int KSLK = NGK * RK + (64 % KROW ? 1 : 0) - SK;   // spare rows behind a tile
  static constexpr int VSLK = NGV * RV + (64 % VROW ? 1 : 0) - SK;
  static constexpr int KTILE_A = KTILE + KSLK * (D + 8 * KPAD);      // LDS elements per K stage
  static constexpr int VTILE_A = VTILE + VSLK * (D + 8 * VPAD);      // LDS elements per V stage
};

// LDS row layouts.  K rows: stride = 16 B mod 256 B, so the 16 lanes of a K fragment read
// (16 rows, one 16-byte chunk each) hit 16 distinct bank groups.  V rows: stride = 64 B mod
// 256 B, so the 4 rows x 64 B touched by 32 lanes of a transposing V read cover the 64 banks once.
template <int D>
__device__ __forceinline__ constexpr int koff(int r, int e) {
  return r * (D + 8) + e;
}
template <int D>
__device__ __forceinline__ constexpr int voff(int r, int e) {
  return r * (D + 32) + e;
}

// Buffer resource over `bytes` bytes from `base` (gfx9 descriptor: word 1 holds the top 16
// address bits with stride 0, word 2 the size, word 3 the data format).  Loads through it are
// bounds-checked by the hardware and take a 32-bit per-lane offset plus a scalar offset.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes,
               0x00020000u};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
// Direct buffer->LDS loads: lane l's 16 (or 4) bytes land at lds + l*16 (l*4).  Written as asm
// on purpose: the compiler cannot tell that a stage's loads and the other stage's LDS reads touch
// different tiles, and would otherwise wait for these loads before every LDS read that follows
// them, serialising the double buffer.  Their completion is awaited explicitly (s_waitcnt +
// barrier) before the stage they fill is read.
__device__ __forceinline__ void load_lds16(u32x4 r, const void* lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr(lds)), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}
// The same load, free to move past the compiler's own LDS reads: for key-stream stages, whose
// loads only ever target the buffer no wave reads before the next wait + barrier.
__device__ __forceinline__ void load_lds16_free(u32x4 r, const void* lds, uint32_t voff,
                                                uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr(lds)), "v"(voff), "s"(r), "s"(soff)
               : "m0");
}
__device__ __forceinline__ void load_lds4(u32x4 r, const void* lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_addr(lds)), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ u32x2 ds_read_tr(const uint16_t* lds_ptr) {
  // Whole-vector cast only: extracting single elements of this builtin's result is lowered to
  // a broadcast of element 0 by this compiler.
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) i16x4*)(lds_ptr)));
}

// The key blocks one query block visits, in order, each split into stages of 32 keys; uniform
// across the workgroup (every value it returns is scalar).  The visit list lives in LDS as 16-bit
// entries (block index, bit 15 = needs the causal mask): the query block's off-diagonal list, a
// window of kOffWindow entries at a time, and the visible own-segment blocks, compacted once.
// Each entry is read from LDS one stage before it is used, so no memory latency sits between two
// stages.
struct StageIter {
  int mode, halves, i, seg_first;
  int n_off, n_own;     // list lengths (MODE != 0)
  int m;                // next entry (MODE 0: next block)
  int win;              // first off-diagonal entry held in the LDS window
  int j, half;
  bool masked;
  bool orig;            // mode 3: the entry is an own-segment block of the original keys
  const int32_t* list;  // off-diagonal list in global memory
  uint16_t* offw;       // LDS window of the off-diagonal list
  const uint16_t* ownl; // LDS list of the visible own-segment blocks
  int ent;              // the next entry's LDS word, read ahead (per lane, all lanes equal)
  // Mode 1: after the off-diagonal blocks, the own segment is walked as a stream of its VISIBLE
  // keys in the order of their original positions: stream key x is the key at original position
  // seg_start + x, held in slot perm_inv[seg_start + x] of the permuted copies.  Query block i
  // sees positions up to its last row, so the stream is (i - seg_first + 1) * Bs keys long: the
  // keys before the block's first row (visible to every row, unmasked stages), then the block's
  // own Bs positions (masked stages, the causal test through perm[slot]).  A key after every row
  // of the block adds exactly zero to every row and is never part of the stream.
  bool ks_on;
  int n_ks;             // stream keys
  int n_ks_full;        // of which visible to every row of the block
  int ks;               // next stream stage
  int kidx;             // stream index of the stage just returned (-1: a contiguous block stage)
  const int32_t* ring;  // LDS: kRing x 32 slots of upcoming stream stages (stage x in x % kRing)

  // Load off-diagonal entries [w0, w0 + kOffWindow) into LDS (all threads; barrier after).
  __device__ __forceinline__ void fill(int w0, int tid, int nt) {
    const int n = min(n_off - w0, kOffWindow);
    for (int e = tid; e < n; e += nt)
      offw[e] = static_cast<uint16_t>(min(max(list[w0 + e], 0), seg_first - 1));
    win = w0;
  }
  __device__ __forceinline__ int read_entry(int k) const {
    return k < n_off ? offw[k - win] : static_cast<int>(ownl[k - n_off]);
  }
  __device__ __forceinline__ void start(int tid, int nt) {
    m = 0;
    half = -1;
    ks = 0;
    kidx = -1;
    if (mode != 0) {
      if (win != 0) {  // a long list left a later window in LDS
        __syncthreads();
        fill(0, tid, nt);
        __syncthreads();
      }
      if (n_off + n_own > 0) ent = read_entry(0);
    }
  }
  __device__ __forceinline__ bool next_block(int tid, int nt) {
    if (mode == 0) {
      if (m > i) return false;
      j = m;
      m = __builtin_amdgcn_readfirstlane(m + 1);
      masked = (j == i);
      return true;
    }
    if (m >= n_off + n_own) return false;
    const int e = __builtin_amdgcn_readfirstlane(ent);
    m = __builtin_amdgcn_readfirstlane(m + 1);
    if (m < n_off && m == win + kOffWindow) {  // every wave is here, past its reads of the window
      fill(m, tid, nt);
      __syncthreads();
    }
    if (m < n_off + n_own) ent = read_entry(m);
    j = e & 0x7fff;
    masked = (e >> 15) != 0;
    orig = (mode == 3) && (m - 1 >= n_off);
    return true;
  }
  // The next stream stage; false at the end of the stream.
  __device__ __forceinline__ bool next_stream() {
    if (ks * 32 >= n_ks) return false;
    kidx = __builtin_amdgcn_readfirstlane(ks * 32);
    ks = __builtin_amdgcn_readfirstlane(ks + 1);
    masked = kidx + 32 > n_ks_full;   // holds a key that some row of the block must not see
    return true;
  }
  // Advance to the next stage; false when the list is exhausted.
  __device__ __forceinline__ bool next(int tid, int nt) {
    if (half >= 0 && half + 1 < halves) {
      ++half;
      return true;
    }
    half = 0;
    if (!ks_on || m < n_off) {
      kidx = -1;
      return next_block(tid, nt);
    }
    orig = false;
    half = halves - 1;   // one stage per stream step
    return next_stream();
  }
  // next() where the caller knows the following stage is a key-block stage (KIND 1) or a
  // key-stream stage (KIND 2): the same result with the other case's code left out.
  template <int KIND>
  __device__ __forceinline__ bool next_of(int tid, int nt) {
    if constexpr (KIND == 1) {
      if (half >= 0 && half + 1 < halves) {
        ++half;
        return true;
      }
      half = 0;
      kidx = -1;
      return next_block(tid, nt);
    } else if constexpr (KIND == 2) {
      return next_stream();
    } else {
      return next(tid, nt);
    }
  }
};

struct Stage {
  int key0;     // first key of the stage in the head's key order (block * Bs + stage * 32)
  int pos0;     // original position of its first key; its 32 keys hold positions pos0 .. pos0+31
                // (a key-stream stage walks positions in order; a block stage of the diagonal
                // block holds them in order in modes 0, 2 and 3)
  bool masked;
  bool orig;    // read from the original keys and values (mode 3 own segment)
  // Own-segment key-stream stage (mode 1): the slots of its 32 keys (perm_inv entries, in LDS);
  // slots == nullptr for a contiguous stage.
  const int32_t* slots;
};

// The stage the iterator just returned.
template <int BS, int SK>
__device__ __forceinline__ Stage stage_of(const StageIter& it) {
  Stage st;
  st.key0 = it.j * BS + it.half * SK;
  st.pos0 = it.kidx >= 0 ? it.seg_first * BS + it.kidx : st.key0;
  st.masked = it.masked;
  st.orig = it.orig;
  st.slots = nullptr;
  if (it.kidx >= 0) st.slots = it.ring + ((it.kidx >> 5) % kRing) * 32;
  return st;
}

// Buffer resources of one head: keys, values, key positions, and (mode 3) the original keys
// and values; mode 1: the own segment's rows of the permuted keys and values (ks, vs) and the
// head's inverse permutation.
struct Rsrc {
  u32x4 k, v, p, k2, v2, ks, vs, inv;
};

// Mode 1: load the slots of stream stage x (perm_inv of its 32 positions) into the ring; wave 0,
// one 4-byte direct load per lane, awaited by the next stage barrier.
__device__ __forceinline__ void issue_ring(const Rsrc& rr, const StageIter& it, int x, int seg_pos,
                                           int w, int lane) {
  if (w == 0 && lane < 32 && x * 32 < it.n_ks)
    load_lds4(rr.inv, it.ring + (x % kRing) * 32, static_cast<uint32_t>(seg_pos + x * 32 + lane) * 4,
              0u);
}

// Start the asynchronous loads of one stage (K, V and, for masked permuted blocks, the original
// positions of its keys) into LDS.  A spare chunk of a padded row re-reads chunk 0 of its row.
// A key-stream stage gathers its rows: row r of the stage is the slot slots[r] of the own
// segment, read through buffer resources that span only that segment, so a slot outside it
// reads zeros instead of another segment's or head's memory.
//
// The loads of a stage are numbered items, issued one by one (item I by piece I, the last piece
// taking every item left), so that a caller can spread them over the MFMAs of the stage it
// computes meanwhile.  Gathered stage: items 0 .. UK-1 are its K loads, UK .. UK+UV-1 its V
// loads, then the positions of a masked stage and, last, the slots of a later stream stage into
// the ring.  Their slots are read from LDS into registers first (read()), before any item.
template <int D, int BS>
struct Gather {
  using C = Cfg<D, BS>;
  // Load u of wave w is load w + u*NW of the stage; only the last u can pass the last load (UK,
  // UV round up): a wave with fewer loads than the others repeats the last one (the same bytes
  // to the same place).  Straight-line code, no lane masks.
  static constexpr int UK = (C::NGK + C::NW - 1) / C::NW, UV = (C::NGV + C::NW - 1) / C::NW;
  static constexpr int NI = UK + UV + 2;
  uint32_t sk[UK], sv[UV];
  __device__ __forceinline__ void read(const Stage& st, int w, int lane) {
    const int rk = lane / C::KROW, rv = lane / C::VROW;
    const int32_t* slk = st.slots + rk + w * C::RK;
    const int32_t* slv = st.slots + rv + w * C::RV;
#pragma unroll
    for (int u = 0; u + 1 < UK; ++u) sk[u] = static_cast<uint32_t>(slk[u * C::NW * C::RK]);
    sk[UK - 1] =
        static_cast<uint32_t>(st.slots[rk + min(w + (UK - 1) * C::NW, C::NGK - 1) * C::RK]);
#pragma unroll
    for (int u = 0; u + 1 < UV; ++u) sv[u] = static_cast<uint32_t>(slv[u * C::NW * C::RV]);
    sv[UV - 1] =
        static_cast<uint32_t>(st.slots[rv + min(w + (UV - 1) * C::NW, C::NGV - 1) * C::RV]);
  }
  // cok / cov: this lane's chunk offset minus the segment's first row, so that one 24-bit
  // multiply-add turns a global slot into an offset in the segment.  `ring` issues the last
  // item (the caller's load of a later stream stage's slots).
  template <int I, class Ring>
  __device__ __forceinline__ void item(const AttnArgs& a, const Rsrc& rr, const Stage& st,
                                       uint16_t* Kst, uint16_t* Vst, int32_t* Pst, int w, int lane,
                                       uint32_t cok, uint32_t cov, Ring&& ring) const {
    const uint32_t rowb = static_cast<uint32_t>(a.kv_rs) * 2;   // < 2^24: checked on the host
    if constexpr (I < UK) {
      const int j = min(w + I * C::NW, C::NGK - 1);
      load_lds16_free(rr.ks, Kst + j * C::RK * C::KROW * 8, __umul24(sk[I], rowb) + cok, 0u);
    } else if constexpr (I < UK + UV) {
      const int j = min(w + (I - UK) * C::NW, C::NGV - 1);
      load_lds16_free(rr.vs, Vst + j * C::RV * C::VROW * 8, __umul24(sv[I - UK], rowb) + cov, 0u);
    } else if constexpr (I == UK + UV) {
      if (st.masked && w == 0 && lane < C::SK)
        load_lds4(rr.p, Pst, static_cast<uint32_t>(st.slots[lane]) * 4, 0u);
    } else {
      ring();
    }
  }
};

template <int D, int BS>
__device__ __forceinline__ void issue_gathered(const AttnArgs& a, const Rsrc& rr, Stage st,
                                               uint16_t* Kst, uint16_t* Vst, int32_t* Pst, int w,
                                               int lane, uint32_t cok, uint32_t cov) {
  // Every slot is read before the first load is issued: the loads are asm with side effects,
  // which the compiler never moves an LDS read across, so reading the slots in between would
  // wait out one LDS round trip per load.
  Gather<D, BS> gt;
  gt.read(st, w, lane);
  static_for<0, Gather<D, BS>::NI - 1>([&](auto i) {
    gt.template item<decltype(i)::value>(a, rr, st, Kst, Vst, Pst, w, lane, cok, cov, [] {});
  });
}

// The loads of a contiguous (key-block) stage as numbered items: item I < UKB is this wave's
// K load I, then its V loads, then (permuted queries only) the positions of a masked stage.
template <int D, int BS, int MODE>
struct BlockLoads {
  using C = Cfg<D, BS>;
  static constexpr int UKB = (C::NLDK + C::NW - 1) / C::NW, UVB = (C::NLDV + C::NW - 1) / C::NW;
  static constexpr int NI = UKB + UVB + (MODE == 4 ? 1 : 0);
  template <int I>
  __device__ __forceinline__ static void item(const AttnArgs& a, const Rsrc& rr, const Stage& st,
                                              uint16_t* Kst, uint16_t* Vst, int32_t* Pst, int w,
                                              int lane, bool more) {
    const uint32_t base = static_cast<uint32_t>(st.key0) * static_cast<uint32_t>(a.kv_rs) * 2;
    if constexpr (I < UKB) {
      const int n = w + I * C::NW;
      const int P = n * 64 + lane;
      const int r = P / (C::CPR + C::KPAD), pc = P - r * (C::CPR + C::KPAD);
      // A partial last load (KCH not a multiple of 64) runs its tail lanes too: they write the
      // spare rows behind the tile (never read) with the next rows of the head, or zeros past
      // its end, so the only test is the wave-uniform one.
      static_assert(C::KCH % 64 == 0 || (C::KTILE_A - C::KTILE) / 8 >= 64 - C::KCH % 64,
                    "spare rows take a partial load's tail");
      if (more && n < C::NLDK)
        load_lds16(st.orig ? rr.k2 : rr.k, Kst + n * 512,
                   static_cast<uint32_t>((r * a.kv_rs + (pc < C::CPR ? pc : 0) * 8) * 2), base);
    } else if constexpr (I < UKB + UVB) {
      const int n = w + (I - UKB) * C::NW;
      const int P = n * 64 + lane;
      const int r = P / (C::CPR + C::VPAD), pc = P - r * (C::CPR + C::VPAD);
      static_assert(C::VCH % 64 == 0 || (C::VTILE_A - C::VTILE) / 8 >= 64 - C::VCH % 64,
                    "spare rows take a partial load's tail");
      if (more && n < C::NLDV)
        load_lds16(st.orig ? rr.v2 : rr.v, Vst + n * 512,
                   static_cast<uint32_t>((r * a.kv_rs + (pc < C::CPR ? pc : 0) * 8) * 2), base);
    } else {
      if (more && st.masked && w == 0 && lane < C::SK)
        load_lds4(rr.p, Pst, static_cast<uint32_t>(lane * 4), static_cast<uint32_t>(st.key0) * 4);
    }
  }
};

// Items [U, U+1) of N, the last piece (U == NP - 1) taking every item from U on.
template <int U, int NP, int N, class F>
__device__ __forceinline__ void piece_items(F&& f) {
  if constexpr (U >= 0 && U < N) {
    if constexpr (U + 1 < NP)
      f(std::integral_constant<int, U>{});
    else
      static_for<U, N>(f);
  }
}

template <int D, int BS, bool MAYBE_STREAM = true>
__device__ __forceinline__ void issue_stage(const AttnArgs& a, const Rsrc& rr, Stage st,
                                            uint16_t* Kst, uint16_t* Vst, int32_t* Pst, int w,
                                            int lane, uint32_t cok, uint32_t cov) {
  using C = Cfg<D, BS>;
  if (MAYBE_STREAM && st.slots != nullptr) {
    issue_gathered<D, BS>(a, rr, st, Kst, Vst, Pst, w, lane, cok, cov);
    return;
  }
  const uint32_t base = static_cast<uint32_t>(st.key0) * static_cast<uint32_t>(a.kv_rs) * 2;
  const u32x4 rk = st.orig ? rr.k2 : rr.k;
  const u32x4 rv = st.orig ? rr.v2 : rr.v;
  const u32x4 rp = rr.p;
#pragma unroll
  for (int n = w; n < C::NLDK; n += C::NW) {
    const int P = n * 64 + lane;
    const int r = P / (C::CPR + C::KPAD), pc = P - r * (C::CPR + C::KPAD);
    // a partial last load (KCH not a multiple of 64) runs with the tail lanes switched off
    if (C::KCH % 64 == 0 || P < C::KCH)
      load_lds16(rk, Kst + n * 512,
                 static_cast<uint32_t>((r * a.kv_rs + (pc < C::CPR ? pc : 0) * 8) * 2), base);
  }
#pragma unroll
  for (int n = w; n < C::NLDV; n += C::NW) {
    const int P = n * 64 + lane;
    const int r = P / (C::CPR + C::VPAD), pc = P - r * (C::CPR + C::VPAD);
    if (C::VCH % 64 == 0 || P < C::VCH)
      load_lds16(rv, Vst + n * 512,
                 static_cast<uint32_t>((r * a.kv_rs + (pc < C::CPR ? pc : 0) * 8) * 2), base);
  }
  if (st.masked && a.mode == 4 && w == 0 && lane < C::SK)
    load_lds4(rp, Pst, static_cast<uint32_t>(lane * 4), static_cast<uint32_t>(st.key0) * 4);
}

// x combined with its value in the other half of the wave (lane l and lane l ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Causal mask of a 32-key sub-tile as the initial value of its score accumulator: -inf for a key
// whose original position is after the lane's query row t, else 0 (then -inf + the dot product
// stays -inf).  Lane value r of sub-tile kt is stage key kt*32 + (r/4)*8 + hl*4 + r%4.
// -inf for d < 0 (a key after the row), +0 for d >= 0, for |d| < 2^23 (positions are below
// N <= 2^20): a negative d has its nine top bits set, which is exactly the bit pattern of -inf;
// a small non-negative d has them clear.  Two independent integer operations per element.
__device__ __forceinline__ float mask_bits(int d) { return __int_as_float(d & 0xff800000); }

template <int MODE>
__device__ __forceinline__ f32x16 mask_init(const int32_t* Ps, int key0, int kt, int hl, int t) {
  f32x16 m;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int key = kt * 32 + rb * 8 + hl * 4;
    int4 pos;
    if constexpr (MODE == 1 || MODE == 4) {
      pos = *reinterpret_cast<const int4*>(&Ps[key]);
    } else {
      const int p0 = key0 + key;
      pos = make_int4(p0, p0 + 1, p0 + 2, p0 + 3);
    }
    m[rb * 4 + 0] = mask_bits(t - pos.x);
    m[rb * 4 + 1] = mask_bits(t - pos.y);
    m[rb * 4 + 2] = mask_bits(t - pos.z);
    m[rb * 4 + 3] = mask_bits(t - pos.w);
  }
  return m;
}

// Row state of one wave across the stages of a pass (log2 units).
struct RowState {
  float mref;     // fixed reference subtracted before exp2 (-inf until the first stage)
  float lsum;     // this lane's half of the row's sum of exp2
  float mseen;    // exact row max (max-only pass)
};

// One stage (32 keys, one 32-key sub-tile per kStageKeys / 32) for one wave.  S^T = K Q^T as one
// MFMA chain per sub-tile (for a masked stage, masked keys enter as -inf through the accumulators'
// initial values); then exp2 against the fixed reference and O^T += V^T P^T.  The other waves of
// the SIMD keep the matrix cores busy while this one runs its exp2 work.  There is no running max: before a pass each
// row's reference is set to its max over the pass's first stage (0 for a row that sees no key of
// it; the MAXONLY form of this function computes that max), and a row sum outside [2^-60, 2^64]
// after the pass sends the workgroup through the exact-max fallback.
template <int D, int BS, int MODE, bool MASKED, bool MAXONLY, bool VPRE = true, class Pre>
__device__ __forceinline__ void attn_stage(const AttnArgs& a, const uint16_t* Ks, const uint16_t* Vs,
                                           const int32_t* Ps, int key0, int lane, int t,
                                           const bf16x8 (&qf)[Cfg<D, BS>::NKS],
                                           f32x16 (&oacc)[Cfg<D, BS>::NMT], RowState& rs,
                                           const bf16x8 (&k01)[2], Pre&& pre, bool skip = false) {
  using C = Cfg<D, BS>;
  const int hl = lane >> 5;
  const int c32 = lane & 31;
  const int gp = lane >> 4, li = lane & 15;
  static_assert(C::NKT == 1, "one 32-key sub-tile per stage");
  f32x16 s[C::NKT];
  // The next stage's loads go out in pieces between the MFMAs of this stage's score chain:
  // pre(-1) (address reads) before the first MFMA, pre(u) after MFMA u, so that their issue
  // and the latency of the address reads sit in the shadow of the chain.  A skipped stage
  // issues every piece and returns.
  // K fragments are read two k-steps ahead of their MFMA, in source order before the load piece
  // of that step (the block loads are ordered against LDS accesses); the first two come from the
  // caller, read as soon as the stage has landed.
  bf16x8 kf[C::NKS];
  kf[0] = k01[0];
  kf[1] = k01[1];
  pre(std::integral_constant<int, -1>{});
  if constexpr (MASKED) {
    // A masked stage (a few per query block) issues every piece up front: a wave whose rows
    // all precede the stage's keys then skips it (wave-uniform: nothing of it reaches them).
    static_for<0, C::NKS>([&](auto u) { pre(u); });
    if (skip) return;
  }
  static_for<0, C::NKS>([&](auto ksc) {
    constexpr int ks = decltype(ksc)::value;
    if constexpr (ks == 0) {
      if constexpr (MASKED)
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0],
                                                       mask_init<MODE>(Ps, key0, 0, hl, t), 0, 0, 0);
      else
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0], f32x16{}, 0, 0, 0);
    } else {
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s[0], 0, 0, 0);
    }
    if constexpr (ks + 2 < C::NKS)
      kf[ks + 2] = *reinterpret_cast<const bf16x8*>(&Ks[koff<D>(c32, (ks + 2) * 16 + hl * 8)]);
    if constexpr (!MASKED) pre(ksc);
  });
  if constexpr (MAXONLY) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    rs.mseen = fmaxf(rs.mseen, pair_max(mx) * a.c);
  } else {
    const float nm = -rs.mref;
    // O^T += V^T P^T in NJ steps, step j = s2 * NMT + mt (keys 16*s2 .. +15, head dims
    // 32*mt .. +31).  The V^T fragment of step j is read two steps ahead, the first two before
    // the exp2 work, so that no step waits out a whole LDS round trip.  (VPRE false: each read
    // just before its step, fewer live registers, for the rarely run exact-max pass.)
    constexpr int NJ = 2 * C::NMT;
    auto read_v = [&](int j) {
      const int s2 = j / C::NMT, mt = j % C::NMT;
      const int vr = 16 * s2 + 4 * (gp >> 1) + (li >> 2);
      const int dv = mt * 32 + (gp & 1) * 16 + 4 * (li & 3);
      const u32x2 lo = ds_read_tr(&Vs[voff<D>(vr, dv)]);
      const u32x2 hi = ds_read_tr(&Vs[voff<D>(vr + 8, dv)]);
      return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    bf16x8 vf[NJ];
    if constexpr (VPRE) {
      vf[0] = read_v(0);
      vf[1] = read_v(1);
    }
    bf16x8 pb[2];
    float sum = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {   // v_cvt_pk_bf16_f32, round to nearest even
        const float pe = fast_exp2(fmaf(s[0][8 * s2 + e], a.c, nm));
        sum += pe;
        pb[s2][e] = static_cast<__bf16>(pe);
      }
    rs.lsum += sum;
    static_for<0, NJ>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (!VPRE) vf[j] = read_v(j);
      oacc[j % C::NMT] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], pb[j / C::NMT], oacc[j % C::NMT], 0, 0, 0);
      if constexpr (VPRE && j + 2 < NJ) vf[j + 2] = read_v(j + 2);
    });
  }
}

// The first two K fragments (A operands of the first two score MFMAs) of a stage in LDS.
template <int D>
__device__ __forceinline__ void read_k01(const uint16_t* Ks, int lane, bf16x8 (&k01)[2]) {
  const int c32 = lane & 31, hl = lane >> 5;
  k01[0] = *reinterpret_cast<const bf16x8*>(&Ks[koff<D>(c32, hl * 8)]);
  k01[1] = *reinterpret_cast<const bf16x8*>(&Ks[koff<D>(c32, 16 + hl * 8)]);
}

// Pipeline state carried from one stage to the next within a pass.
struct Pipe {
  Stage cur;    // the stage whose loads are in flight or landed in buffer `p`
  int p;        // LDS buffer of `cur`
};

// Per-lane constants of the loaders and the stream (computed once per workgroup).
struct LoadCtx {
  uint32_t cok, cov;   // mode 1: chunk offset of this lane's gathered K / V rows, minus the
                       // segment's first slot (see issue_gathered)
  int seg_pos;         // mode 1: first original position of the own segment
};

// `count` stages of one mask kind, one per iteration.  The loads of the next stage go into the
// other buffer before the current stage is computed; the wait + barrier at the top of an iteration
// both lands the current stage and frees the other buffer.  Buffers are picked by parity through
// uniform offsets, so the loop body is one straight copy of the stage code and the accumulators
// stay in place from one iteration to the next.
// KIND: 0 any stage may follow, 1 only key-block stages follow, 2 only key-stream stages.
template <int D, int BS, int MODE, bool MASKED, bool MAXONLY, int KIND, bool VPRE = true>
__device__ __forceinline__ void run_stages(const AttnArgs& a, StageIter& it, int count, Pipe& pp,
                                           const Rsrc& rr, const LoadCtx& lc, uint16_t* smem,
                                           int32_t* Ps0, int32_t* Ps1, int w, int lane, int t,
                                           const bf16x8 (&qf)[Cfg<D, BS>::NKS],
                                           f32x16 (&oacc)[Cfg<D, BS>::NMT], RowState& rs) {
  using C = Cfg<D, BS>;
  const int tid = threadIdx.x;
  for (int n = 0; n < count; ++n) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // the current stage landed; the other buffer is no longer read
    const int p = pp.p;
    // the first score MFMAs' operands are requested before the iterator's scalar work
    bf16x8 k01[2];
    read_k01<D>(smem + (p ? a.tile_off[1] : a.tile_off[0]), lane, k01);
    const bool more = it.template next_of<KIND>(tid, C::NT);
    const Stage nxt = stage_of<BS, C::SK>(it);
    uint16_t* Kn = smem + (p ? a.tile_off[0] : a.tile_off[1]);
    uint16_t* Vn = smem + (p ? a.tile_off[2] : a.tile_off[3]);
    if constexpr (KIND == 0) {
      if (more) issue_stage<D, BS, true>(a, rr, nxt, Kn, Vn, p ? Ps0 : Ps1, w, lane, lc.cok, lc.cov);
    }
    // Key blocks (KIND 1): the next stage's loads go out in pieces between this stage's score
    // MFMAs.  Key stream (KIND 2): the same, after its slots are read from the ring (pre(-1));
    // no branch around them: past the end of the stream the iterator still names the current
    // stage, which is then loaded again into the free buffer.  The slots of the stage after the
    // next one go into the ring with the last piece.
    Gather<D, BS> gt;
    auto pre = [&](auto u) {
      constexpr int U = decltype(u)::value;
      if constexpr (KIND == 1) {
        piece_items<U, C::NKS, BlockLoads<D, BS, MODE>::NI>([&](auto i) {
          BlockLoads<D, BS, MODE>::template item<decltype(i)::value>(a, rr, nxt, Kn, Vn,
                                                                     p ? Ps0 : Ps1, w, lane, more);
        });
      } else if constexpr (KIND == 2) {
        if constexpr (U < 0) {
          gt.read(nxt, w, lane);
        } else {
          piece_items<U, C::NKS, Gather<D, BS>::NI>([&](auto i) {
            gt.template item<decltype(i)::value>(a, rr, nxt, Kn, Vn, p ? Ps0 : Ps1, w, lane,
                                                 lc.cok, lc.cov, [&] {
                                                   issue_ring(rr, it, it.ks, lc.seg_pos, w, lane);
                                                 });
          });
        }
      }
    };
    // A masked stage whose keys all come after every row of this wave adds exactly nothing to
    // the wave's rows: the wave only issues its share of the next loads (queries are in natural
    // order outside mode 4, so the wave's last row is its first row + 31).
    bool skip = false;
    if constexpr (MASKED && MODE != 4)
      skip = pp.cur.pos0 > __builtin_amdgcn_readfirstlane((t & ~31) + 31);
    attn_stage<D, BS, MODE, MASKED, MAXONLY, VPRE>(
        a, smem + (p ? a.tile_off[1] : a.tile_off[0]), smem + (p ? a.tile_off[3] : a.tile_off[2]),
        p ? Ps1 : Ps0, pp.cur.key0, lane, t, qf, oacc, rs, k01, pre, skip);
    pp.cur = nxt;
    pp.p = p ^ 1;
  }
}

// One pass over the visited stages: every visit list is its unmasked blocks followed by its masked
// ones (off-diagonal blocks, then the key stream in mode 1; blocks before the diagonal then the
// diagonal in identity and dense order), so a pass is two loops, one per mask kind.  With PRIME,
// the rows' references are first set from the max of the pass's first stage (computed once more,
// scores only, as soon as that stage has landed).
template <int D, int BS, int MODE, bool MAXONLY, bool PRIME>
__device__ __forceinline__ void attn_pass(const AttnArgs& a, StageIter& it, int n_blk_stages,
                                          int n_unm_stages, int n_msk_stages, const Rsrc& rr,
                                          const LoadCtx& lc, uint16_t* smem, int32_t* Ps0,
                                          int32_t* Ps1, int w, int lane, int t,
                                          const bf16x8 (&qf)[Cfg<D, BS>::NKS],
                                          f32x16 (&oacc)[Cfg<D, BS>::NMT], RowState& rs) {
  using C = Cfg<D, BS>;
  const int tid = threadIdx.x;
  if constexpr (MODE == 1) {
    // the slots of the first two stream stages, landed (with the off-diagonal list window)
    // before any stage is issued
    issue_ring(rr, it, 0, lc.seg_pos, w, lane);
    issue_ring(rr, it, 1, lc.seg_pos, w, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  it.start(tid, C::NT);
  if (it.next(tid, C::NT)) {
    Pipe pp;
    pp.cur = stage_of<BS, C::SK>(it);
    pp.p = 0;
    issue_stage<D, BS>(a, rr, pp.cur, smem + a.tile_off[0], smem + a.tile_off[2], Ps0, w, lane,
                       lc.cok, lc.cov);
    if constexpr (PRIME) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      RowState first{0.f, 0.f, -INFINITY};
      bf16x8 k01[2];
      read_k01<D>(smem + a.tile_off[0], lane, k01);
      if (n_unm_stages > 0)
        attn_stage<D, BS, MODE, false, true>(a, smem + a.tile_off[0], smem + a.tile_off[2], Ps0,
                                             pp.cur.key0, lane, t, qf, oacc, first, k01, [](auto) {});
      else
        attn_stage<D, BS, MODE, true, true>(a, smem + a.tile_off[0], smem + a.tile_off[2], Ps0,
                                            pp.cur.key0, lane, t, qf, oacc, first, k01, [](auto) {});
      rs.mref = (first.mseen == -INFINITY) ? 0.f : first.mseen;
    }
    // n_blk_stages contiguous stages (key blocks), then, in mode 1, the rest of the unmasked
    // stages and all masked ones are the own segment's key stream
    if constexpr (MODE == 1) {
      // key blocks (the last one hands over to the stream), then the stream's stages
      if (n_blk_stages > 0) {
        run_stages<D, BS, MODE, false, MAXONLY, 1, PRIME>(a, it, n_blk_stages - 1, pp, rr, lc, smem, Ps0,
                                                   Ps1, w, lane, t, qf, oacc, rs);
        run_stages<D, BS, MODE, false, MAXONLY, 0, PRIME>(a, it, 1, pp, rr, lc, smem, Ps0, Ps1, w, lane,
                                                   t, qf, oacc, rs);
      }
      run_stages<D, BS, MODE, false, MAXONLY, 2, PRIME>(a, it, n_unm_stages - n_blk_stages, pp, rr, lc,
                                                 smem, Ps0, Ps1, w, lane, t, qf, oacc, rs);
      run_stages<D, BS, MODE, true, MAXONLY, 2, PRIME>(a, it, n_msk_stages, pp, rr, lc, smem, Ps0, Ps1,
                                                w, lane, t, qf, oacc, rs);
    } else {
      run_stages<D, BS, MODE, false, MAXONLY, 1, PRIME>(a, it, n_unm_stages, pp, rr, lc, smem, Ps0, Ps1,
                                                 w, lane, t, qf, oacc, rs);
      run_stages<D, BS, MODE, true, MAXONLY, 1, PRIME>(a, it, n_msk_stages, pp, rr, lc, smem, Ps0, Ps1,
                                                w, lane, t, qf, oacc, rs);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is done with both buffers before another pass refills them
}

template <int D, int BS, int MODE>
__global__ __launch_bounds__(BS * 2, PBS_ATTN_MIN_WAVES) void attn_fwd_kernel(AttnArgs a) {
  using C = Cfg<D, BS>;
  // One LDS array laid out [K stage 0][K stage 1][V stage 0][V stage 1].
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * C::KTILE_A + 2 * C::VTILE_A];
  __shared__ __attribute__((aligned(16))) int32_t Ps0[C::SK];
  __shared__ __attribute__((aligned(16))) int32_t Ps1[C::SK];
  __shared__ uint16_t offw[kOffWindow];
  __shared__ uint16_t ownl[kOwnMax];
  __shared__ __attribute__((aligned(16))) int32_t ring[MODE == 1 ? kRing * 32 : 1];
  __shared__ int own_count;
  __shared__ int qmax_w[C::NW];
  // Visit-list and key-mask rules: mode 4 (permuted queries) walks the permuted keys like mode 1.
  constexpr int LM = (MODE == 4) ? 1 : MODE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index as a scalar
  const int hl = lane >> 5;
  const int c32 = lane & 31;

  // work item -> (b, g, i): heaviest query blocks first, one KV head per XCD run
  int b, g, i;
  {
    const int total = gridDim.x;
    const int L = blockIdx.x;
    const int per_head = a.G * a.nb;
    // The hardware deals workgroups round-robin over the 8 XCDs (workgroup L to XCD L % 8), so
    // L % 8 picks the XCD and L / 8 the position in that XCD's sequence.  Every XCD walks its
    // items heaviest query block first, keeps to one KV head at a time (its K/V stay in that
    // XCD's L2) and gets the same mix of heavy and light blocks.
    int item = L;
    if (a.xcd_map == 1) {          // B*Hkv a multiple of 8: whole KV heads per XCD
      item = (L & 7) * (total >> 3) + (L >> 3);
    } else if (a.xcd_map == 2) {   // 8 a multiple of B*Hkv: xcd_split XCDs share a KV head
      const int x = L & 7, r = a.xcd_split;
      item = (x / r) * per_head + (L >> 3) * r + x % r;
    }
    const int hb = item / per_head;            // b * Hkv + h
    const int rem = item - hb * per_head;
    i = a.nb - 1 - rem / a.G;
    b = hb / a.Hkv;
    g = (hb - b * a.Hkv) * a.G + rem % a.G;
  }
  const int h = g / a.G;
  const size_t q_head = (static_cast<size_t>(b) * a.Hq + g) * a.N;     // lse is [B, Hq, N]
  const size_t kv_head = (static_cast<size_t>(b) * a.Hkv + h) * a.N;   // perm is [B, Hkv, N]
  // This lane's query row (both halves share it): slot ts of the query tensor; its original
  // position t drives the causal test and the output row.  Queries are in natural order except
  // in mode 4, where slot ts holds the token at perm[ts] and the row is written back there.
  const int ts = i * BS + w * 32 + c32;
  const int t = (MODE == 4) ? min(max(a.perm[kv_head + ts], 0), a.N - 1) : ts;
  // one K/V head: rows 0 .. N-1, a.kv_rs elements apart (< 2^32 bytes, checked on the host)
  const size_t kv0 = a.km.off(b, h, 0);
  const uint32_t head_bytes =
      static_cast<uint32_t>((static_cast<size_t>(a.N - 1) * a.kv_rs + D) * 2);
  Rsrc rr;
  rr.k = make_rsrc(a.k + kv0, head_bytes);
  rr.v = make_rsrc(a.v + kv0, head_bytes);
  rr.k2 = make_rsrc(MODE == 3 ? a.k2 + kv0 : nullptr, MODE == 3 ? head_bytes : 0u);
  rr.v2 = make_rsrc(MODE == 3 ? a.v2 + kv0 : nullptr, MODE == 3 ? head_bytes : 0u);
  rr.p =
      make_rsrc(a.perm ? a.perm + kv_head : nullptr, a.perm ? static_cast<uint32_t>(a.N) * 4 : 0u);
  const int seg_first = (i / a.bps) * a.bps;
  LoadCtx lc;
  lc.seg_pos = seg_first * BS;
  lc.cok = lc.cov = 0u;
  if constexpr (MODE == 1) {
    // The own segment's rows of the permuted keys and values: the key stream gathers only there.
    // A lane of a gathered load fetches chunk (lane % row chunks) of its row; the segment's first
    // slot is taken off here, so a global slot s lands at (s - seg_pos) * row bytes + chunk.
    using CC = Cfg<D, BS>;
    const uint32_t rowb = static_cast<uint32_t>(a.kv_rs) * 2;
    const size_t seg_off = a.km.off(b, h, lc.seg_pos);
    const uint32_t seg_bytes =
        static_cast<uint32_t>((static_cast<size_t>(a.bps * BS - 1) * a.kv_rs + D) * 2);
    rr.ks = make_rsrc(a.k + seg_off, seg_bytes);
    rr.vs = make_rsrc(a.v + seg_off, seg_bytes);
    rr.inv = make_rsrc(a.inv + kv_head, static_cast<uint32_t>(a.N) * 4);
    const int ck = lane % CC::KROW, cv = lane % CC::VROW;
    const uint32_t sub = static_cast<uint32_t>(lc.seg_pos) * rowb;
    lc.cok = static_cast<uint32_t>(ck < CC::CPR ? ck : 0) * 16 - sub;
    lc.cov = static_cast<uint32_t>(cv < CC::CPR ? cv : 0) * 16 - sub;
  }

  StageIter it;
  it.mode = LM;
  it.halves = C::HALVES;
  it.i = i;
  it.seg_first = seg_first;
  it.n_off = 0;
  it.n_own = 0;
  it.win = 0;
  it.list = nullptr;
  it.offw = offw;
  it.ownl = ownl;
  it.j = 0;
  it.masked = false;
  it.orig = false;
  it.ent = 0;
  it.ks_on = (MODE == 1);
  it.n_ks = 0;
  it.n_ks_full = 0;
  it.ks = 0;
  it.kidx = -1;
  it.ring = ring;
  if (MODE != 0) {
    const size_t row = (static_cast<size_t>(b) * a.Hq + g) * a.nb + i;
    it.n_off = min(max(a.counts[row], 0), it.seg_first);
    it.list = a.idx + row * a.max_off;
    it.fill(0, tid, C::NT);
    // Visible own-segment blocks, compacted by wave 0.  Permuted order: a block is skipped when
    // its smallest original position is after the query block's last row; every visited block
    // is masked per key.  Identity order: blocks up to the diagonal, only the diagonal masked.
    int last_row = i * BS + BS - 1;   // the latest original position among the block's rows
    int first_row = i * BS;           // the earliest
    if constexpr (MODE == 4) {
      int mx = t;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
      if (lane == 0) qmax_w[w] = mx;
      __syncthreads();
      last_row = qmax_w[0];
#pragma unroll
      for (int ww = 1; ww < C::NW; ++ww) last_row = max(last_row, qmax_w[ww]);
    }
    if constexpr (MODE == 1) {
      // The own segment as a key stream: the positions from the segment's start to the block's
      // last row, those before its first row visible to every row of the block.
      it.n_ks = last_row + 1 - lc.seg_pos;
      it.n_ks_full = first_row - lc.seg_pos;
    } else {
      // Own-segment blocks, compacted by wave 0.  Permuted queries (mode 4): a permuted block is
      // skipped when its smallest original position is after every row of the block, every
      // visited block is masked per key.  Identity order: the blocks up to the diagonal, only
      // the diagonal masked.
      if (w == 0) {
        const int32_t* mp = a.minpos ? a.minpos + kv_head / BS + it.seg_first : nullptr;
        int n = 0;
        for (int o0 = 0; o0 < a.bps; o0 += 64) {
          const int o = o0 + lane;
          const int jj = it.seg_first + o;
          bool vis = false;
          if (o < a.bps) vis = (LM == 1) ? (mp == nullptr || mp[o] <= last_row) : (jj <= i);
          const uint64_t bal = __builtin_amdgcn_ballot_w64(vis);
          const int before = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
          if (vis)
            ownl[n + before] = static_cast<uint16_t>(jj | ((LM == 1 || jj == i) ? 0x8000 : 0));
          n += __builtin_popcountll(bal);
        }
        if (lane == 0) own_count = n;
      }
      __syncthreads();
      it.n_own = own_count;
    }
  }
  // Unmasked stages come first in every visit list, masked ones last.
  int n_unm, n_msk;
  int n_blk = 0;   // mode 1: the off-diagonal stages before the key stream
  if (MODE == 0) {
    n_unm = i * C::HALVES;
    n_msk = C::HALVES;
  } else if (MODE == 1) {
    // the own segment's key stream: whole stages of keys every row sees run unmasked
    n_blk = it.n_off * C::HALVES;
    n_unm = n_blk + it.n_ks_full / 32;
    n_msk = (it.n_ks + 31) / 32 - it.n_ks_full / 32;
  } else if (LM == 1) {
    n_unm = it.n_off * C::HALVES;
    n_msk = it.n_own * C::HALVES;
  } else {
    const int nm = it.n_own > 0 ? 1 : 0;   // the diagonal block closes the identity-order list
    n_unm = (it.n_off + it.n_own - nm) * C::HALVES;
    n_msk = nm * C::HALVES;
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds q[t][ks*16 + hl*8 .. +8]
  bf16x8 qf[C::NKS];
  {
    const uint16_t* qrow = a.q + a.qm.off(b, g, ts) + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  }
  f32x16 oacc[C::NMT];
#pragma unroll
  for (int mt = 0; mt < C::NMT; ++mt) oacc[mt] = f32x16{};
  RowState rs{-INFINITY, 0.f, -INFINITY};
  attn_pass<D, BS, MODE, false, true>(a, it, n_blk, n_unm, n_msk, rr, lc, smem, Ps0, Ps1, w, lane,
                                      t, qf, oacc, rs);
  // A row whose sum left [2^-60, 2^64] (scores far above or below its reference) is recomputed:
  // first its exact maximum, then the pass against that maximum.
  const float l0 = pair_sum(rs.lsum);
  if (__syncthreads_or(!(l0 >= 0x1p-60f && l0 <= 0x1p64f) ? 1 : 0)) {
    attn_pass<D, BS, MODE, true, false>(a, it, n_blk, n_unm, n_msk, rr, lc, smem, Ps0, Ps1, w,
                                        lane, t, qf, oacc, rs);
#pragma unroll
    for (int mt = 0; mt < C::NMT; ++mt) oacc[mt] = f32x16{};
    rs.mref = rs.mseen;
    rs.lsum = 0.f;
    attn_pass<D, BS, MODE, false, false>(a, it, n_blk, n_unm, n_msk, rr, lc, smem, Ps0, Ps1, w,
                                         lane, t, qf, oacc, rs);
  }

  const float l = pair_sum(rs.lsum);   // the two halves of the row
  const float inv_l = (l > 0.f) ? 1.f / l : 0.f;
  uint16_t* orow = a.o + a.qm.off(b, g, t);
#pragma unroll
  for (int mt = 0; mt < C::NMT; ++mt) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      bf16x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = static_cast<__bf16>(oacc[mt][rb * 4 + e] * inv_l);
      // O^T lane value r of tile mt is head-dim index mt*32 + (r/4)*8 + hl*4 + r%4 of row t
      *reinterpret_cast<bf16x4*>(orow + mt * 32 + rb * 8 + hl * 4) = pk;
    }
  }
  if (a.lse && hl == 0) a.lse[q_head + t] = (rs.mref + __log2f(l)) * kLn2;
}

template <int D, int BS>
hipError_t launch_attn_t(const Dims& d, AttnArgs a, hipStream_t stream) {
  using C = Cfg<D, BS>;
  a.tile_off[0] = 0;
  a.tile_off[1] = C::KTILE_A;
  a.tile_off[2] = 2 * C::KTILE_A;
  a.tile_off[3] = 2 * C::KTILE_A + C::VTILE_A;
  const int total = d.B * d.Hq * d.nb;
  const dim3 block(Cfg<D, BS>::NT);
  if (a.mode == 1) return launch(attn_fwd_kernel<D, BS, 1>, dim3(total), block, 0, stream, a);
  if (a.mode == 2) return launch(attn_fwd_kernel<D, BS, 2>, dim3(total), block, 0, stream, a);
  if (a.mode == 3) return launch(attn_fwd_kernel<D, BS, 3>, dim3(total), block, 0, stream, a);
  if (a.mode == 4) return launch(attn_fwd_kernel<D, BS, 4>, dim3(total), block, 0, stream, a);
  return launch(attn_fwd_kernel<D, BS, 0>, dim3(total), block, 0, stream, a);
}

}  // namespace

hipError_t launch_attn(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* perm, const int32_t* perm_inv, const int32_t* blk_minpos,
                       const int32_t* counts, const int32_t* idx, const uint16_t* k_orig,
                       const uint16_t* v_orig, int mode, float scale, uint16_t* o, float* lse,
                       hipStream_t stream) {
  AttnArgs a;
  a.q = q; a.k = k; a.v = v;
  a.k2 = k_orig; a.v2 = v_orig;
  a.perm = perm; a.inv = perm_inv; a.minpos = blk_minpos; a.counts = counts; a.idx = idx;
  a.o = o; a.lse = lse;
  a.B = d.B; a.Hq = d.Hq; a.Hkv = d.Hkv; a.G = d.G; a.N = d.N; a.nb = d.nb; a.bps = d.bps;
  a.max_off = d.max_off > 0 ? d.max_off : 1;
  a.mode = mode;
  const long long total = static_cast<long long>(d.B) * d.Hq * d.nb;
  const int heads = d.B * d.Hkv;
  a.xcd_split = 1;
  a.xcd_map = 0;
  if (total % 8 == 0 && heads % 8 == 0) {
    a.xcd_map = 1;
  } else if (total % 8 == 0 && 8 % heads == 0) {
    a.xcd_map = 2;                  // per_head * heads = total, so per_head % (8 / heads) == 0
    a.xcd_split = 8 / heads;
  }
  a.c = scale * kLog2e;
  a.qm = q_rows(d);
  a.km = kv_rows(d);
  a.kv_rs = a.km.stride();
  if (d.d == 128 && d.Bs == 128) return launch_attn_t<128, 128>(d, a, stream);
  if (d.d == 128 && d.Bs == 64) return launch_attn_t<128, 64>(d, a, stream);
  if (d.d == 64 && d.Bs == 128) return launch_attn_t<64, 128>(d, a, stream);
  return launch_attn_t<64, 64>(d, a, stream);
}

}  // namespace pbs
