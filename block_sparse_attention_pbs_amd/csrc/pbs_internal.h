// Internal interface between the C-ABI layer (pbs_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pbs {

// Validated problem dimensions.
struct Dims {
  int B, Hq, Hkv, N, d, Bs, S;
  int G;        // Hq / Hkv
  int nb;       // N / Bs
  int bps;      // S / Bs
  int nseg;     // N / S
  int max_off;  // (nseg - 1) * bps
  int layout;   // 0: bf16 tensors [B, H, N, d]; 1: [B, N, H, d]
};

// Addressing of a bf16 [B, H, N, d] tensor in either layout: the element offset of row n of head
// h of batch b, and the element distance between two consecutive rows of one head.
struct RowMap {
  int layout, H, N, d;
  __host__ __device__ size_t off(int b, int h, int n) const {
    return layout == 0 ? ((static_cast<size_t>(b) * H + h) * N + n) * d
                       : ((static_cast<size_t>(b) * N + n) * H + h) * d;
  }
  __host__ __device__ int stride() const { return layout == 0 ? d : H * d; }
};
inline RowMap q_rows(const Dims& d) { return RowMap{d.layout, d.Hq, d.N, d.d}; }
inline RowMap kv_rows(const Dims& d) { return RowMap{d.layout, d.Hkv, d.N, d.d}; }

// Kernel launch through hipLaunchKernel so that the status of this very launch is returned
// (every kernel takes one argument struct).
template <typename Args>
inline hipError_t launch(void (*kernel)(Args), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, const Args& args) {
  Args copy = args;
  void* argv[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, shmem, stream);
}

// Workspace of pbs_score: per (batch, KV head, segment, scoring row) softmax max and sum.
size_t score_workspace_bytes(const Dims& d);
// pbs_score_noalloc: capacity of the library's static scratch and its address on the current
// device (looked up on the first call per device, no allocation).
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(16) << 20;
hipError_t score_noalloc_scratch(void** ptr);
// cu / nseq: packed sequences (nseq + 1 starts along N) or null / 0 for one sequence per row.
hipError_t launch_score(const Dims& d, const uint16_t* q, const uint16_t* k, float scale,
                        float* scores, void* ws, const int32_t* cu, int nseq,
                        hipStream_t stream);

// perm_inv (may be null): perm_inv[perm[p]] = p, the slot of every original position.
hipError_t launch_permute(const Dims& d, const float* scores, const uint16_t* k,
                          const uint16_t* v, int32_t* perm, uint16_t* k_perm, uint16_t* v_perm,
                          float* k_pool, int32_t* blk_minpos, int32_t* perm_inv,
                          hipStream_t stream);

// The query-permutation variant: q_perm[b, g, p] = q[b, g, perm[b, g / G, p]].
hipError_t launch_permute_queries(const Dims& d, const int32_t* perm, const uint16_t* q,
                                  uint16_t* q_perm, hipStream_t stream);

// Workspace of pbs_block_select: pooled queries (and pooled keys when not supplied).
size_t select_workspace_bytes(const Dims& d);
hipError_t launch_block_select(const Dims& d, const uint16_t* q, const uint16_t* k_perm,
                               const float* k_pool, float scale, int mode, double param,
                               float* blk_scores, bool scores_in, bool keep_first, int32_t* counts,
                               int32_t* idx, void* ws, const int32_t* cu, int nseq,
                               hipStream_t stream);

// mode: 0 dense causal, 1 PBS with a permutation, 2 PBS in the identity order, 3 PBS with
// permuted off-diagonal blocks and the own segment read from k_orig/v_orig in natural order,
// 4 PBS with permuted queries (q holds them; rows are written back at their original positions).
// perm_inv: mode 1, the slot of every original position (the inverse of perm).
hipError_t launch_attn(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int32_t* perm, const int32_t* perm_inv, const int32_t* blk_minpos,
                       const int32_t* counts, const int32_t* idx, const uint16_t* k_orig,
                       const uint16_t* v_orig, int mode, float scale, uint16_t* o, float* lse,
                       hipStream_t stream);

}  // namespace pbs
