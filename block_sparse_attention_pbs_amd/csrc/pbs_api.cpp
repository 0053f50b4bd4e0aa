// C-ABI entry points of libpbs: argument validation, workspace carving and kernel launches on
// the caller's stream.  Every check happens before the first launch; nothing here allocates,
// frees or synchronises.
#include "pbs.h"
#include "pbs_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

using pbs::Dims;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Fills `d` and returns PBS_OK, or the status describing why the shape is unsupported.
int check_shape(const pbs_shape* s, Dims* d) {
  if (!s) return PBS_E_ARG;
  if (s->batch < 0 || s->seq_len < 0) return PBS_E_SHAPE;
  if (s->heads_q <= 0 || s->heads_kv <= 0 || s->heads_q % s->heads_kv) return PBS_E_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return PBS_E_SHAPE;
  if (s->block != 64 && s->block != 128) return PBS_E_SHAPE;
  if (s->segment <= 0 || s->segment % s->block || s->segment > 16384) return PBS_E_SHAPE;
  if (s->seq_len % s->segment) return PBS_E_SHAPE;
  if (s->seq_len / s->block > 8192) return PBS_E_SHAPE;
  if (s->layout != PBS_LAYOUT_BHND && s->layout != PBS_LAYOUT_BNHD) return PBS_E_SHAPE;
  // K/V rows are addressed with 32-bit byte offsets from the start of a head
  if (s->layout == PBS_LAYOUT_BNHD &&
      static_cast<uint64_t>(s->seq_len) * s->heads_kv * s->head_dim * 2 >= (1ull << 32))
    return PBS_E_SHAPE;
  // ... and one token's K/V row (all KV heads) is under 2^24 bytes (24-bit multiplies)
  if (s->layout == PBS_LAYOUT_BNHD &&
      static_cast<uint64_t>(s->heads_kv) * s->head_dim * 2 >= (1ull << 24))
    return PBS_E_SHAPE;
  d->B = s->batch;
  d->Hq = s->heads_q;
  d->Hkv = s->heads_kv;
  d->N = s->seq_len;
  d->d = s->head_dim;
  d->Bs = s->block;
  d->S = s->segment;
  d->G = s->heads_q / s->heads_kv;
  d->nb = s->seq_len / s->block;
  d->bps = s->segment / s->block;
  d->nseg = s->seq_len / s->segment;
  d->max_off = d->nseg > 0 ? (d->nseg - 1) * d->bps : 0;
  d->layout = s->layout;
  return PBS_OK;
}

bool empty(const Dims& d) { return d.B == 0 || d.N == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? PBS_OK : PBS_E_LAUNCH; }

// All of `ptrs` present (non-null) and 16-byte aligned.
template <int K>
int check_required(const void* const (&ptrs)[K]) {
  for (int i = 0; i < K; ++i)
    if (!ptrs[i]) return PBS_E_ARG;
  for (int i = 0; i < K; ++i)
    if (!aligned16(ptrs[i])) return PBS_E_ALIGN;
  return PBS_OK;
}

int check_optional(const void* p) { return (p && !aligned16(p)) ? PBS_E_ALIGN : PBS_OK; }

bool finite_positive(float x) { return x > 0.f && x < 3.0e38f; }

}  // namespace

extern "C" {

size_t pbs_workspace_bytes(const pbs_shape* shape) {
  Dims d;
  if (check_shape(shape, &d) != PBS_OK) return 0;
  const size_t a = pbs::score_workspace_bytes(d);
  const size_t b = pbs::select_workspace_bytes(d);
  return a > b ? a : b;
}

int32_t pbs_max_offdiag(const pbs_shape* shape) {
  Dims d;
  if (check_shape(shape, &d) != PBS_OK) return -1;
  return d.max_off;
}

const char* pbs_strerror(int status) {
  switch (status) {
    case PBS_OK: return "ok";
    case PBS_E_ARG: return "invalid argument (null pointer, mode, flag or parameter)";
    case PBS_E_SHAPE: return "unsupported shape";
    case PBS_E_ALIGN: return "pointer not 16-byte aligned";
    case PBS_E_WORKSPACE: return "workspace too small";
    case PBS_E_LAUNCH: return "kernel launch failed";
    case PBS_E_SCRATCH: return "problem larger than the static scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Packed sequences: one batch row, 1 <= n_seqs <= N / S sequences, boundaries on the device.
int check_varlen(const Dims& d, const int32_t* cu_seqlens, int32_t n_seqs) {
  if (d.B != 1 && !empty(d)) return PBS_E_SHAPE;
  if (!cu_seqlens) return PBS_E_ARG;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return PBS_E_ALIGN;
  if (n_seqs < 1 || (!empty(d) && n_seqs > d.nseg)) return PBS_E_ARG;
  return PBS_OK;
}

int score_impl(const pbs_shape* shape, const int32_t* cu, int32_t nseq, const uint16_t* q,
               const uint16_t* k, float scale, float* scores, void* workspace,
               size_t workspace_bytes, void* stream) {
  Dims d;
  int st = check_shape(shape, &d);
  if (st != PBS_OK) return st;
  if (cu && (st = check_varlen(d, cu, nseq)) != PBS_OK) return st;
  if (!finite_positive(scale)) return PBS_E_ARG;
  if (empty(d)) return PBS_OK;
  const void* const req[] = {q, k, scores, workspace};
  if ((st = check_required(req)) != PBS_OK) return st;
  if (workspace_bytes < pbs::score_workspace_bytes(d)) return PBS_E_WORKSPACE;
  return status_of(pbs::launch_score(d, q, k, scale, scores, workspace, cu, cu ? nseq : 0,
                                     static_cast<hipStream_t>(stream)));
}

int select_impl(const pbs_shape* shape, const int32_t* cu, int32_t nseq, const uint16_t* q,
                const uint16_t* k_perm, const float* k_pool, float scale, int mode, double param,
                float* blk_scores, int flags, int32_t* counts, int32_t* idx, void* workspace,
                size_t workspace_bytes, void* stream) {
  Dims d;
  int st = check_shape(shape, &d);
  if (st != PBS_OK) return st;
  if (cu && (st = check_varlen(d, cu, nseq)) != PBS_OK) return st;
  if (mode != PBS_SELECT_KEEP_RATIO && mode != PBS_SELECT_COVERAGE) return PBS_E_ARG;
  if (!(param > 0.0 && param <= 1.0)) return PBS_E_ARG;
  if (flags & ~(PBS_FLAG_SCORES_IN | PBS_FLAG_KEEP_FIRST)) return PBS_E_ARG;
  const bool scores_in = (flags & PBS_FLAG_SCORES_IN) != 0;
  if (!scores_in && !finite_positive(scale)) return PBS_E_ARG;
  if (empty(d)) return PBS_OK;
  const void* const req[] = {counts, idx, workspace};
  if ((st = check_required(req)) != PBS_OK) return st;
  if (scores_in) {
    if (!blk_scores) return PBS_E_ARG;
  } else {
    if (!q || (!k_perm && !k_pool)) return PBS_E_ARG;
  }
  if ((st = check_optional(q)) != PBS_OK) return st;
  if ((st = check_optional(k_perm)) != PBS_OK) return st;
  if ((st = check_optional(k_pool)) != PBS_OK) return st;
  if ((st = check_optional(blk_scores)) != PBS_OK) return st;
  if (workspace_bytes < pbs::select_workspace_bytes(d)) return PBS_E_WORKSPACE;
  const bool keep_first = (flags & PBS_FLAG_KEEP_FIRST) != 0;
  return status_of(pbs::launch_block_select(d, q, k_perm, k_pool, scale, mode, param, blk_scores,
                                            scores_in, keep_first, counts, idx, workspace, cu,
                                            cu ? nseq : 0, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int pbs_score(const pbs_shape* shape, const uint16_t* q, const uint16_t* k, float scale,
              float* scores, void* workspace, size_t workspace_bytes, void* stream) {
  return score_impl(shape, nullptr, 0, q, k, scale, scores, workspace, workspace_bytes, stream);
}

int pbs_score_noalloc(const pbs_shape* shape, const uint16_t* q, const uint16_t* k, float scale,
                      float* scores, void* stream) {
  Dims d;
  int st = check_shape(shape, &d);
  if (st != PBS_OK) return st;
  if (!finite_positive(scale)) return PBS_E_ARG;
  if (empty(d)) return PBS_OK;
  const void* const req[] = {q, k, scores};
  if ((st = check_required(req)) != PBS_OK) return st;
  if (pbs::score_workspace_bytes(d) > pbs::kNoAllocScratchBytes) return PBS_E_SCRATCH;
  void* ws = nullptr;
  if (pbs::score_noalloc_scratch(&ws) != hipSuccess) return PBS_E_LAUNCH;
  return status_of(pbs::launch_score(d, q, k, scale, scores, ws, nullptr, 0,
                                     static_cast<hipStream_t>(stream)));
}

int pbs_score_varlen(const pbs_shape* shape, const int32_t* cu_seqlens, int32_t n_seqs,
                     const uint16_t* q, const uint16_t* k, float scale, float* scores,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return PBS_E_ARG;
  return score_impl(shape, cu_seqlens, n_seqs, q, k, scale, scores, workspace, workspace_bytes,
                    stream);
}

int pbs_permute(const pbs_shape* shape, const float* scores, const uint16_t* k,
                const uint16_t* v, int32_t* perm, uint16_t* k_perm, uint16_t* v_perm,
                float* k_pool, int32_t* blk_minpos, int32_t* perm_inv, void* stream) {
  Dims d;
  int st = check_shape(shape, &d);
  if (st != PBS_OK) return st;
  if (empty(d)) return PBS_OK;
  const void* const req[] = {scores, k, v, perm, k_perm, v_perm};
  if ((st = check_required(req)) != PBS_OK) return st;
  if ((st = check_optional(k_pool)) != PBS_OK) return st;
  if ((st = check_optional(blk_minpos)) != PBS_OK) return st;
  if ((st = check_optional(perm_inv)) != PBS_OK) return st;
  return status_of(pbs::launch_permute(d, scores, k, v, perm, k_perm, v_perm, k_pool, blk_minpos,
                                       perm_inv, static_cast<hipStream_t>(stream)));
}

int pbs_permute_queries(const pbs_shape* shape, const int32_t* perm, const uint16_t* q,
                        uint16_t* q_perm, void* stream) {
  Dims d;
  int st = check_shape(shape, &d);
  if (st != PBS_OK) return st;
  if (empty(d)) return PBS_OK;
  const void* const req[] = {perm, q, q_perm};
  if ((st = check_required(req)) != PBS_OK) return st;
  if (static_cast<const void*>(q) == static_cast<const void*>(q_perm)) return PBS_E_ARG;
  return status_of(pbs::launch_permute_queries(d, perm, q, q_perm,
                                               static_cast<hipStream_t>(stream)));
}

int pbs_block_select(const pbs_shape* shape, const uint16_t* q, const uint16_t* k_perm,
                     const float* k_pool, float scale, int mode, double param,
                     float* blk_scores, int flags, int32_t* counts, int32_t* idx,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl(shape, nullptr, 0, q, k_perm, k_pool, scale, mode, param, blk_scores, flags,
                     counts, idx, workspace, workspace_bytes, stream);
}

int pbs_block_select_varlen(const pbs_shape* shape, const int32_t* cu_seqlens, int32_t n_seqs,
                            const uint16_t* q, const uint16_t* k_perm, const float* k_pool,
                            float scale, int mode, double param, float* blk_scores, int flags,
                            int32_t* counts, int32_t* idx, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return PBS_E_ARG;
  return select_impl(shape, cu_seqlens, n_seqs, q, k_perm, k_pool, scale, mode, param,
                     blk_scores, flags, counts, idx, workspace, workspace_bytes, stream);
}

int pbs_attn_fwd(const pbs_shape* shape, const uint16_t* q, const uint16_t* k,
                 const uint16_t* v, const int32_t* perm, const int32_t* perm_inv,
                 const int32_t* counts, const int32_t* idx, float scale, uint16_t* o,
                 float* lse, void* stream) {
  Dims d;
  int st = check_shape(shape, &d);
  if (st != PBS_OK) return st;
  if (!finite_positive(scale)) return PBS_E_ARG;
  if ((counts == nullptr) != (idx == nullptr)) return PBS_E_ARG;
  if ((perm == nullptr) != (perm_inv == nullptr)) return PBS_E_ARG;  // both or neither
  if (!counts && perm) return PBS_E_ARG;  // dense mode takes no permutation
  if (empty(d)) return PBS_OK;
  const void* const req[] = {q, k, v, o};
  if ((st = check_required(req)) != PBS_OK) return st;
  const void* const opt[] = {perm, perm_inv, counts, idx, lse};
  for (const void* p : opt)
    if ((st = check_optional(p)) != PBS_OK) return st;
  const int mode = !counts ? 0 : (perm ? 1 : 2);
  return status_of(pbs::launch_attn(d, q, k, v, perm, perm_inv, nullptr, counts, idx, nullptr,
                                    nullptr, mode, scale, o, lse,
                                    static_cast<hipStream_t>(stream)));
}

int pbs_attn_fwd_permuted_queries(const pbs_shape* shape, const uint16_t* q_perm,
                                  const uint16_t* k_perm, const uint16_t* v_perm,
                                  const int32_t* perm, const int32_t* blk_minpos,
                                  const int32_t* counts, const int32_t* idx, float scale,
                                  uint16_t* o, float* lse, void* stream) {
  Dims d;
  int st = check_shape(shape, &d);
  if (st != PBS_OK) return st;
  if (!finite_positive(scale)) return PBS_E_ARG;
  if (empty(d)) return PBS_OK;
  const void* const req[] = {q_perm, k_perm, v_perm, perm, counts, idx, o};
  if ((st = check_required(req)) != PBS_OK) return st;
  if ((st = check_optional(blk_minpos)) != PBS_OK) return st;
  if ((st = check_optional(lse)) != PBS_OK) return st;
  return status_of(pbs::launch_attn(d, q_perm, k_perm, v_perm, perm, nullptr, blk_minpos, counts,
                                    idx, nullptr, nullptr, 4, scale, o, lse,
                                    static_cast<hipStream_t>(stream)));
}

int pbs_attn_fwd_hybrid(const pbs_shape* shape, const uint16_t* q, const uint16_t* k_perm,
                        const uint16_t* v_perm, const uint16_t* k, const uint16_t* v,
                        const int32_t* counts, const int32_t* idx, float scale, uint16_t* o,
                        float* lse, void* stream) {
  Dims d;
  int st = check_shape(shape, &d);
  if (st != PBS_OK) return st;
  if (!finite_positive(scale)) return PBS_E_ARG;
  if (empty(d)) return PBS_OK;
  const void* const req[] = {q, k_perm, v_perm, k, v, counts, idx, o};
  if ((st = check_required(req)) != PBS_OK) return st;
  if ((st = check_optional(lse)) != PBS_OK) return st;
  return status_of(pbs::launch_attn(d, q, k_perm, v_perm, nullptr, nullptr, nullptr, counts, idx,
                                    k, v, 3, scale, o, lse, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
