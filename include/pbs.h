/*
 * pbs.h -- C ABI of libpbs, Permuted Block-Sparse Attention (PBS-Attn) prefill on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (arXiv 2510.21270, "Sparser Block-Sparse Attention via Token Permutation";
 * sciencestack.ai page: Abstract, Fig. 1 caption, Lemma 3.1; gist.science summary: Methodik
 * 2-4) computes causal prefill attention in four steps, one entry point each:
 *   pbs_score         importance of every key, from the last block of queries
 *   pbs_permute       segment-local descending sort of the keys; permuted copies of K and V
 *   pbs_block_select  per query block, which earlier-segment key blocks to compute
 *   pbs_attn_fwd      block-sparse flash attention over those blocks plus the whole own
 *                     segment (token-level causal mask through the stored positions)
 *
 * Conventions shared by every call
 *  - Tensors are DEVICE pointers owned by the caller, contiguous; bf16 is passed as uint16_t
 *    bit patterns.  The bf16 activations -- q, k, v, o and the permuted copies k_perm, v_perm,
 *    q_perm -- are laid out as pbs_shape.layout says: PBS_LAYOUT_BHND (0, the default of a
 *    zero-initialised shape) Q/O [B, Hq, N, d], K/V [B, Hkv, N, d]; or PBS_LAYOUT_BNHD (1, the
 *    token-major layout of FlashAttention-style callers) Q/O [B, N, Hq, d], K/V [B, N, Hkv, d].
 *    Every other tensor (scores, perm, k_pool, blk_minpos, blk_scores, counts, idx, lse) is
 *    head-major as documented at its call.  Every pointer must be 16-byte aligned
 *    (PBS_E_ALIGN otherwise).
 *  - Query head g reads KV head g / (Hq / Hkv) (grouped-query attention).
 *  - Block size Bs (the pages' B) and segment size S (the pages' S) come in pbs_shape.
 *    Required: Hq % Hkv == 0, d in {64, 128}, Bs in {64, 128}, S % Bs == 0, N % S == 0,
 *    S <= 16384, N / Bs <= 8192, and for PBS_LAYOUT_BNHD N * Hkv * d * 2 < 2^32 bytes and
 *    Hkv * d * 2 < 2^24 bytes (PBS_E_SHAPE otherwise).  batch == 0 or seq_len == 0 is an
 *    empty problem: once the shape and the scalar arguments are valid the call returns PBS_OK
 *    without launching anything or inspecting the pointers.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).  The
 *    library never allocates or frees device memory, never synchronises, and keeps no
 *    mutable global state; calls on different streams with disjoint outputs may overlap.
 *  - Return value: PBS_OK (0) or a negative pbs_status.  All arguments are checked before
 *    any launch, so an error return means nothing was enqueued, except PBS_E_LAUNCH (a
 *    launch was rejected by the runtime; earlier kernels of the same call may have run).
 *    Outputs are only valid once the stream has reached the call.
 */
#ifndef PBS_H
#define PBS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pbs_shape {
  int32_t batch;     /* B                                                */
  int32_t heads_q;   /* Hq, query heads                                  */
  int32_t heads_kv;  /* Hkv, key/value heads (Hq % Hkv == 0)             */
  int32_t seq_len;   /* N                                                */
  int32_t head_dim;  /* d, 64 or 128                                     */
  int32_t block;     /* Bs, attention block size, 64 or 128              */
  int32_t segment;   /* S, permutation segment size, multiple of Bs      */
  int32_t layout;    /* PBS_LAYOUT_BHND or PBS_LAYOUT_BNHD (bf16 tensors) */
} pbs_shape;

#define PBS_LAYOUT_BHND 0 /* [B, H, N, d]: each head's rows contiguous                  */
#define PBS_LAYOUT_BNHD 1 /* [B, N, H, d]: each token's heads contiguous (row stride H*d) */

typedef enum pbs_status {
  PBS_OK = 0,
  PBS_E_ARG = -1,       /* NULL where a pointer is required, bad mode / flag / parameter */
  PBS_E_SHAPE = -2,     /* shape outside the supported set above                          */
  PBS_E_ALIGN = -3,     /* a pointer not 16-byte aligned                                  */
  PBS_E_WORKSPACE = -4, /* workspace smaller than pbs_workspace_bytes()                   */
  PBS_E_LAUNCH = -5,    /* the HIP runtime rejected a kernel launch                       */
  PBS_E_SCRATCH = -6    /* pbs_score_noalloc: the problem needs more than its static scratch */
} pbs_status;

typedef enum pbs_select_mode {
  PBS_SELECT_KEEP_RATIO = 0, /* keep max(1, floor(r * n)) of the n candidate blocks, 0 < r <= 1   */
  PBS_SELECT_COVERAGE = 1    /* keep the fewest top blocks whose probability reaches tau, 0 < tau <= 1 */
} pbs_select_mode;

/* pbs_block_select flag: read the block probabilities from `blk_scores` instead of
   computing them (selection only). */
#define PBS_FLAG_SCORES_IN 1
/* pbs_block_select flag: rank key block 0 ahead of every other candidate, so every query block
   with candidates keeps it and, for coverage, its probability is counted first.  Key block 0
   holds the first tokens in natural order and the top-ranked keys of segment 0 in permuted
   order, where the attention sink lands.  The pages name a first-token mask in the authors'
   code (codewithpapers.app record) without defining it; this is its plainest reading. */
#define PBS_FLAG_KEEP_FIRST 2

/* Bytes of device workspace that pbs_score and pbs_block_select need for `shape`
   (the larger of the two).  0 for an invalid shape. */
size_t pbs_workspace_bytes(const pbs_shape* shape);

/* Row stride of the `idx` lists: (N/S - 1) * (S/Bs), the number of key blocks in earlier
   segments for the last segment.  -1 for an invalid shape. */
int32_t pbs_max_offdiag(const pbs_shape* shape);

/* Static description of a status code. */
const char* pbs_strerror(int status);

/*
 * pbs_score -- query-aware key importance from the last query block.
 * Passage: gist.science summary, Methodik 3 ("Proxy-Bewertung"): the global importance of
 * the keys is estimated from the last block of queries by mean pooling of their attention
 * scores; Methodik 2: no attention crosses into a later segment.
 *
 * For every KV head h and key j in segment s:
 *   scores[b,h,j] = 1/(G*Bs) * sum over q-heads g of h and rows t in [N-Bs, N) of
 *                   softmax over keys j' of segment s with j' <= t of (scale * <q[b,g,t], k[b,h,j']>), at j
 * (0 where j > t).  Each segment's scores sum to 1.
 *   q        [B,Hq,N,d] bf16 (only the last Bs rows of each head are read)
 *   k        [B,Hkv,N,d] bf16
 *   scale    softmax scale, normally 1/sqrt(d)
 *   scores   [B,Hkv,N] float32, written
 *   workspace / workspace_bytes   device scratch of at least pbs_workspace_bytes(shape)
 */
int pbs_score(const pbs_shape* shape, const uint16_t* q, const uint16_t* k, float scale,
              float* scores, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pbs_score_noalloc -- pbs_score for callers that cannot allocate device memory (code recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and the same result, bit for bit, with the score partials in a static scratch array
 * of the library instead of a caller's workspace.
 *   - The scratch holds PBS_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, a file-scope device array
 *     that each GPU the library runs on keeps until the process ends; its device address is
 *     looked up once per device, on the first call there.  No call allocates or frees memory.
 *   - A shape whose score partials (68 bytes per scoring row and segment at S = 8192, Bs = 128)
 *     do not fit returns PBS_E_SCRATCH before anything is enqueued; 32 query / 8 KV heads at
 *     Bs = 128 and S = 8192 fit up to 480K tokens.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents:
 *     calls that overlap on one GPU (different streams, or graphs replayed concurrently) race
 *     and give unspecified scores.  Calls ordered on one stream are safe.  Nothing in the
 *     scratch needs to start at zero.
 * Arguments, outputs and errors otherwise as pbs_score.
 */
#define PBS_NOALLOC_SCRATCH_BYTES (16u << 20)
int pbs_score_noalloc(const pbs_shape* shape, const uint16_t* q, const uint16_t* k, float scale,
                      float* scores, void* stream);

/*
 * pbs_permute -- segmented permutation of keys and values.
 * Passage: gist.science summary, Methodik 2 (permutation only inside contiguous segments of
 * size S) and Methodik 3 ("Sortierung": keys sorted by descending importance in each
 * segment); sciencestack.ai page, Lemma 3.1 (keys and values move together).
 *
 * Within each segment, slots are ordered by score descending, ties by lower original
 * position (-0 equals +0; NaN after every number):
 *   perm[b,h,p]      original position of the key at slot p (int32, stays in p's segment)
 *   k_perm[b,h,p,:]  = k[b,h,perm[b,h,p],:]   (bit copy), same for v_perm
 *   k_pool[b,h,j,:]  float32 mean of k_perm rows of block j (optional, may be NULL;
 *                    pbs_block_select can reuse it)
 *   blk_minpos[b,h,j] smallest original position held by block j (optional, may be NULL;
 *                    lets pbs_attn_fwd_permuted_queries skip own-segment blocks no query of
 *                    a block can see)
 *   perm_inv[b,h,j]  slot that holds original position j: perm_inv[b,h,perm[b,h,p]] = p
 *                    (optional, may be NULL; pbs_attn_fwd walks it to read exactly the own-
 *                    segment keys a query block can see; SK Implementation Steps keep the
 *                    permutation so that it can be undone)
 *   scores [B,Hkv,N] float32, k/v [B,Hkv,N,d] bf16 -> perm [B,Hkv,N], k_perm/v_perm
 *   [B,Hkv,N,d], k_pool [B,Hkv,N/Bs,d], blk_minpos [B,Hkv,N/Bs], perm_inv [B,Hkv,N].
 */
int pbs_permute(const pbs_shape* shape, const float* scores, const uint16_t* k,
                const uint16_t* v, int32_t* perm, uint16_t* k_perm, uint16_t* v_perm,
                float* k_pool, int32_t* blk_minpos, int32_t* perm_inv, void* stream);

/*
 * pbs_permute_queries -- queries moved with their tokens (the query-permutation variant).
 * Passage: sciencestack.ai page, Lemma 3.2 (permuting the queries permutes the output rows the
 * same way) and Theorem 3.3 (permuting queries and keys/values, then applying the inverse
 * permutation to the output, restores the result); gist.science summary, Methodik 1 and
 * Methodik 3 ("Handling von Queries": the default keeps queries in natural order because
 * moving them gave only marginal gains; this entry point is the variant that moves them).
 *
 *   q_perm[b,g,p,:] = q[b,g,perm[b,g/G,p],:]   (bit copy; query head g follows its KV head)
 *   perm   [B,Hkv,N] int32 from pbs_permute
 *   q      [B,Hq,N,d] bf16;  q_perm [B,Hq,N,d] bf16, written (must not alias q)
 * Out-of-range perm entries are clamped into [0, N) (memory-safe, result unspecified).
 */
int pbs_permute_queries(const pbs_shape* shape, const int32_t* perm, const uint16_t* q,
                        uint16_t* q_perm, void* stream);

/*
 * pbs_block_select -- which earlier-segment key blocks each query block computes.
 * Passage: gist.science summary, Methodik 4 ("Block-Auswahl": block importance from mean
 * pooling on the permuted keys); sciencestack.ai page, Fig. 1 caption (blocks of the own,
 * on-diagonal segment are always computed; inter-segment blocks may be skipped) and Fig. 2
 * caption (coverage = attention mass of the selected blocks); skillmd.com page, Implementation
 * Steps (active-block count max(1, int(num_blocks * keep))).
 *
 * For query block i of segment s = i / (S/Bs), the candidates are key blocks j < s*(S/Bs):
 *   P[i,j] = softmax over candidates of scale * <mean of q rows of block i,
 *                                              mean of k_perm rows of block j>
 * ranked by P descending, ties to the lower j (with PBS_FLAG_KEEP_FIRST block 0 first); kept:
 *   PBS_SELECT_KEEP_RATIO (param = r):   the first max(1, floor(r*n)) (in double), n = #candidates
 *   PBS_SELECT_COVERAGE   (param = tau): the shortest prefix whose sequential float32 sum of
 *                                        P (compared in double) is >= tau; all n if none.
 *   q          [B,Hq,N,d] bf16
 *   k_perm     [B,Hkv,N,d] bf16 (permuted keys; the natural K gives plain block-sparse
 *              selection). May be NULL if k_pool is given.
 *   k_pool     [B,Hkv,N/Bs,d] float32 block means of k_perm, or NULL (then computed here)
 *   blk_scores [B,Hq,N/Bs,N/Bs] float32 or NULL.  Output of P (0 off the candidates) unless
 *              flags has PBS_FLAG_SCORES_IN; then P is read from it (candidates only).
 *   counts     [B,Hq,N/Bs] int32, written: number kept (0 for the first segment)
 *   idx        [B,Hq,N/Bs,pbs_max_offdiag] int32, written: kept block indices ascending in
 *              the first counts entries of each row; the rest of a row is left untouched
 *   workspace  at least pbs_workspace_bytes(shape) bytes
 */
int pbs_block_select(const pbs_shape* shape, const uint16_t* q, const uint16_t* k_perm,
                     const float* k_pool, float scale, int mode, double param,
                     float* blk_scores, int flags, int32_t* counts, int32_t* idx,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * pbs_attn_fwd -- block-sparse flash-attention forward with permuted keys.
 * Passage: sciencestack.ai page, Fig. 1 caption (own-segment blocks computed under the causal
 * mask, inter-segment blocks skippable) and Lemma 3.1 (a joint key/value permutation leaves
 * attention unchanged); gist.science summary, Methodik 3 ("Handling von Queries": queries keep
 * their natural order, so the output is already in original token order) and Methodik 4
 * ("Kernel").
 *
 * PBS mode (counts and idx given): query row t of block i in segment s attends to
 *   - every key of the kept blocks idx[b,g,i,0..counts) (whole blocks, no mask), and
 *   - every key of segment s with original position <= t: slot p is visible to row t iff
 *     perm[b,h,p] <= t.  The kernel reads only the slots some row of the block can see: those
 *     holding positions s*S .. the block's last row, found through perm_inv and taken in the
 *     order of their positions; the keys before the block's first row unmasked, the block's
 *     own Bs positions under the causal test on perm[slot]
 *     (perm and perm_inv NULL: identity order, plain block-sparse attention).
 * Dense mode (perm, perm_inv, counts, idx all NULL): plain causal attention over keys 0..t.
 *   q        [B,Hq,N,d] bf16 (natural order)
 *   k, v     [B,Hkv,N,d] bf16: k_perm/v_perm from pbs_permute in PBS mode, natural K/V in
 *            dense mode or with perm == NULL
 *   perm     [B,Hkv,N] int32 or NULL
 *   perm_inv [B,Hkv,N] int32, the inverse of perm (from pbs_permute); required with perm and
 *            NULL without it (PBS_E_ARG otherwise)
 *   counts [B,Hq,N/Bs], idx [B,Hq,N/Bs,pbs_max_offdiag] int32 from pbs_block_select, or NULL
 *   o      [B,Hq,N,d] bf16, written, original token order
 *   lse    [B,Hq,N] float32 natural-log softmax normaliser of every row, or NULL
 * counts, idx, perm and perm_inv are trusted to come from pbs_block_select / pbs_permute; an
 * out-of-range count, index or slot is clamped into range or reads zeros (memory-safe, result
 * unspecified).
 */
int pbs_attn_fwd(const pbs_shape* shape, const uint16_t* q, const uint16_t* k,
                 const uint16_t* v, const int32_t* perm, const int32_t* perm_inv,
                 const int32_t* counts, const int32_t* idx, float scale, uint16_t* o,
                 float* lse, void* stream);

/*
 * pbs_attn_fwd_permuted_queries -- PBS attention with the queries in the segment permutation
 * too; the output comes back in ORIGINAL token order.
 * Passage: sciencestack.ai page, Lemma 3.2 and Theorem 3.3 (the inverse permutation of the
 * output restores the unpermuted result), Fig. 1 caption (own segment under the causal mask);
 * gist.science summary, Methodik 4 ("Kernel": permutation, block selection and inverse
 * permutation handled by the attention kernels).
 *
 * Query slot p of head g holds the token at original position t = perm[b,g/G,p]; it belongs
 * to permuted query block i = p / Bs and attends to every key of the kept blocks
 * idx[b,g,i,0..counts) (a selection made on q_perm with pbs_block_select) and to every key of
 * its own segment with original position <= t.  Its output row is written at o[b,g,t,:] (and
 * lse[b,g,t]), so no separate inverse-permutation pass is needed.
 *   q_perm         [B,Hq,N,d] bf16 from pbs_permute_queries
 *   k_perm, v_perm [B,Hkv,N,d] bf16 from pbs_permute;  perm [B,Hkv,N] int32 (required)
 *   blk_minpos     [B,Hkv,N/Bs] int32 or NULL (own-segment blocks whose smallest position is
 *                  after every row of the query block are skipped)
 *   counts, idx    required; o [B,Hq,N,d] bf16 and lse [B,Hq,N] (or NULL) in original order
 * Errors as pbs_attn_fwd.
 */
int pbs_attn_fwd_permuted_queries(const pbs_shape* shape, const uint16_t* q_perm,
                                  const uint16_t* k_perm, const uint16_t* v_perm,
                                  const int32_t* perm, const int32_t* blk_minpos,
                                  const int32_t* counts, const int32_t* idx, float scale,
                                  uint16_t* o, float* lse, void* stream);

/*
 * pbs_attn_fwd_hybrid -- the same attention as pbs_attn_fwd in PBS mode, with the own segment
 * read from the ORIGINAL keys and values in natural order.
 * Passage: sciencestack.ai page, Lemma 3.1 (attention is unchanged when keys and values are
 * permuted together and the mask follows them) and Fig. 1 caption (the own segment is computed
 * under the causal mask).  Row t of query block i, segment s, sees the keys of segment s with
 * original position <= t whatever order they are stored in, so they can be read from the
 * unpermuted k/v: only blocks s*(S/Bs) .. i are visited (the diagonal one under the causal
 * mask), about half the own-segment blocks the permuted order needs, since almost every
 * permuted block holds some key at or before the query block.  The kept earlier-segment
 * blocks still come from the permuted copies.  Same output as pbs_attn_fwd(k_perm, v_perm,
 * perm, ...) up to floating-point summation order.
 *   q              [B,Hq,N,d] bf16
 *   k_perm, v_perm [B,Hkv,N,d] bf16 from pbs_permute (read for the kept blocks)
 *   k, v           [B,Hkv,N,d] bf16 original keys and values (read for the own segment)
 *   counts, idx    from pbs_block_select (required); o, lse as in pbs_attn_fwd
 * Errors as pbs_attn_fwd; every pointer except lse is required.
 */
int pbs_attn_fwd_hybrid(const pbs_shape* shape, const uint16_t* q, const uint16_t* k_perm,
                        const uint16_t* v_perm, const uint16_t* k, const uint16_t* v,
                        const int32_t* counts, const int32_t* idx, float scale, uint16_t* o,
                        float* lse, void* stream);

/*
 * pbs_score_varlen / pbs_block_select_varlen -- several sequences packed along N.
 * Passage: the pages define the method on one sequence (gist.science summary, Methodik 2-4;
 * sciencestack.ai page, Fig. 1 caption); a packed batch applies it to every sequence on its
 * own: each sequence's segments are scored by that sequence's last Bs query rows, and a query
 * block's candidates are the blocks of earlier segments of its own sequence only.
 *
 *   shape       batch = 1; seq_len = T, the packed length; q/k/v hold the sequences one after
 *               another along N (in either layout: PBS_LAYOUT_BNHD with batch 1 is the
 *               FlashAttention varlen layout [T, H, d])
 *   cu_seqlens  DEVICE int32 [n_seqs + 1], 4-byte aligned: sequence s holds tokens
 *               cu_seqlens[s] .. cu_seqlens[s+1] - 1, with 0 = cu_seqlens[0] < ... <
 *               cu_seqlens[n_seqs] = T and every length a multiple of S.  The values are not
 *               read on the host; boundaries that break these rules give unspecified results,
 *               but every memory access stays inside the tensors.
 *   n_seqs      1 <= n_seqs <= T / S (PBS_E_ARG otherwise); batch != 1 -> PBS_E_SHAPE
 * Every other argument, output and error is as in pbs_score / pbs_block_select; positions and
 * block indices are absolute in the packed row.  pbs_permute, pbs_attn_fwd,
 * pbs_attn_fwd_hybrid, pbs_permute_queries and pbs_attn_fwd_permuted_queries take the packed
 * row unchanged: segments never straddle two sequences and the block lists never leave the
 * query's sequence.  (The dense mode of pbs_attn_fwd treats the packed row as one sequence.)
 */
int pbs_score_varlen(const pbs_shape* shape, const int32_t* cu_seqlens, int32_t n_seqs,
                     const uint16_t* q, const uint16_t* k, float scale, float* scores,
                     void* workspace, size_t workspace_bytes, void* stream);
int pbs_block_select_varlen(const pbs_shape* shape, const int32_t* cu_seqlens, int32_t n_seqs,
                            const uint16_t* q, const uint16_t* k_perm, const float* k_pool,
                            float scale, int mode, double param, float* blk_scores, int flags,
                            int32_t* counts, int32_t* idx, void* workspace,
                            size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PBS_H */
