"""PBS-Attn CPU oracle -- TEST INFRASTRUCTURE, not part of the product.

A plain, slow, obviously-correct numpy implementation of what the PBS-Attn prefill path
computes, used only to check the HIP path.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); the two meet only in the seeded input
generator ``pbs_synth``, which holds none of the method's arithmetic.

Arithmetic is float64 (products of bfloat16 inputs are exact in float64).  Values become
float32 only where the path hands a float32 tensor across its boundary and an integer
decision is then taken on it: the key scores (sorted into the permutation) and the block
probabilities (top-k / coverage selection).  Those decisions are taken here on the float32
values, as the GPU path takes them.

Pages cited (the paper is arXiv 2510.21270, "Sparser Block-Sparse Attention via Token
Permutation"):
  [SS] sciencestack.ai page of the paper: TL;DR, Abstract, captions of Figures 1-5,
       titles of Lemma 3.1, Lemma 3.2 and Theorem 3.3.
  [GS] gist.science (German) summary of the paper, technical part: "Problemstellung",
       "Methodik" 1 (Theoretische Grundlage), 2 (Segmentierte Permutation), 3 (Globale-
       Importanz-basierte Key-Permutation: Proxy-Bewertung, Sortierung, Handling von
       Queries), 4 (Implementierung: Block-Auswahl, Kernel).
  [SK] skillmd.com page "Sparser Block Attention": Implementation Steps.

Notation: block size ``Bs`` (the pages' B), segment size ``S``, ``nb = N/Bs`` blocks,
``bps = S/Bs`` blocks per segment; query head ``g`` reads KV head ``g // G``, G = Hq/Hkv.

Readings taken where the pages are silent (each is listed with its reason in the design
notes of the repository):
  * softmax scale is the caller's ``scale`` (1/sqrt(d) by default), everywhere;
  * key scores: softmax of each of the last ``Bs`` query rows (of every query head in the
    KV group) over the keys of one segment, causal mask applied, averaged over the rows;
  * ordering: descending score, ties to the lower index, -0 == +0, NaN after every number;
  * candidates for block selection: key blocks of strictly earlier segments; the blocks of
    the query's own segment are always computed under the token-level causal mask;
  * keep ratio r: ``k = max(1, floor(r * n))`` of the ``n`` candidates (``n > 0``);
  * coverage tau: the shortest prefix of the descending order whose sequential float32
    sum reaches ``tau`` (all ``n`` if it never does).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

KEEP = "keep"
COVERAGE = "coverage"


# --------------------------------------------------------------------------- helpers

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64.  A bfloat16 is the upper half of a binary32, so
    shifting the 16 bits up gives the float32 value exactly; widening to float64 is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _check_shape(q_shape, kv_shape, block: int, segment: int):
    B, Hq, N, d = q_shape
    Bk, Hkv, Nk, dk = kv_shape
    if (B, N, d) != (Bk, Nk, dk) or Hq % Hkv:
        raise ValueError("inconsistent shapes")
    if segment % block or N % segment:
        raise ValueError("need N % segment == 0 and segment % block == 0")
    return B, Hq, Hkv, N, d, Hq // Hkv


def descending_order(values: np.ndarray) -> np.ndarray:
    """Indices that order ``values`` (float32, last axis) by value descending, ties to the
    lower index, -0 equal to +0, NaN after every number.

    [GS Methodik 3, Sortierung]: keys are sorted by importance, highest first.  The tie,
    signed-zero and NaN rules are this repository's reading (the pages give none)."""
    v = np.asarray(values, dtype=np.float32)
    nan = np.isnan(v)
    neg = np.where(nan, np.float32(0), -v)
    neg = np.where(neg == 0, np.float32(0), neg)        # canonical +0
    pos = np.broadcast_to(np.arange(v.shape[-1]), v.shape)
    # lexsort: the last key is the primary one.
    return np.lexsort((pos, neg, nan), axis=-1)


# --------------------------------------------------------------------------- O1 scores

def key_scores(q, k, *, block: int, segment: int, scale: float) -> np.ndarray:
    """Query-aware importance of every key, float32 ``[B, Hkv, N]``.

    [GS Methodik 3, Proxy-Bewertung]: the importance of keys is estimated from a small set
    of queries, the last block of queries, by mean pooling their attention scores.
    [GS Methodik 2]: attention never crosses into a later segment, so each row's softmax
    is taken over one segment's keys (the segment-local reading), with the causal mask.

    For each KV head h, each segment sigma, each of the G*Bs rows (g, t) with g in the
    group of h and t in [N-Bs, N):  p = softmax_{j in sigma, j <= t}(scale * <q_{g,t}, k_j>);
    score_j = (sum over rows of p_j) / (G * Bs).  Every segment's scores sum to 1."""
    B, Hq, Hkv, N, d, G = _check_shape(q.shape, k.shape, block, segment)
    rows = np.arange(N - block, N)
    t_of_row = np.tile(rows, G)                           # row r -> query position
    out = np.zeros((B, Hkv, N), dtype=np.float32)
    for b in range(B):
        for h in range(Hkv):
            Qr = np.concatenate([bf16_to_f64(q[b, g, N - block:]) for g in range(h * G, (h + 1) * G)])
            acc = np.zeros(N, dtype=np.float64)
            for s0 in range(0, N, segment):
                keys = np.arange(s0, s0 + segment)
                Z = scale * (Qr @ bf16_to_f64(k[b, h, s0:s0 + segment]).T)      # [G*Bs, S]
                visible = keys[None, :] <= t_of_row[:, None]
                Z = np.where(visible, Z, -np.inf)
                Z = Z - Z.max(axis=1, keepdims=True)
                E = np.exp(Z)
                Pm = E / E.sum(axis=1, keepdims=True)
                acc[s0:s0 + segment] = Pm.sum(axis=0)
            out[b, h] = (acc / (G * block)).astype(np.float32)
    return out


# --------------------------------------------------------------------------- O2 permutation

def segment_permutation(scores: np.ndarray, *, segment: int) -> np.ndarray:
    """int32 ``[B, Hkv, N]``: ``perm[p]`` is the ORIGINAL position of the key placed at
    slot p.  Slots of segment sigma hold exactly the keys of sigma, in descending score
    order (ties to the lower position).

    [GS Methodik 2]: permutation only inside contiguous, non-overlapping segments of size
    S, so causality between segments is kept.  [GS Methodik 3, Sortierung]: descending
    importance inside each segment.  [SS Fig. 1]: segmented permutation picture."""
    B, H, N = scores.shape
    if N % segment:
        raise ValueError("N % segment != 0")
    perm = np.empty((B, H, N), dtype=np.int32)
    for s0 in range(0, N, segment):
        order = descending_order(scores[:, :, s0:s0 + segment])
        perm[:, :, s0:s0 + segment] = (order + s0).astype(np.int32)
    return perm


def apply_permutation(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Rows of ``x [B, H, N, d]`` in permuted order: ``out[b,h,p] = x[b,h,perm[b,h,p]]``
    (a bit copy).  K and V move together, so each key keeps its value ([SS Lemma 3.1];
    [GS Methodik 1])."""
    B, H = perm.shape[:2]
    out = np.empty_like(x)
    for b in range(B):
        for h in range(H):
            out[b, h] = x[b, h, perm[b, h]]
    return out


def inverse_permutation(perm: np.ndarray) -> np.ndarray:
    """``inv[perm[p]] = p`` ([SK Implementation Steps]: the inverse restores the order)."""
    inv = np.empty_like(perm)
    B, H, N = perm.shape
    for b in range(B):
        for h in range(H):
            inv[b, h, perm[b, h]] = np.arange(N, dtype=perm.dtype)
    return inv


# --------------------------------------------------------------------------- O3 block scores

def pooled_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of every block of ``block`` consecutive rows, float64 ``[B, H, nb, d]``."""
    B, H, N, d = x.shape
    out = np.empty((B, H, N // block, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = bf16_to_f64(x[b, h]).reshape(N // block, block, d).mean(axis=1)
    return out


def block_probabilities(q, k_perm, *, block: int, segment: int, scale: float) -> np.ndarray:
    """float32 ``[B, Hq, nb, nb]``: for query block i of a segment sigma >= 1, a softmax over
    the candidate key blocks j < sigma*bps of ``scale * <mean q of block i, mean k_perm of
    block j>``; every other entry is 0.

    [GS Methodik 4, Block-Auswahl]: block importance from mean pooling, on the permuted keys.
    [SS Fig. 1]: blocks of the query's own segment are always computed; only blocks of
    earlier segments may be skipped, so only they are candidates."""
    B, Hq, Hkv, N, d, G = _check_shape(q.shape, k_perm.shape, block, segment)
    nb, bps = N // block, segment // block
    kbar = pooled_blocks(k_perm, block)
    P = np.zeros((B, Hq, nb, nb), dtype=np.float32)
    for b in range(B):
        for g in range(Hq):
            qbar = bf16_to_f64(q[b, g]).reshape(nb, block, d).mean(axis=1)
            h = g // G
            for i in range(bps, nb):
                n = (i // bps) * bps
                logits = scale * (kbar[b, h, :n] @ qbar[i])
                e = np.exp(logits - logits.max())
                P[b, g, i, :n] = (e / e.sum()).astype(np.float32)
    return P


# --------------------------------------------------------------------------- O4 selection

def keep_count(n: int, ratio: float) -> int:
    """Blocks kept out of n candidates at keep ratio r: max(1, floor(r*n)) evaluated in
    double precision, 0 when there is no candidate.  [SK Implementation Steps] prints the
    count of active blocks as max(1, int(num_blocks * (1 - sparse_ratio))); r is that
    1 - sparse_ratio, passed directly."""
    if n == 0:
        return 0
    return max(1, int(math.floor(float(ratio) * n)))


def select_blocks(P: np.ndarray, *, block: int, segment: int, mode: str, param: float,
                  keep_first: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Per query block, which candidate key blocks are computed.

    Returns ``counts`` int32 ``[B, Hq, nb]`` and ``idx`` int32 ``[B, Hq, nb, (nseg-1)*bps]``
    (the first ``counts`` entries ascending; the rest -1).

    Candidates of block i are ``j < segb(i)*bps`` ([SS Fig. 1]); they are ranked by P
    descending, ties to the lower j ([GS Methodik 4, Block-Auswahl] estimates importance;
    the order rule is this repository's reading).
      keep:     the first ``keep_count(n, r)`` of that ranking;
      coverage: the shortest prefix whose sequential float32 sum of P, widened to double,
                reaches tau, i.e. the fewest top blocks that cover tau of the block-level
                attention mass
                ([SS Fig. 2] defines coverage as the attention covered by selected blocks);
                all n if the sum never reaches tau.
    ``keep_first``: key block 0 is ranked ahead of every other candidate (so it is always
    kept and its mass counts first), the rest keep their order.  The pages name a
    ``first_token_mask`` in the authors' code ([CP] record) without defining it; this is the
    plainest reading: the block holding the first tokens (the attention sink) is always
    computed."""
    B, Hq, nb, _ = P.shape
    bps = segment // block
    nseg = nb // bps
    width = max((nseg - 1) * bps, 1)
    counts = np.zeros((B, Hq, nb), dtype=np.int32)
    idx = np.full((B, Hq, nb, width), -1, dtype=np.int32)
    tau = float(param)
    for sigma in range(1, nseg):
        n = sigma * bps
        rows = slice(sigma * bps, (sigma + 1) * bps)
        cand = P[:, :, rows, :n]                              # [B, Hq, bps, n]
        order = descending_order(cand)
        if keep_first:
            rest = order[order != 0].reshape(order.shape[:-1] + (n - 1,))
            order = np.concatenate([np.zeros(order.shape[:-1] + (1,), order.dtype), rest], axis=-1)
        if mode == KEEP:
            kk = np.full(cand.shape[:-1], keep_count(n, param), dtype=np.int64)
        elif mode == COVERAGE:
            ranked = np.take_along_axis(cand, order, axis=-1).astype(np.float32)
            csum = np.add.accumulate(ranked, axis=-1, dtype=np.float32)   # sequential
            reached = csum.astype(np.float64) >= tau          # compared in double
            kk = np.where(reached.any(axis=-1), reached.argmax(axis=-1) + 1, n)
        else:
            raise ValueError(mode)
        for b in range(B):
            for g in range(Hq):
                for r in range(bps):
                    c = int(kk[b, g, r])
                    counts[b, g, sigma * bps + r] = c
                    idx[b, g, sigma * bps + r, :c] = np.sort(order[b, g, r, :c])
    return counts, idx


# --------------------------------------------------------------------------- O5/O6 attention

def _head_kv(cache: dict, k, v, b: int, h: int):
    """float64 K and V of KV head (b, h), converted once per head (one head cached)."""
    if (b, h) not in cache:
        cache.clear()
        cache[(b, h)] = (bf16_to_f64(k[b, h]), bf16_to_f64(v[b, h]))
    return cache[(b, h)]


def _attend_rows(Qb, Kf, Vf, keys, t, scale: float):
    """Rows of queries ``Qb`` (original positions ``t``) over the candidate original keys
    ``keys``: row r sees the keys with position <= t[r].  Returns the softmax-weighted values
    and the natural-log normaliser of each row (float64, two passes: max, then sums)."""
    Z = scale * (Qb @ Kf[keys].T)                               # [rows, |keys|]
    Z = np.where(keys[None, :] <= t[:, None], Z, -np.inf)
    m = Z.max(axis=1, keepdims=True)
    E = np.exp(Z - m)
    l = E.sum(axis=1, keepdims=True)
    ob = (E @ Vf[keys]) / l
    lb = (m + np.log(l))[:, 0]
    return ob, lb


def visible_keys(t: int, *, block: int, segment: int, perm_row: Optional[np.ndarray],
                 sel_blocks: Optional[Sequence[int]], dense: bool) -> np.ndarray:
    """Original positions query t attends to (the set A(t)).

    dense causal: {j <= t}.
    PBS: {j in t's own segment, j <= t}  union  {perm[p] : p in a selected key block}.
    ([SS Fig. 1]: own-segment blocks under the causal mask; selected earlier-segment
    blocks in full.  [SS Lemma 3.1]: a permuted slot p stands for original key perm[p].)
    ``perm_row=None`` means the identity order (plain block-sparse attention)."""
    if dense:
        return np.arange(t + 1)
    s0 = (t // segment) * segment
    own = np.arange(s0, t + 1)
    picked = []
    for j in (sel_blocks if sel_blocks is not None else ()):
        slots = np.arange(j * block, (j + 1) * block)
        picked.append(slots if perm_row is None else perm_row[slots].astype(np.int64))
    if picked:
        return np.concatenate([np.concatenate(picked), own])
    return own


def attention(q, k, v, *, block: int, segment: int, scale: float,
              perm: Optional[np.ndarray] = None, counts: Optional[np.ndarray] = None,
              idx: Optional[np.ndarray] = None, dense: bool = False,
              qblocks: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Attention output in ORIGINAL token order, float64, and its natural-log normaliser.

    o_t = sum_{j in A(t)} softmax_j(scale * <q_t, k_j>) v_j  with A(t) from ``visible_keys``.

    ``k``/``v`` are the original (unpermuted) tensors: the permutation only names which
    original keys a selected block holds, so the result does not depend on any permuted
    copy or tiling.  Queries are never permuted ([GS Methodik 3, Handling von Queries]),
    so the output needs no inverse permutation.

    The rows of one query block share the selected blocks and the segment, so they are
    evaluated together: with t_last the block's last row, A(t) = A(t_last) & {j <= t} for
    every row t of the block (selected keys lie in earlier segments, below every t).

    ``qblocks``: optional (b, g, i) query blocks to evaluate; then ``o`` is
    ``[len, Bs, d]`` and ``lse`` ``[len, Bs]`` in that order, else ``[B, Hq, N, d]`` and
    ``[B, Hq, N]``."""
    B, Hq, Hkv, N, d, G = _check_shape(q.shape, k.shape, block, segment)
    nb = N // block
    sampled = qblocks is not None
    todo = list(qblocks) if sampled else [(b, g, i) for b in range(B) for g in range(Hq) for i in range(nb)]
    if sampled:
        o = np.zeros((len(todo), block, d))
        lse = np.zeros((len(todo), block))
    else:
        o = np.zeros((B, Hq, N, d))
        lse = np.zeros((B, Hq, N))
    cache = {}
    for n_out, (b, g, i) in enumerate(todo):
        h = g // G
        Kf, Vf = _head_kv(cache, k, v, b, h)
        sel = None
        if not dense and counts is not None:
            sel = [int(j) for j in idx[b, g, i, :counts[b, g, i]]]
        prow = None if perm is None else perm[b, h]
        t = np.arange(i * block, (i + 1) * block)
        keys = visible_keys(int(t[-1]), block=block, segment=segment, perm_row=prow,
                            sel_blocks=sel, dense=dense)
        if len(np.unique(keys)) != len(keys):
            raise AssertionError("a key would be counted twice")
        Qb = bf16_to_f64(q[b, g, i * block:(i + 1) * block])
        ob, lb = _attend_rows(Qb, Kf, Vf, keys, t, scale)
        if sampled:
            o[n_out], lse[n_out] = ob, lb
        else:
            o[b, g, t], lse[b, g, t] = ob, lb
    return o, lse


def permute_queries(q, perm: np.ndarray) -> np.ndarray:
    """Queries moved with their tokens: ``q_perm[b, g, p] = q[b, g, perm[b, g // G, p]]``, every
    query head in its KV head's segment permutation.

    [GS Methodik 1] (Permutationsäquivarianz der Query) and [SS Lemma 3.2]: permuting the
    queries permutes the output rows the same way.  The default path keeps queries in natural
    order ([GS Methodik 3, Handling von Queries]); this is the variant that moves them too."""
    B, Hq = q.shape[:2]
    Hkv = perm.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    return apply_permutation(q, np.repeat(perm, Hq // Hkv, axis=1))


def attention_permuted_queries(q_perm, k, v, *, block: int, segment: int, scale: float,
                               perm: np.ndarray, counts: np.ndarray, idx: np.ndarray,
                               qblocks: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Attention with queries and keys both in the segment permutation, output returned in
    ORIGINAL token order, float64, with its natural-log normaliser.

    Query slot p of head g holds the token at original position t = perm[b, g // G, p]; it
    belongs to the permuted query block i = p // Bs, whose selected blocks are
    ``idx[b, g, i, :counts]`` (a selection made on the permuted queries).  It sees
      A(t) = {j in t's segment, j <= t}  union  {perm[s] : s in a selected key block},
    the causal test going through the original positions ([SS Fig. 1]; [SS Lemma 3.1] for the
    keys).  [SS Lemma 3.2]: the rows come out in the permuted order; [SS Theorem 3.3]: putting
    each row back at its original position t (the inverse permutation) restores the
    unpermuted result, which is what this returns.

    ``qblocks``: optional (b, g, i) PERMUTED query blocks; then ``o`` is ``[len, Bs, d]`` and
    ``lse`` ``[len, Bs]`` in slot order (row r of entry n is original position
    perm[b, g // G, i*Bs + r]), else ``[B, Hq, N, d]`` / ``[B, Hq, N]`` in original order."""
    B, Hq, Hkv, N, d, G = _check_shape(q_perm.shape, k.shape, block, segment)
    nb = N // block
    sampled = qblocks is not None
    todo = list(qblocks) if sampled else [(b, g, i) for b in range(B) for g in range(Hq) for i in range(nb)]
    if sampled:
        o = np.zeros((len(todo), block, d))
        lse = np.zeros((len(todo), block))
    else:
        o = np.zeros((B, Hq, N, d))
        lse = np.zeros((B, Hq, N))
    cache = {}
    for n_out, (b, g, i) in enumerate(todo):
        h = g // G
        Kf, Vf = _head_kv(cache, k, v, b, h)
        slots = np.arange(i * block, (i + 1) * block)
        t = perm[b, h, slots].astype(np.int64)                      # original positions
        s0 = (i * block // segment) * segment
        sel = [int(j) for j in idx[b, g, i, :counts[b, g, i]]]
        picked = [perm[b, h, j * block:(j + 1) * block].astype(np.int64) for j in sel]
        own = np.arange(s0, int(t.max()) + 1)
        keys = np.concatenate(picked + [own]) if picked else own
        if len(np.unique(keys)) != len(keys):
            raise AssertionError("a key would be counted twice")
        Qb = bf16_to_f64(q_perm[b, g, slots])
        ob, lb = _attend_rows(Qb, Kf, Vf, keys, t, scale)     # causal test on original positions
        if sampled:
            o[n_out], lse[n_out] = ob, lb
        else:
            o[b, g, t], lse[b, g, t] = ob, lb                 # the inverse permutation of the rows
    return o, lse


def dense_causal(q, k, v, *, block: int, scale: float, qblocks=None):
    """Plain causal softmax attention ([GS Problemstellung]; the FlashAttention baseline
    of [SS Fig. 3] computes exactly this)."""
    N = q.shape[2]
    return attention(q, k, v, block=block, segment=N, scale=scale, dense=True, qblocks=qblocks)


# --------------------------------------------------------------------------- density, coverage

def attention_coverage(q, k, *, block: int, segment: int, scale: float,
                       perm: Optional[np.ndarray] = None, counts: Optional[np.ndarray] = None,
                       idx: Optional[np.ndarray] = None,
                       qblocks: Optional[Iterable[Tuple[int, int, int]]] = None) -> np.ndarray:
    """Attention coverage of each query row: the part of its dense causal attention that the
    computed key set A(t) holds, sum over j in A(t) of softmax_{j' <= t}(scale <q_t, k_j'>)_j.

    [SS Fig. 2]: coverage is the total attention of the selected blocks; [SS Fig. 4] and [GS
    Ergebnisse] compare how many blocks the permuted and the natural order need for a given
    coverage.  ``perm=None`` is the natural (unpermuted) order.  ``qblocks`` as in
    ``attention``; returns ``[len, Bs]`` or ``[B, Hq, N]`` (float64)."""
    B, Hq, Hkv, N, d, G = _check_shape(q.shape, k.shape, block, segment)
    nb = N // block
    sampled = qblocks is not None
    todo = list(qblocks) if sampled else [(b, g, i) for b in range(B) for g in range(Hq) for i in range(nb)]
    out = np.zeros((len(todo), block)) if sampled else np.zeros((B, Hq, N))
    cache = {}
    for n_out, (b, g, i) in enumerate(todo):
        h = g // G
        if (b, h) not in cache:
            cache.clear()
            cache[(b, h)] = bf16_to_f64(k[b, h])
        Kf = cache[(b, h)]
        t = np.arange(i * block, (i + 1) * block)
        Qb = bf16_to_f64(q[b, g, i * block:(i + 1) * block])
        Z = scale * (Qb @ Kf[:t[-1] + 1].T)                         # every key up to the block
        Z = np.where(np.arange(t[-1] + 1)[None, :] <= t[:, None], Z, -np.inf)
        E = np.exp(Z - Z.max(axis=1, keepdims=True))
        Pd = E / E.sum(axis=1, keepdims=True)                       # dense causal softmax
        sel = [int(j) for j in idx[b, g, i, :counts[b, g, i]]] if counts is not None else []
        keys = visible_keys(int(t[-1]), block=block, segment=segment,
                            perm_row=None if perm is None else perm[b, h], sel_blocks=sel, dense=False)
        cov = Pd[:, keys].sum(axis=1)                               # keys > t carry no mass
        if sampled:
            out[n_out] = cov
        else:
            out[b, g, t] = cov
    return out


def block_density(counts: np.ndarray, *, block: int, segment: int, N: int,
                  perm: Optional[np.ndarray] = None) -> dict:
    """Block counts of one selection ([SS Fig. 4]: block-level density).

    ``selected`` = kept earlier-segment blocks, ``candidates`` = earlier-segment blocks
    offered; ``computed`` adds the own-segment blocks the attention visits (natural order:
    the blocks up to the diagonal; permuted order: every block of the segment holding a key
    at or before the query block's last row), ``dense`` counts the blocks of dense causal
    attention.  ``counts`` is ``[B, Hq, nb]``; ``perm`` ``[B, Hkv, N]`` or None."""
    B, Hq, nb = counts.shape
    bps = segment // block
    selected = int(counts.sum())
    candidates = B * Hq * sum((i // bps) * bps for i in range(nb))
    own = 0
    for b in range(B):
        for g in range(Hq):
            for i in range(nb):
                s0 = (i // bps) * bps
                if perm is None:
                    own += i - s0 + 1
                else:
                    Hkv = perm.shape[1]
                    h = g // (Hq // Hkv)
                    last = (i + 1) * block - 1
                    for j in range(s0, s0 + bps):
                        if perm[b, h, j * block:(j + 1) * block].min() <= last:
                            own += 1
    dense = B * Hq * nb * (nb + 1) // 2
    return dict(selected=selected, candidates=candidates, computed=selected + own, dense=dense)


# --------------------------------------------------------------------------- whole pipeline

def prefill(q, k, v, *, block: int, segment: int, scale: float, mode: str, param: float):
    """All stages in order: scores -> permutation (+ permuted K/V) -> block probabilities
    -> selection -> attention.  Returns a dict of every intermediate."""
    sc = key_scores(q, k, block=block, segment=segment, scale=scale)
    perm = segment_permutation(sc, segment=segment)
    k_perm = apply_permutation(k, perm)
    v_perm = apply_permutation(v, perm)
    P = block_probabilities(q, k_perm, block=block, segment=segment, scale=scale)
    counts, idx = select_blocks(P, block=block, segment=segment, mode=mode, param=param)
    o, lse = attention(q, k, v, block=block, segment=segment, scale=scale, perm=perm,
                       counts=counts, idx=idx)
    return dict(scores=sc, perm=perm, k_perm=k_perm, v_perm=v_perm, P=P, counts=counts,
                idx=idx, o=o, lse=lse)


def prefill_varlen(q, k, v, cu_seqlens, *, block: int, segment: int, scale: float, mode: str,
                   param: float):
    """Several sequences packed along N (``q [1, Hq, T, d]``, ``k, v [1, Hkv, T, d]``, sequence
    s holding tokens ``cu_seqlens[s] .. cu_seqlens[s+1]-1``, every length a multiple of
    ``segment``): the method applied to each sequence on its own, the results placed back at
    the sequences' positions.  Positions (``perm``) and block indices (``idx``) are absolute in
    the packed sequence; ``P`` is block-diagonal (no block is a candidate of another
    sequence's query).  The pages treat one sequence at a time; a packed batch is read as that,
    sequence by sequence."""
    cu = [int(x) for x in cu_seqlens]
    T = q.shape[2]
    if q.shape[0] != 1 or cu[0] != 0 or cu[-1] != T or any(b <= a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must run 0 < ... < T over one packed batch row")
    if any((b - a) % segment for a, b in zip(cu, cu[1:])):
        raise ValueError("every sequence length must be a multiple of the segment size")
    Hq, Hkv = q.shape[1], k.shape[1]
    nbT = T // block
    width = max((T // segment - 1) * (segment // block), 1)
    out = dict(scores=np.zeros((1, Hkv, T), np.float32), perm=np.zeros((1, Hkv, T), np.int32),
               k_perm=np.zeros_like(k), v_perm=np.zeros_like(v),
               P=np.zeros((1, Hq, nbT, nbT), np.float32), counts=np.zeros((1, Hq, nbT), np.int32),
               idx=np.full((1, Hq, nbT, width), -1, np.int32),
               o=np.zeros(q.shape, np.float64), lse=np.zeros((1, Hq, T), np.float64))
    for a, b in zip(cu, cu[1:]):
        r = prefill(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], block=block, segment=segment,
                    scale=scale, mode=mode, param=param)
        i0, i1 = a // block, b // block
        out["scores"][:, :, a:b] = r["scores"]
        out["perm"][:, :, a:b] = r["perm"] + a
        out["k_perm"][:, :, a:b] = r["k_perm"]
        out["v_perm"][:, :, a:b] = r["v_perm"]
        out["P"][:, :, i0:i1, i0:i1] = r["P"]
        out["counts"][:, :, i0:i1] = r["counts"]
        w = r["idx"].shape[-1]
        out["idx"][:, :, i0:i1, :w] = np.where(r["idx"] >= 0, r["idx"] + i0, -1)
        out["o"][:, :, a:b] = r["o"]
        out["lse"][:, :, a:b] = r["lse"]
    return out


def default_scale(head_dim: int) -> float:
    """float32(1/sqrt(d)) widened: the conventional softmax temperature (the pages print
    none)."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))
