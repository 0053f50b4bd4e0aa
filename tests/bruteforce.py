"""Brute-force reference for tiny inputs, written from the definitions and independent of
``oracle/``: explicit Python loops over every (query, key) pair, float64 via ``math``,
bfloat16 decoded with ``struct``.  Used only to pin the oracle on inputs of a few dozen
tokens.

Pages (arXiv 2510.21270, "Sparser Block-Sparse Attention via Token Permutation"):
sciencestack.ai page, Fig. 1 caption (segments of size S, blocks of size B; blocks of the
query's own segment are computed, earlier-segment blocks may be skipped) and Lemma 3.1
(keys and values permuted together leave attention unchanged); gist.science summary,
Methodik 2 (no query sees a later segment) and 3 (last-block proxy scores, mean pooled).
"""
import math
import struct


def bf16(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def mat(x2d):
    """bf16-bit 2-D array -> list of lists of Python floats."""
    return [[bf16(x) for x in row] for row in x2d]


def dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def softmax_over(values):
    """softmax of a dict key -> logit."""
    m = max(values.values())
    ex = {j: math.exp(z - m) for j, z in values.items()}
    tot = math.fsum(ex.values())
    return {j: e / tot for j, e in ex.items()}


def visibility(N, block, segment, perm=None, sel=None, dense=False):
    """N x N 0/1 matrix vis[t][j] over ORIGINAL key positions j.

    dense: j <= t.  Otherwise j in t's segment with j <= t, plus every key held by a
    selected block: ``sel[i]`` lists selected (permuted) block indices for query block i,
    and slot p of the permuted order holds original key ``perm[p]`` (identity if None)."""
    vis = [[0] * N for _ in range(N)]
    for t in range(N):
        for j in range(N):
            if dense:
                vis[t][j] = int(j <= t)
            else:
                vis[t][j] = int(j // segment == t // segment and j <= t)
        if not dense and sel is not None:
            for jb in sel[t // block]:
                for p in range(jb * block, (jb + 1) * block):
                    orig = p if perm is None else int(perm[p])
                    vis[t][orig] = 1
    return vis


def attention(Q, K, V, vis, scale):
    """o[t] = sum_j softmax over visible j of scale*<q_t,k_j> times v_j (lists of floats)."""
    N = len(Q)
    out = []
    for t in range(N):
        logits = {j: scale * dot(Q[t], K[j]) for j in range(len(K)) if vis[t][j]}
        p = softmax_over(logits)
        d = len(V[0])
        out.append([math.fsum(p[j] * V[j][c] for j in p) for c in range(d)])
    return out


def key_scores(Qheads, K, block, segment, scale):
    """Scores for one KV head: Qheads is a list of the G query heads (each N x d floats).
    For each row of the last block of every head, a softmax over each segment's keys that
    the row may see (j <= t); the probabilities are summed per key and divided by the
    number of rows."""
    N = len(K)
    acc = [0.0] * N
    rows = 0
    for Q in Qheads:
        for t in range(N - block, N):
            rows += 1
            for s0 in range(0, N, segment):
                logits = {j: scale * dot(Q[t], K[j]) for j in range(s0, s0 + segment) if j <= t}
                for j, pj in softmax_over(logits).items():
                    acc[j] += pj
    return [a / rows for a in acc]


def block_probs(Qg, Kp, block, segment, scale):
    """Pooled block probabilities for one query head against one permuted key tensor:
    dict (i, j) -> P over the candidates j of each query block i (earlier segments)."""
    N, d = len(Qg), len(Qg[0])
    nb, bps = N // block, segment // block

    def mean_rows(X, b):
        return [math.fsum(X[r][c] for r in range(b * block, (b + 1) * block)) / block for c in range(d)]

    out = {}
    for i in range(nb):
        n = (i // bps) * bps
        if n == 0:
            continue
        qb = mean_rows(Qg, i)
        logits = {j: scale * dot(qb, mean_rows(Kp, j)) for j in range(n)}
        for j, pj in softmax_over(logits).items():
            out[(i, j)] = pj
    return out
