"""Pins of the CPU oracle: checks against what the pages and the mathematics fix, each
written as a function of the oracle module so that ``test_oracle_pins`` runs them on the
oracle and ``test_oracle_mutants`` runs them on copies of the oracle with a planted mistake
(every planted mistake must fail at least one pin).

Pages (arXiv 2510.21270, "Sparser Block-Sparse Attention via Token Permutation"):
  [SS] sciencestack.ai page: Fig. 1 caption (B=1, S=4 segmented permutation; own-segment
       blocks computed, inter-segment blocks skippable), Fig. 2 caption (coverage), Lemma 3.1
       (joint key/value permutation invariance), Lemma 3.2 (query permutation equivariance),
       Theorem 3.3 (invariance under the inverse transformation).
  [GS] gist.science summary, Methodik 1-4.
  [SK] skillmd.com "Sparser Block Attention", Implementation Steps (active-block count rule,
       inverse permutation).
"""
import math
import os

import numpy as np

import bruteforce as bf
from pbs_synth import f32_to_bf16_bits, random_bf16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _tiny(seed, B=1, Hq=4, Hkv=2, N=32, d=8, scale_k=1.0):
    q = random_bf16((B, Hq, N, d), seed)
    k = random_bf16((B, Hkv, N, d), seed + 1, scale_k)
    v = random_bf16((B, Hkv, N, d), seed + 2)
    return q, k, v


def _vis_matrix(N, block, segment, perm_row, counts_row, idx_row, dense=False):
    sel = None
    if counts_row is not None:
        sel = [list(idx_row[i, :counts_row[i]]) for i in range(N // block)]
    return bf.visibility(N, block, segment, perm=perm_row, sel=sel, dense=dense)


# ----------------------------------------------------------------------------- scores

def pin_scores_sum_to_one(O):
    """Each row's softmax over a segment sums to 1, so each segment's mean-pooled scores
    sum to 1 ([GS Methodik 3, Proxy-Bewertung]; [SK] normalises importance to sum 1)."""
    q, k, _ = _tiny(11, N=64, d=16)
    sc = O.key_scores(q, k, block=8, segment=16, scale=0.25)
    assert sc.dtype == np.float32 and sc.shape == (1, 2, 64)
    sums = sc.astype(np.float64).reshape(1, 2, 4, 16).sum(-1)
    assert np.allclose(sums, 1.0, atol=2e-6), sums
    assert (sc > 0).all()


def pin_scores_identical_keys(O):
    """Closed form: if every key of a segment is the same vector, each visible key of the
    segment gets the same probability.  Segments wholly before the last query block give
    1/S per key; in the last segment row t sees t-s0+1 keys, so
    score_j = (1/(G*Bs)) * sum over rows (g,t) with t >= j of 1/(t-s0+1)."""
    B, Hq, Hkv, N, d, Bs, S = 1, 4, 2, 48, 8, 4, 16
    G = Hq // Hkv
    q = random_bf16((B, Hq, N, d), 21)
    base = random_bf16((B, Hkv, N // S, 1, d), 22)
    k = np.ascontiguousarray(np.broadcast_to(base, (B, Hkv, N // S, S, d)).reshape(B, Hkv, N, d))
    sc = O.key_scores(q, k, block=Bs, segment=S, scale=0.3535533845424652)
    s0 = N - S
    for h in range(Hkv):
        assert np.allclose(sc[0, h, :s0], 1.0 / S, rtol=1e-6)
        for j in range(s0, N):
            exp = sum(1.0 / (t - s0 + 1) for t in range(N - Bs, N) if t >= j) * G / (G * Bs)
            assert math.isclose(float(sc[0, h, j]), exp, rel_tol=1e-6), (j, sc[0, h, j], exp)


def pin_scores_salient_closed_form(O):
    """Closed form with one salient key: all last-block queries are a*e1, all keys are 0
    except key j* = b*e1.  Then z(j*) = scale*a*b and z = 0 elsewhere, so in j*'s segment
    p(j*) = e^z / (e^z + S - 1) for every row; the other segments are uniform."""
    B, Hq, Hkv, N, d, Bs, S = 1, 2, 1, 32, 16, 4, 8
    a, b, scale, jstar = 2.0, 3.0, 0.25, 10
    qf = np.zeros((B, Hq, N, d), np.float32)
    qf[..., 0] = a
    kf = np.zeros((B, Hkv, N, d), np.float32)
    kf[0, 0, jstar, 0] = b
    sc = O.key_scores(f32_to_bf16_bits(qf), f32_to_bf16_bits(kf), block=Bs, segment=S, scale=scale)
    ez = math.exp(scale * a * b)
    assert math.isclose(float(sc[0, 0, jstar]), ez / (ez + S - 1), rel_tol=1e-6)
    assert math.isclose(float(sc[0, 0, 8]), 1.0 / (ez + S - 1), rel_tol=1e-6)
    assert math.isclose(float(sc[0, 0, 0]), 1.0 / S, rel_tol=1e-6)


def pin_scores_bruteforce(O):
    """Brute force over every (row, key) pair on a tiny GQA input."""
    B, Hq, Hkv, N, d, Bs, S = 1, 4, 2, 24, 8, 4, 8
    q, k, _ = _tiny(31, Hq=Hq, Hkv=Hkv, N=N, d=d, scale_k=1.5)
    scale = 0.35
    sc = O.key_scores(q, k, block=Bs, segment=S, scale=scale)
    G = Hq // Hkv
    for h in range(Hkv):
        ref = bf.key_scores([bf.mat(q[0, g]) for g in range(h * G, (h + 1) * G)], bf.mat(k[0, h]),
                            Bs, S, scale)
        assert np.allclose(sc[0, h], ref, rtol=2e-6, atol=1e-9), (h, sc[0, h], ref)


# ----------------------------------------------------------------------------- permutation

def pin_order_rules(O):
    """Descending, ties to the lower index, -0 == +0, NaN last (hand-derived)."""
    v = np.array([0.5, -0.0, 0.0, np.nan, 0.5, 1.0, -1.0], dtype=np.float32)
    assert list(O.descending_order(v)) == [5, 0, 4, 1, 2, 6, 3]


def pin_permutation_fig1(O):
    """Fig. 1 geometry (B=1, S=4, N=8): keys move only inside their segment, in descending
    score order ([SS Fig. 1]; [GS Methodik 2, 3 Sortierung]).  Hand-derived."""
    sc = np.array([[[0.1, 0.4, 0.2, 0.3, 0.05, 0.05, 0.6, 0.3]]], dtype=np.float32)
    perm = O.segment_permutation(sc, segment=4)
    assert perm.dtype == np.int32
    assert perm[0, 0].tolist() == [1, 3, 2, 0, 6, 7, 4, 5]


def pin_permutation_properties(O):
    """Bijection on every segment, non-increasing scores along the permuted order, equal
    scores in increasing position; the permuted copy is a row gather and the inverse
    restores the original ([SK Implementation Steps])."""
    rng = np.random.default_rng(5)
    B, H, N, S, d = 2, 3, 64, 16, 8
    sc = rng.choice(np.array([0.0, -0.0, 0.25, 0.5, 1e-8, 3.0], np.float32), size=(B, H, N))
    perm = O.segment_permutation(sc, segment=S)
    k = random_bf16((B, H, N, d), 7)
    kp = O.apply_permutation(k, perm)
    inv = O.inverse_permutation(perm)
    for b in range(B):
        for h in range(H):
            for s0 in range(0, N, S):
                seg = perm[b, h, s0:s0 + S]
                assert sorted(seg.tolist()) == list(range(s0, s0 + S))
                vals = sc[b, h, seg]
                for p in range(S - 1):
                    assert vals[p] >= vals[p + 1]
                    if vals[p] == vals[p + 1]:
                        assert seg[p] < seg[p + 1]
            for p in range(N):
                assert (kp[b, h, p] == k[b, h, perm[b, h, p]]).all()
                assert inv[b, h, perm[b, h, p]] == p
    assert (O.apply_permutation(kp, inv) == k).all()


# ----------------------------------------------------------------------------- block scores

def pin_block_probs_closed_form(O):
    """Closed form: every row of query block i equals c_i*e1 and every row of permuted key
    block j equals w_j*e1, so the pooled means are c_i*e1 and w_j*e1 and the logit is
    scale*c_i*w_j.  P is a softmax over the earlier-segment blocks only."""
    B, Hq, Hkv, N, d, Bs, S = 1, 1, 1, 24, 4, 2, 6
    nb, bps = N // Bs, S // Bs
    c = np.linspace(-1.0, 1.0, nb).astype(np.float32)
    w = np.linspace(2.0, -1.5, nb).astype(np.float32)
    qf = np.zeros((B, Hq, N, d), np.float32)
    kf = np.zeros((B, Hkv, N, d), np.float32)
    for i in range(nb):
        qf[0, 0, i * Bs:(i + 1) * Bs, 0] = c[i]
        kf[0, 0, i * Bs:(i + 1) * Bs, 0] = w[i]
    qb, kb = f32_to_bf16_bits(qf), f32_to_bf16_bits(kf)
    cq = O.bf16_to_f64(qb[0, 0, ::Bs, 0])
    wk = O.bf16_to_f64(kb[0, 0, ::Bs, 0])
    scale = 0.5
    P = O.block_probabilities(qb, kb, block=Bs, segment=S, scale=scale)
    for i in range(nb):
        n = (i // bps) * bps
        if n == 0:
            assert (P[0, 0, i] == 0).all()
            continue
        e = np.array([math.exp(scale * cq[i] * wk[j]) for j in range(n)])
        assert np.allclose(P[0, 0, i, :n], e / e.sum(), rtol=1e-6), i
        assert (P[0, 0, i, n:] == 0).all()


def pin_block_probs_bruteforce(O):
    """Brute force (explicit means and softmax) on a tiny GQA input."""
    B, Hq, Hkv, N, d, Bs, S = 1, 4, 2, 32, 8, 4, 8
    q, k, _ = _tiny(41, Hq=Hq, Hkv=Hkv, N=N, d=d)
    P = O.block_probabilities(q, k, block=Bs, segment=S, scale=0.4)
    G = Hq // Hkv
    for g in range(Hq):
        ref = bf.block_probs(bf.mat(q[0, g]), bf.mat(k[0, g // G]), Bs, S, 0.4)
        for (i, j), pij in ref.items():
            assert math.isclose(float(P[0, g, i, j]), pij, rel_tol=2e-6), (g, i, j)
        assert np.count_nonzero(P[0, g]) == len(ref)


# ----------------------------------------------------------------------------- selection

def pin_keep_count_golden(O):
    """The printed active-block count rule ([SK Implementation Steps]); golden table."""
    with open(os.path.join(GOLDEN, "keep_count.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for n, r, want in rows:
        assert O.keep_count(int(n), float(r)) == int(want), (n, r, want)


def _select_case(O, rows, mode, param, keep_first=False):
    """rows: list of 5-value P rows for query blocks 5..9 of a block=1, segment=5, N=10
    layout (5 candidates each)."""
    P = np.zeros((1, 1, 10, 10), np.float32)
    for r, vals in enumerate(rows):
        P[0, 0, 5 + r, :5] = np.array(vals, np.float32)
    counts, idx = O.select_blocks(P, block=1, segment=5, mode=mode, param=param,
                                  keep_first=keep_first)
    assert counts.dtype == np.int32 and idx.dtype == np.int32 and idx.shape == (1, 1, 10, 5)
    assert (counts[0, 0, :5] == 0).all()
    return [idx[0, 0, 5 + r, :counts[0, 0, 5 + r]].tolist() for r in range(len(rows))]


def pin_select_handworked(O):
    """Hand-worked selections (values exact in binary): ranking by P descending with ties
    to the lower block, output in ascending block order; coverage stops at the first
    prefix whose float32 sum reaches tau (>=), and keeps every block if it never does."""
    rows = [[0.125, 0.25, 0.25, 0.0625, 0.125],
            [0.2, 0.2, 0.2, 0.2, 0.2],
            [0.0, 0.0, 0.0, 0.0, 1.0],
            [-0.0, 0.0, 0.5, 0.25, 0.25],
            [0.25, 0.5, 0.125, 0.125, 0.0]]
    assert _select_case(O, rows, O.KEEP, 0.5) == [[1, 2], [0, 1], [0, 4], [2, 3], [0, 1]]
    assert _select_case(O, rows, O.KEEP, 0.1) == [[1], [0], [4], [2], [1]]
    assert _select_case(O, rows, O.COVERAGE, 0.75) == [[0, 1, 2, 4], [0, 1, 2, 3], [4], [2, 3], [0, 1]]
    assert _select_case(O, rows, O.COVERAGE, 1.0)[4] == [0, 1, 2, 3]
    assert _select_case(O, [[0.125] * 5], O.COVERAGE, 0.9) == [[0, 1, 2, 3, 4]]


def pin_select_keep_first_handworked(O):
    """Block 0 forced to the front of the ranking (the first-token block): it is always kept,
    the rest follow by P descending (ties to the lower block), and for coverage block 0's mass
    is counted first.  Worked by hand on the rows above:
      row [0.125, 0.25, 0.25, 0.0625, 0.125], keep 0.5 (2 blocks): 0, then 1 (tie 1/2 to the
        lower block)                                      -> [0, 1]
      row [0.0, 0.0, 0.0, 0.0, 1.0], keep 0.5: 0, then 4  -> [0, 4] (the same as without)
      row [0.25, 0.5, 0.125, 0.125, 0.0], coverage 0.75: 0.25 (block 0) + 0.5 (block 1)
        = 0.75 reaches tau                                -> [0, 1]
      row [0.0, 0.0, 0.5, 0.25, 0.25], coverage 0.75: 0 + 0.5 (block 2) + 0.25 (block 3)
        = 0.75                                            -> [0, 2, 3] (without: [2, 3])
      row [0.0, 0.0, 0.0, 0.0, 1.0], keep 0.1 (1 block)   -> [0] (without: [4])"""
    rows = [[0.125, 0.25, 0.25, 0.0625, 0.125],
            [0.0, 0.0, 0.0, 0.0, 1.0],
            [0.25, 0.5, 0.125, 0.125, 0.0],
            [0.0, 0.0, 0.5, 0.25, 0.25]]
    assert _select_case(O, rows[:2], O.KEEP, 0.5, keep_first=True) == [[0, 1], [0, 4]]
    assert _select_case(O, rows[2:], O.COVERAGE, 0.75, keep_first=True) == [[0, 1], [0, 2, 3]]
    assert _select_case(O, rows[3:], O.COVERAGE, 0.75) == [[2, 3]]
    assert _select_case(O, rows[1:2], O.KEEP, 0.1, keep_first=True) == [[0]]
    assert _select_case(O, rows[1:2], O.KEEP, 0.1) == [[4]]


def pin_select_keep_first_laws(O):
    """With block 0 forced first, on random rows: block 0 is always kept, the keep count law
    is unchanged, every other kept block outranks every other dropped one, and the coverage
    prefix (block 0, then by rank) is minimal."""
    rng = np.random.default_rng(19)
    nb, bps = 24, 4
    P = np.zeros((1, 2, nb, nb), np.float32)
    for g in range(2):
        for i in range(bps, nb):
            n = (i // bps) * bps
            e = np.exp(rng.normal(size=n))
            P[0, g, i, :n] = (e / e.sum()).astype(np.float32)
    for mode, param in ((O.KEEP, 0.3), (O.COVERAGE, 0.6)):
        counts, idx = O.select_blocks(P, block=1, segment=bps, mode=mode, param=param,
                                      keep_first=True)
        for g in range(2):
            for i in range(bps, nb):
                n = (i // bps) * bps
                kk = int(counts[0, g, i])
                sel = idx[0, g, i, :kk].tolist()
                assert sel[0] == 0 and sel == sorted(set(sel))
                if mode == O.KEEP:
                    assert kk == max(1, int(param * n))
                row = P[0, g, i, :n]
                others = [j for j in sel if j != 0]
                rest = [j for j in range(1, n) if j not in sel]
                for a in others:
                    for b in rest:
                        assert row[a] > row[b] or (row[a] == row[b] and a < b)
                if mode == O.COVERAGE:
                    ranked = [0] + sorted(others, key=lambda j: (-row[j], j))
                    c = np.float32(0)
                    partial = []
                    for j in ranked:
                        c = np.float32(c + row[j])
                        partial.append(float(c))
                    if kk < n:
                        assert partial[-1] >= param
                    if kk > 1:
                        assert partial[-2] < param


def pin_select_sequential_fp32(O):
    """Coverage sums in sequential float32: 0.75 + 2^-25 rounds back to 0.75 (tie to even),
    so with tau = 0.75 + 2^-24 the float32 running sum never reaches tau and every block is
    kept, while an exact or pairwise sum would stop after three blocks."""
    tiny = 2.0 ** -25
    tau = 0.75 + 2.0 ** -24
    got = _select_case(O, [[0.75, tiny, tiny, tiny, 0.0]], O.COVERAGE, tau)
    assert got == [[0, 1, 2, 3, 4]]


def pin_select_laws(O):
    """Laws on random rows: the count law (keep), dominance (every kept block outranks
    every dropped one), and coverage minimality (kept mass reaches tau; without the last
    kept block it does not)."""
    rng = np.random.default_rng(9)
    nb, bps = 24, 4
    P = np.zeros((1, 2, nb, nb), np.float32)
    for g in range(2):
        for i in range(bps, nb):
            n = (i // bps) * bps
            x = rng.normal(size=n) * 0.5
            x[rng.integers(0, n)] = x.max()            # a planted tie
            e = np.exp(x - x.max())
            P[0, g, i, :n] = (e / e.sum()).astype(np.float32)
    for mode, param in ((O.KEEP, 0.3), (O.KEEP, 1.0), (O.COVERAGE, 0.6), (O.COVERAGE, 0.95)):
        counts, idx = O.select_blocks(P, block=1, segment=bps, mode=mode, param=param)
        for g in range(2):
            for i in range(nb):
                n = (i // bps) * bps
                kk = int(counts[0, g, i])
                sel = idx[0, g, i, :kk].tolist()
                assert sel == sorted(set(sel)) and all(0 <= j < n for j in sel)
                if n == 0:
                    assert kk == 0
                    continue
                if mode == O.KEEP:
                    assert kk == max(1, int(param * n))
                row = P[0, g, i, :n]
                rest = [j for j in range(n) if j not in sel]
                for a in sel:
                    for b in rest:
                        assert row[a] > row[b] or (row[a] == row[b] and a < b)
                if mode == O.COVERAGE:
                    ranked = sorted(sel, key=lambda j: (-row[j], j))
                    c = np.float32(0)
                    partial = []
                    for j in ranked:
                        c = np.float32(c + row[j])
                        partial.append(float(c))
                    if kk < n:
                        assert partial[-1] >= param
                    if kk > 1:
                        assert partial[-2] < param


# ----------------------------------------------------------------------------- geometry

def pin_fig1_geometry(O):
    """Golden region map of Fig. 1 (B=1, S=4, N=8): own-segment keys visible up to t,
    earlier segments are exactly the block-selection candidates, later segments never
    appear.  Holds for the natural order and for a permuted one."""
    with open(os.path.join(GOLDEN, "fig1_b1_s4_n8.txt")) as f:
        grid = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    N, S = 8, 4
    q, k, _ = _tiny(3, Hq=1, Hkv=1, N=N, d=4)
    for perm in (None, np.array([2, 0, 3, 1, 7, 4, 6, 5], np.int32)):
        kp = k if perm is None else O.apply_permutation(k, perm[None, None])
        P = O.block_probabilities(q, kp, block=1, segment=S, scale=0.5)
        for t in range(N):
            vis = set(O.visible_keys(t, block=1, segment=S, perm_row=perm, sel_blocks=[],
                                     dense=False).tolist())
            for j in range(N):
                want = grid[t][j]
                assert (want == "D") == (j in vis), (t, j)
                # candidate slots are permuted block indices; with B=1 and a permutation
                # inside segments, slot j lies in the same segment as key j
                assert (want == "Y") == (P[0, 0, t, j] > 0), (t, j)


# ----------------------------------------------------------------------------- attention

def _tiny_pbs(O, seed, mode="keep", param=0.5, N=32, Bs=4, S=8, Hq=4, Hkv=2, d=8):
    q, k, v = _tiny(seed, Hq=Hq, Hkv=Hkv, N=N, d=d, scale_k=1.7)
    out = O.prefill(q, k, v, block=Bs, segment=S, scale=0.4, mode=mode, param=param)
    return q, k, v, out


def pin_attention_bruteforce(O):
    """PBS and dense outputs (and log-normalisers) against an explicit N x N visibility
    matrix built from the definitions ([SS Fig. 1]: own segment under the causal mask,
    selected earlier-segment blocks in full)."""
    N, Bs, S, Hq, Hkv = 32, 4, 8, 4, 2
    q, k, v, out = _tiny_pbs(O, 51, param=0.34)
    G = Hq // Hkv
    od, lsed = O.dense_causal(q, k, v, block=Bs, scale=0.4)
    for g in range(Hq):
        h = g // G
        Q, K, V = bf.mat(q[0, g]), bf.mat(k[0, h]), bf.mat(v[0, h])
        vis = _vis_matrix(N, Bs, S, out["perm"][0, h], out["counts"][0, g], out["idx"][0, g])
        ref = bf.attention(Q, K, V, vis, 0.4)
        assert np.allclose(out["o"][0, g], ref, atol=1e-12), g
        visd = bf.visibility(N, Bs, S, dense=True)
        assert np.allclose(od[0, g], bf.attention(Q, K, V, visd, 0.4), atol=1e-12)
        for t in (0, 5, N - 1):
            lse = math.log(math.fsum(math.exp(0.4 * bf.dot(Q[t], K[j])) for j in range(N) if vis[t][j]))
            assert math.isclose(out["lse"][0, g, t], lse, rel_tol=1e-12)


def pin_lemma_3_1(O):
    """[SS Lemma 3.1]: attention over the permuted copies, with the causal mask mapped
    through the stored original positions, equals the oracle's result computed from the
    original K and V (the permutation is not an involution, so its direction matters)."""
    N, Bs, S, Hq, Hkv = 32, 4, 8, 4, 2
    q, k, v, out = _tiny_pbs(O, 61, param=0.5)
    G = Hq // Hkv
    for g in range(Hq):
        h = g // G
        perm = out["perm"][0, h]
        assert any(perm[perm[p]] != p for p in range(N))
        vis = _vis_matrix(N, Bs, S, perm, out["counts"][0, g], out["idx"][0, g])
        vis_perm = [[vis[t][int(perm[p])] for p in range(N)] for t in range(N)]
        ref = bf.attention(bf.mat(q[0, g]), bf.mat(out["k_perm"][0, h]), bf.mat(out["v_perm"][0, h]),
                           vis_perm, 0.4)
        assert np.allclose(out["o"][0, g], ref, atol=1e-12), g


def _tiny_qperm(O, seed, mode, param, N=32, Bs=4, S=8, Hq=4, Hkv=2, d=8, scale=0.4):
    """The query-permutation variant end to end in the oracle: scores, permutation, queries
    moved with their tokens, selection on the permuted queries, attention."""
    q, k, v = _tiny(seed, Hq=Hq, Hkv=Hkv, N=N, d=d, scale_k=1.7)
    sc = O.key_scores(q, k, block=Bs, segment=S, scale=scale)
    perm = O.segment_permutation(sc, segment=S)
    qp = O.permute_queries(q, perm)
    kp = O.apply_permutation(k, perm)
    P = O.block_probabilities(qp, kp, block=Bs, segment=S, scale=scale)
    counts, idx = O.select_blocks(P, block=Bs, segment=S, mode=mode, param=param)
    o, lse = O.attention_permuted_queries(qp, k, v, block=Bs, segment=S, scale=scale, perm=perm,
                                          counts=counts, idx=idx)
    return q, k, v, perm, qp, counts, idx, o, lse


def pin_qperm_bruteforce(O):
    """Queries and keys both permuted, computed by brute force entirely in permuted slots:
    slot p (token perm[p]) sees key slot s when s is in p's segment and perm[s] <= perm[p],
    or s lies in a block selected for p's permuted query block; softmax over the permuted
    copies, then each row is put back at its original position ([SS Lemma 3.2, Theorem 3.3]).
    Also checks the query gather head by head from its definition (query head g moves with KV
    head g // G)."""
    N, Bs, S, Hq, Hkv, d = 32, 4, 8, 4, 2, 8
    G = Hq // Hkv
    q, k, v, perm, qp, counts, idx, o, lse = _tiny_qperm(O, 71, O.KEEP, 0.5)
    for g in range(Hq):
        h = g // G
        pr = perm[0, h]
        assert any(pr[pr[p]] != p for p in range(N))
        for p in range(N):
            assert (qp[0, g, p] == q[0, g, int(pr[p])]).all()
        kp = [k[0, h, int(pr[s])] for s in range(N)]
        vp = [v[0, h, int(pr[s])] for s in range(N)]
        vis = [[0] * N for _ in range(N)]
        for p in range(N):
            i = p // Bs
            sel = set(int(j) for j in idx[0, g, i, :counts[0, g, i]])
            for sl in range(N):
                same = sl // S == p // S and int(pr[sl]) <= int(pr[p])
                vis[p][sl] = int(same or (sl // Bs) in sel)
        ref = bf.attention(bf.mat(qp[0, g]), bf.mat(np.array(kp)), bf.mat(np.array(vp)), vis, 0.4)
        for p in range(N):
            assert np.allclose(o[0, g, int(pr[p])], ref[p], atol=1e-12), (g, p)


def pin_qperm_keep_one_is_dense(O):
    """[SS Theorem 3.3]: with every candidate block kept, attention on permuted queries and
    keys followed by the inverse permutation of the output equals plain causal attention."""
    q, k, v, perm, qp, counts, idx, o, lse = _tiny_qperm(O, 73, O.KEEP, 1.0)
    od, ld = O.dense_causal(q, k, v, block=4, scale=0.4)
    assert np.abs(o - od).max() < 1e-12 and np.abs(lse - ld).max() < 1e-12


def pin_qperm_identity_is_natural_order(O):
    """The identity permutation reduces the variant to plain block-sparse attention in the
    natural order (the same lists give the same output)."""
    N, Bs, S = 32, 4, 8
    q, k, v = _tiny(77, Hq=4, Hkv=2, N=N, d=8)
    ident = np.broadcast_to(np.arange(N, dtype=np.int32), (1, 2, N)).copy()
    P = O.block_probabilities(q, k, block=Bs, segment=S, scale=0.4)
    counts, idx = O.select_blocks(P, block=Bs, segment=S, mode=O.KEEP, param=0.3)
    o1, l1 = O.attention_permuted_queries(O.permute_queries(q, ident), k, v, block=Bs, segment=S,
                                          scale=0.4, perm=ident, counts=counts, idx=idx)
    o2, l2 = O.attention(q, k, v, block=Bs, segment=S, scale=0.4, perm=None, counts=counts, idx=idx)
    assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12


def pin_keep_one_is_dense(O):
    """Keep ratio 1 keeps every earlier-segment block, so PBS equals dense causal."""
    q, k, v, out = _tiny_pbs(O, 71, param=1.0)
    od, lsed = O.dense_causal(q, k, v, block=4, scale=0.4)
    assert np.abs(out["o"] - od).max() < 1e-12
    assert np.abs(out["lse"] - lsed).max() < 1e-12


def pin_one_segment_is_dense(O):
    """With S = N there is no earlier segment, so PBS equals dense causal for any ratio."""
    q, k, v = _tiny(81, N=32)
    out = O.prefill(q, k, v, block=4, segment=32, scale=0.4, mode=O.KEEP, param=0.1)
    od, _ = O.dense_causal(q, k, v, block=4, scale=0.4)
    assert (out["counts"] == 0).all()
    assert np.abs(out["o"] - od).max() < 1e-12


def pin_segment0_rows_are_dense(O):
    """Rows of the first segment have no candidate block and equal dense causal; later
    rows at a low keep ratio do not."""
    q, k, v, out = _tiny_pbs(O, 91, param=0.1)
    od, _ = O.dense_causal(q, k, v, block=4, scale=0.4)
    assert np.abs(out["o"][:, :, :8] - od[:, :, :8]).max() < 1e-12
    assert np.abs(out["o"][:, :, 8:] - od[:, :, 8:]).max() > 1e-3


def pin_default_scale(O):
    """The default softmax temperature is 1/sqrt(d) rounded to float32: exactly 1/8 at d = 64 and
    2^-3.5 rounded to float32 at d = 128."""
    assert O.default_scale(64) == 0.125
    assert O.default_scale(128) == float(np.float32(2.0 ** -3.5))


# ----------------------------------------------------------------------------- whole pipeline

def pin_prefill_selects_on_permuted_keys(O):
    """Hand-worked pipeline where the permutation decides which block is kept ([GS Methodik 4,
    Block-Auswahl]: block importance by mean pooling on the PERMUTED keys; [SS Fig. 2]: coverage
    is the mass of the selected blocks).

    N=16, Bs=2, S=8, one head, d=2, every query (1, 0); keys 3 and 5 are (2, 0), all others 0;
    scale = ln(5)/2, so a salient key's logit is ln 5 and every other logit is 0.
      scores, segment 0 (rows 14 and 15 see all of it): 5/16 for keys 3 and 5, 1/16 otherwise,
        so perm[0:8] = [3, 5, 0, 1, 2, 4, 6, 7];
      segment 1: all keys 0, row 14 sees 8..14 and row 15 sees 8..15, so keys 8..14 tie and key
        15 scores lower: perm[8:16] = [8 .. 15];
      pooled permuted keys: block 0 = mean(k3, k5) = (2, 0), blocks 1..3 = 0;
      P of query blocks 4..7 over candidate blocks 0..3: softmax(ln 5, 0, 0, 0) = [5/8, 1/8, 1/8, 1/8];
      keep 0.25 -> max(1, floor(1.0)) = 1 block -> [0];  keep 0.5 -> 2 blocks -> [0, 1];
      coverage 0.6 -> 5/8 already reaches it -> [0];  coverage 0.7 -> 5/8 + 1/8 -> [0, 1].
    (Pooling the unpermuted keys instead gives natural blocks {2,3} and {4,5} the salient mass
    and ranks block 1 first; reading a coverage threshold as a keep ratio keeps 2 blocks at
    0.6.)  The outputs of segment-1 rows then see keys {3, 5} (or {3, 5, 0, 1}) plus their own
    segment up to t; checked against brute force with that visibility."""
    N, Bs, S, d = 16, 2, 8, 2
    scale = math.log(5.0) / 2.0
    qf = np.zeros((1, 1, N, d), np.float32)
    qf[..., 0] = 1.0
    kf = np.zeros((1, 1, N, d), np.float32)
    kf[0, 0, [3, 5], 0] = 2.0
    q, k = f32_to_bf16_bits(qf), f32_to_bf16_bits(kf)
    v = random_bf16((1, 1, N, d), 141)
    cases = [(O.KEEP, 0.25, [0]), (O.KEEP, 0.5, [0, 1]), (O.COVERAGE, 0.6, [0]), (O.COVERAGE, 0.7, [0, 1])]
    for mode, param, want in cases:
        out = O.prefill(q, k, v, block=Bs, segment=S, scale=scale, mode=mode, param=param)
        assert out["perm"][0, 0].tolist() == [3, 5, 0, 1, 2, 4, 6, 7] + list(range(8, 16)), out["perm"]
        for i in range(4, 8):
            assert np.allclose(out["P"][0, 0, i, :4], [0.625, 0.125, 0.125, 0.125], rtol=1e-6), out["P"][0, 0, i]
            assert (out["P"][0, 0, i, 4:] == 0).all()
            assert out["idx"][0, 0, i, :out["counts"][0, 0, i]].tolist() == want, (mode, param, i, out["idx"][0, 0, i])
        assert (out["counts"][0, 0, :4] == 0).all()
        sel = [[] for _ in range(4)] + [want] * 4
        perm = out["perm"][0, 0]
        vis = bf.visibility(N, Bs, S, perm=perm, sel=sel)
        keys_of_block = {0: {3, 5}, 1: {0, 1}}
        for t in range(8, N):
            assert {j for j in range(N) if vis[t][j]} == set().union(*(keys_of_block[b] for b in want)) | set(range(8, t + 1))
        ref = bf.attention(bf.mat(q[0, 0]), bf.mat(k[0, 0]), bf.mat(v[0, 0]), vis, scale)
        assert np.allclose(out["o"][0, 0], ref, atol=1e-12), (mode, param)


def pin_prefill_pipeline_bruteforce(O):
    """The whole pipeline on a random tiny GQA input, in both selection modes, against brute
    force stage by stage: scores from explicit per-segment softmaxes; the permutation sorts
    each segment of the returned float32 scores (descending, ties to the lower position); P is
    the explicit pooled softmax over the candidates of the brute-force PERMUTED keys; the lists
    follow the selection rules applied to the returned P (keep: the top max(1, floor(r*n));
    coverage: the shortest prefix of the ranking whose sequential float32 sum reaches tau); the
    output is brute-force attention over the visibility those lists and that permutation give."""
    N, Bs, S, Hq, Hkv, d = 32, 4, 8, 4, 2, 8
    G, nb, bps = Hq // Hkv, N // Bs, S // Bs
    scale = 0.4
    q, k, v = _tiny(151, Hq=Hq, Hkv=Hkv, N=N, d=d, scale_k=1.7)
    for mode, param in ((O.KEEP, 0.34), (O.COVERAGE, 0.7), (O.COVERAGE, 0.95)):
        out = O.prefill(q, k, v, block=Bs, segment=S, scale=scale, mode=mode, param=param)
        for h in range(Hkv):
            sc = bf.key_scores([bf.mat(q[0, g]) for g in range(h * G, (h + 1) * G)], bf.mat(k[0, h]), Bs, S, scale)
            assert np.allclose(out["scores"][0, h], sc, rtol=2e-6, atol=1e-9)
            s32 = out["scores"][0, h]
            for s0 in range(0, N, S):
                want = sorted(range(s0, s0 + S), key=lambda j: (-float(s32[j]), j))
                assert out["perm"][0, h, s0:s0 + S].tolist() == want, (h, s0)
        for g in range(Hq):
            h = g // G
            perm = out["perm"][0, h]
            kp = np.stack([k[0, h, int(perm[p])] for p in range(N)])
            ref = bf.block_probs(bf.mat(q[0, g]), bf.mat(kp), Bs, S, scale)
            Pg = out["P"][0, g]
            for (i, j), pij in ref.items():
                assert math.isclose(float(Pg[i, j]), pij, rel_tol=2e-6), (g, i, j)
            sel = []
            for i in range(nb):
                n = (i // bps) * bps
                ranked = sorted(range(n), key=lambda j: (-float(Pg[i, j]), j))
                if n == 0:
                    kk = 0
                elif mode == O.KEEP:
                    kk = max(1, math.floor(param * n))
                else:
                    c, kk = np.float32(0), n
                    for m, j in enumerate(ranked):
                        c = np.float32(c + Pg[i, j])
                        if float(c) >= param:
                            kk = m + 1
                            break
                sel.append(sorted(ranked[:kk]))
                assert int(out["counts"][0, g, i]) == kk, (mode, g, i)
                assert out["idx"][0, g, i, :kk].tolist() == sel[-1], (mode, g, i)
            vis = bf.visibility(N, Bs, S, perm=perm, sel=sel)
            o_ref = bf.attention(bf.mat(q[0, g]), bf.mat(k[0, h]), bf.mat(v[0, h]), vis, scale)
            assert np.allclose(out["o"][0, g], o_ref, atol=1e-12), (mode, g)


# ----------------------------------------------------------------------------- packed sequences

def _pack(x):
    """[B, H, N, d] -> [1, H, B*N, d] (the sequences one after another along N)."""
    B, H, N, d = x.shape
    return np.ascontiguousarray(x.transpose(1, 0, 2, 3).reshape(1, H, B * N, d))


def pin_varlen_equal_lengths_is_batch(O):
    """Three sequences of one length packed along N give the batch-of-three result, with
    positions and block indices shifted by each sequence's start and P block-diagonal."""
    q, k, v = _tiny(111, B=3, N=32)
    ref = O.prefill(q, k, v, block=4, segment=8, scale=0.4, mode=O.KEEP, param=0.5)
    out = O.prefill_varlen(_pack(q), _pack(k), _pack(v), [0, 32, 64, 96], block=4, segment=8,
                           scale=0.4, mode=O.KEEP, param=0.5)
    for b in range(3):
        a, i0 = 32 * b, 8 * b
        assert np.array_equal(out["scores"][0, :, a:a + 32], ref["scores"][b])
        assert np.array_equal(out["perm"][0, :, a:a + 32], ref["perm"][b] + a)
        assert np.array_equal(out["k_perm"][0, :, a:a + 32], ref["k_perm"][b])
        assert np.array_equal(out["counts"][0, :, i0:i0 + 8], ref["counts"][b])
        w = ref["idx"].shape[-1]
        want = np.where(ref["idx"][b] >= 0, ref["idx"][b] + i0, -1)
        assert np.array_equal(out["idx"][0, :, i0:i0 + 8, :w], want)
        assert (out["idx"][0, :, i0:i0 + 8, w:] == -1).all()
        assert np.array_equal(out["P"][0, :, i0:i0 + 8, i0:i0 + 8], ref["P"][b])
        P_rest = out["P"][0, :, i0:i0 + 8].copy()
        P_rest[:, :, i0:i0 + 8] = 0
        assert (P_rest == 0).all()
        assert np.array_equal(out["o"][0, :, a:a + 32], ref["o"][b])
        assert np.array_equal(out["lse"][0, :, a:a + 32], ref["lse"][b])


def pin_varlen_keep_one_is_dense_per_sequence(O):
    """Unequal lengths at keep ratio 1: every sequence equals dense causal attention over its
    own tokens only."""
    lens = [16, 32, 8, 24]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = _tiny(121, N=int(cu[-1]))
    out = O.prefill_varlen(q, k, v, cu, block=4, segment=8, scale=0.4, mode=O.KEEP, param=1.0)
    for a, b in zip(cu[:-1], cu[1:]):
        od, lsed = O.dense_causal(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], block=4, scale=0.4)
        assert np.abs(out["o"][:, :, a:b] - od).max() < 1e-12
        assert np.abs(out["lse"][:, :, a:b] - lsed).max() < 1e-12


def pin_varlen_sequences_independent(O):
    """Changing one sequence's tokens changes nothing in the others, and no block list points
    into another sequence."""
    lens = [16, 24, 16]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = _tiny(131, N=int(cu[-1]))
    out = O.prefill_varlen(q, k, v, cu, block=4, segment=8, scale=0.4, mode=O.KEEP, param=0.5)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, :, 16:40], k2[:, :, 16:40], v2[:, :, 16:40] = _tiny(132, N=24)
    out2 = O.prefill_varlen(q2, k2, v2, cu, block=4, segment=8, scale=0.4, mode=O.KEEP, param=0.5)
    for sl in (slice(0, 16), slice(40, 56)):
        assert np.array_equal(out["o"][:, :, sl], out2["o"][:, :, sl])
        assert np.array_equal(out["perm"][:, :, sl], out2["perm"][:, :, sl])
    assert not np.array_equal(out["o"][:, :, 16:40], out2["o"][:, :, 16:40])
    for s_, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        i0, i1 = a // 4, b // 4
        c = out["counts"][0, :, i0:i1]
        ix = out["idx"][0, :, i0:i1]
        live = np.arange(ix.shape[-1])[None, None, :] < c[..., None]
        assert ((ix >= i0) | ~live).all() and ((ix < i1) | ~live).all()
        assert (out["perm"][0, :, a:b] >= a).all() and (out["perm"][0, :, a:b] < b).all()


# ----------------------------------------------------------------------------- density, coverage

def _bf_coverage(Q, K, vis, scale, t):
    """Dense causal softmax of row t summed over the keys vis marks (brute force)."""
    p = bf.softmax_over({j: scale * bf.dot(Q[t], K[j]) for j in range(t + 1)})
    return math.fsum(p[j] for j in p if vis[t][j])


def pin_coverage_definitions(O):
    """[SS Fig. 2] coverage = the dense attention mass held by the computed keys: against brute
    force (explicit visibility matrix, dense softmax over j <= t), against exp(lse_sparse -
    lse_dense) from the attention routines, in both key orders; 1 wherever the key set is the
    whole causal prefix (segment-0 rows, keep ratio 1), below 1 elsewhere at a low ratio."""
    N, Bs, S, Hq, Hkv = 32, 4, 8, 4, 2
    G = Hq // Hkv
    for permuted in (True, False):
        q, k, v = _tiny(101, Hq=Hq, Hkv=Hkv, N=N, d=8, scale_k=1.7)
        if permuted:
            out = O.prefill(q, k, v, block=Bs, segment=S, scale=0.4, mode=O.KEEP, param=0.25)
            perm, counts, idx, lse = out["perm"], out["counts"], out["idx"], out["lse"]
        else:
            P = O.block_probabilities(q, k, block=Bs, segment=S, scale=0.4)
            counts, idx = O.select_blocks(P, block=Bs, segment=S, mode=O.KEEP, param=0.25)
            perm = None
            _, lse = O.attention(q, k, v, block=Bs, segment=S, scale=0.4, counts=counts, idx=idx)
        cov = O.attention_coverage(q, k, block=Bs, segment=S, scale=0.4, perm=perm, counts=counts, idx=idx)
        _, lsed = O.dense_causal(q, k, v, block=Bs, scale=0.4)
        assert np.abs(cov - np.exp(lse - lsed)).max() < 1e-12
        for g in range(Hq):
            h = g // G
            Q, K = bf.mat(q[0, g]), bf.mat(k[0, h])
            vis = _vis_matrix(N, Bs, S, None if perm is None else perm[0, h], counts[0, g], idx[0, g])
            for t in (0, 7, 8, 13, 21, 31):
                assert math.isclose(cov[0, g, t], _bf_coverage(Q, K, vis, 0.4, t), rel_tol=1e-12), (g, t)
        assert np.abs(cov[:, :, :S] - 1).max() < 1e-12
        assert cov[:, :, S:].min() < 0.999 and cov.max() <= 1 + 1e-12
        one = O.select_blocks(O.block_probabilities(q, k if perm is None else O.apply_permutation(k, perm),
                                                    block=Bs, segment=S, scale=0.4),
                              block=Bs, segment=S, mode=O.KEEP, param=1.0)
        cov1 = O.attention_coverage(q, k, block=Bs, segment=S, scale=0.4, perm=perm, counts=one[0], idx=one[1])
        assert np.abs(cov1 - 1).max() < 1e-12


def pin_block_density_handworked(O):
    """Block counts worked by hand for N=16, Bs=4, S=8 (two segments of two blocks), one head,
    one kept block per second-segment row: 2 selected of 4 candidates, 10 dense causal blocks.
    Own-segment blocks: natural order 1+2+1+2; permuted with a segment-1 order whose first
    permuted block holds keys 12..15 only (invisible to rows 8..11) 1+2+1+2; with a mixed order
    1+2+2+2 (segment 0 in natural order).  Then the same counts by brute force over the
    visibility matrix of a random tiny pipeline."""
    counts = np.array([[[0, 0, 1, 1]]], np.int32)
    d = O.block_density(counts, block=4, segment=8, N=16)
    assert d == dict(selected=2, candidates=4, computed=8, dense=10), d
    seg0 = list(range(8))
    late = np.array([[seg0 + [12, 13, 14, 15, 8, 9, 10, 11]]], np.int32)
    mixed = np.array([[seg0 + [15, 8, 13, 10, 12, 9, 14, 11]]], np.int32)
    assert O.block_density(counts, block=4, segment=8, N=16, perm=late)["computed"] == 8
    assert O.block_density(counts, block=4, segment=8, N=16, perm=mixed)["computed"] == 9
    N, Bs, S, Hq, Hkv = 32, 4, 8, 4, 2
    q, k, v, out = _tiny_pbs(O, 111, param=0.34)
    dd = O.block_density(out["counts"], block=Bs, segment=S, N=N, perm=out["perm"])
    G, nb = Hq // Hkv, N // Bs
    computed = 0
    for g in range(Hq):
        h = g // G
        perm = out["perm"][0, h]
        vis = _vis_matrix(N, Bs, S, perm, out["counts"][0, g], out["idx"][0, g])
        for i in range(nb):
            rows = range(i * Bs, (i + 1) * Bs)
            for p in range(nb):   # permuted key block p holds original keys perm[p*Bs:(p+1)*Bs]
                if any(vis[t][int(perm[s])] for t in rows for s in range(p * Bs, (p + 1) * Bs)):
                    computed += 1
    assert dd["computed"] == computed, (dd, computed)
    assert dd["selected"] == int(out["counts"].sum())
    assert dd["dense"] == Hq * nb * (nb + 1) // 2


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
