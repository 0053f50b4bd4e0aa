"""GPU edge cases: degenerate shapes of the method, sort specials, extreme sizes, determinism."""
import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import oracle
import pbs_synth
from gpu_helpers import (check_attn, dev, dev_bf16, inverse_of, lists_equal, run_attn, run_permute,
                         run_score, run_select, say, shape)

pytestmark = pytest.mark.gpu


def _planted(Hq, Hkv, N, d, Bs, S, seed):
    w = pbs_synth.WORKLOADS["gqa_8k"].scaled(heads_q=Hq, heads_kv=Hkv, seq_len=N, head_dim=d,
                                             block=Bs, segment=S, seed=seed)
    return w, pbs_synth.make_inputs(w)


def test_keep_one_equals_dense():
    """Keep ratio 1 keeps every earlier-segment block: PBS equals dense causal attention."""
    say("keep=1 vs dense")
    w, inp = _planted(8, 2, 2048, 128, 128, 512, 11)
    scale = oracle.default_scale(128)
    od, _ = oracle.dense_causal(inp["q"], inp["k"], inp["v"], block=128, scale=scale)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    bufs = P.prefill(q, k, v, block=128, segment=512, keep=1.0, scale=scale)
    dense = P.dense_causal(q, k, v, block=128, scale=scale)
    torch.cuda.synchronize()
    nb = 2048 // 128
    want = np.array([(i // 4) * 4 for i in range(nb)])
    assert (bufs.counts.cpu().numpy() == want[None, None, :]).all()
    check_attn(bufs.o.float().cpu().numpy(), od, "keep=1 PBS vs oracle dense")
    check_attn(dense.float().cpu().numpy(), od, "GPU dense vs oracle dense")


def test_single_segment_is_dense():
    """S = N: no earlier segment, no candidate, PBS equals dense causal for any ratio."""
    say("S = N")
    w, inp = _planted(4, 2, 1024, 128, 128, 1024, 12)
    scale = oracle.default_scale(128)
    od, _ = oracle.dense_causal(inp["q"], inp["k"], inp["v"], block=128, scale=scale)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    bufs = P.prefill(q, k, v, block=128, segment=1024, keep=0.1, scale=scale)
    torch.cuda.synchronize()
    assert (bufs.counts.cpu().numpy() == 0).all()
    check_attn(bufs.o.float().cpu().numpy(), od, "S=N PBS vs oracle dense")


def test_tiny_keep_ratio_keeps_one_block():
    say("tiny keep ratio")
    w, inp = _planted(2, 1, 1024, 64, 64, 128, 13)
    scale = oracle.default_scale(64)
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], block=64, segment=128, scale=scale,
                         mode=oracle.KEEP, param=1e-6)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    bufs = P.prefill(q, k, v, block=64, segment=128, keep=1e-6, scale=scale)
    torch.cuda.synchronize()
    c = bufs.counts.cpu().numpy()
    assert ((c == 1) | (np.arange(16)[None, None, :] < 2)).all()
    check_attn(bufs.o.float().cpu().numpy(), ref["o"], "keep=1e-6 end-to-end")


def test_sort_specials_bitexact():
    """Ties, signed zeros and NaN in the scores: the GPU permutation equals the oracle's."""
    say("sort specials")
    rng = np.random.default_rng(3)
    B, H, N, d, Bs, S = 1, 2, 2048, 64, 64, 1024
    vals = np.array([0.0, -0.0, 1e-30, 0.25, 0.25, np.nan, -1.0, np.inf, 3.0], np.float32)
    sc = rng.choice(vals, size=(B, H, N)).astype(np.float32)
    k = pbs_synth.random_bf16((B, H, N, d), 5)
    v = pbs_synth.random_bf16((B, H, N, d), 6)
    sh = shape(B, H, H, N, d, Bs, S)
    perm, kp, vp, _, _, _ = run_permute(sh, dev(sc), dev_bf16(k), dev_bf16(v), pool=False,
                                        minpos=False, inv=False)
    assert np.array_equal(perm.cpu().numpy(), oracle.segment_permutation(sc, segment=S))


def test_select_handworked_rows_on_gpu():
    """Hand-made probability rows (exact in binary): the GPU selection matches the oracle,
    including the >= boundary of coverage and the sequential float32 sum."""
    say("select handworked")
    B, Hq, N, d, Bs, S = 1, 1, 640, 64, 64, 320   # 10 blocks, 2 segments of 5 blocks
    Pm = np.zeros((B, Hq, 10, 10), np.float32)
    rows = [[0.125, 0.25, 0.25, 0.0625, 0.125], [0.2] * 5, [0.0, 0.0, 0.0, 0.0, 1.0],
            [0.75, 2.0 ** -25, 2.0 ** -25, 2.0 ** -25, 0.0], [0.25, 0.5, 0.125, 0.125, 0.0]]
    for r, vals in enumerate(rows):
        Pm[0, 0, 5 + r, :5] = vals
    sh = shape(B, Hq, 1, N, d, Bs, S)
    for mode, cmode, param in ((oracle.KEEP, P.PBS_SELECT_KEEP_RATIO, 0.5),
                               (oracle.COVERAGE, P.PBS_SELECT_COVERAGE, 0.75),
                               (oracle.COVERAGE, P.PBS_SELECT_COVERAGE, 0.75 + 2.0 ** -24),
                               (oracle.COVERAGE, P.PBS_SELECT_COVERAGE, 1.0)):
        rc, ri = oracle.select_blocks(Pm, block=Bs, segment=S, mode=mode, param=param)
        counts, idx = run_select(sh, None, None, None, 0.125, cmode, param, blk_scores=dev(Pm),
                                 flags=P.PBS_FLAG_SCORES_IN)
        assert lists_equal(counts.cpu().numpy(), idx.cpu().numpy(), rc, ri), (mode, param)


def test_select_widest_rows():
    """The widest supported candidate set (8191 blocks, an 8192-entry sort per row)."""
    say("select widest rows")
    B, Hq, N, d, Bs, S = 1, 1, 8192 * 64, 64, 64, 64
    nb = N // Bs
    rng = np.random.default_rng(8)
    rows = [nb - 1, nb - 2, 4097, 100, 1]
    Pm = np.zeros((B, Hq, nb, nb), np.float32)
    for i in rows:
        x = rng.normal(size=i)
        e = np.exp(x - x.max())
        Pm[0, 0, i, :i] = (e / e.sum()).astype(np.float32)
    sh = shape(B, Hq, 1, N, d, Bs, S)
    assert P.pbs_max_offdiag(sh) == 8191
    for mode, cmode, param in ((oracle.KEEP, P.PBS_SELECT_KEEP_RATIO, 0.1),
                               (oracle.COVERAGE, P.PBS_SELECT_COVERAGE, 0.9)):
        counts, idx = run_select(sh, None, None, None, 0.125, cmode, param, blk_scores=dev(Pm),
                                 flags=P.PBS_FLAG_SCORES_IN)
        c, ix = counts.cpu().numpy(), idx.cpu().numpy()
        for i in rows:
            sub = Pm[:, :, i:i + 1, :]
            # the oracle's selection of one row, laid out as a single-candidate-row problem
            order = oracle.descending_order(sub[0, 0, 0, :i])
            if mode == oracle.KEEP:
                kk = oracle.keep_count(i, param)
            else:
                cs = np.add.accumulate(sub[0, 0, 0, :i][order], dtype=np.float32).astype(np.float64)
                hit = np.nonzero(cs >= param)[0]
                kk = int(hit[0]) + 1 if hit.size else i
            assert c[0, 0, i] == kk
            assert np.array_equal(ix[0, 0, i, :kk], np.sort(order[:kk]))


def test_select_keep_ratio_ties_and_specials():
    """Keep-ratio selection on rows full of ties that straddle the kept count, signed zeros,
    tiny values and NaN (ranked after every number), with and without the first block forced
    first: bit-exact against the oracle's ranking rules, on rows up to 8191 candidates."""
    say("select ties and specials")
    B, Hq, N, d, Bs, S = 1, 2, 8192 * 64, 64, 64, 64
    nb = N // Bs
    rng = np.random.default_rng(12)
    vals = np.array([0.0, -0.0, 1e-30, 0.25, 0.25, 0.25, 0.125, np.nan, 3.0, 2.0 ** -20], np.float32)
    rows = [nb - 1, 4097, 960, 129, 2]
    Pm = np.zeros((B, Hq, nb, nb), np.float32)
    for g in range(Hq):
        for i in rows:
            Pm[0, g, i, :i] = rng.choice(vals, size=i)
    sh = shape(B, Hq, 1, N, d, Bs, S)
    for param in (0.1, 0.3, 0.5, 1.0):
        for keep_first in (False, True):
            flags = P.PBS_FLAG_SCORES_IN | (P.PBS_FLAG_KEEP_FIRST if keep_first else 0)
            counts, idx = run_select(sh, None, None, None, 0.125, P.PBS_SELECT_KEEP_RATIO, param,
                                     blk_scores=dev(Pm), flags=flags)
            c, ix = counts.cpu().numpy(), idx.cpu().numpy()
            for g in range(Hq):
                for i in rows:
                    order = oracle.descending_order(Pm[0, g, i, :i])
                    if keep_first:
                        order = np.concatenate([[0], order[order != 0]])
                    kk = oracle.keep_count(i, param)
                    assert c[0, g, i] == kk, (param, keep_first, g, i)
                    assert np.array_equal(ix[0, g, i, :kk], np.sort(order[:kk])), (param, keep_first, g, i)


def test_select_coverage_row_sizes():
    """Coverage selection on rows of every candidate count class around the powers of two
    (1 to 2047 candidates: the register-sorted sizes 64..1024 and the LDS-sorted rest), with
    softmax rows, rows full of ties and zeros, and rows holding NaN, -0 and a negative value,
    with and without the first block forced first: bit-exact against the oracle."""
    say("select coverage row sizes")
    B, Hq, N, d, Bs, S = 1, 2, 2048 * 64, 64, 64, 64   # one block per segment: row i has i candidates
    nb = N // Bs
    rng = np.random.default_rng(21)
    rows = [1, 2, 63, 64, 65, 100, 127, 128, 129, 255, 256, 300, 511, 512, 513, 700, 960, 1023,
            1024, 1025, 1500, nb - 1]
    tie_vals = np.array([0.0, 0.25, 0.125, 1e-30, 2.0 ** -20, 0.5, 0.0625], np.float32)
    Pm = np.zeros((B, Hq, nb, nb), np.float32)
    for t, i in enumerate(rows):
        x = rng.normal(size=i) * 2.0
        e = np.exp(x - x.max())
        Pm[0, 0, i, :i] = (e / e.sum()).astype(np.float32)
        r = rng.choice(tie_vals, size=i) / max(1.0, i / 16.0)
        if t % 3 == 2 and i > 3:
            r[rng.integers(i)] = np.nan
            r[rng.integers(i)] = -0.0
            r[rng.integers(i)] = -0.125
        Pm[0, 1, i, :i] = r.astype(np.float32)
    sh = shape(B, Hq, 1, N, d, Bs, S)
    for tau, keep_first in ((0.5, False), (0.9, True), (0.999, False), (1.0, True)):
        say(f"coverage tau={tau} keep_first={keep_first}")
        flags = P.PBS_FLAG_SCORES_IN | (P.PBS_FLAG_KEEP_FIRST if keep_first else 0)
        counts, idx = run_select(sh, None, None, None, 0.125, P.PBS_SELECT_COVERAGE, tau,
                                 blk_scores=dev(Pm), flags=flags)
        rc, ri = oracle.select_blocks(Pm, block=Bs, segment=S, mode=oracle.COVERAGE, param=tau,
                                      keep_first=keep_first)
        c = counts.cpu().numpy()
        assert lists_equal(c, idx.cpu().numpy(), rc, ri), (tau, keep_first)
        if tau < 1.0:   # the softmax rows stop before their end
            assert (c[0, 0, rows[3:]] < np.array(rows[3:])).all()


def test_permute_largest_segment():
    """The largest supported segment (16384 keys sorted in one workgroup)."""
    say("permute S=16384")
    B, H, N, d, Bs, S = 1, 1, 32768, 128, 128, 16384
    rng = np.random.default_rng(9)
    sc = (rng.random((B, H, N)) * 1e-3).astype(np.float32)
    sc[0, 0, ::7] = sc[0, 0, 3]                 # many ties
    k = pbs_synth.random_bf16((B, H, N, d), 10)
    v = pbs_synth.random_bf16((B, H, N, d), 11)
    sh = shape(B, H, H, N, d, Bs, S)
    perm, kp, vp, _, mpos, pinv = run_permute(sh, dev(sc), dev_bf16(k), dev_bf16(v), pool=False)
    ref = oracle.segment_permutation(sc, segment=S)
    assert np.array_equal(perm.cpu().numpy(), ref)
    assert np.array_equal(mpos.cpu().numpy(), ref.reshape(B, H, N // Bs, Bs).min(-1))
    assert np.array_equal(pinv.cpu().numpy(), inverse_of(ref))


@pytest.mark.parametrize("S", [1536, 3072, 12288])
def test_permute_segment_not_power_of_two(S):
    """Segments whose length is not a power of two (the sort pads to the next one: 2048, 4096
    and 16384 keys, all register-sorted across the workgroup's waves), with ties and specials:
    the GPU permutation and its inverse equal the oracle's."""
    say(f"permute S={S}")
    B, H, d, Bs = 1, 2, 64, 64
    N = 2 * S
    rng = np.random.default_rng(S)
    vals = np.array([0.0, -0.0, 1e-30, 0.25, np.nan, -1.0, np.inf, 3.0], np.float32)
    sc = (rng.random((B, H, N)) * 1e-3).astype(np.float32)
    mask = rng.random((B, H, N)) < 0.2
    sc[mask] = rng.choice(vals, size=int(mask.sum()))
    k = pbs_synth.random_bf16((B, H, N, d), 20)
    v = pbs_synth.random_bf16((B, H, N, d), 21)
    sh = shape(B, H, H, N, d, Bs, S)
    perm, kp, vp, _, mpos, pinv = run_permute(sh, dev(sc), dev_bf16(k), dev_bf16(v), pool=False)
    ref = oracle.segment_permutation(sc, segment=S)
    assert np.array_equal(perm.cpu().numpy(), ref)
    assert np.array_equal(pinv.cpu().numpy(), inverse_of(ref))
    assert np.array_equal(mpos.cpu().numpy(), ref.reshape(B, H, N // Bs, Bs).min(-1))


def test_deterministic():
    """Two runs of the whole pipeline give bitwise-identical results."""
    say("determinism")
    w, inp = _planted(8, 2, 2048, 128, 128, 512, 14)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    a = P.prefill(q, k, v, block=128, segment=512, coverage=0.9)
    b = P.prefill(q, k, v, block=128, segment=512, coverage=0.9)
    torch.cuda.synchronize()
    for name in ("scores", "perm", "k_perm", "v_perm", "k_pool", "counts", "o", "lse"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert lists_equal(a.counts.cpu().numpy(), a.idx.cpu().numpy(), b.counts.cpu().numpy(),
                       b.idx.cpu().numpy())


def test_empty_problem_launches_nothing():
    sh = shape(0, 4, 2, 1024, 128, 128, 256)
    P.pbs_attn_fwd(sh, 0, 0, 0, None, None, None, None, 0.1, 0)
    P.pbs_score(sh, 0, 0, 0.1, 0, 0, 0)


def _dominant_key_inputs(seed, N=2048, d=128, big_at=700, big=400.0):
    """Queries aligned with a direction u and one key far along u: its score exceeds the scores
    of the keys visited before it by far more than float32 exp2 can represent (pass-0 overflow),
    so the kernel has to fall back to the exact row maximum."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((1, 2, N, d)).astype(np.float32) + np.float32(3.0) * u.astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k[0, 0, big_at] = (big * u).astype(np.float32)
    return [pbs_synth.f32_to_bf16_bits(x) for x in (q, k, v)]


def test_dominant_late_key_dense():
    say("dominant late key, dense")
    q, k, v = _dominant_key_inputs(21)
    scale = oracle.default_scale(128)
    od, ol = oracle.dense_causal(q, k, v, block=128, scale=scale)
    assert ol.max() > 60.0  # the key's logit is far above every earlier one
    sh = shape(1, 2, 1, 2048, 128, 128, 128)
    o, lse = run_attn(sh, dev_bf16(q), dev_bf16(k), dev_bf16(v), None, None, None, None, scale)
    check_attn(o.float().cpu().numpy(), od, "dominant key dense")
    assert np.abs(lse.cpu().numpy() - ol).max() < 1e-3


def test_scores_dominant_late_key():
    """Key scores where one key of a segment lies about 150 (log2 units) above the first keys
    its scoring rows see: the scoring pass's fixed reference would overflow its sum, so the
    chunk is run again with a running max.  Scores against the oracle: relative 1e-4 where they
    are representable, and every segment still sums to one."""
    say("scores, dominant late key")
    q, k, _ = _dominant_key_inputs(23)
    scale = oracle.default_scale(128)
    N, Bs, S = 2048, 128, 512
    ref = oracle.key_scores(q, k, block=Bs, segment=S, scale=scale).astype(np.float64)
    assert ref[0, 0, 700] > 0.95            # the key takes nearly all of its segment's mass
    sh = shape(1, 2, 1, N, 128, Bs, S)
    s = run_score(sh, dev_bf16(q), dev_bf16(k), scale).cpu().numpy().astype(np.float64)
    big = ref > 1e-30
    assert (np.abs(s - ref)[big] <= 1e-4 * ref[big]).all()
    assert (np.abs(s - ref)[~big] <= 1e-30).all()
    assert np.allclose(s.reshape(1, 1, -1, S).sum(-1), 1.0, atol=1e-4)


@pytest.mark.parametrize("permuted", [True, False])
def test_dominant_late_key_pbs(permuted):
    say(f"dominant late key, PBS permuted={permuted}")
    q, k, v = _dominant_key_inputs(22)
    scale = oracle.default_scale(128)
    N, Bs, S = 2048, 128, 512
    sc = oracle.key_scores(q, k, block=Bs, segment=S, scale=scale)
    perm = oracle.segment_permutation(sc, segment=S) if permuted else \
        np.broadcast_to(np.arange(N, dtype=np.int32), (1, 1, N)).copy()
    kp, vp = oracle.apply_permutation(k, perm), oracle.apply_permutation(v, perm)
    Pm = oracle.block_probabilities(q, kp, block=Bs, segment=S, scale=scale)
    counts, idx = oracle.select_blocks(Pm, block=Bs, segment=S, mode=oracle.KEEP, param=0.5)
    oo, ol = oracle.attention(q, k, v, block=Bs, segment=S, scale=scale, perm=perm, counts=counts,
                              idx=idx)
    assert ol.max() > 60.0
    sh = shape(1, 2, 1, N, 128, Bs, S)
    o, lse = run_attn(sh, dev_bf16(q), dev_bf16(kp), dev_bf16(vp),
                      dev(perm) if permuted else None, dev(inverse_of(perm)) if permuted else None,
                      dev(counts), dev(idx), scale)
    check_attn(o.float().cpu().numpy(), oo, f"dominant key PBS permuted={permuted}")
    assert np.abs(lse.cpu().numpy() - ol).max() < 1e-3


@pytest.mark.parametrize("dominant", [False, True])
def test_long_lists_refill_the_window(dominant):
    """Off-diagonal lists longer than the attention kernel's LDS window (1792 entries): N=131072,
    Bs=64, S=256, keep ratio 1, so the last query blocks list up to 2044 blocks.  With keep 1 the
    result equals dense causal attention.  With a dominant key in block 1000 the rows after it
    overflow the first-stage reference, and the fallback passes start over from the first
    window."""
    say(f"long lists, dominant={dominant}")
    N, d, Bs, S = 131072, 64, 64, 256
    rng = np.random.default_rng(31)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    if dominant:
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        q += np.float32(3.0) * u.astype(np.float32)
        k[0, 0, 1000 * Bs + 17] = (300.0 * u).astype(np.float32)
    q, k, v = (pbs_synth.f32_to_bf16_bits(x) for x in (q, k, v))
    scale = oracle.default_scale(d)
    nb = N // Bs
    blocks = [nb - 1, nb - 2, nb - 5, nb - 64, 1500, 1000, 999, 3]
    od, ol = oracle.dense_causal(q, k, v, block=Bs, scale=scale, qblocks=[(0, 0, i) for i in blocks])
    bufs = P.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), block=Bs, segment=S, keep=1.0, scale=scale)
    torch.cuda.synchronize()
    counts = bufs.counts.cpu().numpy()
    assert counts[0, 0, nb - 1] == (nb - 1) // (S // Bs) * (S // Bs) > 1792
    og = bufs.o.float().cpu().numpy()[0, 0]
    lg = bufs.lse.cpu().numpy()[0, 0]
    got = np.stack([og[i * Bs:(i + 1) * Bs] for i in blocks])
    gl = np.stack([lg[i * Bs:(i + 1) * Bs] for i in blocks])
    check_attn(got, od, f"long lists dominant={dominant}")
    assert np.abs(gl - ol).max() < 1e-3


def test_key_stream_refill_and_fallback():
    """The own segment's key stream at its longest (query blocks late in an 8192-key segment see
    up to 8192 keys, 256 stages through the kernel's slot ring) together with the fallback
    passes: N=16384, Bs=128, S=8192, keep 1 (the result equals dense causal attention).  A
    dominant key at position 11192 of the second segment sorts to its first slot, so for the rows
    after it the stream meets a logit far above the first stage's reference, the row sums
    overflow, and the fallback passes must walk the stream again from its first stage."""
    say("key stream refill + fallback, d=128 Bs=128 S=8192 N=16384")
    N, d, Bs, S = 16384, 128, 128, 8192
    rng = np.random.default_rng(77)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q += np.float32(3.0) * u.astype(np.float32)
    k[0, 0, 11192] = (300.0 * u).astype(np.float32)
    q, k, v = (pbs_synth.f32_to_bf16_bits(x) for x in (q, k, v))
    scale = oracle.default_scale(d)
    blocks = [127, 126, 110, 88, 87, 70, 64, 63, 0]
    od, ol = oracle.dense_causal(q, k, v, block=Bs, scale=scale, qblocks=[(0, 0, i) for i in blocks])
    bufs = P.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), block=Bs, segment=S, keep=1.0,
                     scale=scale)
    torch.cuda.synchronize()
    assert int(bufs.perm.cpu().numpy()[0, 0, S]) == 11192   # the dominant key leads its segment
    og = bufs.o.float().cpu().numpy()[0, 0]
    lg = bufs.lse.cpu().numpy()[0, 0]
    got = np.stack([og[i * Bs:(i + 1) * Bs] for i in blocks])
    gl = np.stack([lg[i * Bs:(i + 1) * Bs] for i in blocks])
    check_attn(got, od, "key stream refill + fallback")
    assert np.abs(gl - ol).max() < 1e-3
