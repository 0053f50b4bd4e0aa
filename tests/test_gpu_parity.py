"""GPU parity of every stage of the PBS-Attn path against the CPU oracle, through the C ABI.

Bars: permutations and block lists bit-exact when both sides start from the same float32
values (the oracle's scores / block probabilities); scores and block probabilities within a
relative 1e-4; attention within max-abs 2e-2 and mean-abs 2e-3 of the float64 oracle.

Cases are small enough for the oracle to finish in seconds and still span several blocks and
segments, ragged segment counts (S = 3 Bs), both head dims and block sizes, GQA groups of 4 and 7,
both selection rules, and a batch of 3."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import oracle
import pbs_synth
from gpu_helpers import (check_attn, dev, dev_bf16, host_bits, inverse_of, lists_equal, run_attn,
                         run_permute, run_score, run_select, say, shape)

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-4

# name -> (Hq, Hkv, N, d, Bs, S, mode, param[, batch])
CASES = {
    "toy_1k": (1, 1, 1024, 64, 64, 256, "keep", 0.5),
    "gqa4_2k_keep": (8, 2, 2048, 128, 128, 512, "keep", 0.3),
    "gqa7_1536_ragged": (14, 2, 1536, 128, 128, 384, "keep", 0.25),
    "d64_bs128_cov": (4, 2, 1024, 64, 128, 256, "coverage", 0.9),
    "d128_bs64_cov": (4, 1, 1152, 128, 64, 192, "coverage", 0.8),
    "batch3_gqa2_keep": (4, 2, 1024, 128, 128, 256, "keep", 0.4, 3),
    # B*Hkv = 8: the attention's work order gives each XCD whole KV heads
    "gqa2_8kv_xcd": (16, 8, 1024, 128, 128, 256, "keep", 0.3),
}


def _inputs(name):
    Hq, Hkv, N, d, Bs, S, mode, param = CASES[name][:8]
    batch = CASES[name][8] if len(CASES[name]) > 8 else 1
    w = pbs_synth.WORKLOADS["gqa_8k"].scaled(name=name, batch=batch, heads_q=Hq, heads_kv=Hkv,
                                             seq_len=N, head_dim=d, block=Bs, segment=S, mode=mode,
                                             params=(param,), seed=zlib.crc32(name.encode()) % 100000)
    return w, pbs_synth.make_inputs(w)


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    name = request.param
    w, inp = _inputs(name)
    scale = oracle.default_scale(w.head_dim)
    mode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], block=w.block, segment=w.segment,
                         scale=scale, mode=mode, param=w.params[0])
    ref["dense_o"], ref["dense_lse"] = oracle.dense_causal(inp["q"], inp["k"], inp["v"],
                                                           block=w.block, scale=scale)
    sh = shape(w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, w.block, w.segment)
    g = dict(q=dev_bf16(inp["q"]), k=dev_bf16(inp["k"]), v=dev_bf16(inp["v"]))
    say(f"case {name}: shape {CASES[name]}")
    return dict(name=name, w=w, inp=inp, ref=ref, scale=scale, sh=sh, g=g,
                cmode=P.PBS_SELECT_KEEP_RATIO if w.mode == "keep" else P.PBS_SELECT_COVERAGE)


def test_scores(case):
    say(case["name"], "pbs_score")
    s = run_score(case["sh"], case["g"]["q"], case["g"]["k"], case["scale"]).cpu().numpy()
    ref = case["ref"]["scores"].astype(np.float64)
    rel = np.abs(s - ref) / np.abs(ref)
    say(f"scores max rel err {rel.max():.2e}")
    assert rel.max() <= SCORE_RTOL
    S = case["w"].segment
    sums = s.astype(np.float64).reshape(s.shape[0], s.shape[1], -1, S).sum(-1)
    assert np.allclose(sums, 1.0, atol=1e-4)


def test_permute_bitexact_given_oracle_scores(case):
    say(case["name"], "pbs_permute")
    sh, ref = case["sh"], case["ref"]
    perm, kp, vp, kpool, mpos, pinv = run_permute(sh, dev(ref["scores"]), case["g"]["k"], case["g"]["v"])
    assert np.array_equal(pinv.cpu().numpy(), inverse_of(ref["perm"]))
    assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    assert np.array_equal(host_bits(kp), ref["k_perm"])
    assert np.array_equal(host_bits(vp), ref["v_perm"])
    B, H, N = ref["perm"].shape
    Bs = sh.block
    assert np.array_equal(mpos.cpu().numpy(), ref["perm"].reshape(B, H, N // Bs, Bs).min(-1))
    kbar = oracle.pooled_blocks(ref["k_perm"], Bs)
    assert np.allclose(kpool.cpu().numpy(), kbar, rtol=1e-5, atol=1e-6)


def test_select_bitexact_given_oracle_probabilities(case):
    say(case["name"], "pbs_block_select (probabilities in)")
    ref = case["ref"]
    w = case["w"]
    counts, idx = run_select(case["sh"], None, None, None, case["scale"], case["cmode"],
                             w.params[0], blk_scores=dev(ref["P"]), flags=P.PBS_FLAG_SCORES_IN)
    assert lists_equal(counts.cpu().numpy(), idx.cpu().numpy(), ref["counts"], ref["idx"])


def test_select_keep_first_bitexact(case):
    """PBS_FLAG_KEEP_FIRST (key block 0 ranked first) against the oracle's keep_first selection,
    both given the oracle's float32 block probabilities; then the whole attention with those
    lists against the oracle."""
    say(case["name"], "pbs_block_select keep-first (probabilities in)")
    ref, w, sh = case["ref"], case["w"], case["sh"]
    mode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    rc, ri = oracle.select_blocks(ref["P"], block=w.block, segment=w.segment, mode=mode,
                                  param=w.params[0], keep_first=True)
    counts, idx = run_select(sh, None, None, None, case["scale"], case["cmode"], w.params[0],
                             blk_scores=dev(ref["P"]),
                             flags=P.PBS_FLAG_SCORES_IN | P.PBS_FLAG_KEEP_FIRST)
    assert lists_equal(counts.cpu().numpy(), idx.cpu().numpy(), rc, ri)
    c = counts.cpu().numpy()
    first = idx.cpu().numpy()[..., 0]
    assert ((c == 0) | (first == 0)).all()
    o, _ = run_attn(sh, case["g"]["q"], dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]),
                    dev(ref["perm"]), dev(inverse_of(ref["perm"])), counts, idx, case["scale"],
                    want_lse=False)
    oo, _ = oracle.attention(case["inp"]["q"], case["inp"]["k"], case["inp"]["v"], block=w.block,
                             segment=w.segment, scale=case["scale"], perm=ref["perm"], counts=rc,
                             idx=ri)
    check_attn(o.float().cpu().numpy(), oo, f"{case['name']} keep-first attention")


def test_block_probabilities(case):
    say(case["name"], "pbs_block_select (probabilities computed)")
    ref, sh, w = case["ref"], case["sh"], case["w"]
    kp = dev_bf16(ref["k_perm"])
    nb = w.seq_len // w.block
    Pg = torch.zeros((w.batch, w.heads_q, nb, nb), dtype=torch.float32, device="cuda")
    for k_perm, k_pool in ((kp, None), (None, dev(oracle.pooled_blocks(ref["k_perm"], w.block).astype(np.float32)))):
        counts, idx = run_select(sh, case["g"]["q"], k_perm, k_pool, case["scale"], case["cmode"],
                                 w.params[0], blk_scores=Pg)
        got = Pg.cpu().numpy().astype(np.float64)
        want = ref["P"].astype(np.float64)
        cand = want > 0
        assert np.array_equal(got > 0, cand)
        rel = np.abs(got - want)[cand] / want[cand]
        say(f"P max rel err {rel.max() if rel.size else 0:.2e}")
        assert rel.size == 0 or rel.max() <= SCORE_RTOL
        agree = np.mean(counts.cpu().numpy() == ref["counts"])
        say(f"count agreement {agree:.4f}")


def test_attention_given_oracle_lists(case):
    say(case["name"], "pbs_attn_fwd (oracle permutation and lists)")
    ref, sh = case["ref"], case["sh"]
    o, lse = run_attn(sh, case["g"]["q"], dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]),
                      dev(ref["perm"]), dev(inverse_of(ref["perm"])), dev(ref["counts"]),
                      dev(ref["idx"]), case["scale"])
    check_attn(o.float().cpu().numpy(), ref["o"], f"{case['name']} attention")
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() < 1e-3


def test_hybrid_own_segment_natural(case):
    """pbs_attn_fwd_hybrid: kept blocks from the permuted copies, own segment from the original
    keys in natural order; the visible key set of every row is the same, so the oracle's output
    is the reference (Lemma 3.1 of the sciencestack.ai page)."""
    say(case["name"], "pbs_attn_fwd_hybrid (oracle permutation and lists)")
    ref, sh, g = case["ref"], case["sh"], case["g"]
    o = torch.empty_like(g["q"])
    lse = torch.empty(g["q"].shape[:3], dtype=torch.float32, device="cuda")
    P.pbs_attn_fwd_hybrid(sh, g["q"], dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]), g["k"],
                          g["v"], dev(ref["counts"]), dev(ref["idx"]), case["scale"], o, lse)
    torch.cuda.synchronize()
    check_attn(o.float().cpu().numpy(), ref["o"], f"{case['name']} hybrid attention")
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() < 1e-3


def test_permuted_queries(case):
    """The query-permutation variant: queries gathered with their KV head's permutation
    (bit-exact against the oracle), selection on the permuted queries (bit-exact given the
    oracle's float32 block probabilities), attention with rows written back at their original
    positions against the oracle (sciencestack.ai page, Lemma 3.2 / Theorem 3.3)."""
    say(case["name"], "permuted queries")
    ref, w, sh, g, inp = case["ref"], case["w"], case["sh"], case["g"], case["inp"]
    perm = ref["perm"]
    qp_ref = oracle.permute_queries(inp["q"], perm)
    qp = torch.empty_like(g["q"])
    P.pbs_permute_queries(sh, dev(perm), g["q"], qp)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qp), qp_ref)
    mode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    Pq = oracle.block_probabilities(qp_ref, ref["k_perm"], block=w.block, segment=w.segment,
                                    scale=case["scale"])
    rc, ri = oracle.select_blocks(Pq, block=w.block, segment=w.segment, mode=mode, param=w.params[0])
    counts, idx = run_select(sh, None, None, None, case["scale"], case["cmode"], w.params[0],
                             blk_scores=dev(Pq), flags=P.PBS_FLAG_SCORES_IN)
    assert lists_equal(counts.cpu().numpy(), idx.cpu().numpy(), rc, ri)
    oo, ol = oracle.attention_permuted_queries(qp_ref, inp["k"], inp["v"], block=w.block,
                                               segment=w.segment, scale=case["scale"], perm=perm,
                                               counts=rc, idx=ri)
    B, H, N = perm.shape
    minpos = perm.reshape(B, H, N // w.block, w.block).min(-1).astype(np.int32)
    for mp in (dev(minpos), None):
        o = torch.empty_like(g["q"])
        lse = torch.empty(g["q"].shape[:3], dtype=torch.float32, device="cuda")
        P.pbs_attn_fwd_permuted_queries(sh, qp, dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]),
                                        dev(perm), mp, counts, idx, case["scale"], o, lse)
        torch.cuda.synchronize()
        check_attn(o.float().cpu().numpy(), oo, f"{case['name']} permuted-query attention")
        assert np.abs(lse.cpu().numpy() - ol).max() < 1e-3


def test_permuted_queries_keep_one_is_dense(case):
    """Theorem 3.3 on the GPU: permuted queries and keys with every candidate kept, rows put
    back in original order, equal plain causal attention."""
    say(case["name"], "permuted queries, keep 1")
    ref, w, sh, g, inp = case["ref"], case["w"], case["sh"], case["g"], case["inp"]
    perm = ref["perm"]
    qp = torch.empty_like(g["q"])
    P.pbs_permute_queries(sh, dev(perm), g["q"], qp)
    counts, idx = run_select(sh, qp, dev_bf16(ref["k_perm"]), None, case["scale"],
                             P.PBS_SELECT_KEEP_RATIO, 1.0)
    o = torch.empty_like(g["q"])
    P.pbs_attn_fwd_permuted_queries(sh, qp, dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]),
                                    dev(perm), None, counts, idx, case["scale"], o, None)
    torch.cuda.synchronize()
    check_attn(o.float().cpu().numpy(), ref["dense_o"], f"{case['name']} permuted queries keep 1")


def test_dense_causal(case):
    say(case["name"], "pbs_attn_fwd dense")
    ref, sh = case["ref"], case["sh"]
    o, lse = run_attn(sh, case["g"]["q"], case["g"]["k"], case["g"]["v"], None, None, None, None,
                      case["scale"])
    check_attn(o.float().cpu().numpy(), ref["dense_o"], f"{case['name']} dense")
    assert np.abs(lse.cpu().numpy() - ref["dense_lse"]).max() < 1e-3


def test_identity_order_block_sparse(case):
    """perm = NULL: plain block-sparse attention over the natural key order."""
    say(case["name"], "pbs_attn_fwd identity order")
    inp, sh, w = case["inp"], case["sh"], case["w"]
    mode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    Pn = oracle.block_probabilities(inp["q"], inp["k"], block=w.block, segment=w.segment,
                                    scale=case["scale"])
    cn, ixn = oracle.select_blocks(Pn, block=w.block, segment=w.segment, mode=mode, param=w.params[0])
    on, _ = oracle.attention(inp["q"], inp["k"], inp["v"], block=w.block, segment=w.segment,
                             scale=case["scale"], perm=None, counts=cn, idx=ixn)
    o, _ = run_attn(sh, case["g"]["q"], case["g"]["k"], case["g"]["v"], None, None, dev(cn),
                    dev(ixn), case["scale"])
    check_attn(o.float().cpu().numpy(), on, f"{case['name']} identity-order")


def test_end_to_end(case):
    """Whole GPU pipeline against the whole oracle pipeline.  Near-equal float32 scores may be
    ordered differently by the two sides (rounding), so the permutation and the lists are
    compared by agreement rate; the output must still meet the attention bar."""
    say(case["name"], "end-to-end prefill")
    ref, w, g = case["ref"], case["w"], case["g"]
    kw = {"keep": w.params[0]} if w.mode == "keep" else {"coverage": w.params[0]}
    bufs = P.prefill(g["q"], g["k"], g["v"], block=w.block, segment=w.segment, scale=case["scale"], **kw)
    torch.cuda.synchronize()
    perm_agree = float(np.mean(bufs.perm.cpu().numpy() == ref["perm"]))
    cnt_agree = float(np.mean(bufs.counts.cpu().numpy() == ref["counts"]))
    say(f"perm agreement {perm_agree:.4f}, count agreement {cnt_agree:.4f}")
    check_attn(bufs.o.float().cpu().numpy(), ref["o"], f"{case['name']} end-to-end")
    # a flip needs two keys whose float32 scores round differently on the two sides (scores
    # agree to ~1e-6 relative), so nearly every slot and every count must agree
    assert perm_agree >= 0.99 and cnt_agree >= 0.98, (perm_agree, cnt_agree)
