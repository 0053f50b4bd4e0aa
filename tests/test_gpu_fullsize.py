"""Parity at the full sizes of the benchmark workloads, in the launch configuration bench.py
times (the same entry points, shapes and parameters), on outputs the oracle can afford:

  * scores: every key, against the float64 oracle (relative 1e-4);
  * permutation, permuted K/V and block min-positions: every slot, bit-exact, given the oracle's
    float32 scores;
  * block selection: every row, bit-exact, given the oracle's float32 block probabilities;
  * attention with the oracle's permutation and lists: sampled query blocks (the first and last
    block of every segment and every 16th block) of every query head, max-abs 2e-2 / mean-abs
    2e-3, through pbs_attn_fwd and through pbs_attn_fwd_hybrid;
  * the query-permutation variant: query gather and selection bit-exact, attention on sampled
    permuted query blocks;
  * the whole GPU pipeline end to end: the same sampled blocks of every query head against the
    whole oracle pipeline, with the permutation and the kept-block counts agreeing almost
    everywhere (they can differ only where the two sides' float32 scores round a near-tie
    differently).

Each workload is generated once per module (seconds) and the oracle stages cost tens of seconds
at 128K on the host."""
import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import oracle
import pbs_synth
from gpu_helpers import (check_attn, dev, dev_bf16, host_bits, inverse_of, lists_equal, run_attn,
                         run_permute, run_score, run_select, say)

pytestmark = pytest.mark.gpu

FULL = ["gqa_8k", "gqa_32k_cov", "gqa28_64k_sweep", "gqa_128k"]


def _sample_blocks(w, heads):
    nb, bps = w.seq_len // w.block, w.segment // w.block
    blocks = set(range(0, nb, 16))
    for s0 in range(0, nb, bps):
        blocks.update((s0, s0 + bps - 1))
    return [(0, g, i) for g in heads for i in sorted(blocks)]


@pytest.fixture(scope="module", params=FULL)
def full(request):
    name = request.param
    w = pbs_synth.WORKLOADS[name]
    say(f"full-size workload {name}: generating inputs")
    inp = pbs_synth.make_inputs(w)
    scale = oracle.default_scale(w.head_dim)
    sh = P.make_shape(w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, w.block, w.segment)
    g = dict(q=dev_bf16(inp["q"]), k=dev_bf16(inp["k"]), v=dev_bf16(inp["v"]))
    say(f"{name}: oracle scores / permutation / block probabilities")
    ref = {}
    ref["scores"] = oracle.key_scores(inp["q"], inp["k"], block=w.block, segment=w.segment, scale=scale)
    ref["perm"] = oracle.segment_permutation(ref["scores"], segment=w.segment)
    ref["k_perm"] = oracle.apply_permutation(inp["k"], ref["perm"])
    ref["v_perm"] = oracle.apply_permutation(inp["v"], ref["perm"])
    ref["P"] = oracle.block_probabilities(inp["q"], ref["k_perm"], block=w.block, segment=w.segment,
                                          scale=scale)
    yield dict(name=name, w=w, inp=inp, scale=scale, sh=sh, g=g, ref=ref)
    del g
    torch.cuda.empty_cache()


def test_full_scores(full):
    say(full["name"], "pbs_score")
    s = run_score(full["sh"], full["g"]["q"], full["g"]["k"], full["scale"]).cpu().numpy()
    ref = full["ref"]["scores"].astype(np.float64)
    rel = float((np.abs(s - ref) / ref).max())
    say(f"scores max rel err {rel:.2e}")
    assert rel <= 1e-4


def test_full_permute_bitexact(full):
    say(full["name"], "pbs_permute")
    ref, sh = full["ref"], full["sh"]
    perm, kp, vp, kpool, mpos, pinv = run_permute(sh, dev(ref["scores"]), full["g"]["k"], full["g"]["v"])
    assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    assert np.array_equal(pinv.cpu().numpy(), inverse_of(ref["perm"]))
    assert np.array_equal(host_bits(kp), ref["k_perm"])
    assert np.array_equal(host_bits(vp), ref["v_perm"])
    B, H, N = ref["perm"].shape
    Bs = sh.block
    assert np.array_equal(mpos.cpu().numpy(), ref["perm"].reshape(B, H, N // Bs, Bs).min(-1))
    full["gpu_kp"], full["gpu_vp"] = kp, vp


def test_full_select_bitexact(full):
    """Every parameter the workload is evaluated at (the sweep's five keep ratios included)."""
    w = full["w"]
    mode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    cmode = P.PBS_SELECT_KEEP_RATIO if w.mode == "keep" else P.PBS_SELECT_COVERAGE
    for param in w.params:
        say(full["name"], f"pbs_block_select param {param}")
        rc, ri = oracle.select_blocks(full["ref"]["P"], block=w.block, segment=w.segment, mode=mode,
                                      param=param)
        counts, idx = run_select(full["sh"], None, None, None, full["scale"], cmode, param,
                                 blk_scores=dev(full["ref"]["P"]), flags=P.PBS_FLAG_SCORES_IN)
        assert lists_equal(counts.cpu().numpy(), idx.cpu().numpy(), rc, ri), param


def test_full_attention_sampled(full):
    w, ref, inp = full["w"], full["ref"], full["inp"]
    mode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    heads = list(range(w.heads_q))
    for param in sorted({w.params[0], w.params[-1]}):
        say(full["name"], f"attention, param {param}")
        rc, ri = oracle.select_blocks(ref["P"], block=w.block, segment=w.segment, mode=mode, param=param)
        kp = full.get("gpu_kp") if full.get("gpu_kp") is not None else dev_bf16(ref["k_perm"])
        vp = full.get("gpu_vp") if full.get("gpu_vp") is not None else dev_bf16(ref["v_perm"])
        o, lse = run_attn(full["sh"], full["g"]["q"], kp, vp, dev(ref["perm"]), dev(inverse_of(ref["perm"])),
                          dev(rc), dev(ri), full["scale"])
        samples = _sample_blocks(w, heads)
        oo, ol = oracle.attention(inp["q"], inp["k"], inp["v"], block=w.block, segment=w.segment,
                                  scale=full["scale"], perm=ref["perm"], counts=rc, idx=ri,
                                  qblocks=samples)
        og = o.float().cpu().numpy()
        lg = lse.cpu().numpy()
        got = np.stack([og[b, g, i * w.block:(i + 1) * w.block] for b, g, i in samples])
        gl = np.stack([lg[b, g, i * w.block:(i + 1) * w.block] for b, g, i in samples])
        check_attn(got, oo, f"{full['name']} attention param {param} ({len(samples)} blocks)")
        assert np.abs(gl - ol).max() < 1e-3
        # the hybrid entry point (own segment from the original K/V in natural order), same lists
        oh = torch.empty_like(o)
        lh = torch.empty_like(lse)
        P.pbs_attn_fwd_hybrid(full["sh"], full["g"]["q"], kp, vp, full["g"]["k"], full["g"]["v"],
                              dev(rc), dev(ri), full["scale"], oh, lh)
        torch.cuda.synchronize()
        ohg, lhg = oh.float().cpu().numpy(), lh.cpu().numpy()
        got = np.stack([ohg[b, g, i * w.block:(i + 1) * w.block] for b, g, i in samples])
        gl = np.stack([lhg[b, g, i * w.block:(i + 1) * w.block] for b, g, i in samples])
        check_attn(got, oo, f"{full['name']} hybrid attention param {param}")
        assert np.abs(gl - ol).max() < 1e-3


def test_full_permuted_queries_sampled(full):
    """The query-permutation variant at full size, in the launch configuration bench.py times:
    the query gather bit-exact on every row, the selection on the permuted queries bit-exact
    given the oracle's float32 block probabilities, and the attention (rows written back at
    their original positions) on sampled permuted query blocks."""
    w, ref, inp, g = full["w"], full["ref"], full["inp"], full["g"]
    say(full["name"], "permuted queries")
    perm = ref["perm"]
    qp_ref = oracle.permute_queries(inp["q"], perm)
    qp = torch.empty_like(g["q"])
    P.pbs_permute_queries(full["sh"], dev(perm), g["q"], qp)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qp), qp_ref)
    mode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    Pq = oracle.block_probabilities(qp_ref, ref["k_perm"], block=w.block, segment=w.segment,
                                    scale=full["scale"])
    rc, ri = oracle.select_blocks(Pq, block=w.block, segment=w.segment, mode=mode, param=w.params[0])
    counts, idx = run_select(full["sh"], None, None, None, full["scale"],
                             P.PBS_SELECT_KEEP_RATIO if w.mode == "keep" else P.PBS_SELECT_COVERAGE,
                             w.params[0], blk_scores=dev(Pq), flags=P.PBS_FLAG_SCORES_IN)
    assert lists_equal(counts.cpu().numpy(), idx.cpu().numpy(), rc, ri)
    B, H, N = perm.shape
    minpos = perm.reshape(B, H, N // w.block, w.block).min(-1).astype(np.int32)
    o = torch.empty_like(g["q"])
    P.pbs_attn_fwd_permuted_queries(full["sh"], qp, dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]),
                                    dev(perm), dev(minpos), counts, idx, full["scale"], o, None)
    torch.cuda.synchronize()
    G = w.heads_q // w.heads_kv
    samples = _sample_blocks(w, sorted({0, w.heads_q - 1}))
    oo, _ = oracle.attention_permuted_queries(qp_ref, inp["k"], inp["v"], block=w.block,
                                              segment=w.segment, scale=full["scale"], perm=perm,
                                              counts=rc, idx=ri, qblocks=samples)
    og = o.float().cpu().numpy()
    got = np.stack([og[b, gg, perm[b, gg // G, i * w.block:(i + 1) * w.block]] for b, gg, i in samples])
    check_attn(got, oo, f"{full['name']} permuted-query attention ({len(samples)} blocks)")


def test_full_end_to_end_sampled(full):
    """The whole GPU pipeline (the bench's step) against the whole oracle pipeline."""
    w, ref, inp, g = full["w"], full["ref"], full["inp"], full["g"]
    param = w.params[0]
    say(full["name"], "end-to-end")
    kw = {"keep": param} if w.mode == "keep" else {"coverage": param}
    bufs = P.prefill(g["q"], g["k"], g["v"], block=w.block, segment=w.segment, scale=full["scale"], **kw)
    torch.cuda.synchronize()
    mode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    rc, ri = oracle.select_blocks(ref["P"], block=w.block, segment=w.segment, mode=mode, param=param)
    heads = list(range(w.heads_q))
    samples = _sample_blocks(w, heads)
    oo, _ = oracle.attention(inp["q"], inp["k"], inp["v"], block=w.block, segment=w.segment,
                             scale=full["scale"], perm=ref["perm"], counts=rc, idx=ri, qblocks=samples)
    og = bufs.o.float().cpu().numpy()
    got = np.stack([og[b, gg, i * w.block:(i + 1) * w.block] for b, gg, i in samples])
    perm_agree = float(np.mean(bufs.perm.cpu().numpy() == ref["perm"]))
    cnt_agree = float(np.mean(bufs.counts.cpu().numpy() == rc))
    say(f"perm agreement {perm_agree:.4f}, count agreement {cnt_agree:.4f}")
    check_attn(got, oo, f"{full['name']} end-to-end ({len(samples)} blocks)")
    assert perm_agree >= 0.995 and cnt_agree >= 0.99, (perm_agree, cnt_agree)
