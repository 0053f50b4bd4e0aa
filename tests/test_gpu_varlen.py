"""Packed variable-length sequences (pbs_score_varlen, pbs_block_select_varlen, then the unchanged
permutation and attention) against the oracle's per-sequence definition, stage by stage, plus
two equivalences on the GPU alone: equal lengths give the batched result bit for bit, and the
token-major packed layout gives the head-major one bit for bit.

Cases mix sequence lengths, both head dims and block sizes, a segment of 192 tokens (not a
multiple of the 256-key workgroup of the score reduction) and segments of a single block."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import oracle
import pbs_synth
from gpu_helpers import check_attn, dev, dev_bf16, host_bits, inverse_of, lists_equal, say

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-4

# name -> (Hq, Hkv, d, Bs, S, lengths, mode, param)
CASES = {
    "mixed_bs128": (8, 2, 128, 128, 512, [1024, 512, 2048, 1536], "keep", 0.3),
    "d64_bs64_S192_cov": (4, 2, 64, 64, 192, [384, 192, 576, 192], "coverage", 0.9),
    "S64_gqa4": (4, 1, 128, 64, 64, [64, 128, 256, 64, 192], "keep", 0.5),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    name = request.param
    Hq, Hkv, d, Bs, S, lens, mode, param = CASES[name]
    T = int(sum(lens))
    w = pbs_synth.WORKLOADS["gqa_8k"].scaled(name=name, heads_q=Hq, heads_kv=Hkv, seq_len=T,
                                             head_dim=d, block=Bs, segment=S, mode=mode,
                                             params=(param,),
                                             seed=zlib.crc32(name.encode()) % 100000 + 11)
    inp = pbs_synth.make_inputs(w)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    scale = oracle.default_scale(d)
    omode = oracle.KEEP if mode == "keep" else oracle.COVERAGE
    ref = oracle.prefill_varlen(inp["q"], inp["k"], inp["v"], cu, block=Bs, segment=S,
                                scale=scale, mode=omode, param=param)
    sh = P.make_shape(1, Hq, Hkv, T, d, Bs, S)
    g = dict(q=dev_bf16(inp["q"]), k=dev_bf16(inp["k"]), v=dev_bf16(inp["v"]))
    say(f"case {name}: lengths {lens}")
    return dict(name=name, w=w, inp=inp, ref=ref, scale=scale, sh=sh, g=g, cu=cu,
                cu_dev=dev(cu), n=len(lens),
                cmode=P.PBS_SELECT_KEEP_RATIO if mode == "keep" else P.PBS_SELECT_COVERAGE)


def _ws(sh):
    return torch.empty(max(P.pbs_workspace_bytes(sh), 16), dtype=torch.uint8, device="cuda")


def _select(c, q, k_perm, k_pool, blk_scores=None, flags=0):
    sh, w = c["sh"], c["w"]
    nb = w.seq_len // w.block
    mo = max(P.pbs_max_offdiag(sh), 1)
    counts = torch.full((1, w.heads_q, nb), -7, dtype=torch.int32, device="cuda")
    idx = torch.full((1, w.heads_q, nb, mo), -1, dtype=torch.int32, device="cuda")
    P.pbs_block_select_varlen(sh, c["cu_dev"], c["n"], q, k_perm, k_pool, c["scale"], c["cmode"],
                              w.params[0], blk_scores, flags, counts, idx, _ws(sh))
    torch.cuda.synchronize()
    return counts, idx


def test_varlen_scores(case):
    sh, w = case["sh"], case["w"]
    s = torch.empty((1, w.heads_kv, w.seq_len), dtype=torch.float32, device="cuda")
    P.pbs_score_varlen(sh, case["cu_dev"], case["n"], case["g"]["q"], case["g"]["k"],
                       case["scale"], s, _ws(sh))
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    ref = case["ref"]["scores"].astype(np.float64)
    rel = np.abs(s - ref) / np.abs(ref)
    say(f"{case['name']} varlen scores max rel err {rel.max():.2e}")
    assert rel.max() <= SCORE_RTOL
    sums = s.astype(np.float64).reshape(1, w.heads_kv, -1, w.segment).sum(-1)
    assert np.allclose(sums, 1.0, atol=1e-4)


def test_varlen_permute_bitexact_given_oracle_scores(case):
    sh, ref, w = case["sh"], case["ref"], case["w"]
    nb = w.seq_len // w.block
    perm = torch.empty((1, w.heads_kv, w.seq_len), dtype=torch.int32, device="cuda")
    kp, vp = torch.empty_like(case["g"]["k"]), torch.empty_like(case["g"]["v"])
    mpos = torch.empty((1, w.heads_kv, nb), dtype=torch.int32, device="cuda")
    pinv = torch.empty_like(perm)
    P.pbs_permute(sh, dev(ref["scores"]), case["g"]["k"], case["g"]["v"], perm, kp, vp, None, mpos,
                  pinv)
    torch.cuda.synchronize()
    assert np.array_equal(perm.cpu().numpy(), ref["perm"])
    assert np.array_equal(pinv.cpu().numpy(), inverse_of(ref["perm"]))
    assert np.array_equal(host_bits(kp), ref["k_perm"])
    assert np.array_equal(host_bits(vp), ref["v_perm"])


def test_varlen_select_bitexact_given_oracle_probabilities(case):
    ref = case["ref"]
    counts, idx = _select(case, None, None, None, blk_scores=dev(ref["P"]),
                          flags=P.PBS_FLAG_SCORES_IN)
    assert lists_equal(counts.cpu().numpy(), idx.cpu().numpy(), ref["counts"], ref["idx"])


def test_varlen_block_probabilities(case):
    ref, w = case["ref"], case["w"]
    nb = w.seq_len // w.block
    Pg = torch.full((1, w.heads_q, nb, nb), 7.0, dtype=torch.float32, device="cuda")
    _select(case, case["g"]["q"], dev_bf16(ref["k_perm"]), None, blk_scores=Pg)
    got = Pg.cpu().numpy().astype(np.float64)
    want = ref["P"].astype(np.float64)
    cand = want > 0
    assert np.array_equal(got > 0, cand)           # zero off the candidates and across sequences
    assert (got[~cand] == 0).all()
    rel = np.abs(got - want)[cand] / want[cand]
    say(f"{case['name']} varlen P max rel err {rel.max() if rel.size else 0:.2e}")
    assert rel.size == 0 or rel.max() <= SCORE_RTOL


def test_varlen_attention_given_oracle_lists(case):
    ref, sh, w = case["ref"], case["sh"], case["w"]
    o = torch.empty_like(case["g"]["q"])
    lse = torch.empty(o.shape[:3], dtype=torch.float32, device="cuda")
    P.pbs_attn_fwd(sh, case["g"]["q"], dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]),
                   dev(ref["perm"]), dev(inverse_of(ref["perm"])), dev(ref["counts"]),
                   dev(ref["idx"]), case["scale"], o, lse)
    torch.cuda.synchronize()
    check_attn(o.float().cpu().numpy(), ref["o"], f"{case['name']} varlen attention")
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() < 1e-3


def test_varlen_end_to_end(case):
    """The four calls on the GPU; lists against the oracle's by agreement (fp32 rounding can flip
    near-ties), the attention against the oracle given the GPU's own permutation and lists."""
    w, inp = case["w"], case["inp"]
    kw = {"keep": w.params[0]} if w.mode == "keep" else {"coverage": w.params[0]}
    out = P.prefill_varlen(case["g"]["q"], case["g"]["k"], case["g"]["v"], case["cu_dev"],
                           block=w.block, segment=w.segment, scale=case["scale"], **kw)
    torch.cuda.synchronize()
    agree = float(np.mean(out.counts.cpu().numpy() == case["ref"]["counts"]))
    say(f"{case['name']} varlen end to end: count agreement {agree:.4f}")
    assert agree >= 0.9
    perm = out.perm.cpu().numpy().astype(np.int64)
    counts, idx = out.counts.cpu().numpy(), out.idx.cpu().numpy()
    # no list leaves its query's sequence
    cu = case["cu"]
    for a, b in zip(cu[:-1], cu[1:]):
        i0, i1 = a // w.block, b // w.block
        c, ix = counts[0, :, i0:i1], idx[0, :, i0:i1]
        live = np.arange(ix.shape[-1])[None, None, :] < c[..., None]
        assert (((ix >= i0) & (ix < i1)) | ~live).all()
    oo, _ = oracle.attention(inp["q"], inp["k"], inp["v"], block=w.block, segment=w.segment,
                             scale=case["scale"], perm=perm, counts=counts, idx=idx)
    check_attn(out.o.float().cpu().numpy(), oo, f"{case['name']} varlen end-to-end attention")


def _pack(t):
    B, H, L, d = t.shape
    return t.permute(1, 0, 2, 3).reshape(1, H, B * L, d).contiguous()


def test_varlen_equal_lengths_is_batch():
    """Three sequences of 2048 tokens: packed with boundaries == batch of three, bit for bit."""
    w = pbs_synth.WORKLOADS["gqa_8k"].scaled(name="varlen_batch", batch=3, heads_q=8, heads_kv=2,
                                             seq_len=2048, segment=512, seed=5151)
    inp = pbs_synth.make_inputs(w)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    bat = P.prefill(q, k, v, block=w.block, segment=w.segment, keep=0.3)
    cu = dev(np.array([0, 2048, 4096, 6144], dtype=np.int32))
    pk = P.prefill_varlen(_pack(q), _pack(k), _pack(v), cu, block=w.block, segment=w.segment,
                          keep=0.3)
    torch.cuda.synchronize()
    L, nbl = 2048, 2048 // w.block
    for b in range(3):
        sl = slice(b * L, (b + 1) * L)
        assert torch.equal(pk.scores[0, :, sl], bat.scores[b])
        assert torch.equal(pk.perm[0, :, sl], bat.perm[b] + b * L)
        assert torch.equal(pk.o[0, :, sl].view(torch.int16), bat.o[b].view(torch.int16))
        assert torch.equal(pk.lse[0, :, sl], bat.lse[b])
        c_b = bat.counts[b].cpu().numpy()
        i_b = bat.idx[b].cpu().numpy()
        c_p = pk.counts[0, :, b * nbl:(b + 1) * nbl].cpu().numpy()
        i_p = pk.idx[0, :, b * nbl:(b + 1) * nbl].cpu().numpy()
        assert lists_equal(c_p[None], i_p[None] - b * nbl, c_b[None], i_b[None])
    say("varlen equal lengths: bit-identical to the batch of three")


def test_varlen_token_major_bit_identical(case):
    """The packed row token-major ([T, H, d], the FlashAttention varlen layout) against
    head-major, bit for bit."""
    w = case["w"]
    kw = {"keep": w.params[0]} if w.mode == "keep" else {"coverage": w.params[0]}
    tok = lambda t: t.transpose(1, 2).contiguous()
    head = P.prefill_varlen(case["g"]["q"], case["g"]["k"], case["g"]["v"], case["cu_dev"],
                            block=w.block, segment=w.segment, **kw)
    tm = P.prefill_varlen(tok(case["g"]["q"]), tok(case["g"]["k"]), tok(case["g"]["v"]),
                          case["cu_dev"], block=w.block, segment=w.segment,
                          layout=P.PBS_LAYOUT_BNHD, **kw)
    torch.cuda.synchronize()
    assert torch.equal(head.scores, tm.scores)
    assert torch.equal(head.perm, tm.perm)
    assert lists_equal(head.counts.cpu().numpy(), head.idx.cpu().numpy(),
                       tm.counts.cpu().numpy(), tm.idx.cpu().numpy())
    assert torch.equal(head.o.view(torch.int16), tok(tm.o).view(torch.int16))


def test_varlen_hybrid_given_oracle_lists(case):
    """pbs_attn_fwd_hybrid on the packed row: the own segment from the original keys in natural
    order (a segment never leaves its sequence), the kept blocks from the permuted copies."""
    ref, sh = case["ref"], case["sh"]
    g = case["g"]
    o = torch.empty_like(g["q"])
    P.pbs_attn_fwd_hybrid(sh, g["q"], dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]), g["k"],
                          g["v"], dev(ref["counts"]), dev(ref["idx"]), case["scale"], o, None)
    torch.cuda.synchronize()
    check_attn(o.float().cpu().numpy(), ref["o"], f"{case['name']} varlen hybrid attention")


def test_varlen_permuted_queries(case):
    """The query-permutation variant on the packed row: queries moved with their KV head's
    permutation, selection (varlen) on them given the oracle's probabilities of the moved queries,
    attention with rows written back at their original positions, against the oracle."""
    ref, w, sh, g, inp = case["ref"], case["w"], case["sh"], case["g"], case["inp"]
    perm = ref["perm"]
    qp_ref = oracle.permute_queries(inp["q"], perm)
    qp = torch.empty_like(g["q"])
    P.pbs_permute_queries(sh, dev(perm), g["q"], qp)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qp), qp_ref)
    # the oracle's probabilities of the moved queries, sequence by sequence (block-diagonal)
    omode = oracle.KEEP if w.mode == "keep" else oracle.COVERAGE
    nb = w.seq_len // w.block
    Pq = np.zeros((1, w.heads_q, nb, nb), np.float32)
    width = ref["idx"].shape[-1]
    rc = np.zeros((1, w.heads_q, nb), np.int32)
    ri = np.full((1, w.heads_q, nb, width), -1, np.int32)
    cu = case["cu"]
    for a, b in zip(cu[:-1], cu[1:]):
        i0, i1 = a // w.block, b // w.block
        Ps = oracle.block_probabilities(qp_ref[:, :, a:b], ref["k_perm"][:, :, a:b],
                                        block=w.block, segment=w.segment, scale=case["scale"])
        c_s, x_s = oracle.select_blocks(Ps, block=w.block, segment=w.segment, mode=omode,
                                        param=w.params[0])
        Pq[:, :, i0:i1, i0:i1] = Ps
        rc[:, :, i0:i1] = c_s
        ri[:, :, i0:i1, :x_s.shape[-1]] = np.where(x_s >= 0, x_s + i0, -1)
    counts, idx = _select(case, None, None, None, blk_scores=dev(Pq), flags=P.PBS_FLAG_SCORES_IN)
    assert lists_equal(counts.cpu().numpy(), idx.cpu().numpy(), rc, ri)
    oo, _ = oracle.attention_permuted_queries(qp_ref, inp["k"], inp["v"], block=w.block,
                                              segment=w.segment, scale=case["scale"], perm=perm,
                                              counts=rc, idx=ri)
    o = torch.empty_like(g["q"])
    P.pbs_attn_fwd_permuted_queries(sh, qp, dev_bf16(ref["k_perm"]), dev_bf16(ref["v_perm"]),
                                    dev(perm), None, counts, idx, case["scale"], o, None)
    torch.cuda.synchronize()
    check_attn(o.float().cpu().numpy(), oo, f"{case['name']} varlen permuted-query attention")


def test_varlen_malformed_boundaries_stay_in_bounds():
    """Boundaries that break the documented rules (out of order, past the row, lengths not a
    multiple of S) give unspecified selections, but every access stays inside the tensors: the
    calls complete, the scores are finite and non-negative, and every list entry is a block of an
    earlier segment."""
    w = pbs_synth.WORKLOADS["gqa_8k"].scaled(name="varlen_bad", heads_q=4, heads_kv=1,
                                             seq_len=4096, segment=512, seed=777)
    inp = pbs_synth.make_inputs(w)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    nb, bps = w.seq_len // w.block, w.segment // w.block
    for cu in ([0, 700, 300, 9000, 4096], [0, 4096 + 512, 100], [4000, 1, 2, 3, 4096]):
        out = P.prefill_varlen(q, k, v, dev(np.array(cu, np.int32)), block=w.block,
                               segment=w.segment, keep=0.3)
        torch.cuda.synchronize()
        s = out.scores.cpu().numpy()
        assert np.isfinite(s).all() and (s >= 0).all()
        c, ix = out.counts.cpu().numpy(), out.idx.cpu().numpy()
        seg_first = (np.arange(nb) // bps) * bps
        live = np.arange(ix.shape[-1])[None, None, None, :] < c[..., None]
        assert ((ix >= 0) & (ix < seg_first[None, None, :, None]) | ~live).all()
        assert np.isfinite(out.o.float().cpu().numpy()).all()
        say(f"malformed boundaries {cu}: completed, finite, lists inside earlier segments")
