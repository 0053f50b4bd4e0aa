"""The token-major layout (PBS_LAYOUT_BNHD: Q/O [B, N, Hq, d], K/V [B, N, Hkv, d]) against the
head-major one (PBS_LAYOUT_BHND).

Both run the same kernels with another row addressing and the same arithmetic in the same order,
so every result must be bit-identical once the bf16 tensors are transposed back: scores,
permutation, permuted K/V, pooled keys, block lists, output and log-normalisers, for every entry
point (the four-call path, dense causal, the hybrid attention and the query-permutation variant).
One case is also held against the oracle directly, and the 128K workload is compared whole."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import oracle
import pbs_synth
from gpu_helpers import check_attn, dev, dev_bf16, inverse_of, lists_equal, say

pytestmark = pytest.mark.gpu

# name -> (Hq, Hkv, N, d, Bs, S, mode, param, batch)
CASES = {
    "gqa4_2k_keep": (8, 2, 2048, 128, 128, 512, "keep", 0.3, 1),
    "d64_bs64_cov": (4, 2, 1024, 64, 64, 256, "coverage", 0.9, 2),
    "gqa7_1536_ragged": (14, 2, 1536, 128, 128, 384, "keep", 0.25, 1),
    "d128_bs64_keep_b3": (4, 1, 1152, 128, 64, 192, "keep", 0.5, 3),
}


def _workload(name):
    Hq, Hkv, N, d, Bs, S, mode, param, batch = CASES[name]
    return pbs_synth.WORKLOADS["gqa_8k"].scaled(
        name=name, batch=batch, heads_q=Hq, heads_kv=Hkv, seq_len=N, head_dim=d, block=Bs,
        segment=S, mode=mode, params=(param,), seed=zlib.crc32(name.encode()) % 100000 + 7)


def _tok(t):
    """[B, H, N, d] -> contiguous [B, N, H, d]."""
    return t.transpose(1, 2).contiguous()


def _head(t):
    """[B, N, H, d] -> contiguous [B, H, N, d]."""
    return t.transpose(1, 2).contiguous()


def _same(a, b, what):
    eq = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                     b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    say(f"{what}: {'bit-identical' if eq else 'DIFFERENT'}")
    assert eq, what


def _both_layouts(w, q, k, v, keep_or_cov):
    kw = dict(block=w.block, segment=w.segment)
    kw[keep_or_cov[0]] = keep_or_cov[1]
    head = P.prefill(q, k, v, **kw)
    tok = P.prefill(_tok(q), _tok(k), _tok(v), layout=P.PBS_LAYOUT_BNHD, **kw)
    torch.cuda.synchronize()
    return head, tok


def _compare_prefill(head, tok, name):
    _same(head.scores, tok.scores, f"{name} scores")
    _same(head.perm, tok.perm, f"{name} perm")
    _same(head.k_perm, _head(tok.k_perm), f"{name} k_perm")
    _same(head.v_perm, _head(tok.v_perm), f"{name} v_perm")
    _same(head.k_pool, tok.k_pool, f"{name} k_pool")
    _same(head.blk_minpos, tok.blk_minpos, f"{name} blk_minpos")
    assert lists_equal(head.counts.cpu().numpy(), head.idx.cpu().numpy(),
                       tok.counts.cpu().numpy(), tok.idx.cpu().numpy()), f"{name} block lists"
    _same(head.o, _head(tok.o), f"{name} o")
    _same(head.lse, tok.lse, f"{name} lse")


@pytest.mark.parametrize("name", sorted(CASES))
def test_layouts_bit_identical(name):
    w = _workload(name)
    say(f"case {name}: {CASES[name]}")
    inp = pbs_synth.make_inputs(w)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    sel = ("keep", w.params[0]) if w.mode == "keep" else ("coverage", w.params[0])
    head, tok = _both_layouts(w, q, k, v, sel)
    _compare_prefill(head, tok, name)
    scale = P.default_scale(w.head_dim)

    # dense causal
    od = P.dense_causal(q, k, v, block=w.block)
    odt = P.dense_causal(_tok(q), _tok(k), _tok(v), block=w.block, layout=P.PBS_LAYOUT_BNHD)
    torch.cuda.synchronize()
    _same(od, _head(odt), f"{name} dense causal o")

    # hybrid: own segment from the original K/V
    sh_h = P.shape_of(q, k, w.block, w.segment)
    sh_t = P.shape_of(_tok(q), _tok(k), w.block, w.segment, P.PBS_LAYOUT_BNHD)
    oh = torch.empty_like(q)
    oht = torch.empty_like(_tok(q))
    kt, vt = _tok(k), _tok(v)
    P.pbs_attn_fwd_hybrid(sh_h, q, head.k_perm, head.v_perm, k, v, head.counts, head.idx, scale,
                          oh, None)
    P.pbs_attn_fwd_hybrid(sh_t, _tok(q), tok.k_perm, tok.v_perm, kt, vt, tok.counts, tok.idx,
                          scale, oht, None)
    torch.cuda.synchronize()
    _same(oh, _head(oht), f"{name} hybrid o")

    # query-permutation variant: gather, selection on the moved queries, attention
    qp, qpt = torch.empty_like(q), torch.empty_like(_tok(q))
    P.pbs_permute_queries(sh_h, head.perm, q, qp)
    P.pbs_permute_queries(sh_t, tok.perm, _tok(q), qpt)
    torch.cuda.synchronize()
    _same(qp, _head(qpt), f"{name} q_perm")
    mode = P.PBS_SELECT_KEEP_RATIO if w.mode == "keep" else P.PBS_SELECT_COVERAGE
    c1, i1 = torch.empty_like(head.counts), torch.empty_like(head.idx)
    c2, i2 = torch.empty_like(head.counts), torch.empty_like(head.idx)
    P.pbs_block_select(sh_h, qp, head.k_perm, head.k_pool, scale, mode, w.params[0], None, 0, c1,
                       i1, head.workspace)
    P.pbs_block_select(sh_t, qpt, tok.k_perm, tok.k_pool, scale, mode, w.params[0], None, 0, c2,
                       i2, tok.workspace)
    torch.cuda.synchronize()
    assert lists_equal(c1.cpu().numpy(), i1.cpu().numpy(), c2.cpu().numpy(), i2.cpu().numpy())
    oq, oqt = torch.empty_like(q), torch.empty_like(_tok(q))
    P.pbs_attn_fwd_permuted_queries(sh_h, qp, head.k_perm, head.v_perm, head.perm,
                                    head.blk_minpos, c1, i1, scale, oq, None)
    P.pbs_attn_fwd_permuted_queries(sh_t, qpt, tok.k_perm, tok.v_perm, tok.perm, tok.blk_minpos,
                                    c2, i2, scale, oqt, None)
    torch.cuda.synchronize()
    _same(oq, _head(oqt), f"{name} permuted-query o")


def test_layout_bnhd_against_oracle():
    name = "gqa4_2k_keep"
    w = _workload(name)
    inp = pbs_synth.make_inputs(w)
    scale = oracle.default_scale(w.head_dim)
    ref = oracle.prefill(inp["q"], inp["k"], inp["v"], block=w.block, segment=w.segment,
                         scale=scale, mode=oracle.KEEP, param=w.params[0])
    q, k, v = (_tok(dev_bf16(inp[x])) for x in ("q", "k", "v"))
    out = P.prefill(q, k, v, block=w.block, segment=w.segment, keep=w.params[0], scale=scale,
                    layout=P.PBS_LAYOUT_BNHD)
    torch.cuda.synchronize()
    agree = float(np.mean(out.counts.cpu().numpy() == ref["counts"]))
    say(f"{name} BNHD: count agreement with the oracle {agree:.4f}")
    # same-start comparison of the attention: the oracle's lists through the BNHD kernels
    sh = P.shape_of(q, k, w.block, w.segment, P.PBS_LAYOUT_BNHD)
    B, H, N = ref["perm"].shape
    k_perm = _tok(dev_bf16(ref["k_perm"]))
    v_perm = _tok(dev_bf16(ref["v_perm"]))
    o = torch.empty_like(q)
    P.pbs_attn_fwd(sh, q, k_perm, v_perm, dev(ref["perm"]), dev(inverse_of(ref["perm"])), dev(ref["counts"]),
                   dev(ref["idx"]), scale, o, None)
    torch.cuda.synchronize()
    check_attn(_head(o).float().cpu().numpy().astype(np.float64), ref["o"],
               f"{name} BNHD attention, oracle lists")


def test_layouts_bit_identical_128k():
    w = pbs_synth.WORKLOADS["gqa_128k"]
    say("gqa_128k: BNHD against BHND, whole outputs")
    inp = pbs_synth.make_inputs(w)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    del inp
    head, tok = _both_layouts(w, q, k, v, ("keep", w.params[0]))
    assert lists_equal(head.counts.cpu().numpy(), head.idx.cpu().numpy(),
                       tok.counts.cpu().numpy(), tok.idx.cpu().numpy()), "128K block lists"
    _same(head.perm, tok.perm, "128K perm")
    _same(head.o, _head(tok.o), "128K o")
    _same(head.lse, tok.lse, "128K lse")
