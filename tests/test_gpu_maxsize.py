"""The largest supported problem through the whole path: N = 8192 blocks of 128 = 1,048,576 tokens
with the largest segment (16384 keys), so every query block of the last segment has 8064
candidate blocks.  Every stage is held against the oracle: the scores in full, the permutation
and the block lists bit-exact given the GPU's float32 scores / probabilities, the probabilities in
full, the attention on sampled query blocks (the oracle would take hours on all of them)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import oracle
import pbs_synth
from gpu_helpers import check_attn, dev_bf16, host_bits, lists_equal, say

pytestmark = pytest.mark.gpu


def test_max_sequence_full_path():
    w = pbs_synth.Workload("max_1m", 1, 2, 1, 1 << 20, 64, 128, 16384, "keep", (0.05,), 0.0025,
                           sink=64, seed=4077)
    say("max size: N=1048576, S=16384, Bs=128, d=64, 2 query heads / 1 KV head, keep 0.05")
    inp = pbs_synth.make_inputs(w)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    sh = P.shape_of(q, k, w.block, w.segment)
    nb = w.seq_len // w.block
    assert P.pbs_max_offdiag(sh) == nb - w.segment // w.block
    scale = oracle.default_scale(w.head_dim)
    bufs = P.Buffers(sh, q.device, with_scores=True)
    P.prefill(q, k, v, block=w.block, segment=w.segment, keep=w.params[0], scale=scale,
              buffers=bufs)
    torch.cuda.synchronize()

    sc = bufs.scores.cpu().numpy()
    ref_sc = oracle.key_scores(inp["q"], inp["k"], block=w.block, segment=w.segment, scale=scale)
    rel = np.abs(sc.astype(np.float64) - ref_sc) / np.abs(ref_sc.astype(np.float64))
    say(f"scores max rel err {rel.max():.2e}")
    assert rel.max() <= 1e-4

    perm = bufs.perm.cpu().numpy()
    ref_perm = oracle.segment_permutation(sc, segment=w.segment)
    assert np.array_equal(perm, ref_perm)
    k_perm = oracle.apply_permutation(inp["k"], ref_perm)
    assert np.array_equal(host_bits(bufs.k_perm), k_perm)
    assert np.array_equal(bufs.blk_minpos.cpu().numpy(),
                          ref_perm.reshape(1, 1, nb, w.block).min(-1))
    say("permutation bit-exact given the GPU scores")

    Pg = bufs.blk_scores.cpu().numpy()
    Po = oracle.block_probabilities(inp["q"], k_perm, block=w.block, segment=w.segment,
                                    scale=scale)
    cand = Po > 0
    assert np.array_equal(Pg > 0, cand)
    relp = np.abs(Pg.astype(np.float64) - Po)[cand] / Po[cand].astype(np.float64)
    say(f"block probabilities max rel err {relp.max():.2e}")
    assert relp.max() <= 1e-4
    del Po, cand

    rc, ri = oracle.select_blocks(Pg, block=w.block, segment=w.segment, mode=oracle.KEEP,
                                  param=w.params[0])
    counts, idx = bufs.counts.cpu().numpy(), bufs.idx.cpu().numpy()
    assert lists_equal(counts, idx, rc, ri)
    assert counts[0, 0, nb - 1] == oracle.keep_count(nb - w.segment // w.block, w.params[0])
    say("block lists bit-exact given the GPU probabilities")
    del Pg

    blocks = [nb - 1, nb - 2, nb - 128, nb // 2 + 5, 200, 128, 3]
    qb = [(0, g, i) for g in range(w.heads_q) for i in blocks]
    oo, ol = oracle.attention(inp["q"], inp["k"], inp["v"], block=w.block, segment=w.segment,
                              scale=scale, perm=perm, counts=counts, idx=idx, qblocks=qb)
    og, lg = bufs.o.float().cpu().numpy(), bufs.lse.cpu().numpy()
    got = np.stack([og[b, g, i * w.block:(i + 1) * w.block] for b, g, i in qb])
    gl = np.stack([lg[b, g, i * w.block:(i + 1) * w.block] for b, g, i in qb])
    check_attn(got, oo, "max size attention (sampled query blocks)")
    assert np.abs(gl - ol).max() < 1e-3
