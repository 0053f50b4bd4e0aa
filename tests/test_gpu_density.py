"""Block density and attention coverage on the GPU (permuted and natural key order) against the
oracle: coverage of a row = exp(lse_sparse - lse_dense) from the GPU attention's
log-normalisers, compared with the oracle's dense-softmax mass of the computed key set; block
counts from the GPU's selection (given the oracle's block probabilities) and min-positions
compared with the oracle's counts."""
import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import oracle
import pbs_synth
from gpu_helpers import dev, dev_bf16, inverse_of, run_attn, run_permute, run_select, say, shape

pytestmark = pytest.mark.gpu

COV_ATOL = 5e-3   # coverage = exp(dlse); the GPU log-normalisers are within 1e-3 of the oracle's


def _case(N=2048, Hq=8, Hkv=2, d=128, Bs=128, S=512, seed=41):
    w = pbs_synth.WORKLOADS["gqa_8k"].scaled(heads_q=Hq, heads_kv=Hkv, seq_len=N, head_dim=d, block=Bs,
                                             segment=S, seed=seed)
    return w, pbs_synth.make_inputs(w)


@pytest.mark.parametrize("permuted", [True, False])
@pytest.mark.parametrize("tau", [0.6, 0.9])
def test_coverage_and_density(permuted, tau):
    say(f"density/coverage permuted={permuted} tau={tau}")
    w, inp = _case()
    q, k, v = inp["q"], inp["k"], inp["v"]
    N, Bs, S, Hq, Hkv, d = w.seq_len, w.block, w.segment, w.heads_q, w.heads_kv, w.head_dim
    scale = oracle.default_scale(d)
    sh = shape(1, Hq, Hkv, N, d, Bs, S)
    if permuted:
        sc = oracle.key_scores(q, k, block=Bs, segment=S, scale=scale)
        perm = oracle.segment_permutation(sc, segment=S)
        kp, vp = oracle.apply_permutation(k, perm), oracle.apply_permutation(v, perm)
    else:
        perm, kp, vp = None, k, v
    Pm = oracle.block_probabilities(q, kp, block=Bs, segment=S, scale=scale)
    rc, ri = oracle.select_blocks(Pm, block=Bs, segment=S, mode=oracle.COVERAGE, param=tau)
    cov_ref = oracle.attention_coverage(q, k, block=Bs, segment=S, scale=scale, perm=perm, counts=rc, idx=ri)
    dens_ref = oracle.block_density(rc, block=Bs, segment=S, N=N, perm=perm)

    gq, gk, gv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    counts, idx = run_select(sh, None, None, None, scale, P.PBS_SELECT_COVERAGE, tau, blk_scores=dev(Pm),
                             flags=P.PBS_FLAG_SCORES_IN)
    assert np.array_equal(counts.cpu().numpy(), rc)
    if permuted:
        minpos = perm.reshape(1, Hkv, N // Bs, Bs).min(-1).astype(np.int32)
        _, lse = run_attn(sh, gq, dev_bf16(kp), dev_bf16(vp), dev(perm), dev(inverse_of(perm)), counts,
                          idx, scale)
    else:
        _, lse = run_attn(sh, gq, gk, gv, None, None, counts, idx, scale)
    _, lse_d = run_attn(sh, gq, gk, gv, None, None, None, None, scale)
    cov = torch.exp(lse - lse_d).cpu().numpy()
    err = np.abs(cov - cov_ref)
    say(f"coverage mean gpu {cov.mean():.5f} oracle {cov_ref.mean():.5f}, max err {err.max():.2e}")
    assert err.max() <= COV_ATOL

    # block counts the way the measurement takes them from the GPU outputs
    nb, bps, G = N // Bs, S // Bs, Hq // Hkv
    c = counts.cpu().numpy()
    own = 0
    for i in range(nb):
        s0 = (i // bps) * bps
        if permuted:
            own += int((minpos[:, :, s0:s0 + bps] <= (i + 1) * Bs - 1).sum()) * G
        else:
            own += Hq * (i - s0 + 1)
    assert int(c.sum()) == dens_ref["selected"]
    assert int(c.sum()) + own == dens_ref["computed"]


def test_coverage_full_size_sampled():
    """The 32K coverage workload at its full size: coverage of sampled query blocks (the last of
    every segment, both query heads of KV head 0 and the last head) from the GPU pipeline's
    log-normalisers, given the oracle's permutation and lists."""
    w = pbs_synth.WORKLOADS["gqa_32k_cov"]
    say("coverage full size", w.name)
    inp = pbs_synth.make_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    N, Bs, S, Hq, Hkv, d = w.seq_len, w.block, w.segment, w.heads_q, w.heads_kv, w.head_dim
    scale = oracle.default_scale(d)
    sc = oracle.key_scores(q, k, block=Bs, segment=S, scale=scale)
    perm = oracle.segment_permutation(sc, segment=S)
    kp, vp = oracle.apply_permutation(k, perm), oracle.apply_permutation(v, perm)
    Pm = oracle.block_probabilities(q, kp, block=Bs, segment=S, scale=scale)
    rc, ri = oracle.select_blocks(Pm, block=Bs, segment=S, mode=oracle.COVERAGE, param=w.params[0])
    nb, bps = N // Bs, S // Bs
    samples = [(0, g, i) for g in (0, 1, Hq - 1) for i in range(bps - 1, nb, bps)]
    cov_ref = oracle.attention_coverage(q, k, block=Bs, segment=S, scale=scale, perm=perm, counts=rc, idx=ri,
                                        qblocks=samples)
    sh = shape(1, Hq, Hkv, N, d, Bs, S)
    gq, gk, gv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    minpos = perm.reshape(1, Hkv, nb, Bs).min(-1).astype(np.int32)
    _, lse = run_attn(sh, gq, dev_bf16(kp), dev_bf16(vp), dev(perm), dev(inverse_of(perm)), dev(rc),
                      dev(ri), scale)
    _, lse_d = run_attn(sh, gq, gk, gv, None, None, None, None, scale)
    cov = torch.exp(lse - lse_d).cpu().numpy()
    got = np.stack([cov[b, g, i * Bs:(i + 1) * Bs] for b, g, i in samples])
    err = np.abs(got - cov_ref)
    say(f"coverage sampled mean {got.mean():.5f} (oracle {cov_ref.mean():.5f}), max err {err.max():.2e}")
    assert err.max() <= COV_ATOL
