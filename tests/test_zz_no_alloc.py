"""pbs_score_noalloc (the entry point that allocates nothing: its score partials live in the
library's static scratch) against pbs_score with a caller workspace, through the C ABI, on two
calls in a row, the second with a smaller problem: the same kernels, so the scores must agree
bit for bit.  Also: a problem too large for the scratch is rejected before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import pbs_synth
from gpu_helpers import dev_bf16, say

pytestmark = pytest.mark.gpu


def _scores_both_ways(w):
    inp = pbs_synth.make_inputs(w)
    q, k = dev_bf16(inp["q"]), dev_bf16(inp["k"])
    sh = P.make_shape(w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim, w.block, w.segment)
    scale = P.default_scale(w.head_dim)
    ref = torch.empty((w.batch, w.heads_kv, w.seq_len), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(P.pbs_workspace_bytes(sh), 16), dtype=torch.uint8, device="cuda")
    P.pbs_score(sh, q, k, scale, ref, ws)
    got = torch.full_like(ref, float("nan"))
    L = P.lib()
    st = L.pbs_score_noalloc(ctypes.byref(sh), q.data_ptr(), k.data_ptr(), scale, got.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == P.PBS_OK, P.pbs_strerror(st)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_scores_equal_workspace_scores_twice():
    big = pbs_synth.WORKLOADS["gqa_32k_cov"]                  # 32/8 heads, 32K tokens, S 4096
    small = pbs_synth.WORKLOADS["gqa_8k"]                     # then a smaller problem
    for w in (big, small):
        say(f"pbs_score_noalloc vs pbs_score on {w.name}")
        ref, got = _scores_both_ways(w)
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), w.name
        sums = got.astype(np.float64).reshape(w.batch, w.heads_kv, -1, w.segment).sum(-1)
        assert np.allclose(sums, 1.0, atol=1e-4)


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    sh = P.make_shape(1, 32, 8, 1 << 20, 128, 128, 16384)
    dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = P.lib().pbs_score_noalloc(ctypes.byref(sh), dummy.data_ptr(), dummy.data_ptr(), 0.1,
                                   dummy.data_ptr(), None)
    assert st == P.PBS_E_SCRATCH
