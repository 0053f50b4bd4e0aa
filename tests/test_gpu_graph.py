"""The whole prefill captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every entry point only enqueues kernels on the given stream: no allocation, no memset, no
synchronisation, so the four calls of a prefill (and the dense baseline) can be recorded once and
replayed.  Each replay is checked against the eager result, bit for bit, with the outputs
clobbered and other eager work run on the GPU between the replays."""
import numpy as np
import pytest
import torch

import block_sparse_attention_pbs_amd as P
import pbs_synth
from gpu_helpers import dev_bf16, lists_equal, say

pytestmark = pytest.mark.gpu


def _same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


@pytest.mark.parametrize("mode", ["keep", "coverage"])
def test_prefill_graph_replay(mode):
    w = pbs_synth.WORKLOADS["gqa_8k"].scaled(name=f"graph_{mode}", heads_q=8, heads_kv=2,
                                             seq_len=4096, segment=1024, seed=4242)
    inp = pbs_synth.make_inputs(w)
    q, k, v = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    sel = {"keep": 0.3} if mode == "keep" else {"coverage": 0.9}
    kw = dict(block=w.block, segment=w.segment, **sel)
    shape = P.shape_of(q, k, w.block, w.segment)
    eager = P.prefill(q, k, v, **kw)
    dense_eager = P.dense_causal(q, k, v, block=w.block)
    torch.cuda.synchronize()

    bufs = P.Buffers(shape, q.device)
    o_dense = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # one run outside the capture first
        P.prefill(q, k, v, buffers=bufs, **kw)
        P.dense_causal(q, k, v, block=w.block, o=o_dense)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        P.prefill(q, k, v, buffers=bufs, **kw)
        P.dense_causal(q, k, v, block=w.block, o=o_dense)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (bufs.o, bufs.lse, bufs.scores, o_dense):
            t.zero_()
        bufs.perm.fill_(-1)
        bufs.counts.fill_(-1)
        bufs.idx.fill_(-1)
        other = P.prefill(k.repeat_interleave(4, dim=1)[:, : w.heads_q].contiguous(), k, v, **kw)
        torch.cuda.synchronize()
        del other
        g.replay()
        torch.cuda.synchronize()
        ok = (_same(bufs.scores, eager.scores) and _same(bufs.perm, eager.perm)
              and lists_equal(bufs.counts.cpu().numpy(), bufs.idx.cpu().numpy(),
                              eager.counts.cpu().numpy(), eager.idx.cpu().numpy())
              and _same(bufs.o, eager.o) and _same(bufs.lse, eager.lse)
              and _same(o_dense, dense_eager))
        say(f"graph replay {rep} ({mode}): {'bit-identical to eager' if ok else 'DIFFERENT'}")
        assert ok, rep
