"""The seeded input generator: bfloat16 rounding, planted structure, determinism."""
import numpy as np
import torch

import pbs_synth


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(37.0)
    # exact ties between two bfloat16 values, both parities
    ties = (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    ours = pbs_synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    back = pbs_synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_toy_workload_structure():
    w = pbs_synth.WORKLOADS["toy_1k"]
    a = pbs_synth.make_inputs(w)
    b = pbs_synth.make_inputs(w)
    for name in ("q", "k", "v"):
        assert a[name].dtype == np.uint16 and (a[name] == b[name]).all()
    assert a["q"].shape == (1, 1, 1024, 64) and a["k"].shape == (1, 1, 1024, 64)
    assert a["salient"].shape == (1, 1, 20) and len(set(a["salient"][0, 0])) == 20
    # salient keys carry the planted direction: their projection on u is large
    k = pbs_synth.bf16_bits_to_f32(a["k"][0, 0]).astype(np.float64)
    proj = k @ a["u"][0, 0]
    sal = a["salient"][0, 0]
    others = np.setdiff1d(np.arange(1024), sal)
    assert proj[sal].mean() > 2.5 and abs(proj[others].mean()) < 0.2
    c = pbs_synth.make_inputs(w, seed=7)
    assert not (c["q"] == a["q"]).all()


def test_sink_prefix_planted():
    w = pbs_synth.WORKLOADS["gqa_128k"].scaled(heads_q=4, heads_kv=1, seq_len=2048, segment=512)
    a = pbs_synth.make_inputs(w)
    assert (a["salient"] >= 64).all()
    k = pbs_synth.bf16_bits_to_f32(a["k"][0, 0]).astype(np.float64)
    proj = k @ a["u"][0, 0]
    assert proj[:64].mean() > 3.0
