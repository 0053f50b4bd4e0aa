"""Seeded synthetic inputs for PBS-Attn prefill (shared by the oracle tests, GPU tests and bench).

This module draws data only; it holds none of the attention method's arithmetic.

The pages measure on long-context benchmarks with pretrained models, none of which is
available here. These generators stand in for them with the *shapes* of those models
(32 query / 8 KV heads at d=128 like an 8B Llama-class layer; 28 / 4 like a 7B Qwen-class
layer) and a planted structure that recreates the effect the method targets: a small set
of "heavy hitter" keys scattered over the whole sequence (sciencestack.ai page
"Sparser Block-Sparse Attention via Token Permutation", Abstract; gist.science summary of
the same paper, "Problemstellung" on information fragmentation).

Recipe (fixed; every step seeded from one numpy PCG64 stream, ``seed = 1000 + config``):
  1. per (batch, KV head) a direction ``u`` ~ N(0, I_d), normalised to unit length (float64);
  2. per (batch, KV head) the salient key positions: ``round(frac * N)`` distinct positions
     drawn uniformly from the eligible range (all of ``[0, N)``, or ``[sink, N)`` when a sink
     prefix is planted), returned sorted;
  3. Q, head by head: ``N(0,1)`` float32 ``[N, d]`` plus ``q_boost * u`` of its KV group;
  4. K, head by head: ``N(0,1)`` float32 plus ``k_boost * u`` on the salient rows and
     ``sink_boost * u`` on rows ``[0, sink)``;
  5. V, head by head: ``N(0,1)`` float32, untouched;
  6. every tensor is cast to bfloat16 with round-to-nearest-even and kept as raw uint16 bits.

Tensors are contiguous ``[B, H, N, d]`` (BHND).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic prefill workload: shapes, PBS parameters and the planted structure."""

    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int
    head_dim: int
    block: int          # block size (the pages' B in Fig. 1)
    segment: int        # segment size (the pages' S in Fig. 1)
    mode: str           # "keep" (keep ratio of off-diagonal blocks) or "coverage"
    params: tuple       # keep ratios or coverage thresholds evaluated on this input
    salient_frac: float
    sink: int = 0
    seed: int = 0
    q_boost: float = 1.5
    k_boost: float = 3.0
    sink_boost: float = 4.0

    @property
    def n_salient(self) -> int:
        return int(round(self.salient_frac * self.seq_len))

    def scaled(self, **kw) -> "Workload":
        """Same planted structure at other shapes (for small parity cases)."""
        return dataclasses.replace(self, **kw)


# The five workloads: a 1-head toy, three GQA 32/8 layers at 8K/32K/128K, and a 28/4
# keep-ratio sweep at 64K.
WORKLOADS = {
    "toy_1k": Workload("toy_1k", 1, 1, 1, 1024, 64, 64, 256, "keep", (0.5,), 0.02, seed=1001),
    "gqa_8k": Workload("gqa_8k", 1, 32, 8, 8192, 128, 128, 2048, "keep", (0.3,), 0.01, seed=1002),
    "gqa_32k_cov": Workload("gqa_32k_cov", 1, 32, 8, 32768, 128, 128, 4096, "coverage", (0.9,),
                            0.005, seed=1003),
    "gqa_128k": Workload("gqa_128k", 1, 32, 8, 131072, 128, 128, 8192, "keep", (0.1,), 0.0025,
                         sink=64, seed=1004),
    "gqa28_64k_sweep": Workload("gqa28_64k_sweep", 1, 28, 4, 65536, 128, 128, 4096, "keep",
                                (1.0, 0.5, 0.25, 0.1, 0.05), 0.005, seed=1005),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float32 (exact: a bfloat16 is the top half of a binary32)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw (q, k, v) for workload ``w`` as bf16 bit arrays, plus the planted metadata."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, Hq, Hkv, N, d = w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim
    if Hq % Hkv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    G = Hq // Hkv
    u = rng.standard_normal((B, Hkv, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    lo = w.sink
    n_sal = w.n_salient
    salient = np.zeros((B, Hkv, n_sal), dtype=np.int64)
    for b in range(B):
        for h in range(Hkv):
            salient[b, h] = np.sort(rng.choice(np.arange(lo, N), size=n_sal, replace=False))
    q = np.empty((B, Hq, N, d), dtype=np.uint16)
    k = np.empty((B, Hkv, N, d), dtype=np.uint16)
    v = np.empty((B, Hkv, N, d), dtype=np.uint16)
    for b in range(B):
        for g in range(Hq):
            x = rng.standard_normal((N, d), dtype=np.float32)
            x += (w.q_boost * u[b, g // G]).astype(np.float32)
            q[b, g] = f32_to_bf16_bits(x)
    for b in range(B):
        for h in range(Hkv):
            x = rng.standard_normal((N, d), dtype=np.float32)
            x[salient[b, h]] += (w.k_boost * u[b, h]).astype(np.float32)
            if w.sink:
                x[: w.sink] += (w.sink_boost * u[b, h]).astype(np.float32)
            k[b, h] = f32_to_bf16_bits(x)
    for b in range(B):
        for h in range(Hkv):
            v[b, h] = f32_to_bf16_bits(rng.standard_normal((N, d), dtype=np.float32))
    return {"q": q, "k": k, "v": v, "u": u, "salient": salient, "workload": w}


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) bf16 bits (for edge-case tests that need no planted structure)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))
