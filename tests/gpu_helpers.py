"""Helpers shared by the GPU tests: device copies of seeded inputs, one-call wrappers around the
C ABI (through the binding) and the comparison bars."""
import sys

import numpy as np
import torch

import block_sparse_attention_pbs_amd as P
import oracle

# Attention tolerance of the bf16 GPU path against the float64 oracle.
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3


def say(*msg):
    print("[gpu]", *msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64_torch(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def shape(B, Hq, Hkv, N, d, Bs, S):
    return P.make_shape(B, Hq, Hkv, N, d, Bs, S)


def check_attn(o_gpu: np.ndarray, o_ref: np.ndarray, what: str):
    err = np.abs(o_gpu - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    say(f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= ATTN_MAX_ABS, (what, mx)
    assert mean <= ATTN_MEAN_ABS, (what, mean)
    return mx, mean


def run_score(sh, q, k, scale):
    scores = torch.empty((sh.batch, sh.heads_kv, sh.seq_len), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(P.pbs_workspace_bytes(sh), 16), dtype=torch.uint8, device="cuda")
    P.pbs_score(sh, q, k, scale, scores, ws)
    torch.cuda.synchronize()
    return scores


def run_permute(sh, scores, k, v, pool=True, minpos=True, inv=True):
    B, H, N, d = sh.batch, sh.heads_kv, sh.seq_len, sh.head_dim
    nb = N // sh.block
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    kp = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    kpool = torch.empty((B, H, nb, d), dtype=torch.float32, device="cuda") if pool else None
    mpos = torch.empty((B, H, nb), dtype=torch.int32, device="cuda") if minpos else None
    pinv = torch.empty((B, H, N), dtype=torch.int32, device="cuda") if inv else None
    P.pbs_permute(sh, scores, k, v, perm, kp, vp, kpool, mpos, pinv)
    torch.cuda.synchronize()
    return perm, kp, vp, kpool, mpos, pinv


def inverse_of(perm: np.ndarray) -> np.ndarray:
    """The slot of every original position (what pbs_permute writes as perm_inv), from the
    oracle's inverse permutation."""
    return np.ascontiguousarray(oracle.inverse_permutation(np.ascontiguousarray(perm)), dtype=np.int32)


def run_select(sh, q, k_perm, k_pool, scale, mode, param, blk_scores=None, flags=0):
    B, Hq, N = sh.batch, sh.heads_q, sh.seq_len
    nb = N // sh.block
    mo = max(P.pbs_max_offdiag(sh), 1)
    counts = torch.full((B, Hq, nb), -7, dtype=torch.int32, device="cuda")
    idx = torch.full((B, Hq, nb, mo), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(P.pbs_workspace_bytes(sh), 16), dtype=torch.uint8, device="cuda")
    P.pbs_block_select(sh, q, k_perm, k_pool, scale, mode, param, blk_scores, flags, counts, idx, ws)
    torch.cuda.synchronize()
    return counts, idx


def run_attn(sh, q, k, v, perm, perm_inv, counts, idx, scale, want_lse=True):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda") if want_lse else None
    P.pbs_attn_fwd(sh, q, k, v, perm, perm_inv, counts, idx, scale, o, lse)
    torch.cuda.synchronize()
    return o, lse


def lists_equal(counts_a, idx_a, counts_b, idx_b):
    """Bit-exact comparison of two selections (only the first counts entries of a row count)."""
    ca, cb = np.asarray(counts_a), np.asarray(counts_b)
    if not np.array_equal(ca, cb):
        return False
    ia, ib = np.asarray(idx_a), np.asarray(idx_b)
    w = min(ia.shape[-1], ib.shape[-1])
    pos = np.arange(w)
    live = pos[None, None, None, :] < ca[..., None]
    return bool(np.array_equal(np.where(live, ia[..., :w], -1), np.where(live, ib[..., :w], -1)))
