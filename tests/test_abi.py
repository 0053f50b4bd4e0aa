"""The C-ABI library on the host: it loads, exports every symbol the header declares, and
rejects bad arguments before touching the GPU (no compute call here)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_pbs_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pbs.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pbs_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(P.ENTRY_POINTS)
    L = P.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_shape_rules():
    good = P.make_shape(1, 32, 8, 131072, 128, 128, 8192)
    assert P.pbs_max_offdiag(good) == 15 * 64
    assert P.pbs_workspace_bytes(good) > 0
    bad = [P.make_shape(1, 32, 8, 1000, 128, 128, 256),   # N % S
           P.make_shape(1, 32, 8, 1024, 128, 128, 192),   # S % Bs
           P.make_shape(1, 30, 8, 1024, 128, 128, 256),   # Hq % Hkv
           P.make_shape(1, 32, 8, 1024, 96, 128, 256),    # d
           P.make_shape(1, 32, 8, 1024, 128, 32, 256),    # Bs
           P.make_shape(1, 32, 8, 65536, 128, 128, 32768),  # S too large
           P.make_shape(1, 32, 8, 8192 * 64 * 2, 128, 64, 64),  # too many blocks
           P.make_shape(1, 32, 8, 1024, 128, 128, 256, 2),      # unknown layout
           P.make_shape(1, 32, 8, 1024, 128, 128, 256, -1),     # unknown layout
           # token-major K/V head wider than 32-bit byte offsets: N * Hkv * d * 2 = 2^32
           P.make_shape(1, 64, 16, 8192 * 128, 128, 128, 8192, P.PBS_LAYOUT_BNHD),
           # one token's K/V row (all KV heads) of 2^24 bytes: Hkv * d * 2 = 65536 * 128 * 2
           P.make_shape(1, 65536, 65536, 128, 128, 128, 128, P.PBS_LAYOUT_BNHD)]
    for s in bad:
        assert P.pbs_max_offdiag(s) == -1
        assert P.pbs_workspace_bytes(s) == 0
    # the same sizes are fine head-major, and token-major just below the limit
    assert P.pbs_max_offdiag(P.make_shape(1, 64, 16, 8192 * 128, 128, 128, 8192)) > 0
    assert P.pbs_max_offdiag(P.make_shape(1, 60, 15, 8192 * 128, 128, 128, 8192,
                                          P.PBS_LAYOUT_BNHD)) > 0
    assert P.pbs_max_offdiag(P.make_shape(1, 32, 8, 131072, 128, 128, 8192,
                                          P.PBS_LAYOUT_BNHD)) == 15 * 64


def test_shape_of_both_layouts():
    import torch
    q = torch.empty((2, 32, 4096, 128), dtype=torch.bfloat16)
    k = torch.empty((2, 8, 4096, 128), dtype=torch.bfloat16)
    s = P.shape_of(q, k, 128, 1024)
    assert (s.batch, s.heads_q, s.heads_kv, s.seq_len, s.head_dim, s.layout) == (2, 32, 8, 4096, 128, 0)
    s = P.shape_of(q.transpose(1, 2), k.transpose(1, 2), 128, 1024, P.PBS_LAYOUT_BNHD)
    assert (s.batch, s.heads_q, s.heads_kv, s.seq_len, s.head_dim, s.layout) == (2, 32, 8, 4096, 128, 1)


def _call(fn, *args):
    return getattr(P.lib(), fn)(*args)


def test_errors_before_any_launch():
    s = P.make_shape(1, 4, 2, 1024, 128, 128, 256)
    S = ctypes.byref(s)
    fake = 0x10000  # an aligned, never dereferenced address: every call below fails validation
    assert _call("pbs_score", ctypes.byref(P.make_shape(1, 4, 2, 1000, 128, 128, 256)), fake, fake,
                 0.1, fake, fake, 1 << 30, None) == P.PBS_E_SHAPE
    assert _call("pbs_score", S, None, fake, 0.1, fake, fake, 1 << 30, None) == P.PBS_E_ARG
    assert _call("pbs_score", S, fake + 4, fake, 0.1, fake, fake, 1 << 30, None) == P.PBS_E_ALIGN
    assert _call("pbs_score", S, fake, fake, 0.1, fake, fake, 16, None) == P.PBS_E_WORKSPACE
    assert _call("pbs_score", S, fake, fake, -1.0, fake, fake, 1 << 30, None) == P.PBS_E_ARG
    assert _call("pbs_permute", S, fake, None, fake, fake, fake, fake, None, None, None, None) == P.PBS_E_ARG
    assert _call("pbs_permute", S, fake, fake, fake, fake, fake, fake, fake + 8, None, None, None) == P.PBS_E_ALIGN
    assert _call("pbs_permute", S, fake, fake, fake, fake, fake, fake, None, None, fake + 4, None) == P.PBS_E_ALIGN
    sel = lambda mode, param, flags, ws=1 << 30, bs=None: _call(
        "pbs_block_select", S, fake, fake, None, 0.1, mode, param, bs, flags, fake, fake, fake, ws, None)
    assert sel(2, 0.5, 0) == P.PBS_E_ARG
    assert sel(0, 0.0, 0) == P.PBS_E_ARG
    assert sel(1, 1.5, 0) == P.PBS_E_ARG
    assert sel(0, 0.5, 4) == P.PBS_E_ARG
    assert sel(0, 0.5, P.PBS_FLAG_KEEP_FIRST, ws=16) == P.PBS_E_WORKSPACE   # flag accepted
    assert sel(0, 0.5, P.PBS_FLAG_KEEP_FIRST | 8, ws=16) == P.PBS_E_ARG
    assert sel(0, 0.5, P.PBS_FLAG_SCORES_IN) == P.PBS_E_ARG   # probabilities in, but none given
    assert sel(0, 0.5, 0, ws=16) == P.PBS_E_WORKSPACE
    attn = lambda perm, inv, counts, idx: _call(
        "pbs_attn_fwd", S, fake, fake, fake, perm, inv, counts, idx, 0.1, fake, None, None)
    assert attn(None, None, fake, None) == P.PBS_E_ARG          # counts without idx
    assert attn(fake, fake, None, None) == P.PBS_E_ARG          # permutation in dense mode
    assert attn(fake, None, fake, fake) == P.PBS_E_ARG          # permutation without its inverse
    assert attn(None, fake, fake, fake) == P.PBS_E_ARG          # inverse without the permutation
    assert attn(fake, fake + 4, fake, fake) == P.PBS_E_ALIGN
    pq = lambda perm, q, qp: _call("pbs_permute_queries", S, perm, q, qp, None)
    assert pq(None, fake, fake + 256) == P.PBS_E_ARG
    assert pq(fake, fake, fake) == P.PBS_E_ARG                  # in place is rejected
    assert pq(fake, fake + 8, fake + 256) == P.PBS_E_ALIGN
    aq = lambda perm, counts, minpos=None: _call(
        "pbs_attn_fwd_permuted_queries", S, fake, fake, fake, perm, minpos, counts, fake, 0.1,
        fake, None, None)
    assert aq(None, fake) == P.PBS_E_ARG                         # the permutation is required
    assert aq(fake, None) == P.PBS_E_ARG                         # lists are required
    assert aq(fake, fake, minpos=fake + 4) == P.PBS_E_ALIGN
    na = lambda shape, q: _call("pbs_score_noalloc", shape, q, fake, 0.1, fake, None)
    assert na(S, None) == P.PBS_E_ARG
    assert na(S, fake + 2) == P.PBS_E_ALIGN
    # partials of 1M tokens (64 segments of 16384) exceed the static scratch: rejected on the host
    assert na(ctypes.byref(P.make_shape(1, 32, 8, 1 << 20, 128, 128, 16384)), fake) == P.PBS_E_SCRATCH
    hyb = lambda kp, k, counts, lse=None: _call(
        "pbs_attn_fwd_hybrid", S, fake, kp, fake, k, fake, counts, fake, 0.1, fake, lse, None)
    assert hyb(fake, fake, None) == P.PBS_E_ARG                  # lists are required
    assert hyb(fake, None, fake) == P.PBS_E_ARG                  # original keys are required
    assert hyb(fake + 2, fake, fake) == P.PBS_E_ALIGN
    assert hyb(fake, fake, fake, lse=fake + 4) == P.PBS_E_ALIGN


def test_varlen_errors_before_any_launch():
    s = P.make_shape(1, 4, 2, 1024, 128, 128, 256)   # 4 segments
    S = ctypes.byref(s)
    fake = 0x10000
    sv = lambda cu, n, ws=1 << 30, shape=S: _call(
        "pbs_score_varlen", shape, cu, n, fake, fake, 0.1, fake, fake, ws, None)
    assert sv(fake, 2, shape=ctypes.byref(P.make_shape(2, 4, 2, 1024, 128, 128, 256))) == P.PBS_E_SHAPE
    assert sv(None, 2) == P.PBS_E_ARG
    assert sv(fake + 2, 2) == P.PBS_E_ALIGN
    assert sv(fake, 0) == P.PBS_E_ARG
    assert sv(fake, 5) == P.PBS_E_ARG                  # more sequences than segments
    assert sv(fake + 4, 4, ws=16) == P.PBS_E_WORKSPACE   # 4-byte aligned boundaries accepted
    sl = lambda cu, n, mode=0, ws=1 << 30: _call(
        "pbs_block_select_varlen", S, cu, n, fake, fake, None, 0.1, mode, 0.5, None, 0, fake, fake,
        fake, ws, None)
    assert sl(None, 1) == P.PBS_E_ARG
    assert sl(fake + 1, 1) == P.PBS_E_ALIGN
    assert sl(fake, 9) == P.PBS_E_ARG
    assert sl(fake, 1, mode=3) == P.PBS_E_ARG
    assert sl(fake, 1, ws=16) == P.PBS_E_WORKSPACE
    # an empty packed row is a no-op
    e = P.make_shape(1, 4, 2, 0, 128, 128, 256)
    assert _call("pbs_score_varlen", ctypes.byref(e), fake, 1, None, None, 0.1, None, None, 0,
                 None) == P.PBS_OK


def test_empty_problem_is_ok_without_pointers():
    s = P.make_shape(0, 4, 2, 1024, 128, 128, 256)
    assert _call("pbs_attn_fwd", ctypes.byref(s), None, None, None, None, None, None, None, 0.1,
                 None, None, None) == P.PBS_OK
    s = P.make_shape(2, 4, 2, 0, 128, 128, 256)
    assert _call("pbs_permute", ctypes.byref(s), None, None, None, None, None, None, None, None,
                 None, None) == P.PBS_OK


def test_strerror():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert P.pbs_strerror(code)
    assert P.pbs_strerror(-99) == "unknown status"


def test_binding_raises_pbs_error():
    s = P.make_shape(1, 4, 2, 1000, 128, 128, 256)
    with pytest.raises(P.PbsError) as e:
        P.pbs_attn_fwd(s, 0x10000, 0x10000, 0x10000, None, None, None, None, 0.1, 0x10000, None, stream=0)
    assert e.value.code == P.PBS_E_SHAPE
