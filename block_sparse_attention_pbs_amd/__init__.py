"""Python binding of libpbs: Permuted Block-Sparse Attention (PBS-Attn) prefill on MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of ``libpbs.so``
(built in-tree by ``python -m block_sparse_attention_pbs_amd.build``).  There is no CPU
fallback: importing works without the library, but every call raises ``LibraryMissing`` until
it is built.  Functions carry the names of the C entry points declared in ``include/pbs.h``;
tensors are torch tensors on the GPU (or raw device addresses as ``int``), bf16 data as
``torch.bfloat16``.  Calls are asynchronous on the given stream (default: torch's current
stream).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libpbs.so")

PBS_OK = 0
PBS_E_ARG = -1
PBS_E_SHAPE = -2
PBS_E_ALIGN = -3
PBS_E_WORKSPACE = -4
PBS_E_LAUNCH = -5
PBS_E_SCRATCH = -6
PBS_NOALLOC_SCRATCH_BYTES = 16 << 20
PBS_SELECT_KEEP_RATIO = 0
PBS_SELECT_COVERAGE = 1
PBS_LAYOUT_BHND = 0
PBS_LAYOUT_BNHD = 1
PBS_FLAG_SCORES_IN = 1
PBS_FLAG_KEEP_FIRST = 2

ENTRY_POINTS = ("pbs_workspace_bytes", "pbs_max_offdiag", "pbs_strerror", "pbs_score",
                "pbs_permute", "pbs_block_select", "pbs_attn_fwd", "pbs_attn_fwd_hybrid",
                "pbs_permute_queries", "pbs_attn_fwd_permuted_queries", "pbs_score_varlen",
                "pbs_block_select_varlen", "pbs_score_noalloc")


class PbsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


class LibraryMissing(PbsError):
    pass


class pbs_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("segment", ctypes.c_int32), ("layout", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p


def lib():
    """The loaded libpbs (raises ``LibraryMissing`` if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise LibraryMissing(-100, f"{LIBRARY_PATH} is not built; run "
                                   "`python -m block_sparse_attention_pbs_amd.build`")
    L = ctypes.CDLL(LIBRARY_PATH)
    S = ctypes.POINTER(pbs_shape)
    L.pbs_workspace_bytes.argtypes = [S]
    L.pbs_workspace_bytes.restype = ctypes.c_size_t
    L.pbs_max_offdiag.argtypes = [S]
    L.pbs_max_offdiag.restype = ctypes.c_int32
    L.pbs_strerror.argtypes = [ctypes.c_int]
    L.pbs_strerror.restype = ctypes.c_char_p
    L.pbs_score.argtypes = [S, _P, _P, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
    L.pbs_score_noalloc.argtypes = [S, _P, _P, ctypes.c_float, _P, _P]
    L.pbs_permute.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    L.pbs_block_select.argtypes = [S, _P, _P, _P, ctypes.c_float, ctypes.c_int, ctypes.c_double,
                                   _P, ctypes.c_int, _P, _P, _P, ctypes.c_size_t, _P]
    L.pbs_attn_fwd.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]
    L.pbs_attn_fwd_hybrid.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]
    L.pbs_permute_queries.argtypes = [S, _P, _P, _P, _P]
    L.pbs_attn_fwd_permuted_queries.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                                _P, _P, _P]
    L.pbs_score_varlen.argtypes = [S, _P, ctypes.c_int32, _P, _P, ctypes.c_float, _P, _P,
                                   ctypes.c_size_t, _P]
    L.pbs_block_select_varlen.argtypes = [S, _P, ctypes.c_int32, _P, _P, _P, ctypes.c_float,
                                          ctypes.c_int, ctypes.c_double, _P, ctypes.c_int, _P, _P,
                                          _P, ctypes.c_size_t, _P]
    for name in ("pbs_score", "pbs_permute", "pbs_block_select", "pbs_attn_fwd",
                 "pbs_attn_fwd_hybrid", "pbs_permute_queries", "pbs_attn_fwd_permuted_queries",
                 "pbs_score_varlen", "pbs_block_select_varlen", "pbs_score_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise PbsError(PBS_E_ARG, "tensors must be contiguous")
    return x.data_ptr() or None


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(code: int):
    if code != PBS_OK:
        raise PbsError(code, lib().pbs_strerror(code).decode())


def make_shape(batch, heads_q, heads_kv, seq_len, head_dim, block, segment,
               layout: int = 0) -> pbs_shape:
    return pbs_shape(batch, heads_q, heads_kv, seq_len, head_dim, block, segment, layout)


def shape_of(q: torch.Tensor, k: torch.Tensor, block: int, segment: int,
             layout: int = None) -> pbs_shape:
    """Shape from Q and K: [B,Hq,N,d] / [B,Hkv,N,d] (PBS_LAYOUT_BHND, the default) or
    [B,N,Hq,d] / [B,N,Hkv,d] (PBS_LAYOUT_BNHD)."""
    layout = PBS_LAYOUT_BHND if layout is None else layout
    if layout == PBS_LAYOUT_BNHD:
        B, N, Hq, d = q.shape
        return pbs_shape(B, Hq, k.shape[2], N, d, block, segment, layout)
    B, Hq, N, d = q.shape
    return pbs_shape(B, Hq, k.shape[1], N, d, block, segment, layout)


def pbs_workspace_bytes(shape: pbs_shape) -> int:
    return lib().pbs_workspace_bytes(ctypes.byref(shape))


def pbs_max_offdiag(shape: pbs_shape) -> int:
    return lib().pbs_max_offdiag(ctypes.byref(shape))


def pbs_strerror(code: int) -> str:
    return lib().pbs_strerror(code).decode()


def pbs_score(shape, q, k, scale, scores, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pbs_score(ctypes.byref(shape), _ptr(q), _ptr(k), scale, _ptr(scores),
                           _ptr(workspace), workspace_bytes, _stream(stream)))


def pbs_score_noalloc(shape, q, k, scale, scores, stream=None):
    _check(lib().pbs_score_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), scale, _ptr(scores),
                                   _stream(stream)))


def pbs_permute(shape, scores, k, v, perm, k_perm, v_perm, k_pool=None, blk_minpos=None,
                perm_inv=None, stream=None):
    _check(lib().pbs_permute(ctypes.byref(shape), _ptr(scores), _ptr(k), _ptr(v), _ptr(perm),
                             _ptr(k_perm), _ptr(v_perm), _ptr(k_pool), _ptr(blk_minpos),
                             _ptr(perm_inv), _stream(stream)))


def pbs_block_select(shape, q, k_perm, k_pool, scale, mode, param, blk_scores, flags, counts,
                     idx, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pbs_block_select(ctypes.byref(shape), _ptr(q), _ptr(k_perm), _ptr(k_pool), scale,
                                  mode, param, _ptr(blk_scores), flags, _ptr(counts), _ptr(idx),
                                  _ptr(workspace), workspace_bytes, _stream(stream)))


def pbs_score_varlen(shape, cu_seqlens, n_seqs, q, k, scale, scores, workspace,
                     workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pbs_score_varlen(ctypes.byref(shape), _ptr(cu_seqlens), n_seqs, _ptr(q), _ptr(k),
                                  scale, _ptr(scores), _ptr(workspace), workspace_bytes,
                                  _stream(stream)))


def pbs_block_select_varlen(shape, cu_seqlens, n_seqs, q, k_perm, k_pool, scale, mode, param,
                            blk_scores, flags, counts, idx, workspace, workspace_bytes=None,
                            stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pbs_block_select_varlen(ctypes.byref(shape), _ptr(cu_seqlens), n_seqs, _ptr(q),
                                         _ptr(k_perm), _ptr(k_pool), scale, mode, param,
                                         _ptr(blk_scores), flags, _ptr(counts), _ptr(idx),
                                         _ptr(workspace), workspace_bytes, _stream(stream)))


def pbs_attn_fwd(shape, q, k, v, perm, perm_inv, counts, idx, scale, o, lse=None, stream=None):
    _check(lib().pbs_attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(perm),
                              _ptr(perm_inv), _ptr(counts), _ptr(idx), scale, _ptr(o), _ptr(lse),
                              _stream(stream)))


def pbs_attn_fwd_hybrid(shape, q, k_perm, v_perm, k, v, counts, idx, scale, o, lse=None,
                        stream=None):
    _check(lib().pbs_attn_fwd_hybrid(ctypes.byref(shape), _ptr(q), _ptr(k_perm), _ptr(v_perm),
                                     _ptr(k), _ptr(v), _ptr(counts), _ptr(idx), scale, _ptr(o),
                                     _ptr(lse), _stream(stream)))


def pbs_permute_queries(shape, perm, q, q_perm, stream=None):
    _check(lib().pbs_permute_queries(ctypes.byref(shape), _ptr(perm), _ptr(q), _ptr(q_perm),
                                     _stream(stream)))


def pbs_attn_fwd_permuted_queries(shape, q_perm, k_perm, v_perm, perm, blk_minpos, counts, idx,
                                  scale, o, lse=None, stream=None):
    _check(lib().pbs_attn_fwd_permuted_queries(ctypes.byref(shape), _ptr(q_perm), _ptr(k_perm),
                                               _ptr(v_perm), _ptr(perm), _ptr(blk_minpos),
                                               _ptr(counts), _ptr(idx), scale, _ptr(o), _ptr(lse),
                                               _stream(stream)))


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


class Buffers:
    """Device buffers of one PBS prefill (outputs and intermediates), allocated once and reused."""

    def __init__(self, shape: pbs_shape, device, with_scores: bool = False):
        B, Hq, Hkv, N, d = shape.batch, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim
        nb = N // shape.block
        mo = max(pbs_max_offdiag(shape), 1)
        e = dict(device=device)
        self.shape = shape
        self.scores = torch.empty((B, Hkv, N), dtype=torch.float32, **e)
        self.perm = torch.empty((B, Hkv, N), dtype=torch.int32, **e)
        kv = (B, N, Hkv, d) if shape.layout == PBS_LAYOUT_BNHD else (B, Hkv, N, d)
        self.k_perm = torch.empty(kv, dtype=torch.bfloat16, **e)
        self.v_perm = torch.empty(kv, dtype=torch.bfloat16, **e)
        self.k_pool = torch.empty((B, Hkv, nb, d), dtype=torch.float32, **e)
        self.blk_minpos = torch.empty((B, Hkv, nb), dtype=torch.int32, **e)
        self.perm_inv = torch.empty((B, Hkv, N), dtype=torch.int32, **e)
        self.counts = torch.empty((B, Hq, nb), dtype=torch.int32, **e)
        self.idx = torch.empty((B, Hq, nb, mo), dtype=torch.int32, **e)
        self.blk_scores = torch.empty((B, Hq, nb, nb), dtype=torch.float32, **e) if with_scores else None
        self.o = torch.empty((B, N, Hq, d) if shape.layout == PBS_LAYOUT_BNHD else (B, Hq, N, d),
                             dtype=torch.bfloat16, **e)
        self.lse = torch.empty((B, Hq, N), dtype=torch.float32, **e)
        self.workspace = torch.empty(max(pbs_workspace_bytes(shape), 16), dtype=torch.uint8, **e)


def prefill(q, k, v, *, block: int, segment: int, keep: Optional[float] = None,
            coverage: Optional[float] = None, scale: Optional[float] = None,
            buffers: Optional[Buffers] = None, stream=None, layout: int = None) -> Buffers:
    """The whole PBS-Attn prefill: pbs_score -> pbs_permute -> pbs_block_select ->
    pbs_attn_fwd on one stream.  Exactly one of ``keep`` / ``coverage``.  Returns the buffers
    (``.o`` is the output in original token order, in the layout of q)."""
    if (keep is None) == (coverage is None):
        raise PbsError(PBS_E_ARG, "give exactly one of keep / coverage")
    shape = shape_of(q, k, block, segment, layout)
    if scale is None:
        scale = default_scale(q.shape[-1])
    bf = buffers or Buffers(shape, q.device)
    mode, param = (PBS_SELECT_KEEP_RATIO, keep) if keep is not None else (PBS_SELECT_COVERAGE, coverage)
    pbs_score(shape, q, k, scale, bf.scores, bf.workspace, stream=stream)
    pbs_permute(shape, bf.scores, k, v, bf.perm, bf.k_perm, bf.v_perm, bf.k_pool, bf.blk_minpos,
                bf.perm_inv, stream=stream)
    pbs_block_select(shape, q, bf.k_perm, bf.k_pool, scale, mode, param, bf.blk_scores, 0,
                     bf.counts, bf.idx, bf.workspace, stream=stream)
    pbs_attn_fwd(shape, q, bf.k_perm, bf.v_perm, bf.perm, bf.perm_inv, bf.counts, bf.idx, scale,
                 bf.o, bf.lse, stream=stream)
    return bf


def prefill_varlen(q, k, v, cu_seqlens, *, block: int, segment: int,
                   keep: Optional[float] = None, coverage: Optional[float] = None,
                   scale: Optional[float] = None, buffers: Optional[Buffers] = None, stream=None,
                   layout: int = None) -> Buffers:
    """PBS-Attn prefill of several sequences packed along N (batch 1): ``cu_seqlens`` is a
    device int32 tensor of the n+1 sequence starts, every length a multiple of ``segment``.
    pbs_score_varlen -> pbs_permute -> pbs_block_select_varlen -> pbs_attn_fwd on one stream."""
    if (keep is None) == (coverage is None):
        raise PbsError(PBS_E_ARG, "give exactly one of keep / coverage")
    shape = shape_of(q, k, block, segment, layout)
    n_seqs = int(cu_seqlens.numel()) - 1
    if scale is None:
        scale = default_scale(q.shape[-1])
    bf = buffers or Buffers(shape, q.device)
    mode, param = (PBS_SELECT_KEEP_RATIO, keep) if keep is not None else (PBS_SELECT_COVERAGE, coverage)
    pbs_score_varlen(shape, cu_seqlens, n_seqs, q, k, scale, bf.scores, bf.workspace, stream=stream)
    pbs_permute(shape, bf.scores, k, v, bf.perm, bf.k_perm, bf.v_perm, bf.k_pool, bf.blk_minpos,
                bf.perm_inv, stream=stream)
    pbs_block_select_varlen(shape, cu_seqlens, n_seqs, q, bf.k_perm, bf.k_pool, scale, mode, param,
                            bf.blk_scores, 0, bf.counts, bf.idx, bf.workspace, stream=stream)
    pbs_attn_fwd(shape, q, bf.k_perm, bf.v_perm, bf.perm, bf.perm_inv, bf.counts, bf.idx, scale,
                 bf.o, bf.lse, stream=stream)
    return bf


def dense_causal(q, k, v, *, block: int = 128, scale: Optional[float] = None, o=None, lse=None,
                 stream=None, layout: int = None):
    """Plain causal attention with the same kernel (dense mode of pbs_attn_fwd)."""
    shape = shape_of(q, k, block, block, layout)   # dense mode does not use segments
    if scale is None:
        scale = default_scale(q.shape[-1])
    if o is None:
        o = torch.empty_like(q)
    pbs_attn_fwd(shape, q, k, v, None, None, None, None, scale, o, lse, stream=stream)
    return o
