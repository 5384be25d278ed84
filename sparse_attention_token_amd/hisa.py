"""Thin Python binding over libhisa (include/hisa.h).

Argument marshalling only: tensors are checked for dtype, device, shape and
layout, outputs and workspace are allocated with torch, and the raw device
pointers plus torch's current HIP stream are handed to the C ABI.  Every step
of the indexing path runs in the library's HIP kernels; there is no fallback.
If the built library is missing this module raises on first use.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhisa.so")
_lib = None

HISA_OK = 0
HISA_ERR_ARG = -1
HISA_ERR_UNSUPPORTED = -2
HISA_ERR_WORKSPACE = -3
HISA_ERR_HIP = -4
HISA_ERR_SCRATCH = -5
STATIC_SCRATCH_BYTES = 16 << 20      # HISA_STATIC_SCRATCH_BYTES


class HisaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().hisa_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libhisa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libhisa.so not built ({_LIB_PATH}); run __graft_entry__.build()")
    L = C.CDLL(_LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    L.hisa_abi_version.restype = i32
    L.hisa_abi_version.argtypes = []
    L.hisa_status_string.restype = C.c_char_p
    L.hisa_status_string.argtypes = [i32]
    L.hisa_pool_append.restype = i32
    L.hisa_pool_append.argtypes = [vp, i64, i32, i32, i32, i64, i64, vp, i64, vp]
    L.hisa_index_workspace.restype = sz
    L.hisa_index_workspace.argtypes = [i32, i32, i32, i32, i64, i32, i32, i32]
    L.hisa_index.restype = i32
    L.hisa_index.argtypes = [vp, vp, vp, vp, i64, i64, vp, i64, i32, i32, i32, i32, i32, i32, i32,
                             vp, vp, vp, vp, sz, vp]
    L.hisa_pool_append_mode.restype = i32
    L.hisa_pool_append_mode.argtypes = [vp, i64, i32, i32, i32, i64, i64, vp, i64, i32, vp]
    L.hisa_index_mode.restype = i32
    L.hisa_index_mode.argtypes = [vp, vp, vp, vp, i64, i64, vp, i64, i32, i32, i32, i32, i32, i32, i32,
                                  vp, vp, vp, vp, sz, i32, vp]
    L.hisa_append_index_mode.restype = i32
    L.hisa_append_index_mode.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i32, vp, vp, vp, vp, sz, i32, vp]
    L.hisa_append_index.restype = i32
    L.hisa_append_index.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                    i32, vp, vp, vp, vp, sz, vp]
    L.hisa_append_index_static.restype = i32
    L.hisa_append_index_static.argtypes = [vp, i64, i64, i64, vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                           i32, vp, vp, vp, vp]
    L.hisa_tree_append.restype = i32
    L.hisa_tree_append.argtypes = [vp, i64, i32, i32, i32, i32, i64, i64, vp, i64, vp, i64, i32, vp]
    L.hisa_tree_index_workspace.restype = sz
    L.hisa_tree_index_workspace.argtypes = [i32, i32, i32, i32, i64, i32, i32, i32, i32, i32]
    L.hisa_tree_index.restype = i32
    L.hisa_tree_index.argtypes = [vp, vp, vp, vp, i64, i64, vp, i64, vp, i64, i32, i32, i32, i32, i32, i32,
                                  i32, i32, i32, vp, vp, vp, vp, vp, sz, i32, vp]
    L.hisa_sparse_attention_workspace.restype = sz
    L.hisa_sparse_attention_workspace.argtypes = [i32, i32, i32, i32, i32, i32]
    L.hisa_sparse_attention.restype = i32
    L.hisa_sparse_attention.argtypes = [vp, vp, i64, i64, i64, vp, i32, i32, i32, i32, i32, i32, C.c_float,
                                        vp, vp, vp, sz, vp]
    L.dsa_flat_workspace.restype = sz
    L.dsa_flat_workspace.argtypes = [i32, i32, i32, i32, i64, i32]
    L.dsa_flat_index.restype = i32
    L.dsa_flat_index.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp,
                                 sz, vp]
    L.hisa_profile_enable.restype = i32
    L.hisa_profile_enable.argtypes = [i32]
    L.hisa_profile_read.restype = i32
    L.hisa_profile_read.argtypes = [i32, C.POINTER(C.c_double), C.POINTER(C.c_int)]
    L.hisa_kernel_kinds.restype = i32
    L.hisa_kernel_kinds.argtypes = []
    L.hisa_kernel_name.restype = C.c_char_p
    L.hisa_kernel_name.argtypes = [i32]
    _lib = L
    return L


# ---------------------------------------------------------------- helpers

def _ptr(t: Optional[torch.Tensor]):
    # the prototypes declare void*: ctypes converts a plain int (or None)
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    """torch's current HIP stream on `device`, as an integer handle.  torch's
    raw-stream accessor skips building a Stream object (about 2 us a call);
    the public route serves where it is absent."""
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16 (or its 16-bit pattern), got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _rows(t: torch.Tensor, name: str, d: int):
    """A [S, N, d] tensor with unit stride rows; returns the sequence stride in elements."""
    if t.dim() != 3 or t.shape[2] != d or t.stride(2) != 1 or t.stride(1) != d:
        raise ValueError(f"{name} must be [S, N, {d}] with contiguous rows")
    return t.stride(0)


def _check(fn: str, st: int):
    if st != HISA_OK:
        raise HisaError(fn, st)


def _out(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype, device) -> torch.Tensor:
    """A caller-supplied output: exactly `shape` and `dtype`, contiguous, on `device`; a new
    tensor when t is None.  The kernels write every element of the shape through the raw
    pointer, so anything smaller, strided or of another type is refused before the call."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if (isinstance(t, torch.Tensor) and t.dtype == dtype and t.shape == shape and t.device == device
            and t.is_contiguous()):
        return t                                  # the usual case, checked in one pass
    shape = tuple(int(x) for x in shape)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ---------------------------------------------------------------- the ABI calls

def hisa_abi_version() -> int:
    return int(lib().hisa_abi_version())


POOL_KINDS = {"mean": 0, "max": 1}


def _pool_kind(pool: str) -> int:
    if pool not in POOL_KINDS:
        raise ValueError(f"pool must be one of {sorted(POOL_KINDS)}")
    return POOL_KINDS[pool]


def hisa_pool_append(K: torch.Tensor, pool_mean: torch.Tensor, L_old: int, L_new: int, B: int,
                     pool: str = "mean"):
    """Fold key rows [L_old, L_new) of K [S, L_cap, d] into pool_mean [S, nblk_cap, d] (in place);
    pool="max" keeps max-pooled representatives instead of means."""
    _bf16(K, "K")
    _bf16(pool_mean, "pool_mean")
    S, _, d = K.shape
    kss = _rows(K, "K", d)
    pss = _rows(pool_mean, "pool_mean", d)
    if pool_mean.shape[0] != S:
        raise ValueError("pool_mean and K disagree on S")
    if pool_mean.device != K.device:
        raise ValueError("pool_mean and K must be on the same device")
    if pool_mean.shape[1] * B < L_new or K.shape[1] < L_new:
        raise ValueError("K or pool_mean too short for L_new")
    st = lib().hisa_pool_append_mode(_ptr(K), kss, S, d, B, int(L_old), int(L_new), _ptr(pool_mean),
                                     pss, _pool_kind(pool), _stream(K.device))
    _check("hisa_pool_append", st)
    return pool_mean


def hisa_index_workspace(S, T, H, d, L, B, m, k) -> int:
    return int(lib().hisa_index_workspace(S, T, H, d, L, B, m, k))


def dsa_flat_workspace(S, T, H, d, L, k) -> int:
    return int(lib().dsa_flat_workspace(S, T, H, d, L, k))


def _query_args(q, w, qpos, K, L):
    _bf16(q, "q")
    _bf16(K, "K")
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [S, T, H, d] tensor")
    S, T, H, d = q.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (S, T, H) or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 [S, T, H] tensor")
    if K.shape[0] != S or K.shape[1] < L:
        raise ValueError("K must be [S, >= L, d]")
    kss = _rows(K, "K", d)
    if qpos is not None:
        if qpos.dtype != torch.int32 or tuple(qpos.shape) != (S, T) or not qpos.is_contiguous():
            raise ValueError("qpos must be a contiguous int32 [S, T] tensor")
    for t in (w, K) + (() if qpos is None else (qpos,)):
        if t.device != q.device:
            raise ValueError("all tensors must be on the same device")
    return S, T, H, d, kss


def _workspace(nbytes: Optional[int], device, workspace):
    """Allocate the workspace, or pass the caller's through (the library checks its size:
    a short one returns HISA_ERR_WORKSPACE, so its size need not be queried per call)."""
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous buffer on the query's device")
    return workspace


def hisa_index(q, w, K, L: int, pool_mean, B: int, m: int, k: int, qpos=None, *,
               want_scores: bool = True, want_blocks: bool = False, out_idx=None, out_score=None,
               out_blk=None, workspace=None, pool: str = "mean"):
    """HISA two-stage indexer.  Returns (idx [S,T,k] int32, score [S,T,k] fp32 | None,
    blocks [S,T,m] int32 | None).  pool: how pool_mean was built ("mean" or "max")."""
    S, T, H, d, kss = _query_args(q, w, qpos, K, L)
    _bf16(pool_mean, "pool_mean")
    pss = _rows(pool_mean, "pool_mean", d)
    if pool_mean.shape[0] != S or pool_mean.shape[1] * B < L:
        raise ValueError("pool_mean must be [S, >= ceil(L/B), d]")
    if pool_mean.device != q.device:
        raise ValueError("pool_mean must be on the query's device")
    dev = q.device
    out_idx = _out(out_idx, "out_idx", (S, T, k), torch.int32, dev)
    if want_scores or out_score is not None:
        out_score = _out(out_score, "out_score", (S, T, k), torch.float32, dev)
    if want_blocks or out_blk is not None:
        out_blk = _out(out_blk, "out_blk", (S, T, m), torch.int32, dev)
    if workspace is None:
        nbytes = hisa_index_workspace(S, T, H, d, L, B, m, k)
        if nbytes == 0:
            _check("hisa_index", lib().hisa_index(None, None, None, None, 0, L, None, 0, S, T, H, d, B,
                                                  m, k, None, None, None, None, 0, None))
    ws = _workspace(None if workspace is not None else nbytes, dev, workspace)
    st = lib().hisa_index_mode(_ptr(q), _ptr(w), _ptr(qpos), _ptr(K), kss, int(L), _ptr(pool_mean),
                               pss, S, T, H, d, B, m, k, _ptr(out_idx), _ptr(out_score), _ptr(out_blk),
                               _ptr(ws), ws.numel() * ws.element_size(), _pool_kind(pool), _stream(dev))
    _check("hisa_index", st)
    return out_idx, out_score, out_blk


def hisa_append_index(K, pool_mean, L_old: int, L_new: int, q, w, B: int, m: int, k: int, qpos=None, *,
                      want_scores: bool = True, want_blocks: bool = False, out_idx=None, out_score=None,
                      out_blk=None, workspace=None, pool: str = "mean"):
    """One decode step: hisa_pool_append(K, pool_mean, L_old, L_new, B) then
    hisa_index(q, w, K, L_new, pool_mean, B, m, k, qpos), with the same results
    (the last block's mean is stored from the block stage when the appended
    rows all lie in it).  Returns (idx, score | None, blocks | None)."""
    S, T, H, d, kss = _query_args(q, w, qpos, K, L_new)
    _bf16(pool_mean, "pool_mean")
    pss = _rows(pool_mean, "pool_mean", d)
    if pool_mean.shape[0] != S or pool_mean.shape[1] * B < L_new:
        raise ValueError("pool_mean must be [S, >= ceil(L_new/B), d]")
    if pool_mean.device != q.device:
        raise ValueError("pool_mean must be on the query's device")
    dev = q.device
    out_idx = _out(out_idx, "out_idx", (S, T, k), torch.int32, dev)
    if want_scores or out_score is not None:
        out_score = _out(out_score, "out_score", (S, T, k), torch.float32, dev)
    if want_blocks or out_blk is not None:
        out_blk = _out(out_blk, "out_blk", (S, T, m), torch.int32, dev)
    if workspace is None:
        nbytes = hisa_index_workspace(S, T, H, d, L_new, B, m, k)
        if nbytes == 0:
            _check("hisa_append_index", lib().hisa_append_index(None, 0, int(L_old), int(L_new), None, 0, None,
                                                                None, None, S, T, H, d, B, m, k, None, None, None,
                                                                None, 0, None))
    ws = _workspace(None if workspace is not None else nbytes, dev, workspace)
    st = lib().hisa_append_index_mode(_ptr(K), kss, int(L_old), int(L_new), _ptr(pool_mean), pss, _ptr(q),
                                      _ptr(w), _ptr(qpos), S, T, H, d, B, m, k, _ptr(out_idx), _ptr(out_score),
                                      _ptr(out_blk), _ptr(ws), ws.numel() * ws.element_size(), _pool_kind(pool),
                                      _stream(dev))
    _check("hisa_append_index", st)
    return out_idx, out_score, out_blk


def hisa_append_index_static(K, pool_mean, L_old: int, L_new: int, q, w, B: int, m: int, k: int, qpos=None, *,
                             want_scores: bool = True, want_blocks: bool = False, out_idx=None, out_score=None,
                             out_blk=None):
    """hisa_append_index with the library's own static scratch as the workspace (mean pooling):
    the library allocates nothing.  With every output passed in, neither does this binding.
    Calls that could overlap on one GPU must not be issued (they share the scratch)."""
    S, T, H, d, kss = _query_args(q, w, qpos, K, L_new)
    _bf16(pool_mean, "pool_mean")
    pss = _rows(pool_mean, "pool_mean", d)
    if pool_mean.shape[0] != S or pool_mean.shape[1] * B < L_new:
        raise ValueError("pool_mean must be [S, >= ceil(L_new/B), d]")
    if pool_mean.device != q.device:
        raise ValueError("pool_mean must be on the query's device")
    dev = q.device
    out_idx = _out(out_idx, "out_idx", (S, T, k), torch.int32, dev)
    if want_scores or out_score is not None:
        out_score = _out(out_score, "out_score", (S, T, k), torch.float32, dev)
    if want_blocks or out_blk is not None:
        out_blk = _out(out_blk, "out_blk", (S, T, m), torch.int32, dev)
    st = lib().hisa_append_index_static(_ptr(K), kss, int(L_old), int(L_new), _ptr(pool_mean), pss, _ptr(q),
                                        _ptr(w), _ptr(qpos), S, T, H, d, B, m, k, _ptr(out_idx), _ptr(out_score),
                                        _ptr(out_blk), _stream(dev))
    _check("hisa_append_index_static", st)
    return out_idx, out_score, out_blk


def hisa_tree_append(K, pool_rep, spool_rep, L_old: int, L_new: int, B: int, G: int, pool: str = "mean"):
    """Fold key rows [L_old, L_new) of K [S, L_cap, d] into the block pool [S, nblk_cap, d] and the
    super-block pool [S, nsblk_cap, d] (super-blocks of G blocks), in place."""
    _bf16(K, "K")
    _bf16(pool_rep, "pool_rep")
    _bf16(spool_rep, "spool_rep")
    S, _, d = K.shape
    kss = _rows(K, "K", d)
    pss = _rows(pool_rep, "pool_rep", d)
    sss = _rows(spool_rep, "spool_rep", d)
    if pool_rep.shape[0] != S or spool_rep.shape[0] != S:
        raise ValueError("pool_rep, spool_rep and K disagree on S")
    if pool_rep.device != K.device or spool_rep.device != K.device:
        raise ValueError("pool_rep, spool_rep and K must be on the same device")
    nblk = -(-int(L_new) // B)
    if K.shape[1] < L_new or pool_rep.shape[1] < nblk or spool_rep.shape[1] * G < nblk:
        raise ValueError("K, pool_rep or spool_rep too short for L_new")
    st = lib().hisa_tree_append(_ptr(K), kss, S, d, B, G, int(L_old), int(L_new), _ptr(pool_rep), pss,
                                _ptr(spool_rep), sss, _pool_kind(pool), _stream(K.device))
    _check("hisa_tree_append", st)
    return pool_rep, spool_rep


def hisa_tree_index_workspace(S, T, H, d, L, B, G, W, m, k) -> int:
    return int(lib().hisa_tree_index_workspace(S, T, H, d, L, B, G, W, m, k))


def hisa_tree_index(q, w, K, L: int, pool_rep, spool_rep, B: int, G: int, W: int, m: int, k: int, qpos=None, *,
                    want_scores: bool = True, want_blocks: bool = False, want_super: bool = False,
                    out_idx=None, out_score=None, out_blk=None, out_sblk=None, workspace=None,
                    pool: str = "mean"):
    """Three-level indexer (super-blocks of G blocks, beam W, then m blocks, then k tokens).
    Returns (idx [S,T,k], score [S,T,k] | None, blocks [S,T,m] | None, super-blocks [S,T,W] | None)."""
    S, T, H, d, kss = _query_args(q, w, qpos, K, L)
    _bf16(pool_rep, "pool_rep")
    _bf16(spool_rep, "spool_rep")
    pss = _rows(pool_rep, "pool_rep", d)
    sss = _rows(spool_rep, "spool_rep", d)
    nblk = -(-int(L) // B)
    if pool_rep.shape[0] != S or pool_rep.shape[1] < nblk:
        raise ValueError("pool_rep must be [S, >= ceil(L/B), d]")
    if spool_rep.shape[0] != S or spool_rep.shape[1] * G < nblk:
        raise ValueError("spool_rep must be [S, >= ceil(ceil(L/B)/G), d]")
    if pool_rep.device != q.device or spool_rep.device != q.device:
        raise ValueError("pool_rep and spool_rep must be on the query's device")
    dev = q.device
    out_idx = _out(out_idx, "out_idx", (S, T, k), torch.int32, dev)
    if want_scores or out_score is not None:
        out_score = _out(out_score, "out_score", (S, T, k), torch.float32, dev)
    if want_blocks or out_blk is not None:
        out_blk = _out(out_blk, "out_blk", (S, T, m), torch.int32, dev)
    if want_super or out_sblk is not None:
        out_sblk = _out(out_sblk, "out_sblk", (S, T, W), torch.int32, dev)
    nbytes = hisa_tree_index_workspace(S, T, H, d, L, B, G, W, m, k)
    if nbytes == 0:
        _check("hisa_tree_index", lib().hisa_tree_index(None, None, None, None, 0, int(L), None, 0, None, 0, S, T,
                                                        H, d, B, G, W, m, k, None, None, None, None, None, 0,
                                                        _pool_kind(pool), None))
    ws = _workspace(nbytes, dev, workspace)
    st = lib().hisa_tree_index(_ptr(q), _ptr(w), _ptr(qpos), _ptr(K), kss, int(L), _ptr(pool_rep), pss,
                               _ptr(spool_rep), sss, S, T, H, d, B, G, W, m, k, _ptr(out_idx), _ptr(out_score),
                               _ptr(out_blk), _ptr(out_sblk), _ptr(ws), ws.numel() * ws.element_size(),
                               _pool_kind(pool), _stream(dev))
    _check("hisa_tree_index", st)
    return out_idx, out_score, out_blk, out_sblk


def dsa_flat_index(q, w, K, L: int, k: int, qpos=None, *, want_scores: bool = True,
                   out_idx=None, out_score=None, workspace=None):
    """Flat DSA indexer.  Returns (idx [S,T,k] int32, score [S,T,k] fp32 | None)."""
    S, T, H, d, kss = _query_args(q, w, qpos, K, L)
    dev = q.device
    out_idx = _out(out_idx, "out_idx", (S, T, k), torch.int32, dev)
    if want_scores or out_score is not None:
        out_score = _out(out_score, "out_score", (S, T, k), torch.float32, dev)
    if workspace is None:
        nbytes = dsa_flat_workspace(S, T, H, d, L, k)
        if nbytes == 0:
            _check("dsa_flat_index", lib().dsa_flat_index(None, None, None, None, 0, L, S, T, H, d, k,
                                                          None, None, None, 0, None))
    ws = _workspace(None if workspace is not None else nbytes, dev, workspace)
    st = lib().dsa_flat_index(_ptr(q), _ptr(w), _ptr(qpos), _ptr(K), kss, int(L), S, T, H, d, k,
                              _ptr(out_idx), _ptr(out_score), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(dev))
    _check("dsa_flat_index", st)
    return out_idx, out_score


def hisa_sparse_attention_workspace(S, T, Ha, Dk, Dv, k) -> int:
    return int(lib().hisa_sparse_attention_workspace(S, T, Ha, Dk, Dv, k))


def hisa_sparse_attention(q, kv, L: int, idx, Dv: int, scale: float, *, want_lse: bool = True, out=None,
                          lse=None, workspace=None):
    """Attention of q [S, T, Ha, Dk] over the listed tokens idx [S, T, k] (int32; entries outside
    [0, L) skipped) of the latent cache kv [S, L_cap, row] (key = first Dk entries of a row, value
    = first Dv).  Returns (out [S, T, Ha, Dv] fp32, lse [S, T, Ha] fp32 | None)."""
    _bf16(q, "q")
    _bf16(kv, "kv")
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [S, T, Ha, Dk] tensor")
    S, T, Ha, Dk = q.shape
    if kv.dim() != 3 or kv.shape[0] != S or kv.shape[1] < L or kv.shape[2] < Dk or kv.stride(2) != 1:
        raise ValueError("kv must be [S, >= L, >= Dk] with unit-stride rows")
    if idx.dtype != torch.int32 or idx.dim() != 3 or tuple(idx.shape[:2]) != (S, T) or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 [S, T, k] tensor")
    k = idx.shape[2]
    dev = q.device
    for t in (kv, idx):
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    out = _out(out, "out", (S, T, Ha, Dv), torch.float32, dev)
    if want_lse or lse is not None:
        lse = _out(lse, "lse", (S, T, Ha), torch.float32, dev)
    nbytes = hisa_sparse_attention_workspace(S, T, Ha, Dk, Dv, k)
    if nbytes == 0:
        _check("hisa_sparse_attention", lib().hisa_sparse_attention(None, None, 0, 0, int(L), None, S, T, Ha, Dk,
                                                                    Dv, k, float(scale), None, None, None, 0, None))
    ws = _workspace(nbytes, dev, workspace)
    st = lib().hisa_sparse_attention(_ptr(q), _ptr(kv), kv.stride(0), kv.stride(1), int(L), _ptr(idx), S, T, Ha,
                                     Dk, Dv, k, float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(dev))
    _check("hisa_sparse_attention", st)
    return out, lse


# ---------------------------------------------------------------- profiler

def profile_enable(max_launches: int):
    _check("hisa_profile_enable", lib().hisa_profile_enable(int(max_launches)))


def profile_read() -> dict:
    """{kernel name: (total_ms, launches)} for every kernel kind recorded since enable."""
    L = lib()
    out = {}
    for kind in range(L.hisa_kernel_kinds()):
        ms, n = C.c_double(0.0), C.c_int(0)
        _check("hisa_profile_read", L.hisa_profile_read(kind, C.byref(ms), C.byref(n)))
        if n.value:
            out[L.hisa_kernel_name(kind).decode()] = (ms.value, n.value)
    return out
