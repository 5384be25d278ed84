"""ctypes wrapper over the C oracle (oracle/hisa_oracle.c, oracle/attention_oracle.c) -- TEST INFRASTRUCTURE ONLY.

Arguments are numpy arrays; bf16 tensors are passed as uint16 bit patterns.
Every function here only marshals arguments; all arithmetic is in the C file.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhisa_oracle.so")
_lib = None

_u16p = C.POINTER(C.c_uint16)
_f32p = C.POINTER(C.c_float)
_f64p = C.POINTER(C.c_double)
_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)


def load():
    """Load the oracle library, building it first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build
        build()
    lib = C.CDLL(_LIB_PATH)
    I64, I = C.c_int64, C.c_int
    lib.oracle_score.restype = C.c_double
    lib.oracle_score.argtypes = [_u16p, _f32p, _u16p, I, I]
    lib.oracle_mean_rows.restype = None
    lib.oracle_mean_rows.argtypes = [_u16p, I64, I64, I, _u16p]
    lib.oracle_pool.restype = None
    lib.oracle_pool.argtypes = [_u16p, I64, I, I64, I, I, _u16p]
    lib.oracle_max_rows.restype = None
    lib.oracle_max_rows.argtypes = [_u16p, I64, I64, I, _u16p]
    lib.oracle_pool_mode.restype = None
    lib.oracle_pool_mode.argtypes = [_u16p, I64, I, I64, I, I, I, _u16p]
    lib.oracle_flat_query.restype = I
    lib.oracle_flat_query.argtypes = [_u16p, _f32p, _u16p, I, I, I64, I, _i32p, _f32p, _f64p]
    lib.oracle_refine_query.restype = I
    lib.oracle_refine_query.argtypes = [_u16p, _f32p, _u16p, I, I, I64, I, _i32p, I, I,
                                        _i32p, _f32p, _i64p]
    lib.oracle_hisa_query.restype = I
    lib.oracle_hisa_query.argtypes = [_u16p, _f32p, _u16p, _u16p, I, I, I64, I, I, I,
                                      _i32p, _f32p, _i32p, _f64p]
    lib.oracle_hisa_query_mode.restype = I
    lib.oracle_hisa_query_mode.argtypes = [_u16p, _f32p, _u16p, _u16p, I, I, I64, I, I, I, I,
                                           _i32p, _f32p, _i32p, _f64p]
    lib.oracle_super_pool.restype = I
    lib.oracle_super_pool.argtypes = [_u16p, I64, I, I64, I, I, I, I, _u16p]
    lib.oracle_tree_query.restype = I
    lib.oracle_tree_query.argtypes = [_u16p, _f32p, _u16p, I, I, I64, I, I, I, I, I, I, _i32p, _f32p,
                                      _i32p, _i32p, _f64p]
    lib.oracle_block_sparse_query.restype = I
    lib.oracle_block_sparse_query.argtypes = [_u16p, _f32p, _u16p, I, I, I64, I, I, _i32p, _i32p]
    lib.oracle_hisa_batch.restype = I
    lib.oracle_hisa_batch.argtypes = [_u16p, _f32p, _i32p, _u16p, I64, I64, I, I, I, I, I, I,
                                      I, _i32p, I, _i32p, _f32p, _i32p]
    lib.oracle_hisa_batch_mode.restype = I
    lib.oracle_hisa_batch_mode.argtypes = [_u16p, _f32p, _i32p, _u16p, I64, I64, I, I, I, I, I, I,
                                           I, I, _i32p, I, _i32p, _f32p, _i32p]
    lib.oracle_flat_batch.restype = I
    lib.oracle_flat_batch.argtypes = [_u16p, _f32p, _i32p, _u16p, I64, I64, I, I, I, I, I,
                                      _i32p, I, _i32p, _f32p]
    lib.oracle_sparse_attention.restype = I
    lib.oracle_sparse_attention.argtypes = [_u16p, I, I, I, _u16p, I64, I64, _i32p, I, C.c_double, _f64p, _f64p,
                                            _f64p]
    lib.oracle_sparse_attention_batch.restype = I
    lib.oracle_sparse_attention_batch.argtypes = [_u16p, I, I, I, I, I, _u16p, I64, I64, I64, _i32p, I,
                                                  C.c_double, _i32p, I, _f64p, _f64p, _f64p]
    lib.oracle_num_threads.restype = I
    lib.oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _p(a: np.ndarray, ptype):
    return a.ctypes.data_as(ptype)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(load().oracle_num_threads())


def score(q: np.ndarray, w: np.ndarray, x: np.ndarray) -> float:
    """s(q, w, x) for one query q [H, d] (bf16 bits), w [H], key x [d] (bf16 bits)."""
    q, w, x = _c(q, np.uint16), _c(w, np.float32), _c(x, np.uint16)
    H, d = q.shape
    return float(load().oracle_score(_p(q, _u16p), _p(w, _f32p), _p(x, _u16p), H, d))


def mean_rows(K: np.ndarray, row0: int, row1: int) -> np.ndarray:
    """bf16 bits of the representative of rows [row0, row1) of K [L, d]."""
    K = _c(K, np.uint16)
    out = np.zeros(K.shape[1], dtype=np.uint16)
    load().oracle_mean_rows(_p(K, _u16p), row0, row1, K.shape[1], _p(out, _u16p))
    return out


_MODES = {"mean": 0, "max": 1}


def _mode(mode: str) -> int:
    if mode not in _MODES:
        raise ValueError(f"pooling must be one of {sorted(_MODES)}")
    return _MODES[mode]


def max_rows(K: np.ndarray, row0: int, row1: int) -> np.ndarray:
    """bf16 bits of the max-pooled representative of rows [row0, row1) of K [L, d]."""
    K = _c(K, np.uint16)
    out = np.zeros(K.shape[1], dtype=np.uint16)
    load().oracle_max_rows(_p(K, _u16p), row0, row1, K.shape[1], _p(out, _u16p))
    return out


def pool(K: np.ndarray, L: int, B: int, mode: str = "mean") -> np.ndarray:
    """Block representatives [S, ceil(L/B), d] (bf16 bits) of K [S, L_cap, d] holding L rows;
    mode "mean" or "max"."""
    K = _c(K, np.uint16)
    S, Lcap, d = K.shape
    nblk = -(-L // B)
    out = np.zeros((S, nblk, d), dtype=np.uint16)
    load().oracle_pool_mode(_p(K, _u16p), Lcap * d, S, L, d, B, _mode(mode), _p(out, _u16p))
    return out


def super_pool(K: np.ndarray, L: int, B: int, G: int, mode: str = "mean") -> np.ndarray:
    """Super-block representatives [S, ceil(ceil(L/B)/G), d] of the three-level tree over
    K [S, L_cap, d] holding L rows: per super-block of G blocks, the mean over its keys
    formed from its block representatives weighted by their key counts ("mean"), or the
    max of their maxima ("max")."""
    K = _c(K, np.uint16)
    S, Lcap, d = K.shape
    nsb = -(-(-(-L // B)) // G)
    out = np.zeros((S, nsb, d), dtype=np.uint16)
    if load().oracle_super_pool(_p(K, _u16p), Lcap * d, S, L, d, B, G, _mode(mode), _p(out, _u16p)) != 0:
        raise MemoryError("oracle_super_pool failed")
    return out


def flat_query(q, w, K, t: int, k: int, want_all=False):
    """Flat DSA top-k for one query: (idx [k], score [k], k_eff[, all fp64 scores [t+1]])."""
    q, w, K = _c(q, np.uint16), _c(w, np.float32), _c(K, np.uint16)
    H, d = q.shape
    idx = np.zeros(k, dtype=np.int32)
    sc = np.zeros(k, dtype=np.float32)
    allsc = np.zeros(t + 1, dtype=np.float64) if want_all else None
    keff = load().oracle_flat_query(_p(q, _u16p), _p(w, _f32p), _p(K, _u16p), H, d, t, k,
                                    _p(idx, _i32p), _p(sc, _f32p),
                                    _p(allsc, _f64p) if want_all else None)
    if keff < 0:
        raise MemoryError("oracle_flat_query failed")
    return (idx, sc, keff, allsc) if want_all else (idx, sc, keff)


def refine_query(q, w, K, t: int, B: int, blocks, k: int):
    """Top-k over the tokens j <= t of the given blocks: (idx [k], score [k], k_eff, |C|)."""
    q, w, K = _c(q, np.uint16), _c(w, np.float32), _c(K, np.uint16)
    blocks = _c(blocks, np.int32)
    H, d = q.shape
    idx = np.zeros(k, dtype=np.int32)
    sc = np.zeros(k, dtype=np.float32)
    n = C.c_int64(0)
    keff = load().oracle_refine_query(_p(q, _u16p), _p(w, _f32p), _p(K, _u16p), H, d, t, B,
                                      _p(blocks, _i32p), len(blocks), k, _p(idx, _i32p),
                                      _p(sc, _f32p), C.byref(n))
    if keff < 0:
        raise MemoryError("oracle_refine_query failed")
    return idx, sc, keff, int(n.value)


def hisa_query(q, w, K, t: int, B: int, m: int, k: int, mode: str = "mean"):
    """HISA for one query: (idx [k], score [k], blocks [m], block scores fp64 [t//B+1], k_eff).
    mode: block representatives by "mean" or "max" pooling."""
    q, w, K = _c(q, np.uint16), _c(w, np.float32), _c(K, np.uint16)
    H, d = q.shape
    idx = np.zeros(k, dtype=np.int32)
    sc = np.zeros(k, dtype=np.float32)
    blk = np.zeros(m, dtype=np.int32)
    bsc = np.zeros(t // B + 1, dtype=np.float64)
    keff = load().oracle_hisa_query_mode(_p(q, _u16p), _p(w, _f32p), _p(K, _u16p), None, H, d, t,
                                         B, m, k, _mode(mode), _p(idx, _i32p), _p(sc, _f32p),
                                         _p(blk, _i32p), _p(bsc, _f64p))
    if keff < 0:
        raise MemoryError("oracle_hisa_query failed")
    return idx, sc, blk, bsc, keff


def tree_query(q, w, K, t: int, B: int, G: int, W: int, m: int, k: int, mode: str = "mean"):
    """Three-level HISA for one query (super-blocks of G blocks of B keys; W super-blocks,
    m blocks, k tokens kept): (idx [k], score [k], blocks [m], super-blocks [W], k_eff)."""
    q, w, K = _c(q, np.uint16), _c(w, np.float32), _c(K, np.uint16)
    H, d = q.shape
    idx = np.zeros(k, dtype=np.int32)
    sc = np.zeros(k, dtype=np.float32)
    blk = np.zeros(m, dtype=np.int32)
    sblk = np.zeros(W, dtype=np.int32)
    keff = load().oracle_tree_query(_p(q, _u16p), _p(w, _f32p), _p(K, _u16p), H, d, t, B, G, W, m, k,
                                    _mode(mode), _p(idx, _i32p), _p(sc, _f32p), _p(blk, _i32p),
                                    _p(sblk, _i32p), None)
    if keff < 0:
        raise MemoryError("oracle_tree_query failed")
    return idx, sc, blk, sblk, keff


def tree_super_scores(q, w, K, t: int, B: int, G: int, mode: str = "mean"):
    """Scores (fp64) of every super-block u <= t // (B*G) as the three-level tree ranks them."""
    q, w, K = _c(q, np.uint16), _c(w, np.float32), _c(K, np.uint16)
    H, d = q.shape
    idx, sc = np.zeros(1, dtype=np.int32), np.zeros(1, dtype=np.float32)
    blk, sblk = np.zeros(1, dtype=np.int32), np.zeros(1, dtype=np.int32)
    ssc = np.zeros(t // (B * G) + 1, dtype=np.float64)
    keff = load().oracle_tree_query(_p(q, _u16p), _p(w, _f32p), _p(K, _u16p), H, d, t, B, G, 1, 1, 1,
                                    _mode(mode), _p(idx, _i32p), _p(sc, _f32p), _p(blk, _i32p),
                                    _p(sblk, _i32p), _p(ssc, _f64p))
    if keff < 0:
        raise MemoryError("oracle_tree_query failed")
    return ssc


def block_sparse_query(q, w, K, t: int, B: int, k: int):
    """Block-sparse baseline for one query: (token idx [k] ascending then -1, blocks [k//B], count)."""
    q, w, K = _c(q, np.uint16), _c(w, np.float32), _c(K, np.uint16)
    H, d = q.shape
    idx = np.zeros(k, dtype=np.int32)
    blk = np.zeros(max(1, k // B), dtype=np.int32)
    n = load().oracle_block_sparse_query(_p(q, _u16p), _p(w, _f32p), _p(K, _u16p), H, d, t, B, k,
                                         _p(idx, _i32p), _p(blk, _i32p))
    if n < 0:
        raise ValueError("oracle_block_sparse_query: k < B or out of memory")
    return idx, blk, n


def _sel(sel, S, T):
    if sel is None:
        return None, 0
    s = _c(sel, np.int32)
    if s.size and (s.min() < 0 or s.max() >= S * T):
        raise ValueError("query id out of range")
    return s, len(s)


def hisa_batch(q, w, qpos, K, L: int, B: int, m: int, k: int, sel=None, mode: str = "mean"):
    """HISA over a batch q [S,T,H,d]; returns (idx [S,T,k], score [S,T,k], blocks [S,T,m]).
    With sel (flat ids s*T+i) only those rows are filled; mode: "mean" or "max" pooling."""
    q, w, qpos, K = _c(q, np.uint16), _c(w, np.float32), _c(qpos, np.int32), _c(K, np.uint16)
    S, T, H, d = q.shape
    s_arr, ns = _sel(sel, S, T)
    idx = np.full((S, T, k), -2, dtype=np.int32)
    sc = np.zeros((S, T, k), dtype=np.float32)
    blk = np.full((S, T, m), -2, dtype=np.int32)
    r = load().oracle_hisa_batch_mode(_p(q, _u16p), _p(w, _f32p), _p(qpos, _i32p), _p(K, _u16p),
                                      K.shape[1] * d, L, S, T, H, d, B, m, k, _mode(mode),
                                      _p(s_arr, _i32p) if s_arr is not None else None, ns,
                                      _p(idx, _i32p), _p(sc, _f32p), _p(blk, _i32p))
    if r != 0:
        raise ValueError("oracle_hisa_batch failed (bad position or out of memory)")
    return idx, sc, blk


def flat_batch(q, w, qpos, K, L: int, k: int, sel=None):
    """Flat DSA over a batch; returns (idx [S,T,k], score [S,T,k])."""
    q, w, qpos, K = _c(q, np.uint16), _c(w, np.float32), _c(qpos, np.int32), _c(K, np.uint16)
    S, T, H, d = q.shape
    s_arr, ns = _sel(sel, S, T)
    idx = np.full((S, T, k), -2, dtype=np.int32)
    sc = np.zeros((S, T, k), dtype=np.float32)
    r = load().oracle_flat_batch(_p(q, _u16p), _p(w, _f32p), _p(qpos, _i32p), _p(K, _u16p),
                                 K.shape[1] * d, L, S, T, H, d, k,
                                 _p(s_arr, _i32p) if s_arr is not None else None, ns,
                                 _p(idx, _i32p), _p(sc, _f32p))
    if r != 0:
        raise ValueError("oracle_flat_batch failed (bad position or out of memory)")
    return idx, sc


def sparse_attention(q, kv, idx, Dv: int, scale: float, L: int | None = None):
    """Attention of one query q [Ha, Dk] over the listed tokens idx [k] of the latent cache kv
    [L, >= Dk] (key = first Dk entries of a row, value = first Dv).  Entries outside [0, L) are
    skipped.  Returns (out [Ha, Dv], lse [Ha], absw [Ha, Dv]) in fp64."""
    q, kv, idx = _c(q, np.uint16), _c(kv, np.uint16), _c(idx, np.int32)
    Ha, Dk = q.shape
    L = kv.shape[0] if L is None else L
    out = np.zeros((Ha, Dv), dtype=np.float64)
    absw = np.zeros((Ha, Dv), dtype=np.float64)
    lse = np.zeros(Ha, dtype=np.float64)
    st = load().oracle_sparse_attention(_p(q, _u16p), Ha, Dk, Dv, _p(kv, _u16p), kv.shape[1], L,
                                        _p(idx, _i32p), len(idx), float(scale), _p(out, _f64p), _p(lse, _f64p),
                                        _p(absw, _f64p))
    if st != 0:
        raise MemoryError("oracle_sparse_attention failed")
    return out, lse, absw


def sparse_attention_batch(q, kv, idx, Dv: int, scale: float, L: int, sel=None):
    """Batch form: q [S, T, Ha, Dk], kv [S, L_cap, row], idx [S, T, k]; returns (out [S,T,Ha,Dv],
    lse [S,T,Ha], absw [S,T,Ha,Dv]) (rows not in sel are left zero)."""
    q, kv, idx = _c(q, np.uint16), _c(kv, np.uint16), _c(idx, np.int32)
    S, T, Ha, Dk = q.shape
    k = idx.shape[-1]
    out = np.zeros((S, T, Ha, Dv), dtype=np.float64)
    absw = np.zeros((S, T, Ha, Dv), dtype=np.float64)
    lse = np.zeros((S, T, Ha), dtype=np.float64)
    s, n = _sel(sel, S, T)
    st = load().oracle_sparse_attention_batch(_p(q, _u16p), S, T, Ha, Dk, Dv, _p(kv, _u16p),
                                              kv.shape[1] * kv.shape[2], kv.shape[2], L, _p(idx, _i32p), k,
                                              float(scale), None if s is None else _p(s, _i32p), n,
                                              _p(out, _f64p), _p(lse, _f64p), _p(absw, _f64p))
    if st != 0:
        raise MemoryError("oracle_sparse_attention_batch failed")
    return out, lse, absw
