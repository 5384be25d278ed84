"""Seeded synthetic inputs for the HISA indexer and the flat DSA indexer.

This module only *builds inputs*: random keys, queries, head weights, query
positions and planted "needle" keys.  It holds none of the method's
arithmetic (no pooling, no scoring, no selection), so both the HIP path and the
CPU oracle can consume the very same arrays without sharing any code that
decides a result.

All floating-point tensors that the indexer reads as bf16 (keys K, queries q)
are returned as raw bf16 bit patterns (``uint16``), produced from float32
samples by round-to-nearest-even.  Head weights w stay float32.

The workloads stand in for the pages' kernel-level benchmarks (context lengths
32K / 64K / 128K, plus a prefill chunk): the pages evaluate on trained models
and public suites that are not reproduced here, so keys are drawn from a
block-clustered Gaussian model (a latent vector per 128-token block plus token
noise) and queries mix three block latents, which gives the block structure
that coarse block filtering is meant to exploit.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_BASE = 20260330


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Case:
    """One indexer workload.

    K     uint16 [S, L, d]      bf16 key cache (row j of sequence s = K[s, j])
    q     uint16 [S, T, H, d]   bf16 indexer queries
    w     float32 [S, T, H]     per-head weights
    qpos  int32 [S, T]          query positions t (0-based), each < L
    L     keys present in the cache
    B, m, k                     block size, kept blocks, kept tokens
    L_bulk                      rows folded into the block pool in one call
                                before the remaining rows are appended one by one
    needles int64 [S, n] | None positions of planted needle keys
    """

    name: str
    K: np.ndarray
    q: np.ndarray
    w: np.ndarray
    qpos: np.ndarray
    L: int
    B: int
    m: int
    k: int
    L_bulk: int = -1
    needles: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def S(self) -> int:
        return int(self.K.shape[0])

    @property
    def T(self) -> int:
        return int(self.q.shape[1])

    @property
    def H(self) -> int:
        return int(self.q.shape[2])

    @property
    def d(self) -> int:
        return int(self.q.shape[3])

    def __post_init__(self):
        if self.L_bulk < 0:
            self.L_bulk = self.L


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _default_qpos(S: int, T: int, L: int) -> np.ndarray:
    return np.broadcast_to(np.arange(L - T, L, dtype=np.int32), (S, T)).copy()


def gaussian_case(S, L, T, H, d, B, m, k, seed, qpos=None, w_scale=0.5, name="gaussian"):
    """K ~ N(0,1), q ~ N(0,1), w ~ N(0,1)*w_scale; queries at the last T positions by default."""
    rng = _rng(seed)
    K = rng.standard_normal((S, L, d), dtype=np.float32)
    q = rng.standard_normal((S, T, H, d), dtype=np.float32)
    w = (rng.standard_normal((S, T, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    qp = _default_qpos(S, T, L) if qpos is None else np.asarray(qpos, dtype=np.int32).reshape(S, T)
    return Case(name, bf16_bits(K), bf16_bits(q), w, qp, L, B, m, k)


def clustered_case(S, L, T, H, d, B, m, k, seed, qpos=None, latent_block=128, w_scale=0.125,
                   needles_per_seq=0, needle_gain=3.0, L_bulk=None, name="clustered"):
    """Block-clustered keys and latent-mixture queries.

    K[s, j] = 0.6 * z[s, j // latent_block] + 0.8 * eps[s, j]    with z, eps ~ N(0, I_d)
    q[s, i, h] = (z_a + z_b + z_c) / sqrt(3) + N(0, I_d)          a, b, c uniform over the
                                                                  latent blocks <= the query's own
    w ~ N(0, 1) * w_scale
    Needles: at depths floor(L * (i + 1/2) / n), i < n, the key is replaced by
    needle_gain * sqrt(d) * q_h / |q_h| for a head h of that sequence's first query
    with w_h > 0 (a key aligned with a positively weighted head).
    """
    rng = _rng(seed)
    nlat = -(-L // latent_block)
    z = rng.standard_normal((S, nlat, d), dtype=np.float32)
    K = rng.standard_normal((S, L, d), dtype=np.float32)
    K *= np.float32(0.8)
    for s in range(S):
        K[s] += np.float32(0.6) * np.repeat(z[s], latent_block, axis=0)[:L]
    qp = _default_qpos(S, T, L) if qpos is None else np.asarray(qpos, dtype=np.int32).reshape(S, T)
    nlat_q = np.clip(qp.astype(np.int64), 0, L - 1) // latent_block + 1   # latent blocks visible to each query
    lat = rng.integers(0, nlat_q[..., None], size=(S, T, 3))
    q = rng.standard_normal((S, T, H, d), dtype=np.float32)
    sidx = np.arange(S)[:, None, None]
    mix = z[sidx, lat].sum(axis=2) / np.float32(np.sqrt(3.0))     # [S, T, d]
    q += mix[:, :, None, :]
    w = (rng.standard_normal((S, T, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    Kb = bf16_bits(K)
    qb = bf16_bits(q)
    needles = None
    if needles_per_seq > 0:
        needles = np.zeros((S, needles_per_seq), dtype=np.int64)
        qf = bf16_to_f32(qb)
        for s in range(S):
            pos_heads = np.nonzero(w[s, 0] > 0)[0]
            for i in range(needles_per_seq):
                j = int(np.floor(L * (i + 0.5) / needles_per_seq))
                h = int(pos_heads[rng.integers(0, len(pos_heads))])
                v = qf[s, 0, h].astype(np.float64)
                key = needle_gain * np.sqrt(d) * v / np.linalg.norm(v)
                Kb[s, j] = bf16_bits(key.astype(np.float32))
                needles[s, i] = j
    return Case(name, Kb, qb, w, qp, L, B, m, k, L_bulk=(L if L_bulk is None else L_bulk),
                needles=needles)


# The five workloads: one tiny correctness case, three long-context decode batches
# and one prefill chunk; then two decode batches past a million keys, for the
# three-level tree.  Index i uses seed SEED_BASE + i.
WORKLOADS = {
    0: "tiny_L1024",
    1: "decode_L32K",
    2: "decode_L64K_needles",
    3: "decode_L128K_tail77",
    4: "prefill_T4096_L128K",
    5: "decode_L1M",
    6: "decode_L4M",
}


def workload(i: int, sequences: int | None = None) -> Case:
    """Workload i; `sequences` replaces the batch size of a decode workload
    (1..3, 5, 6) to study how the decode path scales with batch (the name then gains
    an _S<n> suffix)."""
    seed = SEED_BASE + i
    if sequences is not None and i not in (1, 2, 3, 5, 6):
        raise ValueError("only the decode workloads (1..3, 5, 6) take another batch size")
    if i == 0:
        c = gaussian_case(1, 1024, 16, 4, 64, 64, 4, 64, seed, w_scale=0.5)
    elif i == 1:
        c = clustered_case(sequences or 8, 32768, 1, 64, 128, 128, 64, 2048, seed)
    elif i == 2:
        c = clustered_case(sequences or 4, 65536, 1, 64, 128, 128, 64, 2048, seed, needles_per_seq=8)
    elif i == 3:
        c = clustered_case(sequences or 2, 131072 + 77, 1, 64, 128, 128, 128, 2048, seed, L_bulk=131072)
    elif i == 4:
        c = clustered_case(1, 131072, 4096, 64, 128, 128, 64, 2048, seed)
    elif i == 5:
        c = clustered_case(sequences or 4, 1 << 20, 1, 64, 128, 128, 64, 2048, seed, needles_per_seq=8)
    elif i == 6:
        c = clustered_case(sequences or 1, 1 << 22, 1, 64, 128, 128, 64, 2048, seed, needles_per_seq=8)
    else:
        raise ValueError(f"no workload {i}")
    c.name = WORKLOADS[i] + (f"_S{sequences}" if sequences is not None else "")
    return c
