"""GPU: the workgroup top-k selection is exact on the GPU's own scores.

The selection ranks fp32 scores by (score desc, index asc).  These tests take
every candidate's score from the GPU itself (the flat indexer with k at least
the row length keeps every candidate and returns its score), rank them with
numpy's stable sort, and require the GPU's top-k set to equal that ranking
bit for bit.  The score distributions drive the radix passes down their
branches: a Gaussian spread; scores crowded into one narrow band, so the
cutoff is decided in the last digit; long runs of equal scores, cut by
index; one score far above the rest; scores that are all zero or negative;
rows shorter than k (every candidate kept).  Row lengths cover one, eight
and sixteen keys per thread, and a batch of more than 1024 queries (the
512-thread selection).
"""
import sys

import numpy as np
import pytest

from sparse_attention_token_amd import synth
from parity import to_dev

pytestmark = pytest.mark.gpu

KINDS = ["gauss", "narrow", "ties", "outlier", "negative", "short"]


@pytest.fixture(scope="module")
def hisa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_attention_token_amd import hisa as h

    h.lib()
    return h


def _case(kind, L, T, seed):
    import dataclasses

    H, d = 4, 64
    qpos = np.linspace(L // 3, L - 1, T).astype(np.int32)[None, :]
    c = synth.gaussian_case(1, L, T, H, d, 64, 4, 64, seed=seed, qpos=qpos)
    if kind in ("gauss", "short"):
        return c
    rng = np.random.default_rng(seed)
    base = np.abs(rng.standard_normal(d)).astype(np.float32) + 0.25
    base[0] = 0.0
    K = np.broadcast_to(base, (1, L, d)).copy()
    q = np.broadcast_to(base, (1, T, H, d)).copy()
    q[..., 0] = 1.0
    w = np.abs(rng.standard_normal((1, T, H))).astype(np.float32) + 0.1
    if kind == "narrow":
        # one coordinate carries a tiny distinct offset per key: every score
        # lies within about 2^-12 of the others
        K[0, :, 0] = rng.random(L).astype(np.float32) * 0.01
    elif kind == "ties":
        # three distinct rows repeated: three score values, thousands of keys each
        K[0, :, 0] = (np.arange(L) % 3).astype(np.float32) * 0.5
    elif kind == "outlier":
        K[0, :, 0] = rng.random(L).astype(np.float32) * 0.01
        K[0, L // 2] *= 4096.0
    elif kind == "negative":
        K = rng.standard_normal((1, L, d)).astype(np.float32)
        q = rng.standard_normal((1, T, H, d)).astype(np.float32)
        w = -w                                    # every score <= 0, many exactly 0
    return dataclasses.replace(c, K=synth.bf16_bits(K), q=synth.bf16_bits(q), w=w)


def _exact_topk(scores, n, k):
    """Indices of the top min(k, n) of scores[:n] by (score desc, index asc)."""
    s = scores[:n].astype(np.float32)
    s = np.where(s == 0.0, np.float32(0.0), s)            # -0 ties +0
    order = np.lexsort((np.arange(n), -s.astype(np.float64)))
    return np.sort(order[:min(k, n)])


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("L,T", [(1000, 4), (8192, 4), (16384, 3), (6000, 1100)],
                         ids=["R1", "R8", "R16", "many"])
def test_top_k_exact_on_gpu_scores(hisa, kind, L, T):
    import torch

    k = 5000 if kind == "short" else 700
    c = _case(kind, L, T, seed=L + T)
    dev = to_dev(c)
    n_max = int(c.qpos.max()) + 1
    # every candidate's score: k covers the longest row, so nothing is dropped
    aidx, asc = hisa.dsa_flat_index(dev["q"], dev["w"], dev["K"], L, n_max, dev["qpos"])
    idx, sc = hisa.dsa_flat_index(dev["q"], dev["w"], dev["K"], L, k, dev["qpos"])
    torch.cuda.synchronize()
    aidx, asc, idx, sc = (x.cpu().numpy() for x in (aidx, asc, idx, sc))
    for i in range(T):
        n = int(c.qpos[0, i]) + 1
        np.testing.assert_array_equal(aidx[0, i, :n], np.arange(n))
        want = _exact_topk(asc[0, i], n, k)
        got = idx[0, i]
        keff = min(k, n)
        assert np.all(got[keff:] == -1), f"{kind} query {i}: padding"
        np.testing.assert_array_equal(got[:keff], want, err_msg=f"{kind} query {i} (n={n})")
        np.testing.assert_array_equal(sc[0, i, :keff].view(np.uint32), asc[0, i, want].view(np.uint32))
    print(f"select {kind} L={L} T={T}: exact", flush=True)
    sys.stdout.flush()
