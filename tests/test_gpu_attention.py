"""GPU parity of the sparse attention over a selected token set (hisa_sparse_attention, through
the C ABI) against the fp64 CPU oracle.

Tolerance, from the arithmetic: the GPU rounds each softmax weight to bf16 (relative error at
most 2^-9) and normalises by the sum of the rounded weights, so its output is a convex
combination of the values whose weights are within 2^-8 of the exact ones, relative; with the
fp32 score and accumulation errors (below 1e-3 relative at these sizes) every output element
satisfies  |o_gpu - o| <= (2^-8 + 1e-3) * sum_j w_j |v_j| + 1e-6,  the sum being the oracle's
weighted mean magnitude of that value column (absw).  The log-sum-exp moves by the relative
error of the weight sum: |lse_gpu - lse| <= 2^-8 + 1e-5 |lse|.
"""
import sys
import zlib

import numpy as np
import pytest

from sparse_attention_token_amd import synth
from parity import bits

pytestmark = pytest.mark.gpu

OUT_REL = 2.0 ** -8 + 1e-3
LSE_ABS = 2.0 ** -8


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def hisa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_attention_token_amd import hisa as h

    h.lib()
    return h


def _case(name, S, T, Ha, Dk, L, k, row_pad=0, q_scale=0.05):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    kv = synth.bf16_bits(rng.standard_normal((S, L, Dk + row_pad)).astype(np.float32))
    q = synth.bf16_bits((rng.standard_normal((S, T, Ha, Dk)) * q_scale).astype(np.float32))
    idx = np.stack([[rng.choice(L, size=k, replace=False) for _ in range(T)] for _ in range(S)]).astype(np.int32)
    return q, kv, idx


def _to_dev(q, kv, idx):
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    return bf(q), bf(kv), torch.from_numpy(np.ascontiguousarray(idx)).cuda()


def _check(orc, q, kv, idx, Dv, scale, L, out, lse, rows=None):
    S, T = q.shape[:2]
    sel = None if rows is None else np.array([s * T + i for s, i in rows], dtype=np.int32)
    ref, rlse, absw = orc.sparse_attention_batch(q, kv, idx, Dv, scale, L, sel=sel)
    pairs = [(s, i) for s in range(S) for i in range(T)] if rows is None else rows
    worst = 0.0
    for s, i in pairs:
        err = np.abs(out[s, i].astype(np.float64) - ref[s, i])
        bound = OUT_REL * absw[s, i] + 1e-6
        assert np.all(err <= bound), f"query ({s},{i}): max excess {np.max(err - bound)}"
        worst = max(worst, float(np.max(err / bound)))
        fin = np.isfinite(rlse[s, i])
        assert np.all(np.isneginf(lse[s, i][~fin])), "empty sets give -inf"
        d = np.abs(lse[s, i][fin].astype(np.float64) - rlse[s, i][fin])
        assert np.all(d <= LSE_ABS + 1e-5 * np.abs(rlse[s, i][fin]))
    return worst


CASES = [
    # name, S, T, Ha, Dk, Dv, L, k, row padding, query scale (scores of std about this size)
    ("latent_576_512_h128", 2, 1, 128, 576, 512, 5000, 2048, 0, 0.05),
    ("latent_peaked", 1, 3, 128, 576, 512, 5000, 2048, 0, 3.0),
    ("d128_peaked", 2, 2, 32, 128, 128, 3000, 700, 0, 6.0),
    ("d128_h16_ragged", 1, 4, 16, 128, 128, 3000, 300, 0, 0.05),
    ("d64_h32_padded_rows", 2, 3, 32, 64, 64, 1000, 100, 16, 0.05),
    ("d192_v128_h48", 1, 2, 48, 192, 128, 2000, 500, 0, 1.0),
    ("many_queries_one_split", 1, 600, 32, 128, 128, 4096, 256, 0, 1.0),
    ("latent_h16_long_set", 1, 2, 16, 576, 512, 40000, 16384, 0, 0.5),
]


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_sparse_attention(hisa, orc, spec):
    import torch

    name, S, T, Ha, Dk, Dv, L, k, pad, qs = spec
    _say(f"attention {name}")
    q, kv, idx = _case(name, S, T, Ha, Dk, L, k, pad, qs)
    # padding, out-of-range entries and a repeated token in some rows
    idx[0, 0, -7:] = -1
    if T > 1:
        idx[0, 1, 3] = L + 5
        idx[0, 1, 4] = idx[0, 1, 5]
    scale = 1.0 / np.sqrt(Dk)
    dq, dkv, didx = _to_dev(q, kv, idx)
    out, lse = hisa.hisa_sparse_attention(dq, dkv, L, didx, Dv, scale)
    torch.cuda.synchronize()
    rows = None if S * T <= 16 else [(0, i) for i in range(0, T, 37)]
    worst = _check(orc, q, kv, idx, Dv, scale, L, out.cpu().numpy(), lse.cpu().numpy(), rows)
    _say(f"  worst error / bound = {worst:.3f}")


def test_empty_and_single_sets(hisa, orc):
    import torch

    q, kv, idx = _case("empty", 1, 3, 32, 128, 500, 70)
    idx[0, 0, :] = -1                      # nothing selected
    idx[0, 1, :] = -1
    idx[0, 1, 40] = 17                     # exactly one token
    dq, dkv, didx = _to_dev(q, kv, idx)
    out, lse = hisa.hisa_sparse_attention(dq, dkv, 500, didx, 128, 0.3)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(out[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))
    v = synth.bf16_to_f32(kv[0, 17, :128])
    for h in range(32):
        np.testing.assert_array_equal(out[0, 1, h], v)    # one weight of exactly 1
    _check(orc, q, kv, idx, 128, 0.3, 500, out, lse)


def test_attention_over_indexer_output(hisa, orc):
    """End to end, in the benchmark's launch configuration: the HISA index set of the decode
    workload (8 sequences x 32K keys) feeds the attention over a latent cache of the same length
    (576-entry keys, 512-entry values, 128 heads), every query checked."""
    import torch

    c = synth.workload(1)
    from parity import to_dev, build_pool

    dev = to_dev(c)
    pool = build_pool(hisa, dev["K"], c.L, c.B)
    idx, _, _ = hisa.hisa_index(dev["q"], dev["w"], dev["K"], c.L, pool, c.B, c.m, c.k, None)
    rng = np.random.default_rng(11)
    kv = synth.bf16_bits(rng.standard_normal((c.S, c.L, 576)).astype(np.float32))
    q = synth.bf16_bits((rng.standard_normal((c.S, c.T, 128, 576)) * 0.05).astype(np.float32))
    dq, dkv, _ = _to_dev(q, kv, np.zeros(1, np.int32))
    out, lse = hisa.hisa_sparse_attention(dq, dkv, c.L, idx, 512, 1.0 / np.sqrt(576))
    torch.cuda.synchronize()
    _check(orc, q, kv, idx.cpu().numpy(), 512, 1.0 / np.sqrt(576), c.L, out.cpu().numpy(), lse.cpu().numpy())


def test_attention_errors_raise(hisa):
    import torch

    q, kv, idx = _case("err", 1, 1, 16, 128, 100, 10)
    dq, dkv, didx = _to_dev(q, kv, idx)
    with pytest.raises(hisa.HisaError):
        hisa.hisa_sparse_attention(dq, dkv, 100, didx, 96, 0.1)          # unsupported (Dk, Dv)
    q2, _, _ = _case("err2", 1, 1, 24, 128, 100, 10)
    with pytest.raises(hisa.HisaError):
        hisa.hisa_sparse_attention(_to_dev(q2, kv, idx)[0], dkv, 100, didx, 128, 0.1)   # Ha not a multiple of 16
    with pytest.raises(hisa.HisaError):
        hisa.hisa_sparse_attention(dq, dkv, 100, didx, 128, float("nan"))
