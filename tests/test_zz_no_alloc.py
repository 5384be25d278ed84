"""The decode step with the library's static scratch (hisa_append_index_static)
against the same step with a caller workspace (hisa_append_index).

Both run the same kernels on the same inputs, so every output and the pool
must agree bit for bit.  Two calls follow each other on the scratch, the second
with a smaller problem (fewer sequences, shorter cache, fewer heads, a smaller
head dimension and block), so whatever the first call left in the scratch
cannot leak into the second.  Sampled rows are also checked against the oracle.
"""
import sys

import numpy as np
import pytest

from sparse_attention_token_amd import synth
from parity import bits, build_pool, check_hisa_row, to_dev

pytestmark = pytest.mark.gpu


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


# (name, S, L_old, L_new, H, d, B, m, k): one decode query per sequence at t = L_new - 1
CALLS = [
    ("8 x 8197 keys, H=64, d=128, B=128", 8, 8196, 8197, 64, 128, 128, 16, 512),
    ("2 x 3000 keys, H=16, d=64, B=64", 2, 2997, 3000, 16, 64, 64, 8, 256),
]


def _step(hisa, spec, seed):
    import torch

    name, S, L0, L1, H, d, B, m, k = spec
    c = synth.clustered_case(S, L1, 1, H, d, B, m, k, seed=seed, latent_block=B)
    dev = to_dev(c)
    base = build_pool(hisa, dev["K"], L0, B)
    nblk = -(-L1 // B)
    pools = []
    for _ in range(2):
        p = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=dev["K"].device)
        p[:, :base.shape[1]] = base[:, :nblk]
        pools.append(p)
    want = hisa.hisa_append_index(dev["K"], pools[0], L0, L1, dev["q"], dev["w"], B, m, k, want_blocks=True)
    out = (torch.full((S, 1, k), -7, dtype=torch.int32, device=dev["K"].device),
           torch.full((S, 1, k), 7.0, dtype=torch.float32, device=dev["K"].device),
           torch.full((S, 1, m), -7, dtype=torch.int32, device=dev["K"].device))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = hisa.hisa_append_index_static(dev["K"], pools[1], L0, L1, dev["q"], dev["w"], B, m, k,
                                        out_idx=out[0], out_score=out[1], out_blk=out[2])
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "the static call allocated device memory"
    for x, y in zip(want, got):
        np.testing.assert_array_equal(x.cpu().numpy().view(np.int32), y.cpu().numpy().view(np.int32))
    np.testing.assert_array_equal(bits(pools[0]), bits(pools[1]))
    return c, got


def test_static_scratch_matches_workspace_call_twice(hisa, orc):
    for n, spec in enumerate(CALLS):
        _say(f"static scratch call {n + 1}: {spec[0]}")
        c, (idx, sc, blk) = _step(hisa, spec, seed=90 + n)
        idx, sc, blk = idx.cpu().numpy(), sc.cpu().numpy(), blk.cpu().numpy()
        for s in sorted({0, c.S - 1}):
            check_hisa_row(orc, c, s, 0, idx[s, 0], sc[s, 0], blk[s, 0])


def test_static_scratch_refuses_oversized_problems(hisa):
    import torch

    # 4096 queries x 8192 candidates: more workspace than the 16 MiB scratch
    S, T, H, d, L, B, m, k = 1, 4096, 4, 64, 8192, 64, 128, 64
    assert hisa.hisa_index_workspace(S, T, H, d, L, B, m, k) > hisa.STATIC_SCRATCH_BYTES
    dev = torch.device("cuda")
    K = torch.zeros((S, L, d), dtype=torch.bfloat16, device=dev)
    pool = torch.zeros((S, L // B, d), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((S, T, H, d), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((S, T, H), dtype=torch.float32, device=dev)
    with pytest.raises(hisa.HisaError) as e:
        hisa.hisa_append_index_static(K, pool, L - 1, L, q, w, B, m, k)
    assert e.value.status == hisa.HISA_ERR_SCRATCH
