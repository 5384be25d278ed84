"""Poisoned workspaces: every code path runs once with its workspace filled
with zero bytes and once with 0xFF bytes, and must return the same bits.

The library promises nothing about the workspace's contents on entry (the
caller allocates it uninitialised), so no kernel may read a workspace word it
has not written in the same call.  A word read before it is written would
carry 0 in one run and 0xFFFFFFFF (or a NaN pattern) in the other.
"""
import sys

import numpy as np
import pytest

from sparse_attention_token_amd import synth
from parity import bits, build_pool, build_tree_pools, to_dev

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


def _ws(nbytes, fill):
    import torch

    return torch.full((max(1, nbytes),), fill, dtype=torch.uint8, device="cuda")


def _same(a, b, what):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        np.testing.assert_array_equal(x.cpu().numpy().view(np.uint32 if x.element_size() == 4 else np.uint16),
                                      y.cpu().numpy().view(np.uint32 if y.element_size() == 4 else np.uint16),
                                      err_msg=what)


# name, S, L, T, H, d, B, m, k, explicit positions: one case per code path of hisa_index
INDEX_PATHS = [
    ("one_launch_decode", 8, 9000, 1, 64, 128, 128, 16, 512, False),
    ("two_kernel_decode", 2, 40000, 1, 16, 128, 128, 40, 700, False),
    ("query_major_batch", 2, 6000, 40, 16, 64, 16, 20, 150, True),
    ("block_major_chunk", 1, 20000, 300, 16, 128, 128, 12, 400, False),
    ("general_path", 2, 3000, 4, 8, 128, 256, 6, 300, True),
    ("chunked_selection", 1, 300000, 2, 4, 64, 16, 4096, 2048, True),
]


@pytest.mark.parametrize("spec", INDEX_PATHS, ids=[p[0] for p in INDEX_PATHS])
def test_index_ignores_workspace_contents(hisa, spec):
    import torch

    name, S, L, T, H, d, B, m, k, explicit = spec
    _say(f"poisoned workspace: hisa_index {name}")
    rng = np.random.default_rng(len(name))
    qpos = np.stack([np.sort(rng.integers(0, L, size=T)) for _ in range(S)]).astype(np.int32) if explicit else None
    c = synth.clustered_case(S, L, T, H, d, B, m, k, seed=61, qpos=qpos, latent_block=B)
    dev = to_dev(c)
    pool = build_pool(hisa, dev["K"], L, B)
    nbytes = hisa.hisa_index_workspace(S, T, H, d, L, B, m, k)
    qp = dev["qpos"] if explicit else None
    res = []
    for fill in (0x00, 0xFF):
        res.append(hisa.hisa_index(dev["q"], dev["w"], dev["K"], L, pool, B, m, k, qp, want_blocks=True,
                                   workspace=_ws(nbytes, fill)))
        torch.cuda.synchronize()
    _same(res[0], res[1], name)
    # the flat indexer on the same inputs
    fres = []
    fbytes = hisa.dsa_flat_workspace(S, T, H, d, L, k)
    for fill in (0x00, 0xFF):
        fres.append(hisa.dsa_flat_index(dev["q"], dev["w"], dev["K"], L, k, qp, workspace=_ws(fbytes, fill)))
        torch.cuda.synchronize()
    _same(fres[0], fres[1], name + " flat")


@pytest.mark.parametrize("L0,L1", [(8999, 9000), (39990, 40000)])
def test_append_index_ignores_workspace_contents(hisa, L0, L1):
    """The decode step with the pool update fused into the block stage (one
    launch at 9000 keys, two kernels at 40000): outputs and pool bits."""
    import torch

    S, H, d, B, m, k = 4, 32, 128, 128, 24, 600
    _say(f"poisoned workspace: hisa_append_index {L0}->{L1}")
    c = synth.clustered_case(S, L1, 1, H, d, B, m, k, seed=62, latent_block=B)
    dev = to_dev(c)
    base = build_pool(hisa, dev["K"], L0, B)
    nbytes = hisa.hisa_index_workspace(S, 1, H, d, L1, B, m, k)
    outs, pools = [], []
    for fill in (0x00, 0xFF):
        p = torch.zeros((S, -(-L1 // B), d), dtype=torch.bfloat16, device="cuda")
        p[:, :base.shape[1]] = base
        outs.append(hisa.hisa_append_index(dev["K"], p, L0, L1, dev["q"], dev["w"], B, m, k, want_blocks=True,
                                           workspace=_ws(nbytes, fill)))
        pools.append(p)
        torch.cuda.synchronize()
    _same(outs[0], outs[1], "append_index")
    np.testing.assert_array_equal(bits(pools[0]), bits(pools[1]))


# name, S, L, T, H, d, B, G, W, m, k: the one-launch upper levels, and the
# separate launches (more than 2048 super-blocks)
TREE_PATHS = [
    ("tree_one_launch", 2, 20000, 3, 32, 128, 128, 8, 3, 12, 500),
    ("tree_separate_launches", 1, 40000, 2, 16, 64, 16, 1, 8, 30, 256),
]


@pytest.mark.parametrize("spec", TREE_PATHS, ids=[p[0] for p in TREE_PATHS])
def test_tree_ignores_workspace_contents(hisa, spec):
    import torch

    name, S, L, T, H, d, B, G, W, m, k = spec
    _say(f"poisoned workspace: {name}")
    rng = np.random.default_rng(7)
    qpos = np.stack([np.sort(rng.integers(0, L, size=T)) for _ in range(S)]).astype(np.int32)
    c = synth.clustered_case(S, L, T, H, d, B, m, k, seed=63, qpos=qpos, latent_block=B)
    dev = to_dev(c)
    reps, sreps = build_tree_pools(hisa, dev["K"], L, B, G)
    nbytes = hisa.hisa_tree_index_workspace(S, T, H, d, L, B, G, W, m, k)
    res = []
    for fill in (0x00, 0xFF):
        res.append(hisa.hisa_tree_index(dev["q"], dev["w"], dev["K"], L, reps, sreps, B, G, W, m, k, dev["qpos"],
                                        want_blocks=True, want_super=True, workspace=_ws(nbytes, fill)))
        torch.cuda.synchronize()
    _same(res[0], res[1], name)


@pytest.mark.parametrize("S,T,k", [(2, 1, 2048), (1, 64, 300)])
def test_attention_ignores_workspace_contents(hisa, S, T, k):
    """The sparse attention, split over workgroups with partials in the
    workspace (few queries) and unsplit (many)."""
    import torch

    L, Ha, Dk, Dv = 5000, 32, 576, 512
    _say(f"poisoned workspace: attention S={S} T={T} k={k}")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    q = (torch.randn((S, T, Ha, Dk), generator=g, device="cuda") * 0.05).to(torch.bfloat16)
    kv = torch.randn((S, L, Dk), generator=g, device="cuda").to(torch.bfloat16)
    idx = torch.randint(-1, L, (S, T, k), generator=g, device="cuda", dtype=torch.int32)
    nbytes = hisa.hisa_sparse_attention_workspace(S, T, Ha, Dk, Dv, k)
    res = []
    for fill in (0x00, 0xFF):
        res.append(hisa.hisa_sparse_attention(q, kv, L, idx, Dv, 0.04, workspace=_ws(nbytes, fill)))
        torch.cuda.synchronize()
    _same(res[0], res[1], "attention")
