"""GPU: entry points captured in a HIP graph and replayed.

A caller (the benchmark among them) may capture the indexer's calls in a
graph and replay it every step.  Each case runs a call eagerly, captures the
same call on the same buffers, then replays the graph several times with
eager work and synchronisations between the replays and the outputs
overwritten before each one; every replay must give the eager result bit for
bit.  The library enqueues kernels only (no memory sets or copies), so a
replay re-runs exactly the eager work.
"""
import numpy as np
import pytest

from sparse_attention_token_amd import synth
from parity import bits, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def hisa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_attention_token_amd import hisa as h

    h.lib()
    return h


def _snap(ts):
    import torch

    out = []
    for t in ts:
        if t is None:
            out.append(None)
        elif t.dtype == torch.bfloat16:
            out.append(bits(t).copy())
        else:
            out.append(t.cpu().numpy().copy())
    return out


def _scribble(ts):
    import torch

    for t in ts:
        if t is None:
            continue
        if t.dtype == torch.bfloat16:
            t.view(torch.int16).fill_(0x7FC0)
        elif t.dtype == torch.int32:
            t.fill_(-7)
        else:
            t.fill_(float("nan"))


def _replay_matches(call, outs, other):
    """Eager call, capture, REPLAYS replays (outputs scribbled before each, eager
    work in between): every replay equals the eager result."""
    import torch

    call()
    torch.cuda.synchronize()
    ref = _snap(outs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        _scribble(outs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snap(outs)
        for j, (a, b) in enumerate(zip(ref, got)):
            if a is None:
                assert b is None
                continue
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}, output {j}")
        other()                                  # the program's own eager work between replays
        torch.cuda.synchronize()
    return ref


CASES = [
    # name, S, L, T, H, d, B, m, k
    ("decode_one_launch", 4, 3001, 1, 64, 128, 128, 8, 300),
    ("decode_two_kernel", 2, 40001, 1, 16, 64, 64, 20, 400),
    ("prefill_block_major", 1, 2128, 128, 16, 64, 64, 6, 128),
]


@pytest.mark.parametrize("spec", CASES, ids=[s[0] for s in CASES])
def test_index_calls_replay(hisa, spec):
    import torch

    name, S, L, T, H, d, B, m, k = spec
    print(f"graph case {name}", flush=True)
    c = synth.clustered_case(S, L, T, H, d, B, m, k, seed=31, latent_block=B)
    dev = to_dev(c)
    q, w, K = dev["q"], dev["w"], dev["K"]
    nblk = -(-L // B)
    pool = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=K.device)
    hisa.hisa_pool_append(K, pool, 0, L - 1, B)
    idx = torch.empty((S, T, k), dtype=torch.int32, device=K.device)
    sc = torch.empty((S, T, k), dtype=torch.float32, device=K.device)
    blk = torch.empty((S, T, m), dtype=torch.int32, device=K.device)
    ws = torch.empty(hisa.hisa_index_workspace(S, T, H, d, L, B, m, k), dtype=torch.uint8, device=K.device)
    fidx = torch.empty_like(idx)
    fsc = torch.empty_like(sc)
    fws = torch.empty(hisa.dsa_flat_workspace(S, T, H, d, L, k), dtype=torch.uint8, device=K.device)
    scratch = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=K.device)

    def other():                                 # unrelated eager work on other buffers
        hisa.hisa_pool_append(K, scratch, 0, L, B)
        hisa.dsa_flat_index(q, w, K, L, k)

    # pool append + index in one call (the pool's last block is recomputed each time)
    ref = _replay_matches(
        lambda: hisa.hisa_append_index(K, pool, L - 1, L, q, w, B, m, k, out_idx=idx, out_score=sc, out_blk=blk,
                                       want_blocks=True, workspace=ws),
        [idx, sc, blk], other)
    # the same bits as the eager two-call form
    pool2 = torch.zeros_like(pool)
    hisa.hisa_pool_append(K, pool2, 0, L, B)
    i2, s2, b2 = hisa.hisa_index(q, w, K, L, pool2, B, m, k, want_blocks=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ref[0], i2.cpu().numpy())
    np.testing.assert_array_equal(ref[2], b2.cpu().numpy())
    np.testing.assert_array_equal(bits(pool), bits(pool2))
    # index only, and the flat indexer
    _replay_matches(lambda: hisa.hisa_index(q, w, K, L, pool2, B, m, k, out_idx=idx, out_score=sc, out_blk=blk,
                                            want_blocks=True, workspace=ws), [idx, sc, blk], other)
    _replay_matches(lambda: hisa.dsa_flat_index(q, w, K, L, k, out_idx=fidx, out_score=fsc, workspace=fws),
                    [fidx, fsc], other)


def test_tree_and_attention_replay(hisa):
    import torch

    S, L, T, H, d, B, G, W, m, k = 2, 9000, 1, 64, 128, 128, 8, 3, 8, 512
    print("graph case tree + attention", flush=True)
    c = synth.clustered_case(S, L, T, H, d, B, m, k, seed=37, latent_block=B)
    dev = to_dev(c)
    q, w, K = dev["q"], dev["w"], dev["K"]
    nblk = -(-L // B)
    tp = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=K.device)
    sp = torch.zeros((S, -(-nblk // G), d), dtype=torch.bfloat16, device=K.device)
    hisa.hisa_tree_append(K, tp, sp, 0, L - 1, B, G)
    idx = torch.empty((S, T, k), dtype=torch.int32, device=K.device)
    sc = torch.empty((S, T, k), dtype=torch.float32, device=K.device)
    blk = torch.empty((S, T, m), dtype=torch.int32, device=K.device)
    sblk = torch.empty((S, T, W), dtype=torch.int32, device=K.device)
    tws = torch.empty(hisa.hisa_tree_index_workspace(S, T, H, d, L, B, G, W, m, k), dtype=torch.uint8,
                      device=K.device)

    def other():
        hisa.dsa_flat_index(q, w, K, L, k)

    def tree_step():
        hisa.hisa_tree_append(K, tp, sp, L - 1, L, B, G)
        hisa.hisa_tree_index(q, w, K, L, tp, sp, B, G, W, m, k, out_idx=idx, out_score=sc, out_blk=blk,
                             out_sblk=sblk, want_blocks=True, want_super=True, workspace=tws)

    _replay_matches(tree_step, [idx, sc, blk, sblk], other)

    # the sparse attention over the tree's selection, split (8 queries' worth of
    # workgroups are few, so the set is split and merged by the combine kernel)
    Ha, Dk, Dv = 32, 576, 512
    rng = np.random.default_rng(3)
    kv = torch.from_numpy(synth.bf16_bits(rng.standard_normal((S, L, Dk)).astype(np.float32)).view(np.int16))
    kv = kv.cuda().view(torch.bfloat16)
    qa = torch.from_numpy(synth.bf16_bits((rng.standard_normal((S, T, Ha, Dk)) * 0.1).astype(np.float32))
                          .view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty((S, T, Ha, Dv), dtype=torch.float32, device=K.device)
    lse = torch.empty((S, T, Ha), dtype=torch.float32, device=K.device)
    aws = torch.empty(hisa.hisa_sparse_attention_workspace(S, T, Ha, Dk, Dv, k), dtype=torch.uint8,
                      device=K.device)
    _replay_matches(lambda: hisa.hisa_sparse_attention(qa, kv, L, idx, Dv, 1.0 / 24.0, out=out, lse=lse,
                                                       workspace=aws), [out, lse], other)
    assert torch.isfinite(out).all().item()
