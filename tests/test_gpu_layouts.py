"""GPU layout invariance: caches allocated with spare capacity.

A serving cache is allocated for more rows than it holds, so each sequence's
key rows (and pool entries) start a capacity stride apart and the rows past the
current length hold whatever the memory held before.  Every entry point must
give bit-identical results whether its caches are exactly L rows long or are
longer, with the spare rows, the spare pool entries and the spare latent
columns filled with NaN: reading any of them would change a result.  The
tight layout itself is checked against the oracle in the other GPU tests.
"""
import numpy as np
import pytest

from sparse_attention_token_amd import synth
from parity import bits, to_dev

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0          # a bf16 quiet NaN


@pytest.fixture(scope="module")
def hisa():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_attention_token_amd import hisa as h

    h.lib()
    return h


def _nan_filled(shape, device):
    import torch

    return torch.full(shape, NAN_BITS, dtype=torch.int16, device=device).view(torch.bfloat16)


def _spare(t, rows, cols=None):
    """t [S, N, c] copied into the leading corner of a NaN-filled [S, N + rows, c (+ cols)] buffer."""
    S, N, c = t.shape
    big = _nan_filled((S, N + rows, c + (cols or 0)), t.device)
    big[:, :N, :c] = t
    return big


def _same(a, b, what):
    import torch

    if a is None or b is None:
        assert a is None and b is None, what
        return
    if a.dtype == torch.bfloat16:
        np.testing.assert_array_equal(bits(a), bits(b), err_msg=what)
    else:
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy(), err_msg=what)


CASES = [
    # name, S, L, T, H, d, B, m, k, explicit positions
    ("decode_one_launch", 4, 3001, 1, 64, 128, 128, 8, 300, False),
    ("decode_two_kernel", 2, 40001, 1, 16, 64, 64, 20, 400, False),
    ("query_major_20q", 1, 5003, 20, 32, 128, 128, 8, 300, True),
    ("prefill_block_major", 1, 2128, 128, 16, 64, 64, 6, 128, False),
]


@pytest.mark.parametrize("spec", CASES, ids=[s[0] for s in CASES])
def test_spare_capacity_gives_identical_results(hisa, spec):
    import torch

    name, S, L, T, H, d, B, m, k, explicit = spec
    print(f"layout case {name}", flush=True)
    qpos = None
    if explicit:
        rng = np.random.default_rng(5)
        qpos = rng.integers(0, L, size=(S, T)).astype(np.int32)
        qpos[0, 0] = L - 1
    c = synth.clustered_case(S, L, T, H, d, B, m, k, seed=29, qpos=qpos, latent_block=B)
    dev = to_dev(c)
    q, w = dev["q"], dev["w"]
    qp = dev["qpos"] if explicit else None
    nblk = -(-L // B)
    G, W = 4, 2

    def run(K, pool_rows, spool_rows):
        pool = torch.zeros((S, pool_rows, d), dtype=torch.bfloat16, device=K.device)
        if pool_rows > nblk:
            pool[:, nblk:] = _nan_filled((S, pool_rows - nblk, d), K.device)
        # bulk build through row L-2, then the last row appended on its own
        hisa.hisa_pool_append(K, pool, 0, L - 1, B)
        pool2 = pool.clone()
        hisa.hisa_pool_append(K, pool, L - 1, L, B)
        res = {"pool": pool[:, :nblk].clone()}
        res["index"] = hisa.hisa_index(q, w, K, L, pool, B, m, k, qp, want_blocks=True)
        res["flat"] = hisa.dsa_flat_index(q, w, K, L, k, qp)
        # one call that appends the newest row and indexes
        res["append_index"] = hisa.hisa_append_index(K, pool2, L - 1, L, q, w, B, m, k, qp, want_blocks=True)
        res["pool_after_append_index"] = pool2[:, :nblk].clone()
        # the three-level tree
        tp = torch.zeros((S, pool_rows, d), dtype=torch.bfloat16, device=K.device)
        sp = torch.zeros((S, spool_rows, d), dtype=torch.bfloat16, device=K.device)
        nsb = -(-nblk // G)
        if pool_rows > nblk:
            tp[:, nblk:] = _nan_filled((S, pool_rows - nblk, d), K.device)
        if spool_rows > nsb:
            sp[:, nsb:] = _nan_filled((S, spool_rows - nsb, d), K.device)
        hisa.hisa_tree_append(K, tp, sp, 0, L, B, G)
        res["tree_pools"] = (tp[:, :nblk].clone(), sp[:, :nsb].clone())
        res["tree"] = hisa.hisa_tree_index(q, w, K, L, tp, sp, B, G, W, m, k, qp, want_blocks=True,
                                           want_super=True)
        torch.cuda.synchronize()
        return res

    nsb = -(-nblk // G)
    tight = run(dev["K"], nblk, nsb)
    spare = run(_spare(dev["K"], 1000), nblk + 3, nsb + 2)
    _same(tight["pool"], spare["pool"], "pool")
    _same(tight["pool_after_append_index"], spare["pool_after_append_index"], "pool after append+index")
    for key in ("index", "flat", "append_index", "tree"):
        for j, (a, b) in enumerate(zip(tight[key], spare[key])):
            _same(a, b, f"{key} output {j}")
    for a, b in zip(tight["tree_pools"], spare["tree_pools"]):
        _same(a, b, "tree pools")
    # the outputs are real selections, not padding everywhere
    assert (tight["index"][0] >= 0).sum().item() > 0


@pytest.mark.parametrize("Dk,Dv,Ha", [(576, 512, 16), (128, 128, 32)])
def test_attention_spare_rows_and_columns(hisa, Dk, Dv, Ha):
    """Latent rows with spare columns (row stride above Dk) and spare rows past L."""
    import torch

    S, T, L, k = 2, 3, 5000, 700
    print(f"attention layout Dk={Dk} Dv={Dv} Ha={Ha}", flush=True)
    rng = np.random.default_rng(41)
    kv = synth.bf16_bits(rng.standard_normal((S, L, Dk)).astype(np.float32))
    q = synth.bf16_bits((rng.standard_normal((S, T, Ha, Dk)) * 0.1).astype(np.float32))
    idx = rng.integers(-1, L, size=(S, T, k)).astype(np.int32)
    idx[0, 0, :] = -1                                    # an empty set
    idx[1, 2, 5:9] = L + 3                               # entries past L are skipped
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    kv_t, q_t = to(kv), to(q)
    idx_t = torch.from_numpy(idx).cuda()
    scale = 1.0 / np.sqrt(Dk)
    o1, l1 = hisa.hisa_sparse_attention(q_t, kv_t, L, idx_t, Dv, scale)
    o2, l2 = hisa.hisa_sparse_attention(q_t, _spare(kv_t, 300, cols=64), L, idx_t, Dv, scale)
    torch.cuda.synchronize()
    _same(o1, o2, "attention output")
    _same(l1, l2, "attention lse")
    assert torch.isfinite(o1[1]).all().item()


def _wide(t, min_stride):
    """t [S, N, c] in the leading corner of a NaN-filled [S, N', c] buffer whose
    sequence stride N' * c is at least min_stride elements."""
    S, N, c = t.shape
    return _spare(t, max(0, -(-min_stride // c) - N))


def test_strides_past_2g_elements_give_identical_results(hisa):
    """Sequence strides of 2^31 elements or more: the decode, tree and flat
    kernels take their leading arguments preloaded as 32-bit values, so such
    caches run other variants (the batch path for decode, the tree's and the
    flat scorer's struct-reading kernels); they must give the bits the tight
    layout gives.  The wide key cache is 8.6 GB."""
    import torch

    S, L, T, H, d, B, m, k = 2, 3001, 1, 64, 128, 128, 8, 300
    print("layout case strides past 2^31 elements", flush=True)
    c = synth.clustered_case(S, L, T, H, d, B, m, k, seed=31, latent_block=B)
    dev = to_dev(c)
    q, w = dev["q"], dev["w"]
    nblk = -(-L // B)
    G, W = 4, 2

    def run(K):
        pool = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=K.device)
        hisa.hisa_pool_append(K, pool, 0, L - 1, B)
        pool2 = pool.clone()
        hisa.hisa_pool_append(K, pool, L - 1, L, B)
        res = {"pool": pool.clone()}
        res["index"] = hisa.hisa_index(q, w, K, L, pool, B, m, k, want_blocks=True)
        res["flat"] = hisa.dsa_flat_index(q, w, K, L, k)
        res["append_index"] = hisa.hisa_append_index(K, pool2, L - 1, L, q, w, B, m, k, want_blocks=True)
        res["pool_after_append_index"] = pool2.clone()
        tp = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=K.device)
        sp = torch.zeros((S, -(-nblk // G), d), dtype=torch.bfloat16, device=K.device)
        hisa.hisa_tree_append(K, tp, sp, 0, L, B, G)
        res["tree"] = hisa.hisa_tree_index(q, w, K, L, tp, sp, B, G, W, m, k, want_blocks=True, want_super=True)
        torch.cuda.synchronize()
        return res

    tight = run(dev["K"])
    Kw = _wide(dev["K"], (1 << 31) + 64)
    assert Kw.stride(0) >= (1 << 31)
    wide = run(Kw)
    del Kw
    _same(tight["pool"], wide["pool"], "pool")
    _same(tight["pool_after_append_index"], wide["pool_after_append_index"], "pool after append+index")
    for key in ("index", "flat", "append_index", "tree"):
        for j, (a, b) in enumerate(zip(tight[key], wide[key])):
            _same(a, b, f"{key} output {j}")
    assert (tight["index"][0] >= 0).sum().item() > 0


def test_attention_stride_past_2g_elements(hisa):
    """A latent cache whose sequence stride is 2^31 elements or more runs the
    attention variant that reads its struct argument: the same bits."""
    import torch

    S, T, L, k, Dk, Dv, Ha = 2, 3, 5000, 700, 576, 512, 16
    print("attention layout stride past 2^31 elements", flush=True)
    rng = np.random.default_rng(43)
    kv = synth.bf16_bits(rng.standard_normal((S, L, Dk)).astype(np.float32))
    q = synth.bf16_bits((rng.standard_normal((S, T, Ha, Dk)) * 0.1).astype(np.float32))
    idx = rng.integers(-1, L, size=(S, T, k)).astype(np.int32)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    kv_t, q_t = to(kv), to(q)
    idx_t = torch.from_numpy(idx).cuda()
    scale = 1.0 / np.sqrt(Dk)
    o1, l1 = hisa.hisa_sparse_attention(q_t, kv_t, L, idx_t, Dv, scale)
    kvw = _wide(kv_t, (1 << 31) + 64)
    assert kvw.stride(0) >= (1 << 31)
    o2, l2 = hisa.hisa_sparse_attention(q_t, kvw, L, idx_t, Dv, scale)
    torch.cuda.synchronize()
    del kvw
    _same(o1, o2, "attention output")
    _same(l1, l2, "attention lse")
    assert torch.isfinite(o1).all().item()
