"""CPU: the benchmark's algorithmic work models against closed forms.

The roofline fractions the benchmark reports divide these byte and flop
counts by measured kernel times, so they are pinned here to figures derived by
hand from the workload shapes (no GPU, no key data: only the shapes, the
query positions and the kept blocks enter the models).
"""
import types

import numpy as np

import bench


def _case(S, T, H, d, L, B, m, k, qpos):
    return types.SimpleNamespace(S=S, T=T, H=H, d=d, L=L, B=B, m=m, k=k,
                                 qpos=np.asarray(qpos, dtype=np.int32).reshape(S, T))


def test_decode_32k_bytes():
    # 8 queries at t = 32767: 256 pooled means and 64 full kept blocks (8192 rows) each
    S, T, H, d, L, B, m, k = 8, 1, 64, 128, 32768, 128, 64, 2048
    c = _case(S, T, H, d, L, B, m, k, [[L - 1]] * S)
    blocks = np.tile(np.arange(192, 256, dtype=np.int32), (S, T, 1))
    models, per_call, cand = bench.kernel_models(c, blocks)
    qw = S * (H * d * 2 + H * 4)                       # q and w: 16,640 B per query
    assert qw == 8 * 16640
    assert cand == S * 8192
    assert models["index_decode"]["bytes"] == S * (256 + 8192) * d * 2 + qw == 17434624
    assert models["score_flat"]["bytes"] == S * L * d * 2 + qw
    assert models["select_refine"]["bytes"] == S * 8192 * 4 + S * k * 8
    # per call: rows scored, q and w, and the k int32 indices returned
    assert per_call == S * ((256 + 8192) * d * 2 + 16640 + k * 4)


def test_partial_last_block_counts_only_rows_up_to_t():
    # t = 1000 with B = 128: own block 7 holds rows 896..1000 (105 rows)
    c = _case(1, 1, 4, 64, 1001, 128, 3, 64, [[1000]])
    blocks = np.array([[[7, 2, 5]]], dtype=np.int32)
    _, _, cand = bench.kernel_models(c, blocks)
    assert cand == 105 + 128 + 128
    # padding slots (-1) add nothing
    blocks = np.array([[[7, -1, -1]]], dtype=np.int32)
    _, _, cand = bench.kernel_models(c, blocks)
    assert cand == 105


def test_prefill_chunk_flops():
    # 4096 queries at t = 126976..131071 over 131072 keys, 64 kept blocks of 128 full rows each
    S, T, H, d, L, B, m, k = 1, 4096, 64, 128, 131072, 128, 64, 2048
    t = np.arange(L - T, L)
    c = _case(S, T, H, d, L, B, m, k, t[None, :])
    blocks = np.tile(np.arange(0, 64, dtype=np.int32), (S, T, 1))
    models, _, cand = bench.kernel_models(c, blocks)
    # n_b(t) = t // 128 + 1 runs over 993..1024, 128 queries each
    sum_nb = 128 * sum(range(993, 1025))
    assert sum_nb == 4130816
    assert models["score_blocks"]["flops"] == 2 * H * d * sum_nb          # 67.68 GFLOP
    assert models["score_refine"]["flops"] == 2 * H * d * 8192 * T == 549755813888
    assert cand == 8192 * T
    # flat: every key up to t
    assert models["score_flat"]["flops"] == 2 * H * d * int((t + 1).sum())


def test_tree_models():
    # G = 4, W = 2 at t = 4095, B = 128: 32 blocks, 8 super-blocks; super-blocks 7 and 3 kept
    c = _case(1, 1, 16, 64, 4096, 128, 4, 256, [[4095]])
    sblocks = np.array([[[7, 3]]], dtype=np.int32)
    blocks = np.array([[[31, 30, 13, 12]]], dtype=np.int32)
    models, per_call, cand = bench.kernel_models(c, blocks, tree=(4, 2), sblocks=sblocks)
    row = 64 * 2
    qw = 16 * 64 * 2 + 16 * 4
    assert models["score_blocks"]["bytes"] == 8 * row + qw                 # the 8 super-block representatives
    assert models["score_tree"]["bytes"] == 8 * row + qw                   # 4 blocks in each kept super-block
    assert cand == 4 * 128
    assert per_call == (8 + 8 + 512) * row + qw + 256 * 4
