"""Parity helpers: move seeded inputs to the GPU and compare GPU rows with the oracle.

Comparison rule (floating point decides which indices are kept, and the GPU
ranks fp32 scores while the oracle ranks fp64 ones):
  tol(x) = ABS_TOL + REL_TOL * |x|
  1. every returned GPU score is within tol of the oracle's score of that index;
  2. kept blocks: the GPU set may differ from the oracle's only by blocks whose
     oracle score is within tol of the oracle's m-th best block score;
  3. kept tokens: the oracle re-runs the refinement on the GPU's kept blocks
     (conditional oracle); the GPU set may differ from that result only by
     tokens whose oracle score is within tol of its k-th best score.
Everything else -- counts, padding, ordering (ascending ids) -- is exact.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-3
ABS_TOL = 1e-4


def tol(x):
    return ABS_TOL + REL_TOL * abs(x)


def to_dev(case, device="cuda"):
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    return dict(
        K=bf(case.K),
        q=bf(case.q),
        w=torch.from_numpy(np.ascontiguousarray(case.w)).to(device),
        qpos=torch.from_numpy(np.ascontiguousarray(case.qpos)).to(device),
    )


def bits(t):
    """bf16 torch tensor -> numpy uint16 bit patterns."""
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def build_pool(hisa, K, L, B, L_bulk=None, step=1, pool="mean"):
    """Pool representatives for rows [0, L): one bulk append of [0, L_bulk), then appends of `step` rows."""
    import torch

    S, _, d = K.shape
    nblk = -(-L // B)
    reps = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=K.device)
    L_bulk = L if L_bulk is None else L_bulk
    hisa.hisa_pool_append(K, reps, 0, L_bulk, B, pool=pool)
    x = L_bulk
    while x < L:
        y = min(L, x + step)
        hisa.hisa_pool_append(K, reps, x, y, B, pool=pool)
        x = y
    return reps


def _kth(scores_desc, n):
    return scores_desc[n - 1]


def check_hisa_row(orc, case, s, i, g_idx, g_score, g_blk, report=None, pool="mean"):
    """Apply the comparison rule to one GPU output row of hisa_index (block
    representatives pooled by `pool`, "mean" or "max")."""
    q, w, K = case.q[s, i], case.w[s, i], case.K[s]
    t = int(case.qpos[s, i])
    B, m, k = case.B, case.m, case.k
    nb = t // B + 1
    meff = min(m, nb)
    o_idx, o_sc, o_blk, o_bsc, o_keff = orc.hisa_query(q, w, K, t, B, m, k, mode=pool)

    # -- blocks
    g_blk = np.asarray(g_blk)
    assert np.all(g_blk[meff:] == -1), "block padding"
    gb = g_blk[:meff]
    assert np.all(gb >= 0) and np.all(np.diff(gb) > 0), "kept blocks must be ascending and distinct"
    assert gb[-1] < nb
    c_m = _kth(np.sort(o_bsc)[::-1], meff)
    diff = set(gb.tolist()) ^ set(o_blk[:meff].tolist())
    for b in diff:
        assert abs(o_bsc[b] - c_m) <= tol(c_m), f"block {b} differs (score {o_bsc[b]} vs cutoff {c_m})"

    tdiff = _check_tokens(orc, q, w, K, t, B, k, gb, g_idx, g_score)
    if report is not None:
        report.setdefault("block_diffs", 0)
        report.setdefault("token_diffs", 0)
        report["block_diffs"] += len(diff)
        report["token_diffs"] += len(tdiff)
    return o_idx, o_keff


def _check_tokens(orc, q, w, K, t, B, k, gb, g_idx, g_score):
    """Token rule against the conditional oracle on the GPU's kept blocks gb; returns the differing ids."""
    c_idx, c_sc, c_keff, nC = orc.refine_query(q, w, K, t, B, gb, k)
    g_idx = np.asarray(g_idx)
    assert np.all(g_idx[c_keff:] == -1), "token padding"
    gt = g_idx[:c_keff]
    assert np.all(gt >= 0) and np.all(np.diff(gt) > 0), "kept tokens must be ascending and distinct"
    assert np.all(gt <= t), "causality"
    assert np.all(np.isin(gt // B, gb)), "tokens must come from kept blocks"
    c_k = float(orc.score(q, w, K[c_idx[c_keff - 1]])) if c_keff > 0 else 0.0
    tdiff = set(gt.tolist()) ^ set(c_idx[:c_keff].tolist())
    for j in tdiff:
        sj = orc.score(q, w, K[j])
        assert abs(sj - c_k) <= tol(c_k), f"token {j} differs (score {sj} vs cutoff {c_k})"

    # -- scores of the returned tokens
    if g_score is not None:
        g_score = np.asarray(g_score)
        assert np.all(np.isneginf(g_score[c_keff:]))
        ref = dict(zip(c_idx[:c_keff].tolist(), c_sc[:c_keff].astype(np.float64).tolist()))
        for pos, j in enumerate(gt.tolist()):
            sj = ref[j] if j in ref else orc.score(q, w, K[j])
            assert abs(g_score[pos] - sj) <= tol(sj), f"score of token {j}: {g_score[pos]} vs {sj}"
    return tdiff


def build_tree_pools(hisa, K, L, B, G, L_bulk=None, step=1, pool="mean"):
    """Block and super-block pools for rows [0, L) through hisa_tree_append: one bulk append of
    [0, L_bulk), then appends of `step` rows."""
    import torch

    S, _, d = K.shape
    nblk = -(-L // B)
    reps = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=K.device)
    sreps = torch.zeros((S, -(-nblk // G), d), dtype=torch.bfloat16, device=K.device)
    L_bulk = L if L_bulk is None else L_bulk
    hisa.hisa_tree_append(K, reps, sreps, 0, L_bulk, B, G, pool=pool)
    x = L_bulk
    while x < L:
        y = min(L, x + step)
        hisa.hisa_tree_append(K, reps, sreps, x, y, B, G, pool=pool)
        x = y
    return reps, sreps


def check_tree_row(orc, case, s, i, G, W, g_idx, g_score, g_blk, g_sblk, report=None, pool="mean"):
    """Comparison rule for one row of hisa_tree_index, level by level: the GPU's super-blocks
    against the oracle's (differences only at the W-th cutoff), its blocks against the top m of
    the blocks inside the GPU's super-blocks, its tokens against the refinement of its blocks."""
    q, w, K = case.q[s, i], case.w[s, i], case.K[s]
    t = int(case.qpos[s, i])
    B, m, k = case.B, case.m, case.k
    bt = t // B
    ns = bt // G + 1
    weff = min(W, ns)
    o_idx, o_sc, o_blk, o_sblk, o_keff = orc.tree_query(q, w, K, t, B, G, W, m, k, mode=pool)
    ssc = orc.tree_super_scores(q, w, K, t, B, G, mode=pool)

    # -- super-blocks
    g_sblk = np.asarray(g_sblk)
    assert np.all(g_sblk[weff:] == -1), "super-block padding"
    gs = g_sblk[:weff]
    assert np.all(gs >= 0) and np.all(np.diff(gs) > 0) and gs[-1] < ns
    c_w = _kth(np.sort(ssc)[::-1], weff)
    sdiff = set(gs.tolist()) ^ set(o_sblk[:weff].tolist())
    for u in sdiff:
        assert abs(ssc[u] - c_w) <= tol(c_w), f"super-block {u} differs (score {ssc[u]} vs cutoff {c_w})"

    # -- blocks, against the top m of the blocks inside the GPU's super-blocks
    bsc = orc.hisa_query(q, w, K, t, B, 1, 1, mode=pool)[3]
    cand = [b for u in gs.tolist() for b in range(u * G, min(u * G + G, bt + 1))]
    meff = min(m, len(cand))
    ranked = sorted(cand, key=lambda b: (-bsc[b], b))
    g_blk = np.asarray(g_blk)
    assert np.all(g_blk[meff:] == -1), "block padding"
    gb = g_blk[:meff]
    assert np.all(np.diff(gb) > 0) and np.all(np.isin(gb, cand)), "blocks must come from kept super-blocks"
    c_m = bsc[ranked[meff - 1]]
    bdiff = set(gb.tolist()) ^ set(ranked[:meff])
    for b in bdiff:
        assert abs(bsc[b] - c_m) <= tol(c_m), f"block {b} differs (score {bsc[b]} vs cutoff {c_m})"

    tdiff = _check_tokens(orc, q, w, K, t, B, k, gb, g_idx, g_score)
    if report is not None:
        for key, n in (("super_diffs", len(sdiff)), ("block_diffs", len(bdiff)), ("token_diffs", len(tdiff))):
            report[key] = report.get(key, 0) + n
    return o_idx, o_keff


def check_flat_row(orc, case, s, i, g_idx, g_score, report=None, pre=None):
    """Comparison rule for one row of dsa_flat_index; pre = (idx, score, k_eff) from the oracle."""
    q, w, K = case.q[s, i], case.w[s, i], case.K[s]
    t = int(case.qpos[s, i])
    k = case.k
    o_idx, o_sc, o_keff = pre if pre is not None else orc.flat_query(q, w, K, t, k)
    g_idx = np.asarray(g_idx)
    assert np.all(g_idx[o_keff:] == -1)
    gt = g_idx[:o_keff]
    assert np.all(gt >= 0) and np.all(np.diff(gt) > 0) and np.all(gt <= t)
    c_k = float(orc.score(q, w, K[o_idx[o_keff - 1]])) if o_keff > 0 else 0.0
    tdiff = set(gt.tolist()) ^ set(o_idx[:o_keff].tolist())
    for j in tdiff:
        sj = orc.score(q, w, K[j])
        assert abs(sj - c_k) <= tol(c_k), f"token {j} differs (score {sj} vs cutoff {c_k})"
    if g_score is not None:
        g_score = np.asarray(g_score)
        ref = dict(zip(o_idx[:o_keff].tolist(), o_sc[:o_keff].astype(np.float64).tolist()))
        for pos, j in enumerate(gt.tolist()):
            sj = ref[j] if j in ref else orc.score(q, w, K[j])
            assert abs(g_score[pos] - sj) <= tol(sj), f"score of token {j}: {g_score[pos]} vs {sj}"
    if report is not None:
        report.setdefault("flat_token_diffs", 0)
        report["flat_token_diffs"] += len(tdiff)
    return o_idx, o_keff


def iou(a, b):
    a = set(int(x) for x in a if x >= 0)
    b = set(int(x) for x in b if x >= 0)
    u = a | b
    return len(a & b) / len(u) if u else 1.0
