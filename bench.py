#!/usr/bin/env python3
"""HISA indexer benchmark on one MI355X.

A step is one pass of the indexing hot path over one batch: fold the batch's
newest key rows into the block pool, then index every query (block scores ->
top-m blocks -> token refinement -> top-k), through hisa_append_index (the
same as hisa_pool_append followed by hisa_index; in decode steps the last
block's mean is stored from the block stage instead of a launch of its own).  The
flat DSA indexer (dsa_flat_index) runs on the same inputs as the in-run
baseline.  Inputs are seeded synthetic workloads resident in HBM before the
timed region.  Each step reads a different replica of the key cache (and its
pool), so successive calls miss the 256 MB last-level cache as a real
per-layer call would; whole steps are captured in HIP graphs and replayed, so
the timing is of GPU work, not of Python launch overhead.

With --tree G,W the step is the three-level tree instead (super-blocks of G
blocks, beam of W super-blocks): hisa_tree_append of the newest rows, then
hisa_tree_index; the two-level step is timed beside it.

Prints one JSON line.  Default workload: decode, 8 sequences x 32K keys.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer queries/s & µs/query at L=32K/64K/128K; speedup vs flat DSA; % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix
DEFAULT_WORKLOAD = 1          # decode 8 x 32K keys: the headline
SUB_WORKLOADS = (2, 3, 4)     # decode 64K with needles, decode 128K + 77-row tail, prefill chunk


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", type=int, default=None,
                   help="0 tiny, 1 decode 32K, 2 decode 64K, 3 decode 128K, 4 prefill chunk, "
                        "5 decode 1M, 6 decode 4M (default: decode 32K as the headline, with 64K, "
                        "128K and the prefill chunk as sub-records)")
    p.add_argument("--tree", default=None, metavar="G,W",
                   help="time the three-level tree (super-blocks of G blocks, W kept) as the step")
    p.add_argument("--rotate-mib", type=int, default=1024,
                   help="cycle key-cache replicas until at least this much is touched per cycle")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-flat", action="store_true", help="skip the flat DSA baseline")
    p.add_argument("--profile-steps", type=int, default=None,
                   help="eager steps bracketed by per-kernel HIP events")
    p.add_argument("--sequences", type=int, default=None, metavar="S",
                   help="batch size of a decode workload (1..3) in place of its own, for a batch "
                        "sweep; the line then names the workload with an _S<n> suffix")
    p.add_argument("--attention", action="store_true",
                   help="also time the sparse attention over the indexer's output (latent rows of 576 entries, "
                        "512-entry values, 128 heads)")
    p.add_argument("--sweep-lengths", action="store_true",
                   help="time the HISA step and the flat indexer against the cache length L (8K .. 1M keys) "
                        "at 8 sequences, B=128, m=64, k=2048, and fit how each grows with L")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB three times (the known-size "
                        "reference that scales the HBM byte counters) and exit")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_cpu():
    """The host's CPU model and logical CPU count, for the CPU baseline."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


# ---------------------------------------------------------------- algorithmic work models

def kernel_models(case, blocks, tree=None, sblocks=None):
    """Algorithmic bytes and flops per launch of each kernel for this workload.

    Bytes count what the method must move: bf16 rows it scores (block means or
    keys), the queries and weights, and the int32 indices it returns;
    intermediates (candidate scores) are not counted.  Flops count the q.x
    contractions: 2*H*d per scored row.
    """
    S, T, H, d, B, m, k = case.S, case.T, case.H, case.d, case.B, case.m, case.k
    t = case.qpos.astype(np.int64).reshape(-1)
    nb = t // B + 1
    meff = np.minimum(m, nb)
    # exact candidate counts from the kept blocks the GPU returned
    cand = np.zeros_like(t)
    flat_blocks = blocks.reshape(S * T, m)
    for qi in range(S * T):
        bl = flat_blocks[qi][flat_blocks[qi] >= 0].astype(np.int64)
        cand[qi] = np.minimum(B, t[qi] + 1 - bl * B).sum()
    qw = S * T * (H * d * 2 + H * 4)
    row = d * 2
    models = {
        "score_blocks": dict(bytes=int(nb.sum() * row + qw), flops=int(2 * H * d * nb.sum())),
        "score_refine": dict(bytes=int(cand.sum() * row + qw), flops=int(2 * H * d * cand.sum())),
        "select_blocks": dict(bytes=int(nb.sum() * 4 + S * T * m * 4), flops=0),
        "select_refine": dict(bytes=int(cand.sum() * 4 + S * T * k * 8), flops=0),
        "score_flat": dict(bytes=int((t + 1).sum() * row + qw), flops=int(2 * H * d * (t + 1).sum())),
        "select_flat": dict(bytes=int((t + 1).sum() * 4 + S * T * k * 8), flops=0),
    }
    # the one-launch decode kernel does the block stage, the top m and the refinement
    models["index_decode"] = dict(bytes=int((nb.sum() + cand.sum()) * row + qw),
                                  flops=models["score_blocks"]["flops"] + models["score_refine"]["flops"])
    per_query_hisa = (nb.sum() + cand.sum()) * row + qw + S * T * k * 4
    if tree is not None:
        # three-level tree: super-block scores replace the block scores; the
        # blocks scored are those <= b_t inside the kept super-blocks
        G, W = tree
        st = (t // B) // G
        ns = st + 1
        flat_sb = sblocks.reshape(S * T, W)
        ntb = np.zeros_like(t)
        for qi in range(S * T):
            u = flat_sb[qi][flat_sb[qi] >= 0].astype(np.int64)
            ntb[qi] = np.clip(t[qi] // B + 1 - u * G, 0, G).sum()
        models["score_blocks"] = dict(bytes=int(ns.sum() * row + qw), flops=int(2 * H * d * ns.sum()))
        models["select_blocks"] = dict(bytes=int(ns.sum() * 4 + S * T * W * 4), flops=0)
        models["score_tree"] = dict(bytes=int(ntb.sum() * row + qw), flops=int(2 * H * d * ntb.sum()))
        models["select_tree"] = dict(bytes=int(ntb.sum() * 4 + S * T * m * 4), flops=0)
        models["own_super"] = dict(bytes=int(((t // B) - st * G + 1).sum() * row), flops=0)
        # the fused upper two levels (tree_top_kernel: super-block scores, top W,
        # the kept super-blocks' block scores written as keys; its top m is
        # select_tree)
        models["tree_top"] = dict(bytes=int((ns.sum() + ntb.sum()) * row + qw + ntb.sum() * 4 + S * T * W * 4),
                                  flops=int(2 * H * d * (ns.sum() + ntb.sum())))
        per_query_hisa = (ns.sum() + ntb.sum() + cand.sum()) * row + qw + S * T * k * 4
    return models, int(per_query_hisa), int(cand.sum())


def traffic_from_profiles(kernel, workload_name):
    """Measured HBM bytes per launch from a committed counter summary, if its
    kernel source hash still matches (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    src = os.path.join(ROOT, "sparse_attention_token_amd", "csrc", kv.get("source", ""))
    if not os.path.exists(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("source_sha256"):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- sparse attention after the indexer

ATT_HEADS, ATT_DK, ATT_DV = 128, 576, 512      # the latent decode shape of multi-head latent attention


def time_attention(hisa, case, idx, time_graphs_fn, steps, dev, hisa_step, R_index, want_cpu):
    """Time hisa_sparse_attention over the index set idx of this workload, on a synthetic latent
    cache of the same length, and the indexer step followed by the attention."""
    import torch

    S, T, L, k = case.S, case.T, case.L, case.k
    nq = S * T
    rng = np.random.default_rng(7)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    replica_bytes = S * L * ATT_DK * 2
    n_valid = int((idx >= 0).sum().item())
    touched = n_valid * ATT_DK * 2
    # replicas so that one cycle touches more than the last-level cache, within 16 GiB
    R = max(1, min(32, math.ceil(512 * 2**20 / max(touched, 1)), (16 * 2**30) // replica_bytes))
    kvs = [torch.randn((S, L, ATT_DK), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
           for _ in range(R)]
    qa = torch.from_numpy((rng.standard_normal((S, T, ATT_HEADS, ATT_DK)) * 0.05).astype(np.float32)).to(dev)
    qa = qa.to(torch.bfloat16)
    scale = 1.0 / math.sqrt(ATT_DK)
    out = torch.empty((S, T, ATT_HEADS, ATT_DV), dtype=torch.float32, device=dev)
    lse = torch.empty((S, T, ATT_HEADS), dtype=torch.float32, device=dev)
    ws = torch.empty(hisa.hisa_sparse_attention_workspace(S, T, ATT_HEADS, ATT_DK, ATT_DV, k), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()
    log(f"attention: {R} latent replicas ({R * replica_bytes / 2**30:.2f} GiB), {n_valid} selected rows per call")

    def att_step(r):
        hisa.hisa_sparse_attention(qa, kvs[r % R], L, idx, ATT_DV, scale, out=out, lse=lse, workspace=ws)

    att_steps = steps if T == 1 else max(R, min(steps, 20))
    att_ms = time_graphs_fn(att_step, att_steps, 2, "sparse attention", R_override=R)

    def both(r):
        hisa_step(r % R_index)
        hisa.hisa_sparse_attention(qa, kvs[r % R], L, idx, ATT_DV, scale, out=out, lse=lse, workspace=ws)
    both_ms = time_graphs_fn(both, att_steps, 2, "indexer step + attention", R_override=max(R, R_index))

    # per-kernel durations
    hisa.profile_enable(64)
    for i in range(min(8, R)):
        att_step(i)
    res = hisa.profile_read()
    hisa.profile_enable(0)
    kern = {name: {"avg_us": tot * 1e3 / cnt, "launches_per_call": cnt / min(8, R)} for name, (tot, cnt) in res.items()}
    byts = n_valid * ATT_DK * 2 + nq * ATT_HEADS * (ATT_DK * 2 + ATT_DV * 4 + 4)
    flops = 2 * ATT_HEADS * (ATT_DK + ATT_DV) * n_valid
    main_us = kern.get("sparse_attention", {}).get("avg_us")
    roof = None
    if main_us:
        gbs = byts / (main_us * 1e-6) / 1e9
        tfs = flops / (main_us * 1e-6) / 1e12
        roof = {"kernel": "sparse_attention", "avg_launch_us": main_us, "hbm_achieved": gbs,
                "hbm_frac": gbs / HBM_PEAK_GBS, "mfma_achieved": tfs, "mfma_frac": tfs / BF16_PEAK_TFLOPS,
                "bound": "hbm" if flops / byts < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma",
                "algorithmic_bytes_per_launch": byts, "algorithmic_flops_per_launch": flops}
    cpu = None
    if want_cpu:
        import oracle

        kv0 = kvs[0].view(torch.int16).cpu().numpy().view(np.uint16)
        q0 = qa.view(torch.int16).cpu().numpy().view(np.uint16)
        idx0 = idx.cpu().numpy()
        sel = np.arange(min(nq, 8), dtype=np.int32)
        t0 = time.perf_counter()
        oracle.sparse_attention_batch(q0, kv0, idx0, ATT_DV, scale, L, sel=sel)
        tc = time.perf_counter() - t0
        cpu = {"value": len(sel) / tc, "unit": "queries/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"{len(sel)} of {nq} queries (fp64 C oracle) in {tc:.2f} s"}
    return {"heads": ATT_HEADS, "Dk": ATT_DK, "Dv": ATT_DV, "selected_rows_per_call": n_valid,
            "latent_replicas": R, "ms_per_call": att_ms, "us_per_query": att_ms * 1e3 / nq,
            "queries_per_s": nq / (att_ms * 1e-3), "indexer_plus_attention_ms_per_step": both_ms,
            "kernels": kern, "roofline": roof, "cpu_baseline": cpu}


# ---------------------------------------------------------------- main

def bench_case(args, hisa, torch, dev, case, cpu_seconds=15.0):
    """Time one workload: the HISA step, index only, the flat indexer, latency,
    per-kernel durations, the dominant kernel's roofline and the CPU oracle
    baseline.  Returns the record (without the top-level metric fields)."""
    S, T, H, d, L, B, m, k = case.S, case.T, case.H, case.d, case.L, case.B, case.m, case.k
    tree = None
    if args.tree:
        G, W = (int(x) for x in args.tree.split(","))
        tree = (G, W)
        case.name += f"_tree_G{G}_W{W}"
    prefill = T > 1
    log(f"workload {case.name}: S={S} T={T} L={L} H={H} d={d} B={B} m={m} k={k}")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    K0 = bf(case.K)
    q = bf(case.q)
    w = torch.from_numpy(case.w).to(dev)
    nblk = -(-L // B)

    # replicas of the key cache and its pool, enough that one cycle through
    # them touches --rotate-mib (1 GiB) of what the step reads: a decode step
    # reads the kept blocks and the pooled means, a prefill chunk the whole
    # cache (32 replicas of its 32 MiB)
    touched_hisa = S * T * (min(m, nblk) * B + nblk) * d * 2 if not prefill else K0.numel() * 2
    R = max(1, math.ceil(args.rotate_mib * 2**20 / touched_hisa))
    R = min(R, 128, max(1, (16 * 2**30) // (K0.numel() * 2)))
    # a prefill run times one step per replica (each step reads a replica
    # cold); decode runs many steps over the cycle
    steps = args.steps if args.steps is not None else (max(20, R) if prefill else 400)
    warmup = args.warmup if args.warmup is not None else (3 if prefill else 40)
    Ks, pools, spools = [], [], []
    for r in range(R):
        Kr = K0 if r == 0 else K0.clone()
        pr = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=dev)
        if tree is None:
            hisa.hisa_pool_append(Kr, pr, 0, L, B)
        else:
            sp = torch.zeros((S, -(-nblk // tree[0]), d), dtype=torch.bfloat16, device=dev)
            hisa.hisa_tree_append(Kr, pr, sp, 0, L, B, tree[0])
            spools.append(sp)
        Ks.append(Kr)
        pools.append(pr)
    torch.cuda.synchronize()
    log(f"{R} replicas of the key cache ({R * K0.numel() * 2 / 2**30:.2f} GiB)")

    out_idx = torch.empty((S, T, k), dtype=torch.int32, device=dev)
    out_score = torch.empty((S, T, k), dtype=torch.float32, device=dev)
    ws = torch.empty(hisa.hisa_index_workspace(S, T, H, d, L, B, m, k), dtype=torch.uint8, device=dev)
    f_idx = torch.empty((S, T, k), dtype=torch.int32, device=dev)
    f_score = torch.empty((S, T, k), dtype=torch.float32, device=dev)
    fws = torch.empty(hisa.dsa_flat_workspace(S, T, H, d, L, k), dtype=torch.uint8, device=dev)
    L_new_rows = T                       # the step appends the batch's own newest key rows

    def two_level_step(r):
        # hisa_pool_append of the new rows, then hisa_index, in one call (the
        # library stores the last block's mean from the block stage when the
        # new rows all lie in it: decode steps)
        hisa.hisa_append_index(Ks[r], pools[r], L - L_new_rows, L, q, w, B, m, k, None, out_idx=out_idx,
                               out_score=out_score, workspace=ws)

    if tree is not None:
        G, W = tree
        tws = torch.empty(hisa.hisa_tree_index_workspace(S, T, H, d, L, B, G, W, m, k), dtype=torch.uint8,
                          device=dev)

        def tree_index_only(r):
            hisa.hisa_tree_index(q, w, Ks[r], L, pools[r], spools[r], B, G, W, m, k, None, out_idx=out_idx,
                                 out_score=out_score, workspace=tws)

        def hisa_step(r):
            hisa.hisa_tree_append(Ks[r], pools[r], spools[r], L - L_new_rows, L, B, G)
            tree_index_only(r)
    else:
        hisa_step = two_level_step

    def flat_step(r):
        hisa.dsa_flat_index(q, w, Ks[r], L, k, None, out_idx=f_idx, out_score=f_score, workspace=fws)

    def time_graphs(step_fn, nsteps, nwarm, label, R_override=None):
        RR = R if R_override is None else R_override
        for i in range(nwarm):
            step_fn(i % RR)
        torch.cuda.synchronize()
        full = torch.cuda.CUDAGraph()
        with torch.cuda.graph(full):
            for r in range(RR):
                step_fn(r)
        rem = nsteps % RR
        part = None
        if rem:
            part = torch.cuda.CUDAGraph()
            with torch.cuda.graph(part):
                for r in range(rem):
                    step_fn(r)
        full.replay()                     # one untimed replay of the captured graph
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        for _ in range(nsteps // RR):
            full.replay()
        if part is not None:
            part.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms = e0.elapsed_time(e1) / nsteps
        log(f"{label}: {nsteps} steps, {ms * 1e3:.2f} us/step (wall {wall * 1e3 / nsteps * 1e3:.2f} us/step)")
        return ms

    # ---- bulk pool build (hisa_pool_append of rows [0, L)), reported as GB/s:
    # it reads every key row and writes every block's mean
    def pool_build(r):
        if tree is None:
            hisa.hisa_pool_append(Ks[r], pools[r], 0, L, B)
        else:
            hisa.hisa_tree_append(Ks[r], pools[r], spools[r], 0, L, B, tree[0])
    pool_steps = max(R, min(steps, 64)) if not prefill else max(R, 8)
    pool_ms = time_graphs(pool_build, pool_steps, 2, "bulk pool build")
    pool_bytes = S * L * d * 2 + S * nblk * d * 2
    pool_build_rep = {"ms_per_call": pool_ms, "bytes_per_call": pool_bytes,
                      "GB_per_s": pool_bytes / (pool_ms * 1e-3) / 1e9,
                      "hbm_frac": pool_bytes / (pool_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    # ---- correctness snapshot for the reports (kept blocks, IoU vs flat, needles)
    idx_2, _, blk_h = hisa.hisa_index(q, w, K0, L, pools[0], B, m, k, None, want_blocks=True)
    sblocks = None
    idx_h = idx_2
    if tree is not None:
        idx_h, _, blk_h, sb_h = hisa.hisa_tree_index(q, w, K0, L, pools[0], spools[0], B, G, W, m, k, None,
                                                     want_blocks=True, want_super=True)
        sblocks = sb_h.cpu().numpy()
    torch.cuda.synchronize()
    blocks = blk_h.cpu().numpy()
    models, hisa_bytes, n_cand = kernel_models(case, blocks, tree, sblocks)

    # ---- timed HISA steps
    hisa_ms = time_graphs(hisa_step, steps, warmup,
                          "tree step (tree append + tree index)" if tree else "hisa step (pool append + index)")
    two_level_ms = time_graphs(two_level_step, steps, 2, "two-level step") if tree else None

    # ---- index-only timing, for the speedup of the indexer itself
    def hisa_index_only(r):
        hisa.hisa_index(q, w, Ks[r], L, pools[r], B, m, k, None, out_idx=out_idx,
                        out_score=out_score, workspace=ws)
    index_ms = time_graphs(tree_index_only if tree else hisa_index_only, steps, 2,
                           "hisa_tree_index only" if tree else "hisa_index only")

    flat_ms = None
    iou = None
    iou_two = None
    needle = None
    if not args.no_flat:
        flat_steps = max(R, min(steps, 40)) if prefill else steps
        flat_ms = time_graphs(flat_step, flat_steps, 2, "flat DSA")
        fi, _ = hisa.dsa_flat_index(q, w, K0, L, k, None)
        torch.cuda.synchronize()
        a, b = idx_h.cpu().numpy().reshape(S * T, k), fi.cpu().numpy().reshape(S * T, k)

        def mean_iou(xs, ys):
            ious = []
            for x, y in zip(xs, ys):
                sx, sy = set(x[x >= 0].tolist()), set(y[y >= 0].tolist())
                ious.append(len(sx & sy) / max(1, len(sx | sy)))
            return float(np.mean(ious))
        iou = mean_iou(a, b)
        if tree is not None:
            a2 = idx_2.cpu().numpy().reshape(S * T, k)
            iou_two = {"two_level_vs_flat": mean_iou(a2, b), "tree_vs_two_level": mean_iou(a, a2)}
        if case.needles is not None:
            hit = sum(int(j in set(a[s].tolist())) for s in range(S) for j in case.needles[s])
            fhit = sum(int(j in set(b[s].tolist())) for s in range(S) for j in case.needles[s])
            needle = {"hisa": hit / case.needles.size, "flat": fhit / case.needles.size,
                      "needles": int(case.needles.size)}
            if tree is not None:
                a2 = idx_2.cpu().numpy().reshape(S * T, k)
                needle["two_level"] = sum(int(j in set(a2[s].tolist())) for s in range(S)
                                          for j in case.needles[s]) / case.needles.size

    # ---- single-call latency: one eager call, then wait for it (host clock,
    # median), as a caller that needs each result before the next call sees it
    def latency_us(step_fn, n):
        vals = []
        for i in range(n):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            step_fn(i % R)
            torch.cuda.synchronize()
            vals.append((time.perf_counter() - t0) * 1e6)
        return float(np.median(vals))

    n_lat = 8 if prefill else 100
    latency = {"hisa_step_us": latency_us(hisa_step, n_lat), "calls": n_lat,
               "flat_us": None if args.no_flat else latency_us(flat_step, n_lat)}
    log(f"single-call latency: HISA step {latency['hisa_step_us']:.1f} us, flat {latency['flat_us']} us")

    # ---- per-kernel durations: HIP events around each kernel, eager launches
    # queued behind a long matrix product so the GPU never waits on the host
    pro_steps = args.profile_steps if args.profile_steps is not None else (4 if prefill else min(2 * R, 64))
    kernels = {}
    big = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    for label, fn, n in (("hisa", hisa_step, pro_steps), ("flat", flat_step, 0 if args.no_flat else pro_steps)):
        if n == 0:
            continue
        torch.cuda.synchronize()
        hisa.profile_enable(16 * n)
        for _ in range(6 if prefill else 12):
            torch.mm(big, big)
        for i in range(n):
            fn(i % R)
        res = hisa.profile_read()
        hisa.profile_enable(0)
        for name, (tot, cnt) in res.items():
            kernels[name] = {"avg_us": tot * 1e3 / cnt, "launches_per_step": cnt / n}
    del big

    # ---- roofline of the dominant kernel
    roofline = None
    timed = {n: v for n, v in kernels.items() if n in models}
    hisa_kern = {n: v for n, v in timed.items() if not n.endswith("_flat")}
    if hisa_kern:
        dom = max(hisa_kern, key=lambda n: hisa_kern[n]["avg_us"] * hisa_kern[n]["launches_per_step"])
        mdl = models[dom]
        sec = hisa_kern[dom]["avg_us"] * 1e-6
        if prefill and mdl["flops"] > 0:
            ach = mdl["flops"] / sec / 1e12
            roofline = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                        "algorithmic_flops_per_launch": mdl["flops"]}
        else:
            ach = mdl["bytes"] / sec / 1e9
            roofline = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                        "algorithmic_bytes_per_launch": mdl["bytes"]}
        roofline["avg_launch_us"] = hisa_kern[dom]["avg_us"]
        roofline["traffic"] = traffic_from_profiles(dom, case.name)
    # every HISA kernel's own rate against the roof that bounds it
    roofline_by_kernel = {}
    for name, v in hisa_kern.items():
        mdl = models[name]
        sec = v["avg_us"] * 1e-6
        if prefill and mdl["flops"] > 0:
            ach = mdl["flops"] / sec / 1e12
            roofline_by_kernel[name] = {"bound": "mfma", "achieved": ach, "unit": "TFLOP/s",
                                        "frac": ach / BF16_PEAK_TFLOPS, "avg_launch_us": v["avg_us"]}
        else:
            ach = mdl["bytes"] / sec / 1e9
            roofline_by_kernel[name] = {"bound": "hbm", "achieved": ach, "unit": "GB/s",
                                        "frac": ach / HBM_PEAK_GBS, "avg_launch_us": v["avg_us"],
                                        "algorithmic_bytes_per_launch": mdl["bytes"],
                                        "traffic": traffic_from_profiles(name, case.name)}

    # ---- the sparse attention over the indexer's output (opt-in)
    attention = None
    if args.attention:
        attention = time_attention(hisa, case, idx_h, time_graphs_fn=time_graphs, steps=steps, dev=dev,
                                   hisa_step=hisa_step, R_index=R, want_cpu=not args.no_cpu)

    # ---- CPU oracle baseline (bounded sample of the same workload)
    cpu = None
    if not args.no_cpu:
        import oracle

        n = S * T
        if tree is not None:
            # the tree oracle runs one query at a time on one core
            def run(sel):
                for qi in sel:
                    s_, i_ = divmod(int(qi), T)
                    oracle.tree_query(case.q[s_, i_], case.w[s_, i_], case.K[s_], int(case.qpos[s_, i_]), B, G, W,
                                      m, k)
            cores, what = 1, "tree"
        else:
            def run(sel):
                oracle.hisa_batch(case.q, case.w, case.qpos, case.K, L, B, m, k, sel=sel)
            cores, what = oracle.num_threads(), "HISA"
        # size the sample to about 10 s of oracle work: distinct queries first
        # (evenly spaced over the batch), then whole repeats of the batch
        probe = np.linspace(0, n - 1, min(n, 8)).astype(np.int32)
        t0 = time.perf_counter()
        run(probe)
        per_q = max((time.perf_counter() - t0) / len(probe), 1e-6)
        target_s = cpu_seconds
        nsel = int(min(n, max(len(probe), target_s / per_q)))
        sel = np.linspace(0, n - 1, nsel).astype(np.int32)
        reps = max(1, min(1000, int(round(target_s / (per_q * nsel)))))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(sel)
        tc = time.perf_counter() - t0
        nq_cpu = reps * len(sel)
        cpu = {"value": nq_cpu / tc, "unit": "queries/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{len(sel)} of {n} queries of {case.name} (evenly spaced), {reps} pass(es), "
                         f"through the fp64 C oracle ({what}): {nq_cpu} queries in {tc:.1f} s",
               "us_per_query": tc / nq_cpu * 1e6,
               "host": host_cpu()}
        if not args.no_flat:
            # the flat indexer's oracle on a few of the same queries (about 5 s)
            fsel = probe[:1]
            t0 = time.perf_counter()
            oracle.flat_batch(case.q, case.w, case.qpos, case.K, L, k, sel=fsel)
            per_f = max(time.perf_counter() - t0, 1e-6)
            nf = int(min(n, max(1, cpu_seconds / 3.0 / per_f)))
            fsel = np.linspace(0, n - 1, nf).astype(np.int32)
            t0 = time.perf_counter()
            oracle.flat_batch(case.q, case.w, case.qpos, case.K, L, k, sel=fsel)
            tf = time.perf_counter() - t0
            cpu["flat"] = {"value": nf / tf, "unit": "queries/s", "cores": oracle.num_threads(),
                           "sample": f"{nf} of {n} queries (evenly spaced) in {tf:.1f} s"}

    nq = S * T
    return {
        "value": nq / (hisa_ms * 1e-3),
        "unit": "queries/s",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": hisa_ms,
        "config": {"workload": case.name, "S": S, "T": T, "L": L, "H": H, "d": d, "B": B, "m": m,
                   "k": k, "key_cache_replicas": R, "parallelism": "single GPU"},
        "us_per_query": hisa_ms * 1e3 / nq,
        "single_call_latency": latency,
        "pool_build": pool_build_rep,
        "index_only": {"ms_per_call": index_ms, "queries_per_s": nq / (index_ms * 1e-3)},
        "flat": None if flat_ms is None else {"ms_per_call": flat_ms, "queries_per_s": nq / (flat_ms * 1e-3),
                                              "us_per_query": flat_ms * 1e3 / nq},
        "speedup_vs_flat": None if flat_ms is None else flat_ms / hisa_ms,
        "speedup_vs_flat_index_only": None if flat_ms is None else flat_ms / index_ms,
        "iou_vs_flat": iou,
        "tree": None if tree is None else {"G": tree[0], "W": tree[1], "two_level_ms_per_step": two_level_ms,
                                           "speedup_vs_two_level": two_level_ms / hisa_ms, **(iou_two or {})},
        "needle_recall": needle,
        "hisa_algorithmic_bytes_per_call": hisa_bytes,
        "candidates_per_call": n_cand,
        "kernels": kernels,
        "roofline": roofline,
        "roofline_by_kernel": roofline_by_kernel,
        "cpu_baseline": cpu,
        "attention": attention,
    }


SWEEP_LENGTHS = (8192, 16384, 32768, 65536, 131072, 262144, 1 << 20)


def sweep_lengths(args, hisa, torch, dev, synth):
    """HISA step and flat indexer time against L at fixed S=8, B=128, m=64,
    k=2048 (the decode 32K generator at other lengths).  The pages give the
    per-query cost as O(L/B + mB) for HISA against O(L) for the flat indexer;
    the record carries each point and the slope of log(time) against log(L)
    over the doublings from 32K up."""
    S, H, d, B, m, k = 8, 64, 128, 128, 64, 2048
    steps = args.steps if args.steps is not None else 200
    points = []
    for L in SWEEP_LENGTHS:
        c = synth.clustered_case(S, L, 1, H, d, B, m, k, seed=synth.SEED_BASE + 40 + L.bit_length())
        K0 = torch.from_numpy(c.K.view(np.int16)).to(dev).view(torch.bfloat16)
        q = torch.from_numpy(c.q.view(np.int16)).to(dev).view(torch.bfloat16)
        w = torch.from_numpy(c.w).to(dev)
        del c
        nblk = -(-L // B)
        touched = S * (m * B + nblk) * d * 2
        R = max(1, min(64, math.ceil(args.rotate_mib * 2**20 / touched), (16 * 2**30) // (K0.numel() * 2)))
        Ks, pools = [], []
        for r in range(R):
            Kr = K0 if r == 0 else K0.clone()
            pr = torch.zeros((S, nblk, d), dtype=torch.bfloat16, device=dev)
            hisa.hisa_pool_append(Kr, pr, 0, L, B)
            Ks.append(Kr)
            pools.append(pr)
        out_idx = torch.empty((S, 1, k), dtype=torch.int32, device=dev)
        out_score = torch.empty((S, 1, k), dtype=torch.float32, device=dev)
        ws = torch.empty(hisa.hisa_index_workspace(S, 1, H, d, L, B, m, k), dtype=torch.uint8, device=dev)
        fws = torch.empty(hisa.dsa_flat_workspace(S, 1, H, d, L, k), dtype=torch.uint8, device=dev)
        f_idx = torch.empty_like(out_idx)
        f_score = torch.empty_like(out_score)

        def hisa_step(r):
            hisa.hisa_append_index(Ks[r], pools[r], L - 1, L, q, w, B, m, k, None, out_idx=out_idx,
                                   out_score=out_score, workspace=ws)

        def flat_step(r):
            hisa.dsa_flat_index(q, w, Ks[r], L, k, None, out_idx=f_idx, out_score=f_score, workspace=fws)

        def timed(fn, n):
            for i in range(3):
                fn(i % R)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(R):
                    fn(r)
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, n // R)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / (reps * R)

        h_ms, f_ms = timed(hisa_step, steps), timed(flat_step, steps)
        points.append({"L": L, "blocks": nblk, "replicas": R, "hisa_us": h_ms * 1e3, "flat_us": f_ms * 1e3,
                       "speedup": f_ms / h_ms})
        log(f"sweep L={L}: HISA {h_ms * 1e3:.2f} us, flat {f_ms * 1e3:.2f} us ({f_ms / h_ms:.2f}x)")
        del Ks, pools, K0, ws, fws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    def slope(key):
        xs = [math.log2(p_["L"]) for p_ in points if p_["L"] >= 32768]
        ys = [math.log2(p_[key]) for p_ in points if p_["L"] >= 32768]
        return float(np.polyfit(xs, ys, 1)[0])

    def linfit(key):
        # time = a + b * L over the whole sweep (least squares), b in ns per key
        xs = np.array([p_["L"] for p_ in points], dtype=np.float64)
        ys = np.array([p_[key] for p_ in points], dtype=np.float64)
        b, a = np.polyfit(xs, ys, 1)
        return {"intercept_us": float(a), "ns_per_1k_keys": float(b * 1e3 * 1e3)}

    return {"sweep": "cache length", "S": S, "H": H, "d": d, "B": B, "m": m, "k": k,
            "points": points, "loglog_slope_from_32K": {"hisa": slope("hisa_us"), "flat": slope("flat_us")},
            "linear_fit": {"hisa": linfit("hisa_us"), "flat": linfit("flat_us")}}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the indexer has no "
                                   "multi-GPU path here (sequences would shard across GPUs "
                                   "without communication). Use --gpus 1."}), flush=True)
        sys.exit(2)

    import torch

    from sparse_attention_token_amd import hisa, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe * 2**20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return
    hisa.lib()
    if args.sweep_lengths:
        print(json.dumps(sweep_lengths(args, hisa, torch, dev, synth)), flush=True)
        return
    if args.workload is not None:
        wids = [args.workload]
    else:
        wids = [DEFAULT_WORKLOAD] + ([] if args.sequences is not None else list(SUB_WORKLOADS))
    records = []
    for wid in wids:
        case = synth.workload(wid, args.sequences)
        records.append(bench_case(args, hisa, torch, dev, case,
                                  cpu_seconds=15.0 if wid == wids[0] else 8.0))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    head = records[0]
    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        **{k_: v for k_, v in head.items() if k_ not in ("value", "unit", "steps", "warmup", "ms_per_step")},
    }
    if len(records) > 1:
        # the metric's other lengths and the prefill chunk, each with its own
        # timing, flat baseline, roofline and CPU oracle baseline
        res["configs"] = {r["config"]["workload"]: r for r in records[1:]}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
