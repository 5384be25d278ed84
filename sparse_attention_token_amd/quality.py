"""Selection quality of HISA and of the block-sparse baseline against the flat indexer.

The pages compare HISA with block-sparse selection and with the original flat
indexer on retrieval quality (arXiv abstract; gptget.net English summary, "Key
Results"; Chinese summary, experiment design).  This sweep measures the
indexer-level version of that comparison on the seeded synthetic decode
workload with planted needles: for block sizes B and numbers of kept blocks
m, the mean IoU of each method's token set with the flat indexer's top k, the
fraction of needles each keeps, and the time of one indexing call (the key
cache stays in the last-level cache across repeats here, unlike bench.py).

The block-sparse baseline keeps the floor(k/B) best whole blocks by the same
block score; that is hisa_index with m = k/B, whose refinement then keeps
every candidate.  Both run with mean-pooled and with max-pooled block
representatives (the two poolings one page names for the coarse summaries:
"Hierarchical Indexing Makes Sparse Attention Actually Fast", section on the
hierarchical summarization of the KV cache).

The three-level tree (super-blocks of G blocks, W of them kept, then m blocks
and k tokens; same page and section, which searches a tree of summaries with a
beam of W nodes per level) runs with --fanouts: for each G and W, its IoU with
the flat top k and with the two-level HISA of the same B and m.

    python -m sparse_attention_token_amd.quality [--workload 2] [--blocks 64,128,256] [--pools mean,max]
                                                 [--fanouts 16,64 --beams 4,8,16,32]

Prints a markdown table.  Every selection runs in the library's HIP kernels.
"""
from __future__ import annotations

import argparse
import sys

import numpy as np


def _sets(idx):
    return [set(r[r >= 0].tolist()) for r in idx.reshape(-1, idx.shape[-1])]


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--workload", type=int, default=2)
    p.add_argument("--blocks", default="64,128,256")
    p.add_argument("--multiples", default="1,2,4,8",
                   help="candidate budgets m*B as multiples of k (1 = block-sparse)")
    p.add_argument("--reps", type=int, default=20)
    p.add_argument("--pools", default="mean,max", help="block representatives: mean and/or max pooling")
    p.add_argument("--fanouts", default="", help="three-level tree: blocks per super-block (G)")
    p.add_argument("--beams", default="4,8,16,32", help="three-level tree: super-blocks kept (W)")
    p.add_argument("--tree-block", type=int, default=128, help="three-level tree: block size B")
    p.add_argument("--tree-multiple", type=int, default=4, help="three-level tree: m*B as a multiple of k")
    args = p.parse_args(argv)

    import torch

    from sparse_attention_token_amd import hisa, synth

    dev = torch.device("cuda:0")
    hisa.lib()
    case = synth.workload(args.workload)
    S, T, L, k = case.S, case.T, case.L, case.k

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    K = bf(case.K)
    q = bf(case.q)
    w = torch.from_numpy(case.w).to(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    f_idx, _ = hisa.dsa_flat_index(q, w, K, L, k, None)
    torch.cuda.synchronize()
    flat = _sets(f_idx.cpu().numpy())
    needles = case.needles

    def recall(sets):
        if needles is None:
            return None
        hit = sum(int(j in sets[s * T]) for s in range(S) for j in needles[s])
        return hit / needles.size

    rows = []
    f_sc = torch.empty((S, T, k), dtype=torch.float32, device=dev)
    fws = torch.empty(hisa.dsa_flat_workspace(S, T, case.H, case.d, L, k), dtype=torch.uint8, device=dev)
    e0.record()
    for _ in range(args.reps):
        hisa.dsa_flat_index(q, w, K, L, k, None, out_idx=f_idx, out_score=f_sc, workspace=fws)
    e1.record()
    torch.cuda.synchronize()
    rows.append(("flat", "-", "-", 1.0, recall(flat), e0.elapsed_time(e1) * 1e3 / args.reps))

    for pk in args.pools.split(","):
        for B in (int(x) for x in args.blocks.split(",")):
            nblk = -(-L // B)
            pool = torch.zeros((S, nblk, case.d), dtype=torch.bfloat16, device=dev)
            hisa.hisa_pool_append(K, pool, 0, L, B, pool=pk)
            for mult in (int(x) for x in args.multiples.split(",")):
                m = mult * k // B
                if m < 1 or m > 4096 or m * B > (1 << 20):
                    continue
                ws = torch.empty(hisa.hisa_index_workspace(S, T, case.H, case.d, L, B, m, k), dtype=torch.uint8,
                                 device=dev)
                idx, sc, _ = hisa.hisa_index(q, w, K, L, pool, B, m, k, None, workspace=ws, pool=pk)
                torch.cuda.synchronize()
                sets = _sets(idx.cpu().numpy())
                iou = float(np.mean([len(a & b) / max(1, len(a | b)) for a, b in zip(sets, flat)]))
                e0.record()
                for _ in range(args.reps):
                    hisa.hisa_index(q, w, K, L, pool, B, m, k, None, out_idx=idx, out_score=sc, workspace=ws,
                                    pool=pk)
                e1.record()
                torch.cuda.synchronize()
                name = ("block-sparse" if mult == 1 else "HISA") + f" ({pk})"
                rows.append((name, B, m, iou, recall(sets), e0.elapsed_time(e1) * 1e3 / args.reps))

    tree_rows = []
    for pk in args.pools.split(",") if args.fanouts else ():
        B = args.tree_block
        m = args.tree_multiple * k // B
        nblk = -(-L // B)
        pool = torch.zeros((S, nblk, case.d), dtype=torch.bfloat16, device=dev)
        hisa.hisa_pool_append(K, pool, 0, L, B, pool=pk)
        two, _, _ = hisa.hisa_index(q, w, K, L, pool, B, m, k, None, pool=pk)
        torch.cuda.synchronize()
        two = _sets(two.cpu().numpy())
        for G in (int(x) for x in args.fanouts.split(",")):
            sp = torch.zeros((S, -(-nblk // G), case.d), dtype=torch.bfloat16, device=dev)
            hisa.hisa_tree_append(K, pool, sp, 0, L, B, G, pool=pk)
            for W in (int(x) for x in args.beams.split(",")):
                ws = torch.empty(hisa.hisa_tree_index_workspace(S, T, case.H, case.d, L, B, G, W, m, k),
                                 dtype=torch.uint8, device=dev)
                idx, sc, _, _ = hisa.hisa_tree_index(q, w, K, L, pool, sp, B, G, W, m, k, None, workspace=ws,
                                                     pool=pk)
                torch.cuda.synchronize()
                sets = _sets(idx.cpu().numpy())
                iou_f = float(np.mean([len(a & b) / max(1, len(a | b)) for a, b in zip(sets, flat)]))
                iou_2 = float(np.mean([len(a & b) / max(1, len(a | b)) for a, b in zip(sets, two)]))
                e0.record()
                for _ in range(args.reps):
                    hisa.hisa_tree_index(q, w, K, L, pool, sp, B, G, W, m, k, None, out_idx=idx, out_score=sc,
                                         workspace=ws, pool=pk)
                e1.record()
                torch.cuda.synchronize()
                tree_rows.append((pk, B, G, W, m, iou_f, iou_2, recall(sets), e0.elapsed_time(e1) * 1e3 / args.reps))

    print(f"workload {case.name}: S={S} T={T} L={L} H={case.H} d={case.d} k={k}; "
          f"{0 if needles is None else needles.size} needles")
    print("| method | B | m | mean IoU with flat top-k | needle recall | µs per call |")
    print("|---|---|---|---|---|---|")
    for name, B, m, iou, rec, us in rows:
        r = "-" if rec is None else f"{rec:.3f}"
        print(f"| {name} | {B} | {m} | {iou:.3f} | {r} | {us:.1f} |")
    if tree_rows:
        print()
        print("| tree | B | G | W | m | mean IoU with flat top-k | mean IoU with two-level HISA | needle recall "
              "| µs per call |")
        print("|---|---|---|---|---|---|---|---|---|")
        for pk, B, G, W, m, iou_f, iou_2, rec, us in tree_rows:
            r = "-" if rec is None else f"{rec:.3f}"
            print(f"| tree ({pk}) | {B} | {G} | {W} | {m} | {iou_f:.3f} | {iou_2:.3f} | {r} | {us:.1f} |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
