"""Top-P versus fixed top-k budgets on the calibrated 128K layer (oracle only).

TEST INFRASTRUCTURE (calls only the oracle and the input generator).

A synthetic analogue of the comparison the pages make between a fixed
token budget and a query-dependent one ("Full Attention Strikes Back",
section 2.3, Figure 3 and Table 1): for every retrieval query of the
128K-context batch-4 layer (concentrated and diffuse classes, scales
calibrated by calibrate_queries.py) the oracle computes

  * the Top-P set at p = 0.9 (its size is the query's budget), and
  * fixed top-k sets at k = the mean Top-P budget and at k = the largest one,

and reports, per class, the budget and the softmax mass each rule captures.

Usage:  python oracle/budget_study.py [--p 0.9]
"""
import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
from gen.workload import default_seed  # noqa: E402
import oracle as O  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--cfg", type=int, default=3)
    ap.add_argument("--p", type=float, default=0.9)
    a = ap.parse_args()
    spec = gen.spec_for(a.cfg)
    wl = gen.make_workload(spec, default_seed(a.cfg))
    rheads = spec.retrieval_heads()
    rows = []
    for b in range(spec.B):
        kidx = {}
        for r, h in enumerate(rheads):
            g = h // spec.G
            ih = r // spec.idx_group
            if ih not in kidx:
                kidx[ih] = O.index_project(wl.k_pre[b, g], wl.w_k[ih])
            s = O.indexer_logits(O.index_project(wl.q_pre[b, h, 0], wl.w_q[r]), kidx[ih])
            t = O.topp_select(s, a.p)
            w = t["weights"]
            rows.append(dict(cls=wl.classes[(b, r)], s=s, w=w, Z=w.sum(), budget=len(t["sel"]),
                             mass=w[t["sel"]].sum() / w.sum()))
    budgets = np.array([r["budget"] for r in rows])
    ks = {"mean": int(round(budgets.mean())), "max": int(budgets.max())}
    for r in rows:
        for name, k in ks.items():
            sel = O.topk_select(r["s"], k)["sel"]
            r[f"mass_{name}"] = r["w"][sel].sum() / r["Z"]
    print(f"{spec.name}: {len(rows)} retrieval queries, p = {a.p}; fixed k = {ks['mean']} (mean Top-P budget) "
          f"and {ks['max']} (largest)")
    print(f"{'class':14s} {'queries':>7s} {'Top-P budget':>22s} {'Top-P mass':>12s} "
          f"{'top-k mass, k=' + str(ks['mean']):>24s} {'top-k mass, k=' + str(ks['max']):>24s}")
    for cls, name in ((0, "concentrated"), (1, "diffuse")):
        sub = [r for r in rows if r["cls"] == cls]
        if not sub:
            continue
        bud = np.array([r["budget"] for r in sub])
        f = lambda key: np.array([r[key] for r in sub])
        rng = lambda x: f"{x.min():.4f}-{x.max():.4f}"
        print(f"{name:14s} {len(sub):7d} {f'{bud.min()}-{bud.max()} (median {int(np.median(bud))})':>22s} "
              f"{rng(f('mass')):>12s} {rng(f('mass_mean')):>24s} {rng(f('mass_max')):>24s}")
    short = sum(1 for r in rows if r["mass_mean"] < a.p)
    print(f"queries below p with k = {ks['mean']}: {short} of {len(rows)}; "
          f"tokens attended: Top-P {budgets.sum()}, top-k {ks['mean'] * len(rows)} / {ks['max'] * len(rows)}")


if __name__ == "__main__":
    main()
