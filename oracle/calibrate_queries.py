"""Write gen/query_scales.json: query scales of the 128K / 1M decode and the chunked-prefill workloads.

TEST INFRASTRUCTURE (calls only the oracle and the input generator).

The budget of a retrieval query depends on how sharp its indexer logits are.
To reproduce the pages' spread of active token budgets (about 470 tokens for
a needle query versus about 2460 for a multi-key query at p = 0.9, DeepRead
summary of RTPurbo, "Key Results"), each retrieval query q = s * u of the
128K and 1M workloads gets the scale s whose oracle Top-P set (p = 0.9) has
about 500 tokens (concentrated class) or 2500 tokens (diffuse class).  The
scale is found by bisection on log s; the set size is non-increasing in s up
to bf16 rounding of q.

The chunked-prefill workload (config 5) plants a concentrated and a diffuse
topic per head; all its queries of one topic share a scale, found the same
way on the last query of that topic (the longest prefix).

The 1M layer with shared indexer keys (config 6) is calibrated like the 1M
layer, each query against its group's shared indexer keys.

Usage:  python oracle/calibrate_queries.py [cfg ...]     (default: 3 4 5 6)
"""
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
from gen.workload import _SCALES_FILE, default_seed, f32_to_bf16_bits, scale_key  # noqa: E402
import oracle as O  # noqa: E402


def bisect_scale(count, target, iters):
    """Scale s with count(s) closest to target; count is non-increasing in s."""
    lo, hi = math.log(1e-3), math.log(1e2)
    best = None
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        c = count(math.exp(mid))
        if best is None or abs(c - target) < abs(best[1] - target):
            best = (math.exp(mid), c)
        if c > target:
            lo = mid
        else:
            hi = mid
        if c == target:
            break
    s = float(f"{best[0]:.9g}")
    return s, count(s)


def calibrate_topics(cfg: int, iters: int = 34):
    spec = gen.spec_for(cfg)
    seed = default_seed(cfg)
    wl = gen.make_workload(spec, seed, scales={})
    rheads = spec.retrieval_heads()
    dirs = gen.workload.query_directions(wl.u, wl.topics, spec.topic_mix)
    entries = []
    for b in range(spec.B):
        for r, h in enumerate(rheads):
            g = h // spec.G
            kidx = O.index_project(wl.k_pre[b, g], wl.w_k[r // spec.idx_group])
            for tpc in (0, 1):
                t0 = time.time()
                i = spec.nq - 1 if (spec.nq - 1) % 2 == tpc else spec.nq - 2
                m = spec.N - spec.nq + i
                d = dirs[b, h, i]

                def count(s):
                    q = f32_to_bf16_bits((d * s).astype(np.float32))
                    s_idx = O.indexer_logits(O.index_project(q, wl.w_q[r]), kidx[:m + 1])
                    return len(O.topp_select(s_idx, spec.p)["sel"])

                target = spec.budget_targets[tpc]
                s, c = bisect_scale(count, target, iters)
                entries.append([b, r, tpc, s, int(c)])
                print(f"cfg{cfg} b={b} r={r} topic={tpc} target={target} scale={s:.5g} count={c} "
                      f"({time.time() - t0:.1f}s)", flush=True)
    return scale_key(spec, seed), entries


def calibrate(cfg: int, iters: int = 34):
    if gen.spec_for(cfg).needle_mode == "topics":
        return calibrate_topics(cfg, iters)
    spec = gen.spec_for(cfg)
    seed = default_seed(cfg)
    wl = gen.make_workload(spec, seed, scales={})
    rheads = spec.retrieval_heads()
    entries = []
    kidx_of = {}                  # indexer keys per (b, indexer-key head), shared by the group's heads
    for b in range(spec.B):
        for r, h in enumerate(rheads):
            t0 = time.time()
            g = h // spec.G
            m = spec.N - 1
            ih = r // spec.idx_group
            if (b, ih) not in kidx_of:
                kidx_of = {(b, ih): O.index_project(wl.k_pre[b, g, :m + 1], wl.w_k[ih])}
            kidx = kidx_of[(b, ih)]
            cnt_needles, alpha, cls = spec.needle_recipe(b, r)
            target = spec.budget_targets[cls]
            u = wl.u[b, h, 0].astype(np.float64)

            def count(s):
                q = f32_to_bf16_bits((u * s).astype(np.float32))
                s_idx = O.indexer_logits(O.index_project(q, wl.w_q[r]), kidx)
                return len(O.topp_select(s_idx, spec.p)["sel"])

            lo, hi = math.log(1e-3), math.log(1e2)
            best = None
            for _ in range(iters):
                mid = 0.5 * (lo + hi)
                c = count(math.exp(mid))
                if best is None or abs(c - target) < abs(best[1] - target):
                    best = (math.exp(mid), c)
                if c > target:
                    lo = mid
                else:
                    hi = mid
                if c == target:
                    break
            entries.append([b, r, float(f"{best[0]:.9g}"), int(count(float(f"{best[0]:.9g}"))), cls])
            print(f"cfg{cfg} b={b} r={r} cls={cls} target={target} scale={best[0]:.5g} count={entries[-1][3]} "
                  f"({time.time() - t0:.1f}s)", flush=True)
    return scale_key(spec, seed), entries


def main(cfgs):
    table = {}
    if os.path.exists(_SCALES_FILE):
        with open(_SCALES_FILE) as f:
            table = json.load(f)
    for cfg in cfgs:
        key, entries = calibrate(cfg)
        table[key] = entries
        with open(_SCALES_FILE, "w") as f:
            json.dump(table, f, indent=1)
            f.write("\n")


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [3, 4, 5, 6])
