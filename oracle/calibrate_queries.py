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
topic per head; query i takes topic i mod 2, and every query gets its own
scale, found the same way against its own causal prefix (target 500 tokens
for the concentrated topic, 2500 for the diffuse one; bisection stops within
2 % of the target, or after 16 steps: the query is rounded to bf16, whose
relative resolution of 2^-8 the bisection over [1e-3, 1e2] reaches in about
13 steps).  These are 16384 bisections, so they run on a pool of worker
processes (one oracle thread each).

The 1M layer with shared indexer keys (config 6) is calibrated like the 1M
layer, each query against its group's shared indexer keys.

Usage:  python oracle/calibrate_queries.py [cfg ...]     (default: 3 4 5 6)
"""
import json
import math
import os
import sys
import time
from multiprocessing import Pool

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


def bisect_scale_tol(count, target, iters, tol, lo=math.log(1e-3), hi=math.log(1e2)):
    """As bisect_scale over [e^lo, e^hi], stopping once the count is within tol * target."""
    best = None
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        c = count(math.exp(mid))
        if best is None or abs(c - target) < abs(best[1] - target):
            best = (math.exp(mid), c)
        if abs(c - target) <= tol * target:
            break
        if c > target:
            lo = mid
        else:
            hi = mid
    s = float(f"{best[0]:.9g}")
    return s, count(s)


_W = {}


def _topic_task(args):
    """Scales of queries i0..i1-1 of retrieval head r of sequence b (config 5)."""
    cfg, b, r, i0, i1, iters, tol = args
    if _W.get("cfg") != cfg:
        _W.clear()
        spec = gen.spec_for(cfg)
        wl = gen.make_workload(spec, default_seed(cfg), scales={})
        _W.update(cfg=cfg, spec=spec, wl=wl, rheads=spec.retrieval_heads(),
                  dirs=gen.workload.query_directions(wl.u, wl.topics, spec.topic_mix), kidx={})
    spec, wl = _W["spec"], _W["wl"]
    h = _W["rheads"][r]
    key = (b, r // spec.idx_group)
    if key not in _W["kidx"]:
        _W["kidx"] = {key: O.index_project(wl.k_pre[b, h // spec.G], wl.w_k[r // spec.idx_group])}
    kidx = _W["kidx"][key]
    out = []
    prev = {}                                   # last scale per topic in this block: the next bracket's centre
    for i in range(i0, i1):
        m = spec.N - spec.nq + i
        d = _W["dirs"][b, h, i]
        target = spec.budget_targets[i % 2]

        def count(s):
            q = f32_to_bf16_bits((d * s).astype(np.float32))
            s_idx = O.indexer_logits(O.index_project(q, wl.w_q[r]), kidx[:m + 1])
            return len(O.topp_select(s_idx, spec.p)["sel"])

        s = c = None
        if i % 2 in prev:                       # bracket [s/2, 2 s] around the topic's previous scale
            lo, hi = math.log(prev[i % 2]) - math.log(2.0), math.log(prev[i % 2]) + math.log(2.0)
            s, c = bisect_scale_tol(count, target, 10, tol, lo, hi)
            at_edge = min(math.log(s) - lo, hi - math.log(s)) < 0.01
            if abs(c - target) > tol * target and at_edge:
                s = None                        # the target lies outside the bracket: full range
        if s is None:
            s, c = bisect_scale_tol(count, target, iters, tol)
        prev[i % 2] = s
        out.append([b, r, i, s, int(c)])
    return out


def calibrate_topics(cfg: int, iters: int = 16, tol: float = 0.02, workers: int = 0):
    spec = gen.spec_for(cfg)
    seed = default_seed(cfg)
    blk = 64
    tasks = [(cfg, b, r, i0, min(i0 + blk, spec.nq), iters, tol)
             for b in range(spec.B) for r in range(spec.Hr) for i0 in range(0, spec.nq, blk)]
    workers = workers or min(16, os.cpu_count() or 1)
    entries = []
    t0 = time.time()
    with Pool(workers) as pool:
        for k, part in enumerate(pool.imap(_topic_task, tasks)):
            entries.extend(part)
            cs = [e[4] for e in part]
            print(f"cfg{cfg} b={part[0][0]} r={part[0][1]} queries {part[0][2]}..{part[-1][2]}: |S| "
                  f"{min(cs)}..{max(cs)} ({k + 1}/{len(tasks)}, {time.time() - t0:.0f}s)", flush=True)
    return scale_key(spec, seed) + "/per-query", entries


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
        if key.endswith("/per-query"):
            table.pop(key[:-len("/per-query")], None)       # the per-topic form it replaces
        table[key] = entries
        write_table(table)


def write_table(table):
    """The scale table as JSON, one entry per line."""
    items = []
    for k, v in table.items():
        rows = ",\n  ".join(json.dumps(e) for e in v)
        items.append(f" {json.dumps(k)}: [\n  {rows}\n ]")
    with open(_SCALES_FILE, "w") as f:
        f.write("{\n" + ",\n".join(items) + "\n}\n")


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [3, 4, 5, 6])
