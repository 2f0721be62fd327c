"""Seeded synthetic decode workloads (raw draws only).

The pages measure a trained Qwen3 model on public long-context suites; none of
that is available here, so these seeded Gaussian-plus-needle inputs stand in
for them.  They keep the structure the pages describe: a head partition into
retrieval and local heads ("Full Attention Strikes Back", section 3.1/3.2),
concentrated versus diffuse retrieval queries (same paper, section 2.3 and
Figure 3) and a roughly five-fold spread of the active token budget between
the two (DeepRead summary of RTPurbo, "Key Results", niah-S vs multi-K).

Everything here is input plumbing: Gaussian draws, needle planting in the
pre-RoPE key space, rounding of the draws to bf16.  RoPE, the indexer
projection and everything downstream belong to the two implementations under
test and are not computed here.

Draw order for ``make_workload`` (one ``numpy.random.default_rng(seed)``):
  1. W_q for every retrieval q head r (ascending), each (D, R) ~ N(0, 1/D);
     then W_k the same way unless the spec shares one draw (W_k = W_q).  With
     shared indexer keys (idx_group > 1): W_k for every indexer-key head first,
     then W_q per retrieval head, or W_q[r] = W_k[r // idx_group] when shared.
  2. u = the unscaled pre-RoPE queries, (B, Hq, nq, D) ~ N(0, 1).  In
     "topics" mode (chunked prefill) these are the per-query perturbations xi,
     followed by one draw of two topic directions per head, (B, Hq, 2, D);
     query i of head h takes topic i % 2 and the direction
     normalize(t_topic + mix * xi_i).
  3. For b, then KV group g: the group's pre-RoPE keys.  Retrieval groups get
     (N, D) ~ N(0, 1) followed by one draw of all needle positions of the
     group's retrieval heads (without replacement, split in head order);
     a needle key is alpha * sqrt(D) * u_hat + its background draw (in
     "topics" mode every head plants both topics, topic 0 then topic 1, with
     u_hat the topic direction).  Local
     groups get draws only on the rows a local head reads (window + sinks).
  4. For b, then g: values, on the same rows as the keys.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field

import numpy as np

_SCALES_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "query_scales.json")


# ----------------------------------------------------------------------------- bf16 plumbing
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 input draws to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------- specs
@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    nq: int = 1
    ret_groups: tuple = (0,)
    D: int = 128
    R: int = 16
    p: float = 0.9
    window: int = 4096
    n_sink: int = 4
    rope_theta: float = 1.0e6
    # needle recipe: "fixed" -> every retrieval query plants n_needles at alpha;
    # "classes" -> class (b*Hr + r) % 2: 0 concentrated, 1 diffuse;
    # "topics" -> every retrieval head plants a concentrated topic (0) and a
    # diffuse topic (1); query i uses topic i % 2 (chunked prefill)
    needle_mode: str = "fixed"
    n_needles: int = 32
    alpha: float = 3.0
    conc: tuple = (16, 4.0)
    diffuse: tuple = (8192, 0.5)
    budget_targets: tuple = (500, 2500)
    topic_mix: float = 0.3
    # retrieval heads sharing one indexer-key head (1: one per head; G: one per KV group)
    idx_group: int = 1
    top_k: int = 0              # selection rule of the layer (0: Top-P with p); no effect on the draws
    # "unit": q = u; "table": q = s_(b,r) * u with s from the calibration table
    query_scale: str = "unit"
    shared_w: bool = True

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def head_mode(self) -> np.ndarray:
        """1 = retrieval q head, 0 = local (sliding window) q head."""
        hm = np.zeros(self.Hq, dtype=np.int8)
        for g in self.ret_groups:
            hm[g * self.G:(g + 1) * self.G] = 1
        return hm

    def retrieval_heads(self) -> list:
        return [int(h) for h in np.nonzero(self.head_mode())[0]]

    @property
    def Hr(self) -> int:
        return len(self.ret_groups) * self.G

    @property
    def Hi(self) -> int:
        """Indexer-key heads (rows of W_k and of the indexer-key cache)."""
        return self.Hr // self.idx_group

    def needle_recipe(self, b: int, r: int) -> tuple:
        """(count, alpha, class) of the needles planted for retrieval head r of batch b."""
        if self.needle_mode == "fixed":
            return self.n_needles, self.alpha, 0
        cls = (b * self.Hr + r) % 2
        cnt, alpha = self.conc if cls == 0 else self.diffuse
        return cnt, alpha, cls

    def local_rows(self) -> np.ndarray:
        """Cache rows any local head can read: the union of all queries' windows and sinks."""
        lo = max(0, self.N - self.nq - self.window + 1)
        rows = set(range(lo, self.N))
        rows.update(range(min(self.n_sink, self.N)))
        return np.array(sorted(rows), dtype=np.int64)


# The five workloads of the benchmark description, by number.
CONFIGS = {
    1: WorkloadSpec("needle-4k", B=1, Hq=1, Hkv=1, N=4096, ret_groups=(0,),
                    needle_mode="fixed", n_needles=32, alpha=3.0),
    2: WorkloadSpec("qwen3-8b-layer-32k-b8", B=8, Hq=32, Hkv=8, N=32768, ret_groups=(0,),
                    needle_mode="fixed", n_needles=64, alpha=3.0),
    3: WorkloadSpec("qwen3-8b-layer-128k-b4", B=4, Hq=32, Hkv=8, N=131072, ret_groups=(0,),
                    needle_mode="classes", query_scale="table"),
    4: WorkloadSpec("qwen3-32b-layer-1m-b1", B=1, Hq=64, Hkv=8, N=1048576, ret_groups=(0, 1),
                    needle_mode="classes", query_scale="table"),
    # the 1M layer with shared indexer keys (one indexer-key head per KV group)
    6: WorkloadSpec("qwen3-32b-layer-1m-b1-shared-keys", B=1, Hq=64, Hkv=8, N=1048576, ret_groups=(0, 1),
                    needle_mode="classes", query_scale="table", idx_group=8),
    5: WorkloadSpec("prefill-128k-4096q-4h", B=1, Hq=4, Hkv=1, N=131072, nq=4096, ret_groups=(0,),
                    needle_mode="topics", query_scale="table"),
}


def spec_for(cfg: int, **overrides) -> WorkloadSpec:
    """The spec of benchmark workload ``cfg``, optionally shrunk for tests."""
    base = CONFIGS[cfg]
    if not overrides:
        return base
    d = {k: getattr(base, k) for k in base.__dataclass_fields__}
    d.update(overrides)
    if "name" not in overrides:
        d["name"] = base.name + "-" + "-".join(f"{k}{v}" for k, v in sorted(overrides.items()))
    return WorkloadSpec(**d)


def default_seed(cfg: int) -> int:
    return 1000 + cfg


# ----------------------------------------------------------------------------- workload
@dataclass
class Workload:
    spec: WorkloadSpec
    seed: int
    q_pre: np.ndarray            # uint16 bf16 bits [B, Hq, nq, D]
    w_q: np.ndarray              # uint16 [Hr, D, R]
    w_k: np.ndarray              # uint16 [Hi, D, R] (Hi = Hr / idx_group)
    k_pre: np.ndarray            # uint16 [B, Hkv, N, D] pre-RoPE keys (zero rows never read)
    v: np.ndarray                # uint16 [B, Hkv, N, D]
    head_mode: np.ndarray        # int8 [Hq]
    u: np.ndarray = None         # float32 [B, Hq, nq, D] unscaled query draws
    needles: dict = field(default_factory=dict)   # (b, r) -> int64 positions
    classes: dict = field(default_factory=dict)   # (b, r) -> 0 concentrated / 1 diffuse
    scales: dict = field(default_factory=dict)    # (b, r) -> query scale ((b, r, topic) or ("q", b, r, i) in topics mode)
    topics: np.ndarray = None    # float32 [B, Hq, 2, D] topic directions (topics mode)

    @property
    def positions(self) -> np.ndarray:
        """Query positions m of the nq queries (the last nq cache rows)."""
        return np.arange(self.spec.N - self.spec.nq, self.spec.N, dtype=np.int64)


def query_directions(xi: np.ndarray, topics: np.ndarray, mix: float) -> np.ndarray:
    """Unit query directions of topics mode: normalize(t_(i % 2) + mix * xi_i), float64."""
    B, Hq, nq, D = xi.shape
    tsel = topics[:, :, np.arange(nq) % 2].astype(np.float64)
    d = tsel + mix * xi.astype(np.float64)
    return d / np.linalg.norm(d, axis=-1, keepdims=True)


def load_scale_table() -> dict:
    if not os.path.exists(_SCALES_FILE):
        return {}
    with open(_SCALES_FILE) as f:
        return json.load(f)


def scale_key(spec: WorkloadSpec, seed: int) -> str:
    return f"{spec.name}/{seed}"


def make_workload(spec: WorkloadSpec, seed: int, scales: dict | None = None) -> Workload:
    """Draw one seeded workload.

    ``scales`` maps (b, r) -> query scale and overrides the spec's mode; with
    ``query_scale == "table"`` the scales come from ``query_scales.json``.
    """
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, nq, D, R = spec.B, spec.Hq, spec.Hkv, spec.N, spec.nq, spec.D, spec.R
    G = spec.G
    rheads = spec.retrieval_heads()
    Hr = len(rheads)
    inv_sqrt_d = 1.0 / math.sqrt(D)

    # 1. projections
    ig = spec.idx_group
    draw_w = lambda: f32_to_bf16_bits(rng.standard_normal((D, R), dtype=np.float32) * np.float32(inv_sqrt_d))
    if ig == 1:
        w_q = np.empty((Hr, D, R), dtype=np.uint16)
        for r in range(Hr):
            w_q[r] = draw_w()
        if spec.shared_w:
            w_k = w_q.copy()
        else:
            w_k = np.empty_like(w_q)
            for r in range(Hr):
                w_k[r] = draw_w()
    else:
        # shared indexer keys: one W_k per indexer-key head; with shared_w every
        # retrieval head of the group projects its query with that same matrix
        w_k = np.empty((Hr // ig, D, R), dtype=np.uint16)
        for i in range(Hr // ig):
            w_k[i] = draw_w()
        if spec.shared_w:
            w_q = np.repeat(w_k, ig, axis=0)
        else:
            w_q = np.empty((Hr, D, R), dtype=np.uint16)
            for r in range(Hr):
                w_q[r] = draw_w()

    # 2. unscaled queries (topics mode: perturbations, then the topic directions)
    u = rng.standard_normal((B, Hq, nq, D), dtype=np.float32)
    topics = None
    if spec.needle_mode == "topics":
        topics = rng.standard_normal((B, Hq, 2, D), dtype=np.float32)

    # query scales: (b, r) -> s; in topics mode (b, r, topic) -> s for every
    # query of a topic, or ("q", b, r, i) -> s for query i alone (the
    # calibrated table holds one scale per query)
    if scales is None:
        scales = {}
        if spec.query_scale == "table":
            key = scale_key(spec, seed) + ("/per-query" if spec.needle_mode == "topics" else "")
            tab = load_scale_table().get(key)
            if tab is None:
                raise KeyError(f"no calibrated query scales for {key} in {_SCALES_FILE}")
            for e in tab:
                if spec.needle_mode == "topics":
                    scales[("q", int(e[0]), int(e[1]), int(e[2]))] = float(e[3])
                else:
                    scales[(int(e[0]), int(e[1]))] = float(e[2])
    if topics is None:
        q = u.astype(np.float64)
        for (b, r), s in scales.items():
            q[b, rheads[r]] *= s
    else:
        q = query_directions(u, topics, spec.topic_mix)
        for key, s in scales.items():
            if key[0] == "q":
                _, b, r, i = key
                q[b, rheads[r], i] *= s
            else:
                b, r, tpc = key
                q[b, rheads[r], tpc::2] *= s
    q_pre = f32_to_bf16_bits(q.astype(np.float32))

    # 3. keys (+ needles), 4. values
    k_pre = np.zeros((B, Hkv, N, D), dtype=np.uint16)
    v = np.zeros((B, Hkv, N, D), dtype=np.uint16)
    lrows = spec.local_rows()
    needles, classes = {}, {}
    n_avail = N - nq + 1 if nq > 1 else N   # needles must lie in every query's prefix
    for b in range(B):
        for g in range(Hkv):
            if g in spec.ret_groups:
                kg = rng.standard_normal((N, D), dtype=np.float32)
                rs = [r for r in range(Hr) if rheads[r] // G == g]
                if topics is None:
                    plants = [((b, r), spec.needle_recipe(b, r), u[b, rheads[r], 0]) for r in rs]
                else:
                    plants = [((b, r, tpc), (*(spec.conc if tpc == 0 else spec.diffuse), tpc), topics[b, rheads[r], tpc])
                              for r in rs for tpc in (0, 1)]
                total = sum(rec[0] for _, rec, _ in plants)
                pos_all = rng.choice(n_avail, size=total, replace=False).astype(np.int64)
                off = 0
                for key, (cnt, alpha, cls), dvec in plants:
                    pos = np.sort(pos_all[off:off + cnt])
                    off += cnt
                    direction = dvec.astype(np.float64)
                    direction /= np.linalg.norm(direction)
                    kg[pos] += (alpha * math.sqrt(D) * direction).astype(np.float32)
                    needles[key] = pos
                    classes[key] = cls
                k_pre[b, g] = f32_to_bf16_bits(kg)
                del kg
            else:
                k_pre[b, g, lrows] = f32_to_bf16_bits(rng.standard_normal((len(lrows), D), dtype=np.float32))
    for b in range(B):
        for g in range(Hkv):
            if g in spec.ret_groups:
                v[b, g] = f32_to_bf16_bits(rng.standard_normal((N, D), dtype=np.float32))
            else:
                v[b, g, lrows] = f32_to_bf16_bits(rng.standard_normal((len(lrows), D), dtype=np.float32))

    return Workload(spec=spec, seed=seed, q_pre=q_pre, w_q=w_q, w_k=w_k, k_pre=k_pre, v=v,
                    head_mode=spec.head_mode(), u=u, needles=needles, classes=classes,
                    scales={k: float(s) for k, s in scales.items()}, topics=topics)
