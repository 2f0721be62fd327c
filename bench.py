"""Benchmark of one sparse-attention decode step (RTPurbo) on one MI355X.

Metric: decode attention microseconds per step and achieved HBM GB/s at 1M
context (Qwen3-32B-shaped layer, the headline line) and at 128K context
(Qwen3-8B-shaped layer, batch 4, reported beside it).  A step is one
rtp_decode_step: every head of the layer and every sequence of the batch,
from query preparation to the attention output.  Inputs are seeded synthetic
caches already resident in HBM; several replicas of the caches are rotated so
that successive steps do not hit the 256 MB Infinity Cache.

GB/s counts algorithmic bytes (what the method must move): 32 B of indexer
key per cached token per retrieval head, 512 B per K/V row of the union of
the selected sets of each KV group, 512 B per window-plus-sink row of each
local KV group.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import contextlib
import dataclasses
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import long_context_sparse_retrieval_amd as rtp  # noqa: E402

METRIC = "decode attn µs/step + achieved HBM GB/s at 128K and 1M ctx, 1 GPU"
HBM_PEAK_GBPS = 8000.0
TOPK_BENCH = 2048          # fixed budget of the top-k variant line (about the diffuse queries' Top-P budget)
CSRC = os.path.join(ROOT, "long_context_sparse_retrieval_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "phase_a_kernel.qwen3-32b-layer-1m-b1.traffic.json")
CPU_SAMPLE_SECONDS = 6.0
TUNING = {}                # rtp_layer tuning fields from the command line (sweeps); empty = the library's choice


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@contextlib.contextmanager
def quiet_gc():
    """Collect garbage first and keep Python's collector off while GPU work is
    timed: a full collection inside a loop of launches stalls the launches
    (seen once as 720 us of host time per step over a round of 50 steps,
    against 35 us normally)."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def up(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


# sources that decide what the phase-A kernel reads and writes: the kernel, the
# headers it includes and the launch plan
PHASE_A_SOURCES = [os.path.join(CSRC, f) for f in ("topp_kernels.hip", "swa.h", "block_util.h", "rtp_internal.h",
                                                   "api.hip")] + [os.path.join(ROOT, "include", "rtp.h")]


def _code_only(src: str) -> str:
    """C/C++ source without comments and with whitespace collapsed, so that
    edits to comments alone keep a recorded measurement valid."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            i = src.find("\n", i)
            i = n if i < 0 else i
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif src[i] in "\"'":                                 # string or character literal, kept whole
            q, j = src[i], i + 1
            while j < n and src[j] != q:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the code (not the comments) of the phase-A sources."""
    h = hashlib.sha256()
    for path in PHASE_A_SOURCES:
        with open(path, encoding="utf-8") as fh:
            h.update(os.path.basename(path).encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


class Case:
    """One benchmark workload resident on the GPU, with rotating cache replicas."""

    def __init__(self, cfg: int, replicas: int, wl=None):
        self.cfg = cfg
        self.spec = spec = gen.spec_for(cfg)
        t0 = time.time()
        self.wl = wl = gen.make_workload(spec, gen.workload.default_seed(cfg)) if wl is None else wl
        log(f"[bench] cfg{cfg} {spec.name}: drew inputs in {time.time() - t0:.1f}s")
        self.layer = rtp.Layer(B=spec.B, Hq=spec.Hq, Hkv=spec.Hkv, N=spec.N,
                               head_mode=[int(h) for h in spec.head_mode()], p=spec.p, window=spec.window,
                               n_sink=spec.n_sink, rope_theta=spec.rope_theta, idx_group=spec.idx_group,
                               **TUNING)
        t0 = time.time()
        self.q = up(wl.q_pre)
        self.w_q = up(wl.w_q)
        k_pre = up(wl.k_pre)
        # caches written by the library's own cache writers (RoPE keys, indexer keys)
        k = rtp.rope_keys(self.layer, k_pre)
        k_idx = rtp.index_keys(self.layer, k_pre, up(wl.w_k))
        del k_pre
        v = up(wl.v)
        torch.cuda.synchronize()
        self.reps = [(k_idx, k, v)]
        for _ in range(replicas - 1):
            self.reps.append((k_idx.clone(), k.clone(), v.clone()))
        torch.cuda.synchronize()
        log(f"[bench] cfg{cfg}: caches + {replicas} replicas on GPU in {time.time() - t0:.1f}s")
        self.ws = rtp.workspace(self.layer)
        self.out = torch.empty((spec.B, spec.Hq, 1, spec.D), dtype=torch.float32, device="cuda")
        self._sets()

    def _sets(self):
        spec = self.spec
        Hr = spec.Hr
        idx = torch.full((spec.B, Hr, 1, spec.N), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros((spec.B, Hr, 1), dtype=torch.int32, device="cuda")
        k_idx, k, v = self.reps[0]
        rtp.decode_step(self.layer, self.q, self.w_q, k_idx, k, v, self.ws, self.out, idx=idx, count=cnt)
        torch.cuda.synchronize()
        self.sel = (idx, cnt)                   # the step's own sets, for selection_stats
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        self.counts = cnt[:, :, 0]
        rheads = spec.retrieval_heads()
        union = total = 0
        for b in range(spec.B):
            for g in spec.ret_groups:
                rs = [r for r, h in enumerate(rheads) if h // spec.G == g]
                sets = [idx[b, r, 0, :cnt[b, r, 0]] for r in rs]
                union += len(np.unique(np.concatenate(sets)))
                total += sum(len(s) for s in sets)
        self.gather_rows_union, self.gather_rows_sum = union, total
        # algorithmic bytes of one step
        n_scan = spec.B * spec.Hi * spec.N      # indexer-key rows: one per position and indexer-key head
        lo = max(0, spec.N - spec.window)
        swa_rows = min(spec.n_sink, lo) + (spec.N - lo)
        n_local_groups = spec.Hkv - len(spec.ret_groups)
        self.bytes_scan = 32 * n_scan
        self.bytes_swa = 512 * swa_rows * spec.B * n_local_groups
        self.bytes_gather = 512 * union
        self.bytes_total = self.bytes_scan + self.bytes_swa + self.bytes_gather

    def run(self, steps: int, warmup: int):
        """Warm up, then time exactly `steps` plain steps (the headline: only a
        begin and an end event around them); then a second, instrumented pass of
        as many steps records an event before every step and after its phase A,
        for the per-step percentiles and the phase-A kernel time (each event
        record costs a few microseconds of GPU time, so that pass is slower).
        Returns (ms/step, ms of the phase-A kernel per step)."""
        R = len(self.reps)
        for s in range(warmup):
            k_idx, k, v = self.reps[s % R]
            rtp.decode_step(self.layer, self.q, self.w_q, k_idx, k, v, self.ws, self.out)
        t_begin = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_begin.record()
        for s in range(steps):
            k_idx, k, v = self.reps[s % R]
            rtp.decode_step(self.layer, self.q, self.w_q, k_idx, k, v, self.ws, self.out)
        t_end.record()
        torch.cuda.synchronize()
        ms_step = t_begin.elapsed_time(t_end) / steps
        # instrumented pass
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        mids = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for e in mids:
            e.record()          # materialise the underlying hipEvent
        i_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        for s in range(steps):
            k_idx, k, v = self.reps[s % R]
            starts[s].record()
            rtp.decode_step(self.layer, self.q, self.w_q, k_idx, k, v, self.ws, self.out, phase_event=mids[s])
        i_end.record()
        torch.cuda.synchronize()
        ms_pa = float(np.mean([starts[s].elapsed_time(mids[s]) for s in range(steps)]))
        per = [starts[s].elapsed_time(starts[s + 1]) for s in range(steps - 1)] + [starts[-1].elapsed_time(i_end)]
        self.pct = {f"p{q}": round(float(np.percentile(per, q)) * 1e3, 2) for q in (10, 50, 90)}
        self.instr_us = round(starts[0].elapsed_time(i_end) / steps * 1e3, 2)
        return ms_step, ms_pa

    def run_dense(self, steps: int, warmup: int) -> float:
        """ms per call of the dense comparator (every head over every cached position) on the same caches."""
        R = len(self.reps)
        for s in range(warmup):
            _, k, v = self.reps[s % R]
            rtp.dense_attn(self.layer, self.q, k, v, self.ws, out=self.out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for s in range(steps):
            _, k, v = self.reps[s % R]
            rtp.dense_attn(self.layer, self.q, k, v, self.ws, out=self.out)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps


def copy_ceiling_gbps() -> float:
    """Plain device copy of 2 GiB (read + write bytes / time), the box's practical streaming rate."""
    n = 1 << 29
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del a, b
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def read_ceiling() -> dict:
    """The box's streaming-read rate: libreadprobe.so's read kernels over a 2 GiB
    buffer (read once per pass, nothing written), swept over two access
    patterns (grid-stride; one contiguous chunk per workgroup, as the indexer
    scan reads), plain or non-temporal loads, grid sizes and loads in flight
    per thread; the best configuration is the ceiling the bandwidth-bound
    kernels are compared with."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_sparse_retrieval_amd", "libreadprobe.so"))
    lib.readprobe_stream.restype = ctypes.c_int
    lib.readprobe_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    configs = [(0, b, u, nt) for b in (2048, 8192) for u in (8, 16) for nt in (0, 1)]
    configs += [(1, b, u, nt) for b in (1024, 2048, 4096) for u in (8, 16) for nt in (0, 1)]
    configs += [(2, b, u, nt) for b in (1024, 2048) for u in (4, 8) for nt in (0, 1)]
    best, sweep = None, {}
    for chunked, blocks, unroll, nt in configs:
        def one():
            st = lib.readprobe_stream(buf.data_ptr(), nbytes, sink.data_ptr(), blocks, unroll, chunked, nt, stream)
            if st != 0:
                raise RuntimeError(f"readprobe_stream: status {st}")
        for _ in range(2):
            one()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            one()
        e1.record()
        torch.cuda.synchronize()
        gbps = nbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        key = f"{('stride', 'chunk', 'rows32')[chunked]}-{blocks}x{unroll}{'-nt' if nt else ''}"
        sweep[key] = round(gbps, 1)
        if best is None or gbps > best[0]:
            best = (gbps, key)
    del buf
    return {"GBps": round(best[0], 1), "config": best[1], "bytes": nbytes, "sweep": sweep}


def exp_lds_ceiling(blocks: int = 4096, rounds: int = 128) -> dict:
    """Scores per second of libreadprobe.so's exp_lds_kernel: the chunked
    prefill's per-score histogram work (cell, in-cell exponential weight, one
    64-bit LDS atomic into one of 16 per-query histograms) with no indexer and
    no memory traffic -- the arithmetic ceiling of the selection's histogram pass."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_sparse_retrieval_amd", "libreadprobe.so"))
    lib.readprobe_exp_lds.restype = ctypes.c_int
    lib.readprobe_exp_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def one():
        st = lib.readprobe_exp_lds(blocks, rounds, sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"readprobe_exp_lds: status {st}")
    one()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        one()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    scores = blocks * 256 * 16 * rounds
    return {"scores_per_s": round(scores / (ms * 1e-3), 1), "ms_per_launch": round(ms, 4),
            "scores_per_launch": scores, "workgroups": blocks}


def calibration_copy(n_bytes: int = 1 << 30, reps: int = 3) -> None:
    """A plain streaming copy of known size (negation: read n_bytes, write n_bytes).

    Run under rocprofv3 --pmc, its FETCH_SIZE / WRITE_SIZE readings give the
    scale from those counters to bytes moved on this device.
    """
    a = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def traffic_per_launch(workload: str):
    """rocprof-measured HBM bytes per phase-A launch, if taken on the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def time_append(case: Case) -> dict:
    """rtp_append_kv on the layer's caches (run last: it overwrites a cache replica).

    One token: the GPU time of a single call, queued behind a busy-wait kernel so
    the host's launch time is not in it (median of 50).  Bulk: every position of
    the context appended in one call (the caches' initial fill), algorithmic
    bytes = new keys and values read once, K, V and indexer keys written."""
    spec, lay = case.spec, case.layer
    k_idx, k, v = case.reps[-1]
    w_k = up(case.wl.w_k)
    # any [B, Hkv, N, D] bf16 tensor outside the written caches serves as new rows
    src = case.reps[0][2] if len(case.reps) > 1 else case.reps[0][2].clone()
    one = src[:, :, :1].contiguous()
    for _ in range(5):
        rtp.append_kv(lay, one, one, w_k, k, v, k_idx, spec.N - 1)
    times = []
    for _ in range(50):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(200_000)
        e0.record()
        rtp.append_kv(lay, one, one, w_k, k, v, k_idx, spec.N - 1)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    rtp.append_kv(lay, src, src, w_k, k, v, k_idx, 0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        rtp.append_kv(lay, src, src, w_k, k, v, k_idx, 0)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    nbytes = 4 * spec.B * spec.Hkv * spec.N * 256 + spec.B * spec.Hi * spec.N * 32
    return {"what": "rtp_append_kv: post-RoPE keys, values and indexer keys of new tokens in one launch",
            "one_token_us": round(float(np.median(times)), 2), "bulk_rows": spec.N, "bulk_ms": round(ms, 3),
            "bulk_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "bulk_algorithmic_bytes": nbytes}


def time_local_ring(case: Case, steps: int, warmup: int) -> dict:
    """The same step over ring-buffer caches (rtp_layer.local_ring): all-local KV
    groups keep n_sink + window rows.  The ring caches are written by one bulk
    rtp_append_kv of the whole context; the step must equal the full layout's
    bit for bit, and is timed like the Top-P step."""
    spec = case.spec
    lay = dataclasses.replace(case.layer, local_ring=1)
    shape = rtp.kv_shape(lay)
    k_idx0, _, v0 = case.reps[0]
    kr, vr = torch.empty(shape, dtype=torch.bfloat16, device="cuda"), torch.empty(shape, dtype=torch.bfloat16,
                                                                                  device="cuda")
    ki = torch.empty_like(k_idx0)
    k_pre = up(case.wl.k_pre)
    rtp.append_kv(lay, k_pre, v0, up(case.wl.w_k), kr, vr, ki, 0)
    del k_pre
    same_keys = bool(torch.equal(ki, k_idx0))
    del ki
    reps = [(case.reps[i][0], kr.clone() if i else kr, vr.clone() if i else vr) for i in range(len(case.reps))]
    ws = rtp.workspace(lay)
    out_full = rtp.decode_step(case.layer, case.q, case.w_q, *case.reps[0], case.ws)
    out_ring = rtp.decode_step(lay, case.q, case.w_q, *reps[0], ws)
    identical = bool(torch.equal(out_full, out_ring))
    for s in range(warmup):
        rtp.decode_step(lay, case.q, case.w_q, *reps[s % len(reps)], ws, case.out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for s in range(steps):
        rtp.decode_step(lay, case.q, case.w_q, *reps[s % len(reps)], ws, case.out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    full_bytes = 2 * 2 * spec.B * spec.Hkv * spec.N * spec.D
    return {"what": "same step over ring-buffer K/V caches for the all-local KV groups (local_ring = 1)",
            "us_per_step": round(us, 2), "kv_cache_bytes_full": full_bytes,
            "kv_cache_bytes_ring": 2 * 2 * spec.B * rtp.kv_rows(lay) * spec.D,
            "outputs_identical_to_full_layout": identical, "indexer_keys_identical": same_keys}


CLUSTER_K, CLUSTER_ITERS = 128, 8     # cluster index: the article's example K, k-means rounds


def time_cluster(case: Case, steps: int) -> dict:
    """Cluster index on the case's caches: the k-means build once (timed), then
    the coarse-to-fine decode step over it (timed like the Top-P step)."""
    spec, lay = case.spec, case.layer
    ws = rtp.cluster_workspace(lay, CLUSTER_K)
    k_idx, k, v = case.reps[0]
    rtp.cluster_build(lay, k_idx, CLUSTER_K, CLUSTER_ITERS, ws)          # warm-up (code load)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    index = rtp.cluster_build(lay, k_idx, CLUSTER_K, CLUSTER_ITERS, ws)
    e1.record()
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1)
    cnt = torch.zeros((spec.B, spec.Hr, 1), dtype=torch.int32, device="cuda")
    rtp.cluster_step(lay, case.q, case.w_q, index, k, v, ws, case.out, count=cnt)
    for _ in range(5):
        rtp.cluster_step(lay, case.q, case.w_q, index, k, v, ws, case.out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        rtp.cluster_step(lay, case.q, case.w_q, index, k, v, ws, case.out)
    e1.record()
    torch.cuda.synchronize()
    return {"what": f"rtp_cluster_build (K = {CLUSTER_K}, {CLUSTER_ITERS} k-means rounds per indexer-key head) "
                    "and rtp_cluster_step over it, same caches",
            "build_ms": round(build_ms, 3), "us_per_step": round(e0.elapsed_time(e1) / steps * 1e3, 2),
            "selected_tokens": cnt.cpu().numpy().ravel().tolist()}


def time_cluster_topics(steps: int) -> dict:
    """The cluster index where its premise holds: the 1M layer (64 q / 8 kv
    heads, KV groups 0-1 retrieval) with pre-RoPE keys of the retrieval groups
    drawn around 128 topic centres (k = mu_t + 0.3 eps, topics uniform over
    positions) and each retrieval query along one topic centre; local groups
    and values plain Gaussian.  Caches written by rtp_append_kv.  Reports the
    cluster step against the Top-P step on the same caches, the member-set
    sizes and the fraction of the query's topic the set covers (recall)."""
    B, Hq, Hkv, N, T = 1, 64, 8, 1 << 20, 128
    hm = [1] * 16 + [0] * 48
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, head_mode=hm)
    gen_ = torch.Generator(device="cuda").manual_seed(4242)
    mu = torch.randn((2, T, 128), device="cuda", generator=gen_)
    topic = torch.randint(0, T, (2, N), device="cuda", generator=gen_)
    k_pre = torch.randn((B, Hkv, N, 128), device="cuda", generator=gen_)
    for g in range(2):
        k_pre[0, g] = mu[g, topic[g]] + 0.3 * k_pre[0, g]
    k_pre = k_pre.to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, 128), device="cuda", generator=gen_).to(torch.bfloat16)
    w = (torch.randn((16, 128, 16), device="cuda", generator=gen_) / 128 ** 0.5).to(torch.bfloat16)
    tq = torch.randint(0, T, (16,), device="cuda", generator=gen_)
    q = torch.randn((B, Hq, 1, 128), device="cuda", generator=gen_)
    for r in range(16):
        q[0, r, 0] = mu[r // 8, tq[r]]
    q = q.to(torch.bfloat16)
    kc, vc = torch.empty_like(k_pre), torch.empty_like(v)
    ki = torch.empty((B, 16, N, 16), dtype=torch.bfloat16, device="cuda")
    rtp.append_kv(lay, k_pre, v, w, kc, vc, ki, 0)
    del k_pre
    ws = rtp.cluster_workspace(lay, CLUSTER_K)
    index = rtp.cluster_build(lay, ki, CLUSTER_K, CLUSTER_ITERS, ws)
    out = torch.empty((B, Hq, 1, 128), dtype=torch.float32, device="cuda")
    idx = torch.full((B, 16, 1, N), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, 16, 1), dtype=torch.int32, device="cuda")
    rtp.cluster_step(lay, q, w, index, kc, vc, ws, out, idx=idx, count=cnt)
    torch.cuda.synchronize()
    cnt_h = cnt.cpu().numpy().ravel()
    recall = []
    for r in range(16):
        sel = idx[0, r, 0, :int(cnt_h[r])].long()
        in_topic = int((topic[r // 8, sel] == tq[r]).sum().item())
        recall.append(in_topic / max(1, int((topic[r // 8] == tq[r]).sum().item())))

    def timed(fn):
        for _ in range(5):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    us_cluster = timed(lambda: rtp.cluster_step(lay, q, w, index, kc, vc, ws, out))
    us_topp = timed(lambda: rtp.decode_step(lay, q, w, ki, kc, vc, ws, out))
    return {"what": "1M layer with 128-topic retrieval keys (k = mu_t + 0.3 eps), queries along a topic centre: "
                    f"cluster step (K = {CLUSTER_K}) vs the Top-P step on the same caches",
            "cluster_us_per_step": round(us_cluster, 2), "topp_us_per_step": round(us_topp, 2),
            "speedup": round(us_topp / us_cluster, 3), "selected_tokens": cnt_h.tolist(),
            "topic_recall_min": round(min(recall), 4)}


PREFILL_N = 32768             # full prefill of a 32K context, the pages' shortest prefill figure


def time_prefill() -> dict:
    """rtp_prefill_attn on the 32K layer (32 q / 8 kv heads, KV group 0 retrieval):
    RTPurbo prefill (retrieval heads dense, local heads window 4096 + 4 sinks)
    against every head dense, all 32768 queries causal; seeded synthetic inputs.
    Algorithmic flops: 4 * 128 per (query, key) pair the attention visits."""
    B, Hq, Hkv, N, W, S = 1, 32, 8, PREFILL_N, 4096, 4
    hm = [1] * 4 + [0] * 28
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, nq=N, head_mode=hm, window=W, n_sink=S)
    gen_ = torch.Generator(device="cuda").manual_seed(2032)
    q, k, v = (torch.randn((B, h, N, 128), device="cuda", generator=gen_).to(torch.bfloat16) for h in (Hq, Hkv, Hkv))
    out = torch.empty((B, Hq, N, 128), dtype=torch.float32, device="cuda")
    pairs_dense = B * Hq * N * (N + 1) / 2
    local_pairs = sum(min(m + 1, W) + min(S, max(0, m + 1 - W)) for m in range(N))
    pairs = {True: pairs_dense, False: B * (4 * N * (N + 1) / 2 + 28 * local_pairs)}
    res = {}
    for dense in (False, True):
        rtp.prefill_attn(lay, q, k, v, out, all_dense=dense)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(3):
            rtp.prefill_attn(lay, q, k, v, out, all_dense=dense)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        res[dense] = (ms, pairs[dense] * 512 / (ms * 1e-3) / 1e12)
    return {"what": "rtp_prefill_attn, 32 q / 8 kv heads (4 retrieval), 32768 causal queries: RTPurbo prefill "
                    "(retrieval heads dense, local heads window 4096 + 4 sinks) vs every head dense",
            "rtpurbo_ms": round(res[False][0], 3), "dense_ms": round(res[True][0], 3),
            "speedup": round(res[True][0] / res[False][0], 3),
            "rtpurbo_TFLOPs": round(res[False][1], 1), "dense_TFLOPs": round(res[True][1], 1),
            "peak_bf16_TFLOPs": 2500.0}


def selection_stats(case: Case) -> dict:
    """What the Top-P sets of the step keep, per query class of the workload
    (needle-class queries with a few strong keys, diffuse ones): |S|, the
    sparsity 1 - |S| / N and the retained indexer mass sum_{n in S} softmax(s)_n
    (>= p by construction), from the library's own scores (rtp_index_score)
    and sets, summed in fp64."""
    spec, lay = case.spec, case.layer
    idx, cnt = case.sel
    logits = rtp.index_score(lay, case.q, case.w_q, case.reps[0][0])
    rows = []
    for b in range(spec.B):
        for r in range(spec.Hr):
            s = logits[b, r, 0].double()
            w = torch.exp(s - s.max())
            c = int(cnt[b, r, 0].item())
            sel = idx[b, r, 0, :c].long()
            rows.append({"b": b, "r": r, "cls": int(case.wl.classes.get((b, r), -1)), "S": c,
                         "sparsity": 1.0 - c / spec.N, "mass": float(w[sel].sum() / w.sum())})
    del logits
    out = {"p": spec.p, "N": spec.N}
    for cls, name in ((0, "needle_class"), (1, "diffuse")):
        q = [x for x in rows if x["cls"] == cls]
        if not q:
            continue
        out[name] = {"queries": len(q),
                     "S_mean": round(float(np.mean([x["S"] for x in q])), 1),
                     "S_min": min(x["S"] for x in q), "S_max": max(x["S"] for x in q),
                     "sparsity_mean": round(float(np.mean([x["sparsity"] for x in q])), 6),
                     "retained_mass_mean": round(float(np.mean([x["mass"] for x in q])), 6),
                     "retained_mass_min": round(min(x["mass"] for x in q), 6)}
    out["per_query"] = [[x["b"], x["r"], x["cls"], x["S"], round(x["mass"], 6)] for x in rows]
    out["per_query_fields"] = ["b", "retrieval head", "class (0 needle, 1 diffuse)", "|S|", "retained mass"]
    return out


def time_other_decode(cfg: int, steps: int, warmup: int, replicas: int) -> dict:
    """The decode step of another workload of the benchmark description, timed
    like the headline (needle 4K: a launch-latency case, its bytes fraction is
    not meaningful; 32K batch 8: the window-attention-dominated case)."""
    case = Case(cfg, replicas)
    ms, ms_pa = case.run(steps, warmup)
    gbps = case.bytes_total / (ms * 1e-3) / 1e9
    out = {"workload": case.spec.name, "us_per_step": round(ms * 1e3, 2), "GBps": round(gbps, 1),
           "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_step": case.bytes_total,
           "phase_a_kernel_us": round(ms_pa * 1e3, 2), "instrumented_us_per_step": case.instr_us,
           "selected_tokens": case.counts.ravel().tolist()}
    if case.spec.N >= 32768:
        # the same step with every head attending over every cached position
        ms_dense = case.run_dense(max(5, steps // 10), 3)
        dense_bytes = 512 * case.spec.B * case.spec.Hkv * case.spec.N
        dense_peak_us = dense_bytes / HBM_PEAK_GBPS / 1e3
        out["dense_comparator"] = {"what": "rtp_dense_attn: every head over every cached position, same caches",
                                   "us_per_step": round(ms_dense * 1e3, 2),
                                   "GBps": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1),
                                   "sparse_speedup": round(ms_dense / ms, 3),
                                   "dense_at_hbm_peak_us": round(dense_peak_us, 2),
                                   "sparse_speedup_vs_dense_at_peak": round(dense_peak_us / (ms * 1e3), 3)}
    return out


def time_chunked_prefill(calls: int = 3) -> dict:
    """rtp_decode_step with nq = 4096 causal queries against 128K positions (4
    retrieval heads, topic-structured keys and queries): the decode-path
    selection applied to every prefill query.  Work: the sum over queries and
    heads of the prefix length (logits scored in each of the selection's
    passes) and the rows the attention gathers."""
    spec = gen.spec_for(5)
    wl = gen.make_workload(spec, gen.workload.default_seed(5))
    lay = rtp.Layer(B=spec.B, Hq=spec.Hq, Hkv=spec.Hkv, N=spec.N, nq=spec.nq,
                    head_mode=[int(h) for h in spec.head_mode()], p=spec.p, window=spec.window,
                    n_sink=spec.n_sink, rope_theta=spec.rope_theta, idx_group=spec.idx_group)
    k_pre = up(wl.k_pre)
    k = rtp.rope_keys(lay, k_pre)
    k_idx = rtp.index_keys(lay, k_pre, up(wl.w_k))
    del k_pre
    v, q, w_q = up(wl.v), up(wl.q_pre), up(wl.w_q)
    ws = rtp.workspace(lay)
    out = torch.empty((spec.B, spec.Hq, spec.nq, spec.D), dtype=torch.float32, device="cuda")
    cnt = torch.zeros((spec.B, spec.Hr, spec.nq), dtype=torch.int32, device="cuda")
    idx = torch.empty((spec.B, spec.Hr, spec.nq, 1), dtype=torch.int32, device="cuda")
    rtp.decode_step(lay, q, w_q, k_idx, k, v, ws, out, idx=idx, count=cnt)      # counts (one position each kept)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(calls):
        rtp.decode_step(lay, q, w_q, k_idx, k, v, ws, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    prefix = sum(spec.N - spec.nq + i + 1 for i in range(spec.nq))
    logits = spec.B * spec.Hr * prefix
    c = cnt.cpu().numpy()[0]                                    # [Hr, nq]
    rows = int(c.sum())
    # |S| per topic: query i takes topic i mod 2 (0 concentrated, 1 diffuse)
    per_topic = {}
    for tpc, name in ((0, "concentrated_topic"), (1, "diffuse_topic")):
        s = c[:, tpc::2].ravel()
        per_topic[name] = {"queries": int(s.size), "S_mean": round(float(s.mean()), 1),
                           "S_p10": int(np.percentile(s, 10)), "S_p50": int(np.percentile(s, 50)),
                           "S_p90": int(np.percentile(s, 90)), "S_min": int(s.min()), "S_max": int(s.max()),
                           "per_head_mean": [round(float(x), 1) for x in c[:, tpc::2].mean(axis=1)]}
    ceil = exp_lds_ceiling()
    out = {"workload": spec.name, "what": "rtp_decode_step, nq = 4096 causal queries (chunked prefill selection "
                                          "and sparse attention of 4 retrieval heads)",
           "ms_per_call": round(ms, 3), "logits_per_call": logits,
           "logits_per_s": round(logits / (ms * 1e-3), 1), "gathered_rows": rows,
           "gathered_GB": round(rows * 512 / 1e9, 3),
           "S_mean_per_query": round(rows / c.size, 1),
           "calibration": ("one query scale per query, calibrated by the oracle against the query's own causal "
                           "prefix to |S| = 500 (concentrated topic) / 2500 (diffuse topic), within 2 % where the "
                           "set size allows (gen/query_scales.json, oracle/calibrate_queries.py)"),
           "S_per_topic": per_topic,
           "exp_lds_ceiling": ceil,
           "histogram_pass_scores": logits}
    # the kernel split of this call from its committed rocprofv3 trace (same command)
    split = chunked_prefill_split()
    if split:
        sel_us, attn_us = split["pf_select_kernel"], split["pf_attn_kernel"]
        out["kernel_split"] = {
            "source": split["source"], "pf_select_kernel_us": sel_us, "pf_attn_kernel_us": attn_us,
            "pf_select_passes": 4,
            "passes": "per-query maximum, exact histogram (the exp + LDS-add work), per-chunk counts, "
                      "ordered emission; each recomputes the scores on the matrix cores",
            "pf_select_scores_per_s": round(logits / (sel_us * 1e-6), 1),
            "pf_select_frac_of_exp_lds_ceiling": round(logits / (sel_us * 1e-6) / ceil["scores_per_s"], 4),
            "pf_select_score_evaluations_per_s": round(4 * logits / (sel_us * 1e-6), 1),
            "attention_gather_GBps": round(rows * 512 / (attn_us * 1e-6) / 1e9, 1),
            "pf_select_matrix_core_busy": counter_line(CP_COUNTERS, "matrix-core busy"),
            "pf_select_valu_busy": counter_line(CP_COUNTERS, "VALU busy"),
            "pf_select_lds_bank_conflict_stall": counter_line(CP_COUNTERS, "LDS bank-conflict stall"),
            "counters_source": os.path.relpath(CP_COUNTERS, ROOT)}
    return out


CP_COUNTERS = os.path.join(ROOT, "profiles", "pf_select_kernel.prefill-128k-4096q-4h.counters.txt")


def counter_line(path: str, label: str):
    """The value of a derived line ("<label> ... <value>") of a committed counter summary."""
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as fh:
        for line in fh:
            if line.strip().startswith(label):
                try:
                    return float(line.split()[-1])
                except ValueError:
                    return None
    return None


CP_TRACE = os.path.join(ROOT, "profiles", "pf_select_kernel.prefill-128k-4096q-4h.kernel_trace.txt")


def chunked_prefill_split() -> dict | None:
    """Average pf_select_kernel / pf_attn_kernel durations (us) per call from the
    committed kernel trace of `bench.py --chunked-prefill` (kernels per call:
    one of each per chunk of queries, summed)."""
    if not os.path.exists(CP_TRACE):
        return None
    per, calls = {}, {}
    with open(CP_TRACE, encoding="utf-8") as fh:
        for line in fh:
            f = line.split()
            if len(f) >= 7 and f[0].startswith(("pf_select_kernel", "pf_attn_kernel")):
                name = f[0].split("<")[0]
                n, avg = int(f[-5]), float(f[-4])
                per[name] = per.get(name, 0.0) + n * avg
                calls[name] = calls.get(name, 0) + n
    if "pf_select_kernel" not in per or "pf_attn_kernel" not in per:
        return None
    ncall = 4                                   # the traced command makes one set-up call and three timed calls
    return {"source": os.path.relpath(CP_TRACE, ROOT),
            "pf_select_kernel": round(per["pf_select_kernel"] / ncall, 1),
            "pf_attn_kernel": round(per["pf_attn_kernel"] / ncall, 1)}


CPU_WORKERS_MAX = 16       # host cores that go with one GPU on the measuring machines
CPU_ALL_WALL_SECONDS = 6.0  # wall time of the timed all-cores passes


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# per-process state of the oracle workers: the step's arrays, memory-mapped
_CPU = {}


def _cpu_init(d: str, meta: dict):
    import threadpoolctl
    threadpoolctl.threadpool_limits(1)
    _CPU.clear()
    _CPU["meta"] = meta
    for name in ("kp", "kc", "ki", "v"):
        _CPU[name] = np.load(os.path.join(d, name + ".npy"), mmap_mode="r+")
    for name in ("q_pre", "w_q", "w_k", "head_mode"):
        _CPU[name] = np.load(os.path.join(d, name + ".npy"))


def _cpu_task(task):
    """One unit of oracle work.  ("rope", b, g, r0, r1) and ("idx", b, i, r0, r1)
    write cache rows (untimed set-up); ("decode", b, heads) runs the oracle's
    step for those heads and returns (seconds, {(b, r): selected positions})."""
    import oracle as O
    m, kind = _CPU["meta"], task[0]
    if kind == "rope":
        _, b, g, r0, r1 = task
        rows = np.arange(r0, r1, dtype=np.int64) if r1 > r0 else np.asarray(m["local_rows"], np.int64)
        _CPU["kc"][b, g, rows] = O.rope_keys(_CPU["kp"][b, g, rows], m["rope_theta"], rows)
        return None
    if kind == "idx":
        _, b, i, r0, r1 = task
        g = m["rheads"][i * m["idx_group"]] // m["G"]
        _CPU["ki"][b, i, r0:r1] = O.index_project(_CPU["kp"][b, g, r0:r1], _CPU["w_k"][i])
        return None
    _, b, heads = task
    t0 = time.perf_counter()
    res = O.decode_step(_CPU["q_pre"], _CPU["w_q"], _CPU["ki"], _CPU["kc"], _CPU["v"], _CPU["head_mode"],
                        N=m["N"], p=m["p"], window=m["window"], n_sink=m["n_sink"], rope_base=m["rope_theta"],
                        heads=heads, batches=[b], idx_group=m["idx_group"])
    return time.perf_counter() - t0, {k[:2]: v for k, v in res["sel"].items()}


def cpu_baseline(spec, wl) -> dict:
    """The oracle on the host cores, over the whole 1M step.

    Set-up (not timed): the step's inputs go to memory-mapped files and a pool
    of worker processes (one oracle thread each) writes the RoPE key cache and
    the indexer-key cache with the oracle's own functions, in row blocks.
    Timed: every (sequence, head) of the step -- each retrieval head on its
    own, each local KV group's heads together -- is one task; after one
    untimed pass, enough passes to fill about CPU_ALL_WALL_SECONDS of wall time
    go to the pool at once.  GB/s counts the step's algorithmic bytes (the
    GPU's definition, with the oracle's own selected sets) per pass.
    Beside it, one process with one thread runs two retrieval heads and one
    local group on the same caches for about CPU_SAMPLE_SECONDS.
    """
    import multiprocessing as mp
    import shutil
    import tempfile

    import threadpoolctl

    t_setup = time.time()
    B, Hkv, N, D, R = spec.B, spec.Hkv, spec.N, spec.D, spec.R
    rheads = [int(h) for h in spec.retrieval_heads()]
    lrows = spec.local_rows()
    loc_groups = [g for g in range(Hkv) if g not in spec.ret_groups]
    workers = max(1, min(CPU_WORKERS_MAX, len(os.sched_getaffinity(0))))
    meta = dict(N=N, p=spec.p, window=spec.window, n_sink=spec.n_sink, rope_theta=spec.rope_theta,
                idx_group=spec.idx_group, G=spec.G, rheads=rheads, local_rows=[int(x) for x in lrows])
    d = tempfile.mkdtemp(prefix="rtp_oracle_")
    try:
        def mm(name, shape):
            return np.lib.format.open_memmap(os.path.join(d, name + ".npy"), mode="w+", dtype=np.uint16, shape=shape)
        kp, vv = mm("kp", (B, Hkv, N, D)), mm("v", (B, Hkv, N, D))
        for b in range(B):
            for g in range(Hkv):
                if g in spec.ret_groups:
                    kp[b, g], vv[b, g] = wl.k_pre[b, g], wl.v[b, g]
                else:
                    kp[b, g, lrows], vv[b, g, lrows] = wl.k_pre[b, g, lrows], wl.v[b, g, lrows]
        kp.flush(), vv.flush()
        del kp, vv
        mm("kc", (B, Hkv, N, D)).flush()
        mm("ki", (B, spec.Hi, N, R)).flush()
        for name in ("q_pre", "w_q", "w_k", "head_mode"):
            np.save(os.path.join(d, name + ".npy"), np.ascontiguousarray(getattr(wl, name)))
        blk = 1 << 16
        setup = [("rope", b, g, r0, min(N, r0 + blk)) for b in range(B) for g in spec.ret_groups
                 for r0 in range(0, N, blk)]
        setup += [("rope", b, g, 0, 0) for b in range(B) for g in loc_groups]
        setup += [("idx", b, i, r0, min(N, r0 + blk)) for b in range(B) for i in range(spec.Hi)
                  for r0 in range(0, N, blk)]
        items = [("decode", b, [h]) for b in range(B) for h in rheads]
        items += [("decode", b, list(range(g * spec.G, (g + 1) * spec.G))) for b in range(B) for g in loc_groups]
        with mp.get_context("spawn").Pool(workers, initializer=_cpu_init, initargs=(d, meta)) as pool:
            for _ in pool.imap_unordered(_cpu_task, setup, chunksize=1):
                pass
            t_setup = time.time() - t_setup
            warm = pool.map(_cpu_task, items, chunksize=1)
            sets = {}
            for _, s in warm:
                sets.update(s)
            cpu_pass = sum(t for t, _ in warm)
            passes = max(2, int(round(CPU_ALL_WALL_SECONDS * workers / cpu_pass)))
            t0 = time.perf_counter()
            for _ in pool.imap_unordered(_cpu_task, items * passes, chunksize=1):
                pass
            wall = time.perf_counter() - t0
        union = 0
        for b in range(B):
            for g in spec.ret_groups:
                rs = [r for r, h in enumerate(rheads) if h // spec.G == g]
                union += len(np.unique(np.concatenate([sets[(b, r)] for r in rs])))
        lo = max(0, N - spec.window)
        swa_rows = min(spec.n_sink, lo) + (N - lo)
        step_bytes = 32 * B * spec.Hi * N + 512 * swa_rows * B * len(loc_groups) + 512 * union

        # one thread, two retrieval heads (one of each query class) and one local group
        _cpu_init(d, meta)
        with threadpoolctl.threadpool_limits(1):
            r_sample = [0, 1]
            one = [("decode", 0, [rheads[r]]) for r in r_sample] + [items[-1]]
            n1, spent = 0, 0.0
            while spent < CPU_SAMPLE_SECONDS or n1 < 2:
                spent += sum(_cpu_task(t)[0] for t in one)
                n1 += 1
        _CPU.clear()
        sel1 = sum(len(sets[(0, r)]) for r in r_sample)
        bytes1 = 32 * N * len(r_sample) + 512 * sel1 + 512 * swa_rows
    finally:
        shutil.rmtree(d, ignore_errors=True)
    return {"value": round(step_bytes * passes / wall / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"{spec.name}: the whole step (all {spec.Hq} heads: {spec.Hr} retrieval heads one task each, "
                       f"{len(loc_groups)} local KV groups one task each), {passes} passes in {wall:.1f}s wall "
                       f"on a pool of {workers} worker processes with one oracle thread each "
                       f"(host cpu_count {os.cpu_count()}); caches written by the same pool before the clock "
                       f"({t_setup:.0f}s)"),
            "us_per_step": round(wall / passes * 1e6, 1),
            "single_thread": {"value": round(bytes1 * n1 / spent / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"2 of {spec.Hr} retrieval queries (1 needle-class, 1 diffuse) + the "
                                        f"{spec.G} local heads of one KV group, {n1} passes in {spent:.1f}s"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", type=int, default=0, help="run only this config (3, 4 or 6)")
    ap.add_argument("--calib", action="store_true", help="run the known-size copy used to scale HBM counters")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the Top-P step (no dense comparator, no top-k line): for profiling runs")
    ap.add_argument("--prefill", action="store_true",
                    help="time only the 32K prefill attention (RTPurbo and all-dense) and print its line")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="measure only the streaming-read and copy ceilings and print them")
    ap.add_argument("--chunked-prefill", action="store_true",
                    help="time only the 128K chunked-prefill call (4 heads x 4096 queries) and print its line")
    ap.add_argument("--scan-tile", type=int, default=0, help="tuning sweep: rtp_layer.scan_tile")
    ap.add_argument("--swa-chunk", type=int, default=0, help="tuning sweep: rtp_layer.swa_chunk")
    args = ap.parse_args()
    TUNING.update({k: v for k, v in (("scan_tile", args.scan_tile), ("swa_chunk", args.swa_chunk)) if v})
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    cfgs = [args.only] if args.only else [4, 3, 6]
    gpu_only = args.prefill or args.chunked_prefill or args.read_ceiling
    drawn, cpu = {}, None
    if 4 in cfgs and not args.no_cpu_baseline and not gpu_only:
        # the oracle's leg runs first, before this process touches the GPU,
        # since it starts a pool of worker processes
        spec4 = gen.spec_for(4)
        drawn[4] = gen.make_workload(spec4, gen.workload.default_seed(4))
        t0 = time.time()
        cpu = cpu_baseline(spec4, drawn[4])
        log(f"[bench] cpu baseline {cpu['value']} GB/s on {cpu['cores']} cores, single thread "
            f"{cpu['single_thread']['value']} GB/s ({time.time() - t0:.1f}s incl. cache build)")
    torch.cuda.set_device(0)
    rtp.load()
    if args.prefill:
        with quiet_gc():
            print(json.dumps({"prefill_32k": time_prefill()}), flush=True)
        return
    if args.chunked_prefill:
        with quiet_gc():
            print(json.dumps({"chunked_prefill_128k": time_chunked_prefill()}), flush=True)
        return
    if args.calib:
        calibration_copy()
    with quiet_gc():
        copy_gbps = copy_ceiling_gbps()
        rc = read_ceiling()
    log(f"[bench] device copy ceiling {copy_gbps:.0f} GB/s, streaming read ceiling {rc['GBps']:.0f} GB/s "
        f"({rc['config']})")
    if args.read_ceiling:
        print(json.dumps({"read_ceiling": rc, "copy_ceiling_GBps": round(copy_gbps, 1)}), flush=True)
        return

    summ = {}
    for cfg in cfgs:
        case = Case(cfg, args.replicas, drawn.pop(cfg, None))
        with quiet_gc():
            ms, ms_pa = case.run(args.steps, args.warmup)
        gbps = case.bytes_total / (ms * 1e-3) / 1e9
        # the dense comparator ignores the indexer, so the shared-key layer would repeat the 1M figure
        with quiet_gc():
            ms_dense = (case.run_dense(max(5, args.steps // 10), 3) if cfg != 6 and not args.no_extras
                        else float("nan"))
        dense_bytes = 512 * case.spec.B * case.spec.Hkv * case.spec.N
        pa_bytes = case.bytes_scan + case.bytes_swa
        summ[cfg] = dict(ms=ms, us=ms * 1e3, gbps=gbps, frac=gbps / HBM_PEAK_GBPS, pa_us=ms_pa * 1e3,
                         pa_gbps=pa_bytes / (ms_pa * 1e-3) / 1e9, pa_bytes=pa_bytes,
                         bytes=case.bytes_total, spec=case.spec, counts=case.counts,
                         union=case.gather_rows_union, rsum=case.gather_rows_sum,
                         dense_us=ms_dense * 1e3, dense_gbps=dense_bytes / (ms_dense * 1e-3) / 1e9,
                         pct=case.pct, instr_us=case.instr_us)
        log(f"[bench] cfg{cfg}: {ms * 1e3:.1f} us/step, phase-A kernel {ms_pa * 1e3:.1f} us, {gbps:.0f} GB/s "
            f"algorithmic; |S| {case.counts.ravel().tolist()}; dense comparator {ms_dense * 1e3:.1f} us "
            f"({dense_bytes / (ms_dense * 1e-3) / 1e9:.0f} GB/s), sparse step {ms_dense / ms:.2f}x faster")
        if cfg in (3, 4):
            summ[cfg]["selection"] = selection_stats(case)
            sel = summ[cfg]["selection"]
            log(f"[bench] cfg{cfg}: selection " + "; ".join(
                f"{k}: |S| {v['S_mean']}, sparsity {v['sparsity_mean']}, retained mass {v['retained_mass_mean']}"
                for k, v in sel.items() if isinstance(v, dict)))
        case.sel = None
        torch.cuda.empty_cache()
        if cfg in (3, 4) and not args.no_extras:
            with quiet_gc():
                summ[cfg]["cluster"] = time_cluster(case, max(20, args.steps // 4))
            log(f"[bench] cfg{cfg}: cluster index {summ[cfg]['cluster']}")
        if cfg == 4 and not args.no_extras:
            # the fixed top-k variant of the same kernels on the same caches
            top_p_layer = case.layer
            case.layer = dataclasses.replace(top_p_layer, top_k=TOPK_BENCH)
            with quiet_gc():
                ms_k, ms_pa_k = case.run(max(20, args.steps // 4), args.warmup)
            case.layer = top_p_layer
            summ[cfg].update(topk_us=ms_k * 1e3, topk_pa_us=ms_pa_k * 1e3)
            log(f"[bench] cfg{cfg}: fixed top-k (k = {TOPK_BENCH}) {ms_k * 1e3:.1f} us/step")
        if cfg == 4 and not args.no_extras:
            with quiet_gc():
                summ[cfg]["ring"] = time_local_ring(case, max(20, args.steps // 4), args.warmup)
            log(f"[bench] cfg{cfg}: ring-buffer local caches {summ[cfg]['ring']}")
            torch.cuda.empty_cache()
        if cfg == 4 and not args.no_extras:
            with quiet_gc():
                summ[cfg]["append"] = time_append(case)
            log(f"[bench] cfg{cfg}: cache append {summ[cfg]['append']}")
        del case
        torch.cuda.empty_cache()

    prefill = topics = others = None
    if not args.only and not args.no_extras:
        others = {}
        for cfg, key in ((2, "ctx_32k_b8"), (1, "needle_4k")):
            with quiet_gc():
                others[key] = time_other_decode(cfg, args.steps, args.warmup, args.replicas)
            log(f"[bench] {key}: {others[key]}")
            torch.cuda.empty_cache()
        with quiet_gc():
            others["chunked_prefill_128k"] = time_chunked_prefill()
        log(f"[bench] chunked prefill: {others['chunked_prefill_128k']}")
        torch.cuda.empty_cache()
        with quiet_gc():
            prefill = time_prefill()
        log(f"[bench] prefill attention 32K: {prefill}")
        torch.cuda.empty_cache()
        with quiet_gc():
            topics = time_cluster_topics(max(20, args.steps // 4))
        log(f"[bench] cluster index on topic keys: {topics}")
        torch.cuda.empty_cache()

    main_cfg = cfgs[0]
    s = summ[main_cfg]
    spec = s["spec"]
    out = {
        "metric": METRIC,
        "value": round(s["gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32/f64",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}: one decode step of a {spec.Hq}-q/{spec.Hkv}-kv-head layer, "
                               f"batch {spec.B}, context {spec.N}, {spec.Hr} retrieval q heads "
                               f"(indexer rank 16, p={spec.p}), other heads SWA {spec.window}+{spec.n_sink} sinks",
                   "context": spec.N, "batch": spec.B, "q_heads": spec.Hq, "kv_heads": spec.Hkv,
                   "retrieval_q_heads": spec.Hr, "p": spec.p, "window": spec.window, "sinks": spec.n_sink,
                   "cache_replicas": args.replicas},
        "us_per_step": round(s["us"], 2),
        "hbm_frac": round(s["frac"], 4),
        "algorithmic_bytes_per_step": s["bytes"],
        "selected_tokens": {"per_query": s["counts"].ravel().tolist(), "kv_rows_union": s["union"],
                            "kv_rows_sum": s["rsum"]},
        "roofline": {"bound": "hbm",
                     "kernel": "phase_a_kernel (indexer scores, codes, tile histograms; local-head SWA)",
                     "achieved": round(s["pa_gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(s["pa_gbps"] / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel_us": round(s["pa_us"], 2), "algorithmic_bytes_per_launch": s["pa_bytes"]},
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "read_ceiling": {"GBps": rc["GBps"], "what": "in-tree streaming-read kernels (libreadprobe.so) over 2 GiB, "
                                                     "best of an access-pattern / grid / loads-in-flight sweep",
                         "config": rc["config"], "sweep_GBps": rc["sweep"],
                         "phase_a_frac_of_read_ceiling": round(s["pa_gbps"] / rc["GBps"], 4),
                         "step_frac_of_read_ceiling": round(s["gbps"] / rc["GBps"], 4)},
        "step_us_percentiles": s["pct"],
        "instrumented_us_per_step": s["instr_us"],
    }
    if s["dense_us"] == s["dense_us"]:          # measured (not NaN)
        dense_peak_us = 512 * spec.B * spec.Hkv * spec.N / HBM_PEAK_GBPS / 1e3
        out["dense_comparator"] = {"what": "rtp_dense_attn: every head over every cached position, same caches",
                                   "us_per_step": round(s["dense_us"], 2), "GBps": round(s["dense_gbps"], 1),
                                   "sparse_speedup": round(s["dense_us"] / s["us"], 3),
                                   "dense_at_hbm_peak_us": round(dense_peak_us, 2),
                                   "sparse_speedup_vs_dense_at_peak": round(dense_peak_us / s["us"], 3)}
    if main_cfg == 4:
        out["roofline"]["traffic"] = traffic_per_launch(spec.name)
    if main_cfg == 4 and "topk_us" in s:
        out["fixed_top_k"] = {"k": TOPK_BENCH, "us_per_step": round(s["topk_us"], 2),
                              "phase_a_kernel_us": round(s["topk_pa_us"], 2),
                              "what": "same step with rtp_layer.top_k = k instead of Top-P, same caches"}
    if "selection" in s:
        out["selection"] = s["selection"]
    if "append" in s:
        out["cache_append"] = s["append"]
    if "ring" in s:
        out["local_ring"] = s["ring"]
    if "cluster" in s:
        out["cluster_index"] = s["cluster"]
    if prefill is not None:
        out["prefill_32k"] = prefill
    if others is not None:
        out.update(others)
    if topics is not None:
        out["cluster_index_topic_keys"] = topics
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if 3 in summ and main_cfg != 3:
        s3 = summ[3]
        out["ctx_128k"] = {"workload": s3["spec"].name, "us_per_step": round(s3["us"], 2),
                           "step_us_percentiles": s3["pct"],
                           "instrumented_us_per_step": s3["instr_us"],
                           "GBps": round(s3["gbps"], 1), "hbm_frac": round(s3["frac"], 4),
                           "algorithmic_bytes_per_step": s3["bytes"], "phase_a_kernel_us": round(s3["pa_us"], 2),
                           "phase_a_GBps": round(s3["pa_gbps"], 1),
                           "dense_comparator_us": round(s3["dense_us"], 2) if s3["dense_us"] == s3["dense_us"] else None,
                           "sparse_speedup_vs_dense": (round(s3["dense_us"] / s3["us"], 3)
                                                       if s3["dense_us"] == s3["dense_us"] else None),
                           "selected_tokens": s3["counts"].ravel().tolist()}
        if "cluster" in s3:
            out["ctx_128k"]["cluster_index"] = s3["cluster"]
        if "selection" in s3:
            out["ctx_128k"]["selection"] = s3["selection"]
    if 6 in summ and main_cfg != 6:
        s6 = summ[6]
        out["shared_keys_1m"] = {"workload": s6["spec"].name, "indexer_key_heads": s6["spec"].Hi,
                                 "us_per_step": round(s6["us"], 2), "GBps": round(s6["gbps"], 1),
                                 "hbm_frac": round(s6["frac"], 4), "algorithmic_bytes_per_step": s6["bytes"],
                                 "phase_a_kernel_us": round(s6["pa_us"], 2), "phase_a_GBps": round(s6["pa_gbps"], 1),
                                 "selected_tokens": s6["counts"].ravel().tolist()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
