"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The GPU runs one whole decode step of the 32K (batch 8), 128K (batch 4) and 1M
layers (the latter also with one indexer-key head per KV group): every
head, caches written by the library's own cache writers, the same tile and
workgroup plan as the benchmark.  The oracle, which cannot redo the whole step
in seconds, builds its own caches for a sample and recomputes, one by one:
one concentrated and one diffuse retrieval query of sequence 0 (whole
context), and the local heads of one KV group.  Every other query is checked
through properties that hold at any size (positions unique, in range, count
within [1, m + 1]).
"""
import dataclasses

import numpy as np
import pytest
import torch

import gen
import long_context_sparse_retrieval_amd as rtp
import oracle as O
from parity import check_output, check_set, dev_bf16, layer_of, say

pytestmark = pytest.mark.gpu

# config -> sampled retrieval heads r of sequence 0 (r = 0 concentrated, r = 1 diffuse)
FULL = {"32k-b8": (2, [0, 1]), "128k-b4": (3, [0, 1]), "1m-b1": (4, [0, 1]), "1m-b1-shared-keys": (6, [0, 1])}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rtp.load()
    torch.cuda.init()


@pytest.mark.parametrize("case", list(FULL))
def test_decode_step_full_size_sampled(case):
    cfg, r_sample = FULL[case]
    spec = gen.spec_for(cfg)
    say(f"full-size decode {case}: {spec.name} N={spec.N} B={spec.B} Hr={spec.Hr}")
    wl = gen.make_workload(spec, gen.workload.default_seed(cfg))
    lay = layer_of(spec, rtp)

    # GPU: the benchmark's configuration
    k_pre = dev_bf16(wl.k_pre)
    k = rtp.rope_keys(lay, k_pre)
    k_idx = rtp.index_keys(lay, k_pre, dev_bf16(wl.w_k))
    del k_pre
    v = dev_bf16(wl.v)
    ws = rtp.workspace(lay)
    cap = spec.N
    idx = torch.full((spec.B, spec.Hr, 1, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((spec.B, spec.Hr, 1), dtype=torch.int32, device="cuda")
    out = rtp.decode_step(lay, dev_bf16(wl.q_pre), dev_bf16(wl.w_q), k_idx, k, v, ws, idx=idx, count=cnt)
    torch.cuda.synchronize()
    out, idx, cnt = out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    del k, v, k_idx
    torch.cuda.empty_cache()
    say(f"{case}: GPU step done; |S| = {cnt.ravel().tolist()}")

    # properties of every query's set
    m = spec.N - 1
    for b in range(spec.B):
        for r in range(spec.Hr):
            c = int(cnt[b, r, 0])
            assert 1 <= c <= m + 1, f"b{b} r{r}: count {c}"
            got = idx[b, r, 0, :c]
            assert np.all((got >= 0) & (got <= m)), f"b{b} r{r}: position out of range"
            assert len(np.unique(got)) == c, f"b{b} r{r}: duplicate positions"
    assert np.all(np.isfinite(out)), "non-finite output"

    # the oracle on the sample, from its own caches
    rheads = spec.retrieval_heads()
    g_loc = [g for g in range(spec.Hkv) if g not in spec.ret_groups][0]
    loc_heads = list(range(g_loc * spec.G, (g_loc + 1) * spec.G))
    groups = sorted({rheads[r] // spec.G for r in r_sample} | {g_loc})
    kc, ki = O.build_caches(wl, groups=groups, heads=r_sample)
    say(f"{case}: oracle caches built for groups {groups}, retrieval heads {r_sample}")
    res = O.decode_step(wl.q_pre, wl.w_q, ki, kc, wl.v, wl.head_mode, N=spec.N, p=spec.p, window=spec.window,
                        n_sink=spec.n_sink, rope_base=spec.rope_theta, heads=[rheads[r] for r in r_sample] + loc_heads,
                        batches=[0], want_logits=True,
                        idx_group=spec.idx_group)
    verdicts = []
    for (b, h, i), ref in res["out"].items():
        check_output(out[b, h, i], ref, f"{case} b{b} h{h}")
    for (b, r, i), t in res["topp"].items():
        verdicts.append(check_set(idx[b, r, i], int(cnt[b, r, i]), cap, t, res["logits"][(b, r, i)], spec.p,
                                  f"{case} b{b} r{r}"))
    say(f"{case}: sampled sets {verdicts.count('exact')} exact, {verdicts.count('edge')} edge, {verdicts.count('margin')} margin; "
        f"{len(res['out'])} head outputs checked")


def test_prefill_full_size_sampled():
    """4096 causal queries x 4 heads against a 128K cache (the chunked-prefill workload)."""
    spec = gen.spec_for(5)
    say(f"full-size prefill: {spec.name} N={spec.N} nq={spec.nq} Hr={spec.Hr}")
    wl = gen.make_workload(spec, gen.workload.default_seed(5))
    lay = layer_of(spec, rtp)
    k_pre = dev_bf16(wl.k_pre)
    k = rtp.rope_keys(lay, k_pre)
    k_idx = rtp.index_keys(lay, k_pre, dev_bf16(wl.w_k))
    del k_pre
    v = dev_bf16(wl.v)
    ws = rtp.workspace(lay)
    cap = spec.N                  # every set fits (the device list is 8 GiB; only sampled rows come back)
    idx = torch.full((spec.B, spec.Hr, spec.nq, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((spec.B, spec.Hr, spec.nq), dtype=torch.int32, device="cuda")
    q, wq = dev_bf16(wl.q_pre), dev_bf16(wl.w_q)
    rtp.decode_step(lay, q, wq, k_idx, k, v, ws, idx=idx, count=cnt)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    out = rtp.decode_step(lay, q, wq, k_idx, k, v, ws)
    e1.record()
    torch.cuda.synchronize()
    out, cnt_h = out.cpu().numpy(), cnt.cpu().numpy()
    c = cnt_h.ravel()
    say(f"full-size prefill: step {e0.elapsed_time(e1):.2f} ms; |S| min {c.min()} median {int(np.median(c))} "
        f"max {c.max()}")
    rows = {}

    def gpu_set(r, i):
        if (r, i) not in rows:
            rows[(r, i)] = idx[0, r, i, :int(cnt_h[0, r, i])].cpu().numpy()
        return rows[(r, i)]

    for r in range(spec.Hr):
        for i in range(spec.nq):
            m = spec.N - spec.nq + i
            ci = int(cnt_h[0, r, i])
            assert 1 <= ci <= m + 1, f"r{r} i{i}: count {ci}"
        for i in range(r, spec.nq, 97):                   # positions of a spread of queries
            m = spec.N - spec.nq + i
            got = gpu_set(r, i)
            assert np.all((got >= 0) & (got <= m)), f"r{r} i{i}: position out of range"
            assert len(np.unique(got)) == len(got), f"r{r} i{i}: duplicate positions"
    assert np.all(np.isfinite(out)), "non-finite output"
    del k, v, k_idx

    queries = [0, 1, spec.nq // 2, spec.nq // 2 + 1, spec.nq - 2, spec.nq - 1]
    kc, ki = O.build_caches(wl)
    res = O.decode_step(wl.q_pre, wl.w_q, ki, kc, wl.v, wl.head_mode, N=spec.N, p=spec.p, window=spec.window,
                        n_sink=spec.n_sink, rope_base=spec.rope_theta, queries=queries, want_logits=True,
                        idx_group=spec.idx_group)
    for (b, h, i), ref in res["out"].items():
        check_output(out[b, h, i], ref, f"prefill b{b} h{h} i{i}")
    verdicts = [check_set(gpu_set(r, i), int(cnt_h[b, r, i]), cap, t, res["logits"][(b, r, i)], spec.p,
                          f"prefill b{b} r{r} i{i}", exact_logits=False) for (b, r, i), t in res["topp"].items()]
    say(f"full-size prefill: sampled sets {verdicts.count('exact')} exact, {verdicts.count('edge')} edge, {verdicts.count('margin')} margin")


def test_prefill_attn_full_size_sampled():
    """The benchmark's 32K prefill (32 q / 8 kv heads, group 0 retrieval, 32768
    causal queries): sampled queries of a retrieval and a local head, both
    modes, against the oracle."""
    rng = np.random.default_rng(2032)
    B, Hq, Hkv, N, W, S = 1, 32, 8, 32768, 4096, 4
    hm = [1] * 4 + [0] * 28
    q = gen.f32_to_bf16_bits(rng.standard_normal((B, Hq, N, 128), dtype=np.float32))
    k = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, 128), dtype=np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, 128), dtype=np.float32))
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, nq=N, head_mode=hm, window=W, n_sink=S)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    for dense in (False, True):
        out = rtp.prefill_attn(lay, qd, kd, vd, all_dense=dense).cpu().numpy()
        assert np.all(np.isfinite(out))
        for h in (1, 5, 30):                  # a retrieval head, local heads of groups 1 and 7
            for i in (0, 1, 63, 4095, 4096, 4100, 17000, N - 1):
                rows = np.arange(i + 1) if (dense or hm[h]) else O.swa_positions(i, W, S)
                q_rot = O.rope_rotate(O.bf16_to_f64(q[0, h, i]), i, 1e6)
                ref = O.attention(q_rot, O.bf16_to_f64(k[0, h // 4, rows]), O.bf16_to_f64(v[0, h // 4, rows]))
                check_output(out[0, h, i], ref, f"prefill dense={dense} h{h} i{i}")
        say(f"full-size prefill attention (dense={dense}): sampled queries match")


def test_ring_layout_full_size():
    """The 1M layer over ring-buffer local caches (local_ring), written by one
    bulk rtp_append_kv of the whole context: the step (outputs, sets, counts)
    equals the full layout's step bit for bit, in the benchmark's launch plan;
    the full layout's step is itself checked against the oracle above."""
    cfg = 4
    spec = gen.spec_for(cfg)
    say(f"full-size ring layout: {spec.name} N={spec.N}")
    wl = gen.make_workload(spec, gen.workload.default_seed(cfg))
    full = layer_of(spec, rtp)
    ring = dataclasses.replace(full, local_ring=1)
    k_pre = dev_bf16(wl.k_pre)
    w_k = dev_bf16(wl.w_k)
    k = rtp.rope_keys(full, k_pre)
    k_idx = rtp.index_keys(full, k_pre, w_k)
    v = dev_bf16(wl.v)
    kr = torch.empty(rtp.kv_shape(ring), dtype=torch.bfloat16, device="cuda")
    vr = torch.empty_like(kr)
    ki = torch.empty_like(k_idx)
    rtp.append_kv(ring, k_pre, v, w_k, kr, vr, ki, 0)
    del k_pre
    assert torch.equal(ki, k_idx)
    del ki
    n_ring = spec.Hkv - len(spec.ret_groups)                 # all-local KV groups
    assert rtp.kv_rows(ring) == len(spec.ret_groups) * spec.N + n_ring * (spec.n_sink + spec.window)
    q, w_q = dev_bf16(wl.q_pre), dev_bf16(wl.w_q)
    res = []
    for lay, kc, vc in ((full, k, v), (ring, kr, vr)):
        idx = torch.full((spec.B, spec.Hr, 1, spec.N), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros((spec.B, spec.Hr, 1), dtype=torch.int32, device="cuda")
        out = rtp.decode_step(lay, q, w_q, k_idx, kc, vc, rtp.workspace(lay), idx=idx, count=cnt)
        res.append((out, idx, cnt))
    for a, b in zip(*res):
        assert torch.equal(a, b)
    say(f"ring layout at 1M: K/V rows per sequence {rtp.kv_rows(ring)} vs {rtp.kv_rows(full)}")
