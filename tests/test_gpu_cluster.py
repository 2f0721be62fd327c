"""GPU parity of the cluster index (build and decode step) against the oracle.

The build must reproduce the oracle's k-means exactly (centres, counts, the
member lists); the decode step's member sets must equal the oracle's (except
when the oracle reports a cluster decision within rounding of p Z, then the
set must still be a union of whole clusters reaching p) and its outputs must
meet the attention bar.
"""
import numpy as np
import pytest
import torch

import gen
import long_context_sparse_retrieval_amd as rtp
import oracle as O
from parity import MARGIN, check_output, dev_bf16, host_bf16, layer_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rtp.load()
    torch.cuda.init()


def _csr(assign, K):
    order = np.argsort(assign, kind="stable")
    counts = np.bincount(assign, minlength=K)
    return counts, np.concatenate(([0], np.cumsum(counts))), order


@pytest.mark.parametrize("N,K,iters,Hi", [(300, 1, 2, 1), (300, 7, 0, 2), (5000, 128, 4, 2), (20000, 256, 3, 1),
                                          (4099, 128, 1, 3), (200, 200, 1, 1)])
def test_cluster_build_matches_oracle(N, K, iters, Hi):
    say(f"cluster build N={N} K={K} iters={iters} Hi={Hi}")
    rng = np.random.default_rng(N + K + iters)
    B = 2
    lay = rtp.Layer(B=B, Hq=Hi, Hkv=1, N=N, head_mode=[1] * Hi)
    k_idx = gen.f32_to_bf16_bits((rng.standard_normal((B, Hi, N, 16)) * 0.7).astype(np.float32))
    ws = rtp.cluster_workspace(lay, K)
    idx = rtp.cluster_build(lay, dev_bf16(k_idx), K, iters, ws)
    idx2 = rtp.cluster_build(lay, dev_bf16(k_idx), K, iters, ws)       # the workspace is reusable
    cent, counts = host_bf16(idx["centroids"]), idx["counts"].cpu().numpy()
    offs, mem = idx["offsets"].cpu().numpy(), idx["members"].cpu().numpy()
    assert torch.equal(idx["members"], idx2["members"]) and torch.equal(idx["centroids"], idx2["centroids"])
    for b in range(B):
        for i in range(Hi):
            ref = O.kmeans_index(k_idx[b, i], K, iters)
            assert np.array_equal(cent[b, i], ref["centroids"]), f"b{b} i{i}: centres differ"
            c, o, order = _csr(ref["assign"], K)
            assert np.array_equal(counts[b, i], c), f"b{b} i{i}: counts differ"
            assert np.array_equal(offs[b, i], o), f"b{b} i{i}: offsets differ"
            assert np.array_equal(mem[b, i], order), f"b{b} i{i}: members differ"


STEP_CASES = {
    "cfg2-K64": (2, dict(B=2, N=3000, window=512), 64, 4),
    "cfg2-K128-shared-keys": (2, dict(B=2, N=5000, window=512, idx_group=4), 128, 3),
    "cfg4-small-K128": (4, dict(N=40000, window=2048, query_scale="unit"), 128, 4),
    "one-cluster-per-key": (2, dict(B=1, N=200, window=64, n_needles=4), 200, 1),
    "p1": (2, dict(B=1, N=2500, window=300, p=1.0), 32, 2),
}


@pytest.mark.parametrize("case", list(STEP_CASES))
def test_cluster_step_matches_oracle(case):
    cfg, over, K, iters = STEP_CASES[case]
    spec = gen.spec_for(cfg, **over)
    say(f"cluster step {case}: {spec} K={K}")
    wl = gen.make_workload(spec, 500 + cfg)
    kc, ki = O.build_caches(wl)
    lay = layer_of(spec, rtp)
    ws = rtp.cluster_workspace(lay, K)
    index = rtp.cluster_build(lay, dev_bf16(ki), K, iters, ws)
    cap = spec.N
    idx = torch.full((spec.B, spec.Hr, 1, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((spec.B, spec.Hr, 1), dtype=torch.int32, device="cuda")
    args = (dev_bf16(wl.q_pre), dev_bf16(wl.w_q), index, dev_bf16(kc), dev_bf16(wl.v), ws)
    out = rtp.cluster_step(lay, *args, idx=idx, count=cnt).cpu().numpy()
    out2 = rtp.cluster_step(lay, *args).cpu().numpy()
    assert np.array_equal(out, out2), "two runs differ"
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    rheads = spec.retrieval_heads()
    G = spec.G
    m = spec.N - 1
    tolerated = 0
    for b in range(spec.B):
        refs = {}
        for r, h in enumerate(rheads):
            i = r // spec.idx_group
            if i not in refs:
                refs[i] = O.kmeans_index(ki[b, i, :spec.N], K, iters)
            res = O.cluster_decode_head(wl.q_pre[b, h, 0], wl.w_q[r], refs[i], kc[b, h // G], wl.v[b, h // G], m,
                                        spec.p, spec.rope_theta)
            got = np.sort(idx[b, r, 0, :cnt[b, r, 0]])
            if not np.array_equal(got, res["rows"]):
                t = res["select"]
                assert t["margin"] < MARGIN, f"b{b} r{r}: member sets differ (margin {t['margin']:.2e})"
                hit = np.unique(refs[i]["assign"][got])
                assert np.array_equal(np.sort(O.cluster_members(refs[i]["assign"], hit)), got), "not whole clusters"
                w = t["weights"]
                assert w[hit].sum() >= (spec.p - 1e-4) * w.sum(), f"b{b} r{r}: cluster mass below p"
                tolerated += 1
                q_rot = O.rope_rotate(O.bf16_to_f64(wl.q_pre[b, h, 0]), m, spec.rope_theta)
                ref = O.attention(q_rot, O.bf16_to_f64(kc[b, h // G, got]), O.bf16_to_f64(wl.v[b, h // G, got]))
            else:
                ref = res["out"]
            check_output(out[b, h, 0], ref, f"{case} b{b} h{h}")
        for h in range(spec.Hq):
            if spec.head_mode()[h]:
                continue
            rows = O.swa_positions(m, spec.window, spec.n_sink)
            q_rot = O.rope_rotate(O.bf16_to_f64(wl.q_pre[b, h, 0]), m, spec.rope_theta)
            ref = O.attention(q_rot, O.bf16_to_f64(kc[b, h // G, rows]), O.bf16_to_f64(wl.v[b, h // G, rows]))
            check_output(out[b, h, 0], ref, f"{case} local b{b} h{h}")
    say(f"{case}: |S| = {sorted(int(c) for c in cnt.ravel())}, {tolerated} tolerated")


def test_cluster_step_on_topic_keys_is_selective_and_matches_oracle():
    """Keys drawn around 16 topic centres, each query along one centre: the index
    recovers the topics, the hit set is the query's topic, and the step matches
    the oracle."""
    rng = np.random.default_rng(77)
    B, Hq, Hkv, N, T, K = 1, 8, 2, 8192, 16, 64          # about four clusters per topic
    hm = [1] * 4 + [0] * 4
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, head_mode=hm, window=512)
    mu = rng.standard_normal((T, 128))
    topic = rng.integers(0, T, N)
    k_pre = rng.standard_normal((B, Hkv, N, 128))
    k_pre[0, 0] = mu[topic] + 0.3 * k_pre[0, 0]
    k_pre = gen.f32_to_bf16_bits(k_pre.astype(np.float32))
    v = gen.f32_to_bf16_bits(rng.standard_normal((B, Hkv, N, 128)).astype(np.float32))
    w = gen.f32_to_bf16_bits((rng.standard_normal((4, 128, 16)) / np.sqrt(128)).astype(np.float32))
    tq = rng.integers(0, T, 4)
    q = rng.standard_normal((B, Hq, 1, 128))
    for r in range(4):
        q[0, r, 0] = mu[tq[r]]
    q = gen.f32_to_bf16_bits(q.astype(np.float32))
    kc, vc = torch.empty((B, Hkv, N, 128), dtype=torch.bfloat16, device="cuda"), torch.empty(
        (B, Hkv, N, 128), dtype=torch.bfloat16, device="cuda")
    ki = torch.empty((B, 4, N, 16), dtype=torch.bfloat16, device="cuda")
    rtp.append_kv(lay, dev_bf16(k_pre), dev_bf16(v), dev_bf16(w), kc, vc, ki, 0)
    ws = rtp.cluster_workspace(lay, K)
    index = rtp.cluster_build(lay, ki, K, 8, ws)
    idx = torch.full((B, 4, 1, N), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((B, 4, 1), dtype=torch.int32, device="cuda")
    out = rtp.cluster_step(lay, dev_bf16(q), dev_bf16(w), index, kc, vc, ws, idx=idx, count=cnt).cpu().numpy()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    kc_h, ki_h = host_bf16(kc), host_bf16(ki)
    recalls = []
    for r in range(4):
        ref_idx = O.kmeans_index(ki_h[0, r, :N], K, 8)
        res = O.cluster_decode_head(q[0, r, 0], w[r], ref_idx, kc_h[0, 0], v[0, 0], N - 1, 0.9, 1e6)
        got = np.sort(idx[0, r, 0, :cnt[0, r, 0]])
        assert np.array_equal(got, res["rows"]), f"r{r}: member sets differ"
        check_output(out[0, r, 0], res["out"], f"topic r{r}")
        # k-means may split a topic or merge two (a local optimum of Lloyd's
        # rounds from positional seeds), so coverage is checked loosely
        in_topic = np.sum(topic[got] == tq[r]) / np.sum(topic == tq[r])
        assert in_topic >= 0.5, f"r{r}: only {in_topic:.2f} of the query's topic in the hit set"
        assert len(got) <= N // 4, f"r{r}: hit set not selective ({len(got)} of {N})"
        recalls.append(round(float(in_topic), 3))
    say(f"topic keys: |S| = {cnt.ravel().tolist()}, topic coverage {recalls}")
