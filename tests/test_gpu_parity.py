"""GPU parity of every C-ABI call against the CPU oracle (element by element).

Sizes are small enough for the oracle to finish in seconds while spanning
several scan tiles (1024..8192 positions) and a ragged tail.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import gen
import long_context_sparse_retrieval_amd as rtp
import oracle as O
from parity import (check_output, check_set, check_topk_set, dev_bf16, host_bf16, layer_of, say, sdpa_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rtp.load()          # fails loudly if the HIP library is missing
    torch.cuda.init()


def _rand_bf16(rng, shape, scale=1.0):
    return gen.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


# ----------------------------------------------------------------------------- cache writers
@pytest.mark.parametrize("n0,n1,Ncap", [(0, 700, 700), (1000, 1700, 2000), ((1 << 20) - 300, 1 << 20, 1 << 20)])
def test_rope_keys_bit_exact(n0, n1, Ncap):
    say(f"rope_keys n0={n0} n1={n1} Ncap={Ncap}")
    rng = np.random.default_rng(n0 + 1)
    B, Hkv = (2, 3) if Ncap < 10000 else (1, 1)
    k_pre = np.zeros((B, Hkv, Ncap, 128), np.uint16)
    k_pre[:, :, n0:n1] = _rand_bf16(rng, (B, Hkv, n1 - n0, 128), 3.0)
    lay = rtp.Layer(B=B, Hq=Hkv, Hkv=Hkv, N=max(n1, 1), Ncap=Ncap, head_mode=[0] * Hkv)
    d = dev_bf16(k_pre)
    out = torch.zeros_like(d)
    rtp.rope_keys(lay, d, out, n0, n1)
    got = host_bf16(out)[:, :, n0:n1]
    ref = O.rope_keys(k_pre[:, :, n0:n1], 1e6, np.arange(n0, n1))
    ndiff = int(np.sum(got != ref))
    assert ndiff <= max(1, got.size // 10 ** 6), f"{ndiff} of {got.size} bf16 values differ"
    if ndiff:
        assert np.max(np.abs(got.astype(np.int32) - ref.astype(np.int32))) <= 1
    # in place
    rtp.rope_keys(lay, d, d, n0, n1)
    assert np.array_equal(host_bf16(d)[:, :, n0:n1], got)


@pytest.mark.parametrize("shared,ig", [(True, 1), (False, 1), (True, 4), (False, 4)])
def test_index_keys_bit_exact(shared, ig):
    say(f"index_keys shared_w={shared} idx_group={ig}")
    spec = gen.spec_for(2, B=2, N=1500, shared_w=shared, idx_group=ig)
    wl = gen.make_workload(spec, 11)
    lay = layer_of(spec, rtp)
    out = rtp.index_keys(lay, dev_bf16(wl.k_pre), dev_bf16(wl.w_k))
    _, ref = O.build_caches(wl, groups=[])
    assert np.array_equal(host_bf16(out), ref)


@pytest.mark.parametrize("nq", [1, 3])
def test_index_score_bit_exact(nq):
    say(f"index_score nq={nq}")
    rng = np.random.default_rng(5 + nq)
    B, Hq, Hkv, N = 2, 4, 2, 3000
    hm = [1, 0, 1, 1]
    q = _rand_bf16(rng, (B, Hq, nq, 128), 2.0)
    w = _rand_bf16(rng, (3, 128, 16), 1 / np.sqrt(128))
    kidx = _rand_bf16(rng, (B, 3, N, 16))
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, nq=nq, head_mode=hm)
    got = rtp.index_score(lay, dev_bf16(q), dev_bf16(w), dev_bf16(kidx)).cpu().numpy()
    rheads = [0, 2, 3]
    for b in range(B):
        for r, h in enumerate(rheads):
            for i in range(nq):
                m = N - nq + i
                qi = O.index_project(q[b, h, i], w[r])
                ref = O.indexer_logits(qi, kidx[b, r, :m + 1])
                assert np.array_equal(got[b, r, i, :m + 1], ref)
                assert np.all(np.isneginf(got[b, r, i, m + 1:]))


def test_index_score_shared_keys():
    say("index_score idx_group=2")
    rng = np.random.default_rng(17)
    B, Hq, Hkv, N, nq = 2, 4, 2, 2500, 2
    hm = [1, 1, 0, 0]
    q = _rand_bf16(rng, (B, Hq, nq, 128), 2.0)
    w = _rand_bf16(rng, (2, 128, 16), 1 / np.sqrt(128))
    kidx = _rand_bf16(rng, (B, 1, N, 16))          # one indexer-key head for the group's two heads
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, nq=nq, head_mode=hm, idx_group=2)
    got = rtp.index_score(lay, dev_bf16(q), dev_bf16(w), dev_bf16(kidx)).cpu().numpy()
    for b in range(B):
        for r in range(2):
            for i in range(nq):
                m = N - nq + i
                ref = O.indexer_logits(O.index_project(q[b, r, i], w[r]), kidx[b, 0, :m + 1])
                assert np.array_equal(got[b, r, i, :m + 1], ref)


# ----------------------------------------------------------------------------- cache append
@pytest.mark.parametrize("n0,n_new", [(0, 1), (4999, 1), (17, 3), (100, 8), (0, 9), (33, 64), (1000, 777),
                                      (0, 5000)])
@pytest.mark.parametrize("ig", [1, 4])
def test_append_kv_matches_writers_and_oracle(n0, n_new, ig):
    """One launch writes K (post-RoPE), V and the indexer keys of the new rows:
    bit for bit what rtp_rope_keys / rtp_index_keys write, the oracle's indexer
    keys exactly, and nothing outside [n0, n0 + n_new)."""
    say(f"append_kv n0={n0} n_new={n_new} idx_group={ig}")
    rng = np.random.default_rng(n0 * 7 + n_new + ig)
    B, Hq, Hkv, Ncap = 2, 16, 4, 5000
    hm = [1] * 4 + [0] * 4 + [1] * 4 + [0] * 4           # KV groups 0 and 2 retrieval
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=Ncap, head_mode=hm, idx_group=ig)
    k_new = _rand_bf16(rng, (B, Hkv, n_new, 128), 2.0)
    v_new = _rand_bf16(rng, (B, Hkv, n_new, 128))
    w_k = _rand_bf16(rng, (lay.Hi, 128, 16), 128 ** -0.5)
    sentinel = lambda shape: rng.integers(0, 1 << 16, size=shape, dtype=np.uint16) & np.uint16(0x7f7f)
    kc0, vc0, ki0 = sentinel((B, Hkv, Ncap, 128)), sentinel((B, Hkv, Ncap, 128)), sentinel((B, lay.Hi, Ncap, 16))
    kc, vc, ki = dev_bf16(kc0), dev_bf16(vc0), dev_bf16(ki0)
    rtp.append_kv(lay, dev_bf16(k_new), dev_bf16(v_new), dev_bf16(w_k), kc, vc, ki, n0)
    kc, vc, ki = host_bf16(kc), host_bf16(vc), host_bf16(ki)
    sl = slice(n0, n0 + n_new)
    for a, a0 in ((kc, kc0), (vc, vc0), (ki, ki0)):        # rows outside the range untouched
        assert np.array_equal(a[:, :, :n0], a0[:, :, :n0]) and np.array_equal(a[:, :, n0 + n_new:], a0[:, :, n0 + n_new:])
    assert np.array_equal(vc[:, :, sl], v_new)
    # the stand-alone writers on the same rows
    k_pre = np.zeros((B, Hkv, Ncap, 128), np.uint16)
    k_pre[:, :, sl] = k_new
    ref_k = torch.zeros((B, Hkv, Ncap, 128), dtype=torch.bfloat16, device="cuda")
    rtp.rope_keys(lay, dev_bf16(k_pre), ref_k, n0, n0 + n_new)
    ref_i = rtp.index_keys(lay, dev_bf16(k_pre), dev_bf16(w_k), n0=n0, n1=n0 + n_new)
    assert np.array_equal(kc[:, :, sl], host_bf16(ref_k)[:, :, sl]), "keys differ from rtp_rope_keys"
    assert np.array_equal(ki[:, :, sl], host_bf16(ref_i)[:, :, sl]), "indexer keys differ from rtp_index_keys"
    # the oracle: indexer keys exactly; RoPE to the rope_keys test's bar
    rheads = [h for h in range(Hq) if hm[h]]
    for b in range(B):
        for i in range(lay.Hi):
            g = rheads[i * ig] // (Hq // Hkv)
            assert np.array_equal(ki[b, i, sl], O.index_project(k_new[b, g], w_k[i])), f"b{b} i{i}"
    ref = O.rope_keys(k_new, 1e6, np.arange(n0, n0 + n_new))
    got = kc[:, :, sl]
    ndiff = int(np.sum(got != ref))
    assert ndiff <= max(1, got.size // 10 ** 6), f"{ndiff} of {got.size} bf16 values differ"


def test_append_kv_builds_the_caches_a_decode_step_reads():
    """Caches grown by appends (a bulk prefix, then token by token) give the same
    decode step, bit for bit, as caches written by the stand-alone writers."""
    spec = gen.spec_for(2, B=2, N=3000, window=512)
    say(f"append then decode: {spec}")
    wl = gen.make_workload(spec, 91)
    lay = layer_of(spec, rtp)
    k_pre, v, wk = dev_bf16(wl.k_pre), dev_bf16(wl.v), dev_bf16(wl.w_k)
    k_ref = rtp.rope_keys(lay, k_pre)
    ki_ref = rtp.index_keys(lay, k_pre, wk)
    kc = torch.zeros_like(k_ref)
    vc = torch.zeros_like(v)
    ki = torch.zeros_like(ki_ref)
    pieces = [(0, spec.N - 11), (spec.N - 11, 8)] + [(n, 1) for n in range(spec.N - 3, spec.N)]
    for n0, cnt in pieces:
        rtp.append_kv(lay, k_pre[:, :, n0:n0 + cnt].contiguous(), v[:, :, n0:n0 + cnt].contiguous(), wk,
                      kc, vc, ki, n0)
    assert torch.equal(kc, k_ref) and torch.equal(vc, v) and torch.equal(ki, ki_ref)
    q, wq = dev_bf16(wl.q_pre), dev_bf16(wl.w_q)
    a = rtp.decode_step(lay, q, wq, ki, kc, vc, rtp.workspace(lay))
    b = rtp.decode_step(lay, q, wq, ki_ref, k_ref, v, rtp.workspace(lay))
    assert torch.equal(a, b)


# ----------------------------------------------------------------------------- Top-P
def _logit_case(kind, rng, n):
    if kind == "gauss1":
        return (rng.standard_normal(n) * 1.0).astype(np.float32)
    if kind == "gauss4":
        return (rng.standard_normal(n) * 4.0).astype(np.float32)
    if kind == "uniform":
        return np.full(n, 0.731, np.float32)
    if kind == "dominant":
        s = (rng.standard_normal(n) * 0.5).astype(np.float32)
        s[n // 3] = 80.0
        return s
    if kind == "ties":
        return (np.round(rng.standard_normal(n) * 8) / 8).astype(np.float32)
    if kind == "wide":      # spans far more than the 32 logits of the histogram: clamp bin in use
        return (rng.standard_normal(n) * 30.0).astype(np.float32)
    if kind == "huge":      # spans more than the 512 logits the merge ring holds: exact fallback merge
        s = (rng.standard_normal(n) * 300.0).astype(np.float32)
        s[0] = -2000.0
        return s
    if kind == "needles":
        s = (rng.standard_normal(n) * 2.0).astype(np.float32)
        s[rng.choice(n, min(n, 20), replace=False)] += 9.0
        return s
    raise ValueError(kind)


@pytest.mark.parametrize("N", [1, 5, 1000, 4097, 33000])
@pytest.mark.parametrize("kind", ["gauss1", "gauss4", "uniform", "dominant", "ties", "wide", "huge", "needles"])
@pytest.mark.parametrize("p", [0.9, 0.5, 1.0])
def test_topp_select_matches_oracle(N, kind, p):
    say(f"topp_select N={N} kind={kind} p={p}")
    rng = np.random.default_rng(N * 7 + len(kind))
    B, nq = 2, 2 if N >= 2 else 1
    lay = rtp.Layer(B=B, Hq=2, Hkv=1, N=N, nq=nq, head_mode=[1, 1], p=p)
    logits = np.stack([np.stack([np.stack([_logit_case(kind, rng, N) for _ in range(nq)]) for _ in range(2)])
                       for _ in range(B)])
    cap = N
    ws = rtp.workspace(lay)
    idx, cnt = rtp.topp_select(lay, torch.from_numpy(logits).cuda(), cap, ws)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        for r in range(2):
            for i in range(nq):
                m = N - nq + i
                t = O.topp_select(logits[b, r, i, :m + 1], p)
                check_set(idx[b, r, i], int(cnt[b, r, i]), cap, t, logits[b, r, i, :m + 1], p,
                          f"b{b} r{r} i{i}")
                if kind == "uniform" and p < 1:
                    assert cnt[b, r, i] == math.ceil(p * (m + 1))


def test_topp_select_truncates_at_cap():
    rng = np.random.default_rng(3)
    N = 5000
    lay = rtp.Layer(B=1, Hq=1, Hkv=1, N=N, head_mode=[1], p=0.99)
    logits = (rng.standard_normal((1, 1, 1, N)) * 0.5).astype(np.float32)
    t = O.topp_select(logits[0, 0, 0], 0.99)
    ws = rtp.workspace(lay)
    idx, cnt = rtp.topp_select(lay, torch.from_numpy(logits).cuda(), 100, ws)
    assert int(cnt[0, 0, 0]) == len(t["sel"]) > 100
    got = idx.cpu().numpy()[0, 0, 0, :100]
    assert np.all(np.isin(got, t["sel"]))


@pytest.mark.parametrize("N", [100, 1000])
@pytest.mark.parametrize("p", [0.1, 0.3, 0.99])
def test_topp_uniform_decimal_p(N, p):
    """Uniform scores: the count is ceil(p N) with p N rounded once to double
    (here the decimal value: 10, 30, 99, 100, 300, 990) and the set is the
    first positions, both from given scores and through the whole step (W_q = 0
    makes every indexer score exactly 0)."""
    say(f"uniform p={p} N={N}")
    want = math.ceil(p * N)
    assert want == round(p * N)
    lay = rtp.Layer(B=1, Hq=4, Hkv=1, N=N, head_mode=[1, 1, 0, 0], p=p, window=64)
    ws = rtp.workspace(lay)
    logits = np.full((1, 2, 1, N), 0.8125, np.float32)
    idx, cnt = rtp.topp_select(lay, torch.from_numpy(logits).cuda(), N, ws)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for r in range(2):
        t = O.topp_select(logits[0, r, 0], p)
        assert int(cnt[0, r, 0]) == want
        assert check_set(idx[0, r, 0], int(cnt[0, r, 0]), N, t, logits[0, r, 0], p, f"r{r}") == "exact"
        assert list(idx[0, r, 0, :want]) == list(range(want))
    rng = np.random.default_rng(N + int(p * 1000))
    q = _rand_bf16(rng, (1, 4, 1, 128), 1.5)
    wq = np.zeros((2, 128, 16), np.uint16)
    kidx = _rand_bf16(rng, (1, 2, N, 16))
    k = _rand_bf16(rng, (1, 1, N, 128))
    v = _rand_bf16(rng, (1, 1, N, 128))
    idx2 = torch.full((1, 2, 1, N), -1, dtype=torch.int32, device="cuda")
    cnt2 = torch.zeros((1, 2, 1), dtype=torch.int32, device="cuda")
    out = rtp.decode_step(lay, dev_bf16(q), dev_bf16(wq), dev_bf16(kidx), dev_bf16(k), dev_bf16(v), ws,
                          idx=idx2, count=cnt2).cpu().numpy()
    res = O.decode_step(q, wq, kidx, k, v, np.array([1, 1, 0, 0]), N=N, p=p, window=64, n_sink=4, rope_base=1e6)
    for r in range(2):
        assert int(cnt2[0, r, 0]) == want and len(res["sel"][(0, r, 0)]) == want
        assert list(idx2.cpu().numpy()[0, r, 0, :want]) == list(range(want))
    for (b, h, i), ref in res["out"].items():
        check_output(out[b, h, i], ref, f"uniform h{h}")


def test_topp_boundary_in_clamp_bin_takes_all():
    """The boundary bin is the clamp bin 255 (p within N e^-31.75 of 1): every
    position is selected, as in the oracle (one token at 0, a thousand 255
    cells below it, some deeper)."""
    N = 1001
    s = np.full(N, -31.875, dtype=np.float32)
    s[0] = 0.0
    s[600:] = -40.0
    p = 1.0 - 1e-13
    t = O.topp_select(s, p)
    assert t.get("clamp_all") and len(t["sel"]) == N
    lay = rtp.Layer(B=1, Hq=1, Hkv=1, N=N, head_mode=[1], p=p)
    idx, cnt = rtp.topp_select(lay, torch.from_numpy(s.reshape(1, 1, 1, N)).cuda(), N, rtp.workspace(lay))
    assert int(cnt[0, 0, 0]) == N
    assert check_set(idx.cpu().numpy()[0, 0, 0], N, N, t, s, p) == "exact"
    idx, cnt = rtp.topp_select(dataclasses.replace(lay, p=0.9), torch.from_numpy(s.reshape(1, 1, 1, N)).cuda(), N,
                               rtp.workspace(lay))
    assert int(cnt[0, 0, 0]) == 1 and int(idx[0, 0, 0, 0]) == 0


# ----------------------------------------------------------------------------- fixed top-k
@pytest.mark.parametrize("N", [1, 5, 1000, 4097, 33000])
@pytest.mark.parametrize("kind", ["gauss1", "uniform", "dominant", "ties", "wide", "huge", "needles"])
@pytest.mark.parametrize("k", [1, 37, 2048])
def test_topk_select_matches_oracle(N, kind, k):
    """Same kernels with every weight 1: the first k of the (bin, position) order, exactly.

    "wide" puts the boundary into the clamp bin whenever fewer than k scores lie
    within 32 logits of the maximum; "huge" takes the merge path for cells
    spanning more than the ring.
    """
    say(f"topk_select N={N} kind={kind} k={k}")
    rng = np.random.default_rng(N * 11 + len(kind) + k)
    B, nq = 2, 2 if N >= 2 else 1
    lay = rtp.Layer(B=B, Hq=2, Hkv=1, N=N, nq=nq, head_mode=[1, 1], top_k=k)
    logits = np.stack([np.stack([np.stack([_logit_case(kind, rng, N) for _ in range(nq)]) for _ in range(2)])
                       for _ in range(B)])
    ws = rtp.workspace(lay)
    idx, cnt = rtp.topp_select(lay, torch.from_numpy(logits).cuda(), N, ws)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for b in range(B):
        for r in range(2):
            for i in range(nq):
                m = N - nq + i
                t = O.topk_select(logits[b, r, i, :m + 1], k)
                check_topk_set(idx[b, r, i], int(cnt[b, r, i]), N, t, k, f"b{b} r{r} i{i}")


# ----------------------------------------------------------------------------- attention
@pytest.mark.parametrize("counts", [(0, 1, 37, 600), (5000, 70000, 3, 1)])
def test_sparse_attn_matches_oracle(counts):
    say(f"sparse_attn counts={counts}")
    rng = np.random.default_rng(sum(counts))
    N = max(counts) + 50
    B, Hq, Hkv = 2, 4, 2
    hm = [1, 1, 0, 1]
    rheads = [0, 1, 3]
    q = _rand_bf16(rng, (B, Hq, 1, 128), 1.5)
    k = _rand_bf16(rng, (B, Hkv, N, 128))
    v = _rand_bf16(rng, (B, Hkv, N, 128))
    cap = max(counts)
    idx = np.zeros((B, 3, 1, cap), np.int32)
    cnt = np.zeros((B, 3, 1), np.int32)
    for b in range(B):
        for r in range(3):
            c = counts[(b * 3 + r) % len(counts)]
            idx[b, r, 0, :c] = rng.choice(N, c, replace=False)
            cnt[b, r, 0] = c
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, head_mode=hm)
    ws = rtp.workspace(lay)
    out = torch.full((B, Hq, 1, 128), 7.0, device="cuda")
    rtp.sparse_attn(lay, dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(idx).cuda(),
                    torch.from_numpy(cnt).cuda(), ws, out)
    out = out.cpu().numpy()
    G = Hq // Hkv
    for b in range(B):
        for r, h in enumerate(rheads):
            rows = idx[b, r, 0, :cnt[b, r, 0]]
            q_rot = O.rope_rotate(O.bf16_to_f64(q[b, h, 0]), N - 1, 1e6)
            ref = O.attention(q_rot, O.bf16_to_f64(k[b, h // G, rows]), O.bf16_to_f64(v[b, h // G, rows]))
            check_output(out[b, h, 0], ref, f"b{b} h{h} |S|={len(rows)}")
        assert np.all(out[b, 2] == 7.0)        # local head rows untouched


@pytest.mark.parametrize("N,window,n_sink,nq", [(1, 4096, 4, 1), (5, 3, 2, 1), (300, 4096, 4, 1),
                                                (5000, 1, 0, 1), (5000, 1000, 4, 2), (9000, 4096, 4, 3)])
@pytest.mark.parametrize("G,hm", [(4, [0, 0, 1, 0, 1, 1, 1, 1]), (8, [0] * 8 + [1] * 2 + [0] * 6)])
def test_swa_matches_oracle(N, window, n_sink, nq, G, hm):
    say(f"swa N={N} W={window} sinks={n_sink} nq={nq} G={G}")
    rng = np.random.default_rng(N + window + G)
    B, Hq = 2, len(hm)
    Hkv = Hq // G
    q = _rand_bf16(rng, (B, Hq, nq, 128), 1.5)
    k = _rand_bf16(rng, (B, Hkv, N, 128))
    v = _rand_bf16(rng, (B, Hkv, N, 128))
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, nq=nq, head_mode=hm, window=window, n_sink=n_sink)
    ws = rtp.workspace(lay)
    out = torch.full((B, Hq, nq, 128), 7.0, device="cuda")
    rtp.swa_attn(lay, dev_bf16(q), dev_bf16(k), dev_bf16(v), ws, out)
    out = out.cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            for i in range(nq):
                if hm[h]:
                    assert np.all(out[b, h, i] == 7.0)
                    continue
                m = N - nq + i
                rows = O.swa_positions(m, window, n_sink)
                q_rot = O.rope_rotate(O.bf16_to_f64(q[b, h, i]), m, 1e6)
                ref = O.attention(q_rot, O.bf16_to_f64(k[b, h // G, rows]), O.bf16_to_f64(v[b, h // G, rows]))
                check_output(out[b, h, i], ref, f"b{b} h{h} i{i}")


# ----------------------------------------------------------------------------- the fused step
DECODE_CASES = {
    "cfg1": (1, dict(), None),
    "cfg1-indepW": (1, dict(shared_w=False), None),
    "cfg2-small": (2, dict(B=2, N=3000, window=512), None),
    "cfg3-small": (3, dict(B=2, N=20000, window=1024, query_scale="unit"), 0.35),
    "cfg4-small": (4, dict(N=40000, window=2048, query_scale="unit"), 0.3),
    "p1": (2, dict(B=1, N=2500, window=300, p=1.0), None),
    "tiny": (2, dict(B=1, N=3, window=2, n_sink=1, n_needles=0), None),
    # shared indexer keys: one indexer-key head per KV group
    "cfg2-shared-keys": (2, dict(B=2, N=3000, window=512, idx_group=4), None),
    "cfg2-shared-keys-indepW": (2, dict(B=2, N=3000, window=512, idx_group=4, shared_w=False), None),
    "cfg4-shared-keys": (4, dict(N=40000, window=2048, query_scale="unit", idx_group=8), 0.3),
    # fixed top-k instead of Top-P
    "cfg2-topk": (2, dict(B=2, N=3000, window=512, top_k=100), None),
    "cfg4-small-topk": (4, dict(N=40000, window=2048, query_scale="unit", top_k=2048), 0.3),
    "cfg4-shared-keys-topk": (4, dict(N=40000, window=2048, query_scale="unit", idx_group=8, top_k=500), 0.3),
    "topk-all": (2, dict(B=1, N=2500, window=300, top_k=2500), None),
    # scaled queries: tiles whose scores span over 64 logits (clamp cells
    # summed several per thread) and over 256 logits (the tile recomputes
    # its scores from the keys)
    "cfg2-span-200": (2, dict(B=2, N=9000, window=512), 3.0),
    "cfg2-span-3000": (2, dict(B=2, N=9000, window=512), 60.0),
    "topk-1": (1, dict(top_k=1), None),
}


def _run_decode(spec, wl, kc, ki, want_sets=True):
    lay = layer_of(spec, rtp)
    ws = rtp.workspace(lay)
    Hr = spec.Hr
    cap = spec.N
    idx = torch.full((spec.B, Hr, 1, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((spec.B, Hr, 1), dtype=torch.int32, device="cuda")
    args = (dev_bf16(wl.q_pre), dev_bf16(wl.w_q), dev_bf16(ki), dev_bf16(kc), dev_bf16(wl.v))
    out1 = rtp.decode_step(lay, *args, ws, idx=idx, count=cnt)
    out2 = rtp.decode_step(lay, *args, ws)
    torch.cuda.synchronize()
    return out1.cpu().numpy(), out2.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_step_matches_oracle(case):
    cfg, over, scale = DECODE_CASES[case]
    spec = gen.spec_for(cfg, **over)
    say(f"decode_step {case}: {spec}")
    scales = None
    if scale is not None:
        scales = {(b, r): scale * (1.0 + 0.5 * ((b * spec.Hr + r) % 2)) for b in range(spec.B) for r in range(spec.Hr)}
    wl = gen.make_workload(spec, 100 + cfg, scales=scales)
    kc, ki = O.build_caches(wl)
    out, out2, idx, cnt = _run_decode(spec, wl, kc, ki)
    assert np.array_equal(out, out2), "two runs differ (non-deterministic)"
    res = O.decode_step(wl.q_pre, wl.w_q, ki, kc, wl.v, wl.head_mode, N=spec.N, p=spec.p, window=spec.window,
                        n_sink=spec.n_sink, rope_base=spec.rope_theta, want_logits=True,
                        idx_group=spec.idx_group, top_k=spec.top_k)
    verdicts = []
    for (b, h, i), ref in res["out"].items():
        check_output(out[b, h, i], ref, f"{case} b{b} h{h}")
    for (b, r, i), t in res["topp"].items():
        if spec.top_k:
            verdicts.append(check_topk_set(idx[b, r, i], int(cnt[b, r, i]), spec.N, t, spec.top_k,
                                           f"{case} b{b} r{r}"))
        else:
            verdicts.append(check_set(idx[b, r, i], int(cnt[b, r, i]), spec.N, t, res["logits"][(b, r, i)],
                                      spec.p, f"{case} b{b} r{r}"))
    say(f"{case}: sets {verdicts.count('exact')} exact, {verdicts.count('edge')} edge, {verdicts.count('margin')} margin; "
        f"|S| = {sorted(int(c) for c in cnt.ravel())}")


# ----------------------------------------------------------------------------- chunked prefill (nq > 1)
# name -> (config, spec overrides, query scales (None: 3 / 4.5 per topic), queries per selection chunk)
PREFILL_CASES = {
    "pf-3k-64q": (5, dict(N=3000, nq=64, diffuse=(200, 0.5)), None, None),
    "pf-ragged-37q": (5, dict(N=2500, nq=37, diffuse=(150, 0.5)), None, None),
    "pf-p1": (5, dict(N=1200, nq=20, p=1.0, diffuse=(100, 0.5)), None, None),
    "pf-every-position": (5, dict(N=48, nq=48, conc=(0, 4.0), diffuse=(0, 0.5)), None, None),
    "pf-query-chunks": (5, dict(N=5000, nq=80, diffuse=(300, 0.5)), None, "16"),
    "pf-layer-with-local-heads": (2, dict(B=2, N=3000, nq=24, n_needles=16, window=512), {}, None),
    "pf-shared-keys": (5, dict(N=3000, nq=40, diffuse=(200, 0.5), idx_group=4), None, None),
    "pf-topk": (5, dict(N=3000, nq=40, diffuse=(200, 0.5), top_k=300), None, None),
    "pf-topk-chunks": (5, dict(N=5000, nq=80, diffuse=(300, 0.5), top_k=1), None, "16"),
    # prefixes longer than 2^17 positions: the selection keeps its bin counts
    # apart from the masses (shorter prefixes pack them into one word)
    "pf-long-prefix": (5, dict(N=140000, nq=16, diffuse=(2000, 0.5)), None, None),
}


def _prefill_scales(spec, given):
    if given is not None:
        return given
    return {(b, r, t): (3.0 if t == 0 else 4.5) for b in range(spec.B) for r in range(spec.Hr) for t in (0, 1)}


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_prefill_step_matches_oracle(case):
    cfg, over, scales, qch = PREFILL_CASES[case]
    spec = gen.spec_for(cfg, query_scale="unit", **over)
    say(f"prefill {case}: {spec}")
    wl = gen.make_workload(spec, 300 + cfg, scales=_prefill_scales(spec, scales))
    kc, ki = O.build_caches(wl)
    lay = dataclasses.replace(layer_of(spec, rtp), pf_qch=int(qch or 0))
    ws = rtp.workspace(lay)
    cap = spec.N
    idx = torch.full((spec.B, spec.Hr, spec.nq, cap), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((spec.B, spec.Hr, spec.nq), dtype=torch.int32, device="cuda")
    args = (dev_bf16(wl.q_pre), dev_bf16(wl.w_q), dev_bf16(ki), dev_bf16(kc), dev_bf16(wl.v))
    out = rtp.decode_step(lay, *args, ws, idx=idx, count=cnt).cpu().numpy()
    out2 = rtp.decode_step(lay, *args, ws).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(out, out2), "two runs differ (non-deterministic)"
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    res = O.decode_step(wl.q_pre, wl.w_q, ki, kc, wl.v, wl.head_mode, N=spec.N, p=spec.p, window=spec.window,
                        n_sink=spec.n_sink, rope_base=spec.rope_theta, want_logits=True,
                        idx_group=spec.idx_group, top_k=spec.top_k)
    for (b, h, i), ref in res["out"].items():
        check_output(out[b, h, i], ref, f"{case} b{b} h{h} i{i}")
    if spec.top_k:
        verdicts = [check_topk_set(idx[b, r, i], int(cnt[b, r, i]), cap, t, spec.top_k, f"{case} b{b} r{r} i{i}")
                    for (b, r, i), t in res["topp"].items()]
    else:
        verdicts = [check_set(idx[b, r, i], int(cnt[b, r, i]), cap, t, res["logits"][(b, r, i)], spec.p,
                              f"{case} b{b} r{r} i{i}", exact_logits=False) for (b, r, i), t in res["topp"].items()]
    say(f"{case}: sets {verdicts.count('exact')} exact, {verdicts.count('edge')} edge, {verdicts.count('margin')} margin")


# ----------------------------------------------------------------------------- dense comparator
@pytest.mark.parametrize("N,nq,Hq,Hkv", [(1, 1, 4, 1), (5, 1, 4, 2), (300, 3, 8, 2), (5000, 1, 8, 1),
                                          (70000, 1, 16, 2), (9000, 2, 32, 8)])
def test_dense_attn_matches_oracle(N, nq, Hq, Hkv):
    say(f"dense N={N} nq={nq} Hq={Hq} Hkv={Hkv}")
    rng = np.random.default_rng(N + 7 * nq + Hq)
    B = 1
    q = _rand_bf16(rng, (B, Hq, nq, 128), 1.5)
    k = _rand_bf16(rng, (B, Hkv, N, 128), 1.0)
    v = _rand_bf16(rng, (B, Hkv, N, 128), 1.0)
    hm = [0] * Hq
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, nq=nq, head_mode=hm)
    ws = rtp.workspace(lay)
    out = rtp.dense_attn(lay, dev_bf16(q), dev_bf16(k), dev_bf16(v), ws)
    out2 = rtp.dense_attn(lay, dev_bf16(q), dev_bf16(k), dev_bf16(v), ws)
    torch.cuda.synchronize()
    out, out2 = out.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(out, out2), "two runs differ (non-deterministic)"
    dummy_w = np.zeros((0, 128, 16), np.uint16)
    res = O.decode_step(q, dummy_w, None, k, v, np.zeros(Hq, np.int8), N=N, p=0.9, window=N, n_sink=0,
                        rope_base=1e6)
    for (b, h, i), ref in res["out"].items():
        check_output(out[b, h, i], ref, f"dense b{b} h{h} i{i}")


# ----------------------------------------------------------------------------- prefill attention
# (N, nq, Hq, Hkv, head_mode, window, n_sink, all_dense)
FLASH_CASES = {
    "mixed-group": (300, 300, 8, 2, [1, 1, 0, 0, 0, 0, 0, 0], 64, 4, False),
    "ragged-tail": (1000, 77, 8, 1, [1, 0, 1, 0, 0, 0, 0, 1], 200, 4, False),
    "long-window": (5000, 40, 16, 4, [1] * 4 + [0] * 12, 1000, 4, False),
    "no-sinks": (700, 150, 4, 1, [0, 0, 0, 0], 100, 0, False),
    "window-covers-all": (500, 33, 4, 2, [0, 0, 1, 1], 4096, 4, False),
    "dense-all": (2000, 200, 8, 2, [1] * 2 + [0] * 6, 300, 4, True),
    "one-query": (4096, 1, 4, 1, [1, 0, 0, 0], 1024, 4, False),
    "six-heads-per-group": (900, 50, 12, 2, [1] * 6 + [0] * 6, 128, 4, False),
    # the largest head count: q head 255 is an ordinary head (quads pad by count, not by a head value)
    "256-heads": (160, 20, 256, 64, [1] * 8 + [0] * 247 + [1], 48, 4, False),
    "256-heads-dense": (160, 20, 256, 64, [0] * 256, 48, 4, True),
}


@pytest.mark.parametrize("case", list(FLASH_CASES))
def test_prefill_attn_matches_oracle(case):
    N, nq, Hq, Hkv, hm, window, n_sink, all_dense = FLASH_CASES[case]
    say(f"prefill_attn {case}: N={N} nq={nq} Hq={Hq} Hkv={Hkv} window={window} sinks={n_sink} dense={all_dense}")
    rng = np.random.default_rng(N + nq + Hq)
    B = 2
    q = _rand_bf16(rng, (B, Hq, nq, 128), 1.5)
    k = _rand_bf16(rng, (B, Hkv, N, 128))
    v = _rand_bf16(rng, (B, Hkv, N, 128))
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, nq=nq, head_mode=hm, window=window, n_sink=n_sink)
    out = rtp.prefill_attn(lay, dev_bf16(q), dev_bf16(k), dev_bf16(v), all_dense=all_dense)
    out2 = rtp.prefill_attn(lay, dev_bf16(q), dev_bf16(k), dev_bf16(v), all_dense=all_dense)
    torch.cuda.synchronize()
    out, out2 = out.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(out, out2), "two runs differ (non-deterministic)"
    G = Hq // Hkv
    queries = range(nq) if nq <= 80 else sorted(set(range(0, nq, 7)) | {nq - 1, nq - 2, 1})
    for b in range(B):
        for h in range(Hq):
            for i in queries:
                m = N - nq + i
                rows = np.arange(m + 1) if (all_dense or hm[h]) else O.swa_positions(m, window, n_sink)
                q_rot = O.rope_rotate(O.bf16_to_f64(q[b, h, i]), m, 1e6)
                ref = O.attention(q_rot, O.bf16_to_f64(k[b, h // G, rows]), O.bf16_to_f64(v[b, h // G, rows]))
                check_output(out[b, h, i], ref, f"{case} b{b} h{h} i{i}")


def test_prefill_attn_rising_scores():
    """Scores that grow along the key axis, so the running maximum of every
    query moves again and again (each time a score outgrows the reference by
    the kernel's rescale headroom) and the weight piles up on the newest
    keys.  The query lives in the slowest-rotating RoPE pairs, so its rotation
    barely changes across positions and the ramp holds for every query."""
    B, Hq, Hkv, N, nq, window, n_sink = 1, 8, 2, 2048, 40, 256, 4
    hm = [1] * 4 + [0] * 4
    rng = np.random.default_rng(2024)
    say(f"prefill_attn rising scores: N={N} nq={nq}")
    u = np.zeros(128)
    u[112:] = rng.standard_normal(16)
    u /= np.linalg.norm(u)
    q = O.f64_to_bf16(np.broadcast_to(4.0 * u, (B, Hq, nq, 128)) + 0.05 * rng.standard_normal((B, Hq, nq, 128)))
    # score of key n for |q| = 4: about 0.03 n (natural units), 61 at the last key
    ramp = 0.03 * np.arange(N) * np.sqrt(128.0) / 4.0
    k = O.f64_to_bf16(ramp[None, None, :, None] * u + 0.5 * rng.standard_normal((B, Hkv, N, 128)))
    v = _rand_bf16(rng, (B, Hkv, N, 128))
    lay = rtp.Layer(B=B, Hq=Hq, Hkv=Hkv, N=N, nq=nq, head_mode=hm, window=window, n_sink=n_sink)
    out = rtp.prefill_attn(lay, dev_bf16(q), dev_bf16(k), dev_bf16(v)).cpu().numpy()
    G = Hq // Hkv
    for h in range(Hq):
        for i in range(nq):
            m = N - nq + i
            rows = np.arange(m + 1) if hm[h] else O.swa_positions(m, window, n_sink)
            q_rot = O.rope_rotate(O.bf16_to_f64(q[0, h, i]), m, 1e6)
            ref = O.attention(q_rot, O.bf16_to_f64(k[0, h // G, rows]), O.bf16_to_f64(v[0, h // G, rows]))
            check_output(out[0, h, i], ref, f"rising b0 h{h} i{i}")


# ----------------------------------------------------------------------------- one workspace, many calls
def test_workspace_serves_every_call_in_sequence():
    """Every call leaves the workspace ready for the next call on a layer of the
    same shape: the dense comparator's and the stand-alone calls' scratch must
    not disturb the step's persistent state (merge ring, cell ranges,
    counters), and N, p and top_k may change between calls."""
    spec = gen.spec_for(2, B=2, N=6000, window=512)
    say(f"workspace sequence: {spec}")
    wl = gen.make_workload(spec, 77)
    lay = layer_of(spec, rtp)
    k_pre = dev_bf16(wl.k_pre)
    k = rtp.rope_keys(lay, k_pre)
    k_idx = rtp.index_keys(lay, k_pre, dev_bf16(wl.w_k))
    v = dev_bf16(wl.v)
    q, wq = dev_bf16(wl.q_pre), dev_bf16(wl.w_q)
    lay_k = dataclasses.replace(lay, top_k=300)
    lay_short = dataclasses.replace(lay, N=5000, Ncap=spec.N, p=0.8)      # same caches, shorter context

    def step(layer, ws):
        return rtp.decode_step(layer, q, wq, k_idx, k, v, ws).cpu().numpy()

    ref = {name: step(l, rtp.workspace(l)) for name, l in (("p", lay), ("k", lay_k), ("short", lay_short))}
    ref_dense = rtp.dense_attn(lay, q, k, v, rtp.workspace(lay)).cpu().numpy()
    ws = rtp.workspace(lay)
    seq = ["p", "dense", "p", "swa", "k", "dense", "short", "logits", "p", "dense", "k", "short", "p"]
    for j, x in enumerate(seq):
        if x == "dense":
            assert np.array_equal(rtp.dense_attn(lay, q, k, v, ws).cpu().numpy(), ref_dense), "dense after others"
        elif x == "swa":
            rtp.swa_attn(lay, q, k, v, ws)
        elif x == "logits":
            lg = rtp.index_score(lay, q, wq, k_idx)
            rtp.topp_select(lay, lg, spec.N, ws)
        else:
            got = step({"p": lay, "k": lay_k, "short": lay_short}[x], ws)
            assert np.array_equal(got, ref[x]), f"decode step '{x}' differs after {seq[:j]}"
    torch.cuda.synchronize()
