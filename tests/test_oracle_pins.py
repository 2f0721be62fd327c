"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against a library routine, a closed form, exact
rational arithmetic, a brute force on tiny inputs, an invariant of the method
or a hand-worked example, so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- number formats
def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        # exact ties between two bf16 neighbours
                        (1.0 + np.arange(1, 256) * 2.0 ** -8) * 2.0 ** rng.integers(-20, 20, 255)])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.f64_to_bf16(x32.astype(np.float64)), ref)


def test_bf16_rounding_is_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-40 is above the midpoint between 1 and 1 + 2^-7: it must round up,
    # whereas a detour through float32 would first land on the midpoint and then tie to 1.
    assert O.f64_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert O.f64_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 0x3F80          # tie -> even
    assert O.f64_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 0x3F82      # tie -> even (up)
    assert O.f64_to_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == 0xBF82
    rng = np.random.default_rng(1)
    x = rng.standard_normal(300) * 7.3
    for v, bits in zip(x, O.f64_to_bf16(x)):
        assert bits == O.fraction_to_bf16(Fraction(float(v)))


def test_fraction_to_f32_matches_numpy_cast():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000)
    x = np.concatenate([x, [2.0 ** -149, 2.0 ** -130 * 1.5, 1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24]])
    for v in x:
        assert O.fraction_to_f32(Fraction(float(v))) == np.float32(v)


# ----------------------------------------------------------------------------- RoPE, eq. (1)-(2)
def test_rope_theta_closed_form():
    th = O.rope_theta(128, 1e6)
    assert th[0] == 1.0
    np.testing.assert_allclose(th[1:] / th[:-1], 1e6 ** (-2 / 128), rtol=1e-13)
    assert np.all(np.diff(th) < 0)           # decreases with the channel index


def test_rope_rotation_convention():
    D = 8
    e0 = np.zeros(D); e0[0] = 1
    e1 = np.zeros(D); e1[1] = 1
    r0 = O.rope_rotate(e0, 1, 1e6)
    r1 = O.rope_rotate(e1, 1, 1e6)
    np.testing.assert_allclose(r0[:2], [math.cos(1), math.sin(1)], atol=1e-15)
    np.testing.assert_allclose(r1[:2], [-math.sin(1), math.cos(1)], atol=1e-15)
    assert np.all(r0[2:] == 0) and np.all(r1[2:] == 0)
    # second pair rotates with theta_2 = base^(-2/D)
    e2 = np.zeros(D); e2[2] = 1
    t2 = 1e6 ** (-2 / D)
    np.testing.assert_allclose(O.rope_rotate(e2, 5, 1e6)[2:4], [math.cos(5 * t2), math.sin(5 * t2)], atol=1e-15)


def test_rope_identity_norm_inverse():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128))
    m = rng.integers(0, 1 << 20, 50)
    np.testing.assert_array_equal(O.rope_rotate(x, np.zeros(50), 1e6), x)
    y = O.rope_rotate(x, m, 1e6)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(O.rope_rotate(y, -m, 1e6), x, atol=1e-9)


def test_rope_score_depends_only_on_offset():
    """eq. (2): q_m . k_n is a function of m - n only."""
    rng = np.random.default_rng(4)
    for _ in range(20):
        q, k = rng.standard_normal(128), rng.standard_normal(128)
        m, n = (int(v) for v in rng.integers(0, 1 << 18, 2))
        t = int(rng.integers(1, 1 << 20))
        s0 = O.rope_rotate(q, m, 1e6) @ O.rope_rotate(k, n, 1e6)
        s1 = O.rope_rotate(q, m + t, 1e6) @ O.rope_rotate(k, n + t, 1e6)
        assert abs(s1 - s0) <= 1e-9 * max(1.0, abs(s0)) * 10


def test_rope_pair_score_closed_form():
    th = O.rope_theta(128, 1e6)
    for i in (0, 5, 63):
        q = np.zeros(128); q[2 * i] = 1
        for m, n in ((10, 3), (1000, 999), (70000, 5)):
            s = O.rope_rotate(q, m, 1e6) @ O.rope_rotate(q, n, 1e6)
            assert abs(s - math.cos((m - n) * th[i])) < 1e-9


# ----------------------------------------------------------------------------- indexer, eq. (4)
def _fraction_index(x_bits, w_bits):
    x = [Fraction(float(v)) for v in O.bf16_to_f64(x_bits)]
    w = O.bf16_to_f64(w_bits)
    return [O.fraction_to_bf16(sum((x[c] * Fraction(float(w[c, j])) for c in range(len(x))), Fraction(0)))
            for j in range(w.shape[1])]


def test_index_project_equals_exact_rational():
    rng = np.random.default_rng(5)
    for trial in range(6):
        x = _rand_bf16(rng, (128,), scale=10.0 ** trial)
        w = _rand_bf16(rng, (128, 16), scale=1 / math.sqrt(128))
        np.testing.assert_array_equal(O.index_project(x, w), np.array(_fraction_index(x, w), dtype=np.uint16))


def test_index_project_identity_weights():
    rng = np.random.default_rng(6)
    x = _rand_bf16(rng, (7, 128))
    w = np.zeros((128, 16), dtype=np.uint16)
    w[np.arange(16), np.arange(16)] = 0x3F80          # W = [I_16; 0]
    np.testing.assert_array_equal(O.index_project(x, w), x[:, :16])


def test_indexer_logits_equal_exact_rational():
    rng = np.random.default_rng(7)
    q = _rand_bf16(rng, (16,), 3.0)
    k = _rand_bf16(rng, (200, 16))
    s = O.indexer_logits(q, k)
    qf = [Fraction(float(v)) for v in O.bf16_to_f64(q)]
    kf = O.bf16_to_f64(k)
    for n in range(200):
        ex = sum((qf[j] * Fraction(float(kf[n, j])) for j in range(16)), Fraction(0))
        assert s[n] == O.fraction_to_f32(ex)


def test_indexer_logits_wide_exponent_spread():
    # products 2^60 and 2^-60 need more than 53 bits: the certificate must fail and
    # the rational fallback must round the exact sum once
    big, tiny = np.float32(2.0 ** 30), np.float32(2.0 ** -30)
    q = O.f64_to_bf16(np.array([big, tiny] + [0.0] * 14))
    k = O.f64_to_bf16(np.array([[big, tiny] + [0.0] * 14, [big, -tiny] + [0.0] * 14]))
    s = O.indexer_logits(q, k)
    assert s[0] == np.float32(2.0 ** 60) and s[1] == np.float32(2.0 ** 60)
    q2 = O.f64_to_bf16(np.array([1.0, 2.0 ** -30] + [0.0] * 14))
    k2 = O.f64_to_bf16(np.array([[1.0 + 2.0 ** -7, 2.0 ** -30 * 1.5] + [0.0] * 14]))
    assert O.indexer_logits(q2, k2)[0] == np.float32(1.0 + 2.0 ** -7)


# ----------------------------------------------------------------------------- Top-P rule
def _nucleus_fixed_order(s, p):
    """Brute force: walk tokens by (bin, position), stop once the mass reaches p*Z."""
    s64 = [float(np.float32(v)) for v in s]
    M = max(s64)
    c = math.floor(M * 8)
    items = []
    for n, v in enumerate(s64):
        b = min(c - math.floor(v * 8), 255)
        items.append((b, n, math.exp(v - M)))
    Z = math.fsum(w for _, _, w in items)
    if p >= 1:
        return list(range(len(s64)))
    need = p * Z
    out, acc = [], 0.0
    for b, n, w in sorted(items):
        if acc >= need:
            break
        out.append(n)
        acc += w
    return sorted(out)


def test_topp_hand_example():
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "topp_hand_example.txt")) if l.strip() and not l.startswith("#")]
    logits = np.array([float(v) for v in lines[0].split(":")[1].split(",")], dtype=np.float32)
    for line in lines[1:]:
        p, bstar, sel = (f.strip() for f in line.split(";"))
        t = O.topp_select(logits, float(p))
        assert t["bstar"] == int(bstar)
        assert list(t["sel"]) == [int(v) for v in sel.split(",")]
    assert list(O.topp_select(logits, 1.0)["sel"]) == list(range(6))


@pytest.mark.parametrize("N", [1, 2, 3, 7, 100, 1000, 4097])
@pytest.mark.parametrize("p", [0.1, 0.5, 0.9, 0.95, 0.999])
def test_topp_uniform_takes_ceil_pN(N, p):
    s = np.full(N, 1.2345, dtype=np.float32)
    assert len(O.topp_select(s, p)["sel"]) == math.ceil(p * N)


@pytest.mark.parametrize("N", [100, 1000])
@pytest.mark.parametrize("p", [0.1, 0.3, 0.99])
def test_topp_uniform_decimal_p(N, p):
    """p * N rounded once to double is an integer for these decimal p, so the
    count is the decimal ceil(pN) and the positions are the first ones."""
    assert p * N == round(p * N)
    t = O.topp_select(np.full(N, -0.4375, dtype=np.float32), p)
    assert list(t["sel"]) == list(range(round(p * N)))


def test_topp_boundary_in_clamp_bin_takes_all():
    """Hand-built case: one token at 0 and 1000 tokens 255 cells (31.875) below
    it, all in the clamp bin 255.  Z = 1 + 1000 e^-31.875 = 1 + 1.43e-11, so
    with p = 1 - 1e-13 the needed mass p Z exceeds bins 0..254 (mass 1) and the
    boundary falls in the clamp bin, which is taken whole: every position.
    At p = 0.9 the top token alone reaches p Z."""
    s = np.full(1001, -31.875, dtype=np.float32)
    s[0] = 0.0
    t = O.topp_select(s, 1.0 - 1e-13)
    assert t["bins"][0] == 0 and np.all(t["bins"][1:] == 255)
    assert abs(t["Z"] - (1.0 + 1000 * math.exp(-31.875))) < 1e-15
    assert t["need"] > 1.0
    assert len(t["sel"]) == 1001 and t.get("clamp_all")
    assert list(O.topp_select(s, 0.9)["sel"]) == [0]
    # cells deeper than 255 below the top clamp into the same bin
    s2 = s.copy()
    s2[500:] = -40.0
    t2 = O.topp_select(s2, 1.0 - 1e-13)
    assert np.all(t2["bins"][1:] == 255) and len(t2["sel"]) == 1001


def test_topp_uniform_integer_pN():
    assert len(O.topp_select(np.zeros(10, np.float32), 0.9)["sel"]) == 9
    assert list(O.topp_select(np.zeros(10, np.float32), 0.9)["sel"]) == list(range(9))


def test_topp_p1_and_dominant():
    rng = np.random.default_rng(8)
    s = rng.standard_normal(500).astype(np.float32)
    assert len(O.topp_select(s, 1.0)["sel"]) == 500
    assert len(O.topp_select(s, 1.5)["sel"]) == 500
    s[123] = 60.0
    assert list(O.topp_select(s, 0.9)["sel"]) == [123]


@pytest.mark.parametrize("N", [1, 2, 3, 17, 257])
def test_topp_matches_brute_force_with_ties(N):
    rng = np.random.default_rng(N)
    for trial in range(40):
        scale = [0.05, 0.5, 2.0, 8.0][trial % 4]
        s = (rng.standard_normal(N) * scale).astype(np.float32)
        if trial % 3 == 0:                      # ties
            s = np.round(s * 4) / 4
        for p in (0.3, 0.9, 0.99):
            assert list(O.topp_select(s, p)["sel"]) == _nucleus_fixed_order(s, p)


def test_topp_agrees_with_sorted_outside_boundary_bin():
    rng = np.random.default_rng(9)
    for trial in range(60):
        s = (rng.standard_normal(2000) * rng.uniform(0.3, 4)).astype(np.float32)
        t = O.topp_select(s, 0.9)
        srt = set(O.sorted_topp(s, 0.9).tolist())
        hist = set(t["sel"].tolist())
        bins = t["bins"]
        for n in range(len(s)):
            if bins[n] < t["bstar"]:
                assert n in hist and n in srt
            elif bins[n] > t["bstar"]:
                assert n not in hist and n not in srt


# ---------------------------------------------------------------- fixed top-k on the histogram order
def test_topk_hand_example():
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "topk_hand_example.txt")) if l.strip() and not l.startswith("#")]
    logits = np.array([float(v) for v in lines[0].split(":")[1].split(",")], dtype=np.float32)
    for line in lines[1:]:
        k, bstar, sel = (f.strip() for f in line.split(";"))
        t = O.topk_select(logits, int(k))
        assert t["bstar"] == int(bstar)
        assert list(t["sel"]) == [int(v) for v in sel.split(",")]


def test_topk_count_all_and_dominant():
    rng = np.random.default_rng(21)
    s = (rng.standard_normal(777) * 2).astype(np.float32)
    for k in (1, 2, 17, 500, 776):
        assert len(O.topk_select(s, k)["sel"]) == k
    for k in (777, 778, 10 ** 6):
        assert list(O.topk_select(s, k)["sel"]) == list(range(777))
    s[400] = 50.0
    assert list(O.topk_select(s, 1)["sel"]) == [400]


@pytest.mark.parametrize("N", [1, 5, 100, 4097])
def test_topk_uniform_takes_first_positions(N):
    s = np.full(N, -0.7, dtype=np.float32)
    for k in (1, 3, N // 2 + 1, N):
        assert list(O.topk_select(s, k)["sel"]) == list(range(min(k, N)))


def test_topk_agrees_with_sorted_outside_boundary_bin():
    rng = np.random.default_rng(22)
    for trial in range(60):
        n = int(rng.integers(1, 3000))
        s = (rng.standard_normal(n) * rng.uniform(0.1, 6)).astype(np.float32)
        if trial % 3 == 0:
            s = np.round(s * 4) / 4                              # ties
        k = int(rng.integers(1, n + 1))
        t = O.topk_select(s, k)
        hist = set(t["sel"].tolist())
        srt = set(O.sorted_topk(s, k).tolist())
        bins = t["bins"]
        if k >= n:
            assert hist == srt == set(range(n))
            continue
        for x in range(n):
            if bins[x] < t["bstar"]:
                assert x in hist and x in srt
            elif bins[x] > t["bstar"]:
                assert x not in hist and x not in srt
        in_b = lambda S: sum(1 for x in S if bins[x] == t["bstar"])
        assert in_b(hist) == in_b(srt)


def test_topk_at_topp_budget_equals_topp():
    """The count rule and the mass rule share one order: top-k with k = |S_p| is S_p."""
    rng = np.random.default_rng(23)
    for trial in range(40):
        s = (rng.standard_normal(2500) * rng.uniform(0.2, 5)).astype(np.float32)
        for p in (0.3, 0.9, 0.99):
            sp = O.topp_select(s, p)["sel"]
            assert list(O.topk_select(s, len(sp))["sel"]) == list(sp)


def test_topk_nested_and_shift_invariant():
    rng = np.random.default_rng(24)
    for trial in range(20):
        s = (np.round(rng.standard_normal(1500) * 64) / 64).astype(np.float32)
        prev = set()
        for k in (1, 10, 100, 700, 1499):
            cur = set(O.topk_select(s, k)["sel"].tolist())
            assert prev <= cur
            prev = cur
            shifted = (s.astype(np.float64) + 3 * 0.125).astype(np.float32)   # exact: |s| < 8, step 1/64
            assert list(O.topk_select(shifted, k)["sel"]) == sorted(cur)


def test_topp_invariants():
    rng = np.random.default_rng(10)
    for trial in range(40):
        s = (rng.standard_normal(3000) * rng.uniform(0.2, 5)).astype(np.float32)
        w = np.exp(s.astype(np.float64) - s.max())
        Z = w.sum()
        prev = set()
        for p in (0.2, 0.5, 0.8, 0.9, 0.95):
            t = O.topp_select(s, p)
            sel = t["sel"]
            assert w[sel].sum() >= p * Z * (1 - 1e-12)                         # mass reaches p
            order = np.lexsort((np.arange(len(s)), t["bins"]))
            last = [n for n in order if n in set(sel.tolist())][-1]
            assert w[sel].sum() - w[last] < p * Z * (1 + 1e-12)                 # minimal
            cur = set(sel.tolist())
            assert prev <= cur                                                    # monotone in p
            prev = cur


def test_topp_shift_by_bin_width_invariant():
    rng = np.random.default_rng(11)
    for trial in range(20):
        s = (np.round(rng.standard_normal(1000) * 3 * 1024) / 1024).astype(np.float32)
        base = O.topp_select(s, 0.9)["sel"]
        for k in (1, -3, 40):
            np.testing.assert_array_equal(O.topp_select(s + np.float32(k / 8), 0.9)["sel"], base)


# ----------------------------------------------------------------------------- attention, eq. (5)
def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(12)
    q = rng.standard_normal(128) * 2
    k = rng.standard_normal((300, 128))
    v = rng.standard_normal((300, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None])[0, 0, 0].numpy()
    np.testing.assert_allclose(O.attention(q, k, v), ref, rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((5, 128))
    v = rng.standard_normal((5, 128))
    np.testing.assert_array_equal(O.attention(rng.standard_normal(128), k[2:3], v[2:3]), v[2])
    np.testing.assert_allclose(O.attention(np.zeros(128), k, v), v.mean(axis=0), rtol=1e-14)


def test_swa_positions():
    assert list(O.swa_positions(9, 100, 4)) == list(range(10))
    assert list(O.swa_positions(9, 1, 0)) == [9]
    assert list(O.swa_positions(9, 3, 2)) == [0, 1, 7, 8, 9]
    assert list(O.swa_positions(5, 4, 4)) == [0, 1, 2, 3, 4, 5]


def _dense_ref(q_rot, k_rows, v_rows):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q_rot)[None, None, None], torch.from_numpy(k_rows)[None, None],
        torch.from_numpy(v_rows)[None, None])[0, 0, 0].numpy()


def test_decode_step_p1_and_wide_window_equal_dense_attention():
    """p = 1 turns eq. (5) into dense attention; so does a window covering the whole cache."""
    import gen
    spec = gen.spec_for(2, B=1, N=700, window=4096)
    wl = gen.make_workload(spec, 77)
    kc, ki = O.build_caches(wl)
    res = O.decode_step(wl.q_pre, wl.w_q, ki, kc, wl.v, wl.head_mode, N=spec.N, p=1.0,
                        window=spec.window, n_sink=spec.n_sink, rope_base=spec.rope_theta,
                        heads=[0, 5])
    m = spec.N - 1
    for h in (0, 5):
        g = h // spec.G
        q_rot = O.rope_rotate(O.bf16_to_f64(wl.q_pre[0, h, 0]), m, spec.rope_theta)
        ref = _dense_ref(q_rot, O.bf16_to_f64(kc[0, g, :m + 1]), O.bf16_to_f64(wl.v[0, g, :m + 1]))
        np.testing.assert_allclose(res["out"][(0, h, 0)], ref, rtol=1e-10, atol=1e-12)


def test_decode_step_selects_planted_needles():
    """Concentrated needle queries: every selected position is a planted needle (generator sanity)."""
    import gen
    spec = gen.spec_for(1)
    wl = gen.make_workload(spec, gen.workload.default_seed(1))
    kc, ki = O.build_caches(wl)
    res = O.decode_step(wl.q_pre, wl.w_q, ki, kc, wl.v, wl.head_mode, N=spec.N, p=spec.p,
                        window=spec.window, n_sink=spec.n_sink, rope_base=spec.rope_theta)
    sel = res["sel"][(0, 0, 0)]
    assert 1 <= len(sel) <= 32
    assert np.isin(sel, wl.needles[(0, 0)]).all()


def test_shared_indexer_keys_reduce_to_per_head_keys():
    """Shared indexer keys (one W_k per KV group) give the same sets and outputs
    as per-head keys whose W_k are all that group's matrix (a pure re-indexing)."""
    import gen
    spec_s = gen.spec_for(2, B=1, N=600, window=64, idx_group=4, n_needles=8)
    wl = gen.make_workload(spec_s, 5)
    kc, ki_s = O.build_caches(wl)
    assert ki_s.shape[1] == spec_s.Hi == 1
    # the per-head view: W_k of every retrieval head = the group's shared matrix
    w_k_per_head = np.repeat(wl.w_k, spec_s.idx_group, axis=0)
    rheads = spec_s.retrieval_heads()
    ki_p = np.stack([O.index_project(wl.k_pre[0, rheads[r] // spec_s.G], w_k_per_head[r])
                     for r in range(spec_s.Hr)])[None]
    common = dict(N=spec_s.N, p=spec_s.p, window=spec_s.window, n_sink=spec_s.n_sink, rope_base=spec_s.rope_theta)
    a = O.decode_step(wl.q_pre, wl.w_q, ki_s, kc, wl.v, wl.head_mode, idx_group=4, **common)
    b = O.decode_step(wl.q_pre, wl.w_q, ki_p, kc, wl.v, wl.head_mode, idx_group=1, **common)
    for key in a["sel"]:
        assert np.array_equal(a["sel"][key], b["sel"][key])
    for key in a["out"]:
        assert np.array_equal(a["out"][key], b["out"][key])
    # with shared W every retrieval head of the group projects with the group's matrix
    assert all(np.array_equal(wl.w_q[r], wl.w_k[r // 4]) for r in range(spec_s.Hr))
