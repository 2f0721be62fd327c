"""The seeded input generator: determinism and the structure of the draws (CPU only)."""
import numpy as np

import gen


def test_deterministic_and_seed_dependent():
    spec = gen.spec_for(2, B=2, N=5000, window=64)
    a = gen.make_workload(spec, 5)
    b = gen.make_workload(spec, 5)
    c = gen.make_workload(spec, 6)
    for name in ("q_pre", "w_q", "w_k", "k_pre", "v"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert not np.array_equal(a.k_pre, c.k_pre)


def test_needles_disjoint_and_local_rows_only():
    spec = gen.spec_for(2, B=2, N=5000, window=64)
    wl = gen.make_workload(spec, 9)
    assert wl.head_mode.tolist() == [1] * 4 + [0] * 28
    for b in range(2):
        pos = np.concatenate([wl.needles[(b, r)] for r in range(4)])
        assert len(np.unique(pos)) == len(pos) == 4 * 64
    rows = spec.local_rows()
    assert rows.tolist() == [0, 1, 2, 3] + list(range(5000 - 64, 5000))
    mask = np.zeros(5000, bool)
    mask[rows] = True
    assert np.all(wl.k_pre[:, 1:, ~mask] == 0) and np.all(wl.v[:, 1:, ~mask] == 0)
    assert np.any(wl.k_pre[:, 1:, mask] != 0)


def test_bf16_plumbing_roundtrip():
    x = np.array([1.0, -2.5, 3.14159, 1e-20, 65504.0], dtype=np.float32)
    bits = gen.f32_to_bf16_bits(x)
    y = gen.bf16_bits_to_f32(bits)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)
    np.testing.assert_array_equal(gen.f32_to_bf16_bits(y), bits)


def test_class_recipe():
    spec = gen.spec_for(3, B=2, N=20000)
    wl = gen.make_workload(spec, 3, scales={})
    assert [wl.classes[(0, r)] for r in range(4)] == [0, 1, 0, 1]
    assert len(wl.needles[(0, 0)]) == 16 and len(wl.needles[(0, 1)]) == 8192


def test_topics_mode_per_query_scale():
    """A ("q", b, r, i) scale multiplies query i of retrieval head r alone; a
    (b, r, topic) scale every query of that topic."""
    spec = gen.spec_for(5, N=3000, nq=8, query_scale="unit", diffuse=(200, 0.5))
    base = gen.make_workload(spec, 11, scales={})
    one = gen.make_workload(spec, 11, scales={("q", 0, 1, 3): 2.0})
    top = gen.make_workload(spec, 11, scales={(0, 2, 1): 0.5})
    h1, h2 = spec.retrieval_heads()[1], spec.retrieval_heads()[2]
    u = gen.bf16_bits_to_f32(base.q_pre)
    for wl, (h, rows, s) in ((one, (h1, [3], 2.0)), (top, (h2, [1, 3, 5, 7], 0.5))):
        q = gen.bf16_bits_to_f32(wl.q_pre)
        for i in range(spec.nq):
            want = u[0, h, i] * s if i in rows else u[0, h, i]
            np.testing.assert_allclose(q[0, h, i], want, rtol=2.0 ** -7)
        others = [x for x in range(spec.Hq) if x != h]
        np.testing.assert_array_equal(wl.q_pre[0, others], base.q_pre[0, others])


def test_chunked_prefill_table_has_one_scale_per_query():
    """The calibrated chunked-prefill workload stores one scale per (b, head,
    query), with the oracle's set size at that scale near its topic's target
    (500 concentrated, 2500 diffuse)."""
    spec = gen.spec_for(5)
    key = gen.workload.scale_key(spec, gen.workload.default_seed(5)) + "/per-query"
    ent = gen.workload.load_scale_table()[key]
    assert sorted((e[0], e[1], e[2]) for e in ent) == [
        (b, r, i) for b in range(spec.B) for r in range(spec.Hr) for i in range(spec.nq)]
    assert all(e[3] > 0 for e in ent)
    for tpc, target in ((0, 500), (1, 2500)):
        c = np.array([e[4] for e in ent if e[2] % 2 == tpc])
        assert abs(np.median(c) - target) <= 0.05 * target, (tpc, np.median(c))
    diffuse = np.array([e[4] for e in ent if e[2] % 2 == 1])
    assert np.mean(np.abs(diffuse - 2500) <= 50) > 0.75
