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
