"""Pins of the cluster-index oracle (CPU only).

The cluster index restates the RTPurboV2 article's coarse-to-fine decode
(finding three: tokens grouped into K clusters in the indexer space, the
query matched against the centres, attention inside the hit clusters).  Its
pieces are pinned against the already pinned token path and against
properties of k-means that hold by construction.
"""
import numpy as np
import pytest

import gen
import oracle as O


def _bf16(rng, shape, scale=1.0):
    return gen.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


# ---------------------------------------------------------------- cluster-level top-p
@pytest.mark.parametrize("n", [1, 2, 17, 300])
def test_weighted_topp_with_unit_counts_is_token_topp(n):
    rng = np.random.default_rng(n)
    for trial in range(20):
        s = (rng.standard_normal(n) * rng.uniform(0.1, 5)).astype(np.float32)
        if trial % 3 == 0:
            s = np.round(s * 4) / 4
        for p in (0.3, 0.9, 0.99, 1.0):
            assert list(O.topp_weighted(s, np.ones(n), p)["sel"]) == list(O.topp_select(s, p)["sel"])


def test_weighted_topp_equals_token_rule_on_replicated_items():
    """Item j with count n_j behaves as n_j consecutive tokens at its score:
    it is taken exactly when the token rule takes its first replica."""
    rng = np.random.default_rng(5)
    for trial in range(40):
        k = int(rng.integers(1, 60))
        s = (rng.standard_normal(k) * rng.uniform(0.2, 4)).astype(np.float32)
        cnt = rng.integers(0, 9, size=k)
        cnt[rng.integers(0, k)] = max(1, cnt.max())
        tokens = np.repeat(s, cnt)
        first = np.concatenate(([0], np.cumsum(cnt)[:-1]))
        for p in (0.5, 0.9, 0.97):
            tok = set(O.topp_select(tokens, p)["sel"].tolist())
            ref = [j for j in range(k) if cnt[j] > 0 and first[j] in tok]
            assert list(O.topp_weighted(s, cnt, p)["sel"]) == ref


def test_weighted_topp_skips_empty_items_and_p1_takes_all_live():
    s = np.array([5.0, 1.0, 0.5, 3.0], np.float32)
    cnt = np.array([0, 2, 1, 0])
    # live items: 1 (score 1, two tokens, mass 2) and 2 (score 0.5, one token, mass e^-0.5); Z = 2.6065
    assert list(O.topp_weighted(s, cnt, 0.9)["sel"]) == [1, 2]      # need 2.346: the mass before item 2 is 2
    assert list(O.topp_weighted(s, cnt, 0.7)["sel"]) == [1]         # need 1.825
    assert list(O.topp_weighted(s, cnt, 1.0)["sel"]) == [1, 2]


# ---------------------------------------------------------------- k-means
def test_kmeans_assignment_is_nearest_centre_brute_force():
    rng = np.random.default_rng(6)
    x = _bf16(rng, (120, 16))
    idx = O.kmeans_index(x, 7, 4)
    c = O.bf16_to_f64(idx["centroids"])
    xf = O.bf16_to_f64(x)
    for i in range(len(x)):
        d = [sum((xf[i, t] - c[j, t]) ** 2 for t in range(16)) for j in range(7)]
        best = min(range(7), key=lambda j: (d[j], j))
        assert idx["assign"][i] == best
    assert idx["counts"].sum() == 120


def test_kmeans_converged_centres_are_rounded_member_means():
    rng = np.random.default_rng(7)
    x = _bf16(rng, (200, 16))
    idx = O.kmeans_index(x, 5, 40)                      # enough rounds to settle on this input
    again = O.kmeans_index(x, 5, 41)
    assert np.array_equal(idx["assign"], again["assign"]), "not converged"
    xf = O.bf16_to_f64(x)
    for j in range(5):
        mem = xf[idx["assign"] == j]
        if len(mem):
            assert np.array_equal(idx["centroids"][j], O.f64_to_bf16(mem.mean(axis=0)))


def test_kmeans_recovers_planted_blobs():
    """Well separated blobs, one initial centre in each: the clusters are the blobs."""
    rng = np.random.default_rng(8)
    K, per = 4, 50
    centres = np.eye(16)[:K] * 20.0
    x = np.concatenate([centres[j] + rng.standard_normal((per, 16)) * 0.3 for j in range(K)])
    bits = gen.f32_to_bf16_bits(x.astype(np.float32))
    idx = O.kmeans_index(bits, K, 3)
    assert np.array_equal(idx["assign"], np.repeat(np.arange(K), per))
    assert list(idx["counts"]) == [per] * K


def test_kmeans_one_cluster_per_distinct_key():
    rng = np.random.default_rng(9)
    x = _bf16(rng, (33, 16))
    idx = O.kmeans_index(x, 33, 2)
    assert np.array_equal(idx["assign"], np.arange(33))
    assert np.array_equal(idx["centroids"], x)


# ---------------------------------------------------------------- the coarse-to-fine decode
def test_one_cluster_per_key_reduces_to_the_token_path():
    """With every key its own cluster the hit clusters are the token Top-P set."""
    rng = np.random.default_rng(10)
    n = 400
    k_idx = _bf16(rng, (n, 16))
    q_idx = _bf16(rng, (16,), 2.0)
    idx = O.kmeans_index(k_idx, n, 1)
    t = O.cluster_select(q_idx, idx["centroids"], idx["counts"], 0.9)
    ref = O.topp_select(O.indexer_logits(q_idx, k_idx), 0.9)["sel"]
    assert list(O.cluster_members(idx["assign"], t["sel"])) == list(ref)
