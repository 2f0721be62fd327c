"""CPU oracle of the cluster index (the RTPurboV2 decode path).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/.  It shares no code with
the HIP library.

Source: the news article on RTPurboV2, finding three ("adaptive clustering in
the sequence dimension"): the cached tokens are grouped into K clusters in the
low-rank indexer space (K = 128 as the page's example), a query first matches
the K cluster centres (the coarse stage) and full attention then runs only
inside the clusters it hits (the fine stage); the retrieval heads keep a
dynamic top-p.  The page names neither the clustering method nor the hit
rule.  Readings (the plainest ones the rest of the pages support):

  * Clustering: Lloyd's k-means on the bf16 indexer keys K_idx (16-d), squared
    Euclidean distance, ties to the lowest cluster index.  Initial centre j is
    the key at position floor(j N / K).  Each round assigns every key to its
    nearest centre, then moves every non-empty cluster's centre to the mean
    of its members rounded once to bf16 (empty clusters keep theirs).  After
    the last round the keys are assigned once more; that assignment is the
    index.  Distances are exact in fp64 (bf16 products and short sums).
  * Coarse stage: the centre scores s_j = fp32(exact q_idx . c_j), the same
    dot product as a token's indexer score.
  * Hit rule: dynamic top-p over clusters.  Cluster j stands for its n_j
    members at score s_j, so its softmax mass is estimated as n_j exp(s_j);
    the histogram rule of the token path picks the clusters (bins of the
    centre scores, bins above b* whole, clusters of bin b* in ascending index
    while the mass before them is below p Z; empty clusters are never hit).
  * Fine stage: attention (FASB eq. (5)) over every member of the hit
    clusters, i.e. the cached positions assigned to them.
"""
from __future__ import annotations

import numpy as np

from .rtp_oracle import (CELLS_PER_UNIT, N_BINS, attention, bf16_to_f64, f64_to_bf16, index_project,
                         indexer_logits, rope_rotate)


def kmeans_index(k_idx_bits, K: int, iters: int) -> dict:
    """Lloyd's k-means of bf16 indexer keys [n, 16] into K clusters (reading in the module docstring).

    Returns centroids (bf16 bits [K, 16]), assign [n] and counts [K].
    """
    x = bf16_to_f64(np.asarray(k_idx_bits, dtype=np.uint16))
    n = x.shape[0]
    if not 1 <= K <= n:
        raise ValueError("need 1 <= K <= n")
    c_bits = np.asarray(k_idx_bits, dtype=np.uint16)[(np.arange(K) * n) // K].copy()
    xx = np.sum(x * x, axis=1)

    def assign_to(cb):
        c = bf16_to_f64(cb)
        d = xx[:, None] - 2.0 * (x @ c.T) + np.sum(c * c, axis=1)[None, :]
        return np.argmin(d, axis=1)                  # first minimum: lowest index on ties

    for _ in range(iters):
        a = assign_to(c_bits)
        for j in range(K):
            mem = x[a == j]
            if len(mem):
                c_bits[j] = f64_to_bf16(mem.sum(axis=0) / len(mem))
    a = assign_to(c_bits)
    return dict(centroids=c_bits, assign=a.astype(np.int64), counts=np.bincount(a, minlength=K).astype(np.int64))


def topp_weighted(scores, counts, p: float) -> dict:
    """Histogram top-p over items of score s_j standing for counts[j] tokens each.

    Bins and order as the token rule (bin ascending, then item index); an item
    is taken whole while the mass before it is below p * Z.  Items with a zero
    count are never taken.  Returns the taken items ``sel`` (ascending), the
    boundary bin and the closest decision's relative margin.
    """
    s = np.asarray(scores, dtype=np.float32)
    w_n = np.asarray(counts, dtype=np.float64)
    live = np.nonzero(w_n > 0)[0]
    if live.size == 0:
        return dict(sel=np.zeros(0, np.int64), bstar=-1, margin=np.inf)
    s64 = s.astype(np.float64)
    M = s64[live].max()
    c = int(np.floor(M * CELLS_PER_UNIT))
    bins = np.minimum(c - np.floor(s64 * CELLS_PER_UNIT).astype(np.int64), N_BINS - 1)
    w = np.where(w_n > 0, w_n * np.exp(np.minimum(s64 - M, 0.0)), 0.0)
    if p >= 1.0:
        return dict(sel=live.astype(np.int64), bstar=N_BINS, margin=np.inf)
    order = np.lexsort((np.arange(s.size), bins))
    order = order[w[order] > 0]
    before = np.concatenate(([0.0], np.cumsum(w[order])[:-1]))
    Z = float(w.sum())
    need = p * Z
    take = before < need
    sel = np.sort(order[take])
    m = [need - float(before[take][-1])]
    if (~take).any():
        m.append(float(before[~take][0]) - need)
    bstar = int(bins[order[take][-1]])
    return dict(sel=sel.astype(np.int64), bstar=bstar, margin=min(abs(v) for v in m) / Z, bins=bins, weights=w)


def cluster_select(q_idx_bits, centroid_bits, counts, p: float) -> dict:
    """Coarse stage: centre scores and the hit clusters (module docstring)."""
    s = indexer_logits(q_idx_bits, centroid_bits)
    t = topp_weighted(s, counts, p)
    t["scores"] = s
    return t


def cluster_members(assign, hit) -> np.ndarray:
    """Cached positions assigned to any hit cluster, ascending."""
    return np.nonzero(np.isin(assign, hit))[0].astype(np.int64)


def cluster_decode_head(q_pre_bits, w_q_bits, index: dict, k_cache_bits, v_cache_bits, m: int, p: float,
                        rope_base: float) -> dict:
    """One retrieval head's decode over the cluster index: coarse stage, then
    eq. (5) attention over the hit clusters' members (all at positions <= m)."""
    q_idx = index_project(q_pre_bits, w_q_bits)
    t = cluster_select(q_idx, index["centroids"], index["counts"], p)
    rows = cluster_members(index["assign"], t["sel"])
    q_rot = rope_rotate(bf16_to_f64(q_pre_bits), m, rope_base)
    out = attention(q_rot, bf16_to_f64(k_cache_bits[rows]), bf16_to_f64(v_cache_bits[rows]))
    return dict(out=out, rows=rows, select=t)
