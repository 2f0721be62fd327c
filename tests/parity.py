"""Helpers of the GPU parity tests: uploads and the acceptance rules.

Acceptance (sparse-decode parity, stated with the workload description):
  * attention outputs: max-abs <= 1e-2 and rel-L2 <= 2e-3 against the oracle
    (bf16 in, fp32 accumulate on the GPU, fp64 in the oracle);
  * selected sets: identical except tokens whose fp32 score lies within 1e-4 of
    a bin edge, or when the oracle reports that its closest mass decision lies
    within 1e-5 of Z (rounding of masses can then legitimately flip it; the
    differences must then stay in the boundary bin and its neighbours, see
    check_set);
  * selected mass >= p - 1e-4 (fp64, oracle weights, on the GPU's set).
"""
import collections
import math
import os
import sys

import numpy as np
import torch

import oracle as O

MAX_ABS = 1e-2
REL_L2 = 2e-3
EDGE = 1e-4
MARGIN = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def check_output(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref).max()
    rel = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= MAX_ABS, f"{what}: max-abs {err:.3e}"
    assert rel <= REL_L2 or np.linalg.norm(ref) < 1e-6, f"{what}: rel-L2 {rel:.3e}"
    return err, rel


# verdicts of check_set per test file, printed at the end of the session
SET_STATS = collections.defaultdict(collections.Counter)


def _test_file() -> str:
    cur = os.environ.get("PYTEST_CURRENT_TEST", "?")
    return os.path.basename(cur.split("::")[0])


def check_set(gpu_list: np.ndarray, gpu_count: int, cap: int, t: dict, logits: np.ndarray, p: float, what: str = "",
              exact_logits: bool = True):
    """Compare a GPU Top-P set with the oracle's; returns 'exact', 'edge' or 'margin'.

    'exact': the same positions (and the layout: positions above the boundary
    bin first, then those taken from it, each ascending).
    'edge': every differing position has a score within 1e-4 of a bin edge
    (possible only when the GPU's scores are not bit-exact, exact_logits=False).
    'margin': the oracle reports its closest mass decision within MARGIN * Z of
    p * Z; then every differing position that is not an edge token lies in the
    oracle's bins b*-1..b*+1, the counts differ by at most the population of
    bin b* plus one, and -- when the scores are bit-exact -- the GPU set is
    itself a prefix of the (bin, position) order, i.e. the same rule decided
    at a neighbouring mass.
    Every non-exact set must still hold mass >= p - 1e-4 (oracle weights).
    """
    ref = t["sel"]
    n = min(gpu_count, cap)
    got = np.asarray(gpu_list[:n], dtype=np.int64)
    assert gpu_count >= 1, f"{what}: count {gpu_count}"
    if gpu_count <= cap:
        assert len(np.unique(got)) == len(got), f"{what}: duplicate positions"
        assert np.all((got >= 0) & (got < len(logits))), f"{what}: position out of range"
    if gpu_count == len(ref) and gpu_count <= cap and np.array_equal(np.sort(got), ref):
        if t["bstar"] < O.N_BINS and p < 1:
            nsure = int(np.sum(t["bins"] < t["bstar"]))
            assert np.all(np.diff(got[:nsure]) > 0) and np.all(np.diff(got[nsure:]) > 0), f"{what}: order"
            assert np.all(t["bins"][got[:nsure]] < t["bstar"]), f"{what}: layout"
        elif t["bstar"] >= O.N_BINS:
            assert np.all(np.diff(got) > 0), f"{what}: order (all positions)"
        SET_STATS[_test_file()]["exact"] += 1
        return "exact"
    assert gpu_count <= cap, f"{what}: sets differ and GPU list truncated ({gpu_count} > {cap})"
    diff = np.setxor1d(got, ref)
    s = logits.astype(np.float64)
    bins = t["bins"]
    edge = np.abs(s[diff] * 8 - np.round(s[diff] * 8)) < 8 * EDGE
    if exact_logits:
        edge[:] = False          # bit-exact scores: bins agree, only the mass decision may differ
    rest = diff[~edge]
    verdict = "edge"
    if rest.size:
        verdict = "margin"
        assert t["margin"] < MARGIN, (
            f"{what}: {len(rest)} differing positions (e.g. {rest[:8]}), margin {t['margin']:.2e}")
        bstar = t["bstar"] if t["bstar"] < O.N_BINS else O.N_BINS - 1
        assert np.all(np.abs(bins[rest] - bstar) <= 1), (
            f"{what}: differing positions outside bins b*-1..b*+1 (b* = {bstar}): bins {np.unique(bins[rest])[:8]}")
        pop = int(np.sum(bins == bstar))
        assert abs(gpu_count - len(ref)) <= pop + 1, (
            f"{what}: count {gpu_count} vs {len(ref)} differs by more than bin b* holds ({pop})")
        if exact_logits:
            order = np.lexsort((np.arange(len(bins)), bins))         # bin ascending, then position
            assert np.array_equal(np.sort(order[:gpu_count]), np.sort(got)), (
                f"{what}: GPU set is not a prefix of the (bin, position) order")
    w = t["weights"]
    assert w[got].sum() >= (p - 1e-4) * w.sum(), f"{what}: selected mass below p"
    SET_STATS[_test_file()][verdict] += 1
    return verdict


def check_topk_set(gpu_list: np.ndarray, gpu_count: int, cap: int, t: dict, k: int, what: str = ""):
    """A GPU fixed top-k set must equal the oracle's exactly (only counts decide)."""
    ref = t["sel"]
    assert gpu_count == len(ref) == min(k, len(t["bins"])), f"{what}: count {gpu_count} vs {len(ref)}"
    assert gpu_count <= cap, f"{what}: list truncated"
    got = np.asarray(gpu_list[:gpu_count], dtype=np.int64)
    assert np.array_equal(np.sort(got), ref), f"{what}: sets differ"
    if t["bstar"] < O.N_BINS:
        # layout: positions above the boundary bin, then those taken from it, each ascending
        nsure = int(np.sum(t["bins"] < t["bstar"]))
        assert np.all(np.diff(got[:nsure]) > 0) and np.all(np.diff(got[nsure:]) > 0), f"{what}: order"
        assert np.all(t["bins"][got[:nsure]] < t["bstar"]), f"{what}: layout"
    return "exact"


def sdpa_f64(q_rot, k_rows, v_rows):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.asarray(q_rot, np.float64))[None, None, None],
        torch.from_numpy(np.asarray(k_rows, np.float64))[None, None],
        torch.from_numpy(np.asarray(v_rows, np.float64))[None, None])[0, 0, 0].numpy()


def layer_of(spec, rtp, N=None, Ncap=None, p=None, window=None, n_sink=None):
    return rtp.Layer(B=spec.B, Hq=spec.Hq, Hkv=spec.Hkv, N=spec.N if N is None else N,
                     head_mode=[int(x) for x in spec.head_mode()], nq=spec.nq, Ncap=Ncap,
                     p=spec.p if p is None else p, window=spec.window if window is None else window,
                     n_sink=spec.n_sink if n_sink is None else n_sink, rope_theta=spec.rope_theta,
                     idx_group=spec.idx_group, top_k=spec.top_k)


def edge_fraction(logits):
    s = np.asarray(logits, np.float64)
    return float(np.mean(np.abs(s * 8 - np.round(s * 8)) < 8 * EDGE))


def ceil_pn(p, n):
    return math.ceil(p * n)
