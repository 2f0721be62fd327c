"""Plain, slow, obviously-correct CPU oracle of one sparse-attention decode step.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the CPU baseline
leg of the benchmark.  It shares no code with the HIP library and must never
sit on the product path.

Sources (all statements below are restated, not quoted):
  [FASB]  "Full Attention Strikes Back: Transferring Full Attention into Sparse
          within Hundred Training Steps" (RTPurbo, arXiv 2605.16928),
          section 2.2 eq. (1)-(2) (RoPE), section 3.2 eq. (4)-(5) (indexer,
          Top-P, sparse attention; local heads use a sliding window with
          attention sinks).
  [DR]    DeepRead summary of RTPurbo, "Method" / hardware-optimised kernels:
          sort-free top-p through a 256-bin histogram (1 KB per head),
          p = 0.9, indexer rank 16.

Readings of the pages (where they are silent the plainest reading is taken):
  * RoPE frequencies theta_i = base^(-2(i-1)/D), i = 1..D/2, pairs of
    adjacent channels (2i-2, 2i-1) rotated by m*theta_i; angles in fp64.
  * Indexer query q_idx = bf16(exact q_pre . W_q) and keys K_idx =
    bf16(exact k_pre . W_k), each rounded once (nearest, ties to even).
    Logits s = fp32(exact q_idx . K_idx), rounded once: the "fp32 dense
    indexer".  Products of two bf16 values are exact in fp64; sums are
    certified exact and otherwise done in rational arithmetic.
  * Top-P acts on softmax(s) (no temperature).  Histogram: 256 bins of width
    1/8 on the logit, edges on the multiples of 1/8, bin 0 holding the cell of
    the maximum logit, everything 255 or more cells below it clamped into bin
    255.  b* = first bin (from the top) whose cumulative mass reaches p*Z
    (the product rounded once to double); bins above b* are taken whole, bin
    b* is filled in ascending position while the mass accumulated before a
    token is below p*Z.  p >= 1 takes all, and so does a boundary in the clamp
    bin 255, whose tokens have no common weight scale to fill it by.
  * Fixed top-k (the budget-by-count counterpart of Top-P that FASB section
    2.3 / Table 1 compares against): the first k positions in the order
    (bin ascending, position ascending) of the same histogram; it differs
    from the k largest logits only inside the boundary bin, where scores
    lie within 1/8 of a logit of each other.  k >= m+1 takes all.
  * The candidate set of a query at position m is every cached position
    0..m (the current token included).
  * Local heads attend to the window of the W most recent positions
    (m-W+1..m) plus the first n_sink positions.
  * Attention: softmax(q_rot . K / sqrt(D)) over the set, applied to V; fp64.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

N_BINS = 256          # [DR] 256-bin histogram
CELLS_PER_UNIT = 8    # bin width 1/8 of a logit unit (reading, see module docstring)


# ============================================================================ number formats
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to their exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values once to bf16 (nearest, ties to even); uint16 bits.

    bf16 keeps 8 significant bits and the float32 exponent range, so the
    rounding grid at x = m * 2^e (0.5 <= |m| < 1) has spacing 2^(e-8), and
    2^-133 below the smallest normal 2^-126.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value")
    _, e = np.frexp(x)
    step = np.maximum(e, -125) - 8
    y = np.ldexp(np.rint(np.ldexp(x, -step)), step)   # rint: ties to even
    y32 = y.astype(np.float32)                          # exact (8 significant bits), inf on overflow
    return (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def fraction_to_f32(q: Fraction) -> np.float32:
    """Round an exact rational once to float32 (nearest, ties to even)."""
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1); float32 keeps 24 significant bits
    step = max(e, -126) - 23
    scaled = a / (Fraction(2) ** step)
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * math.ldexp(n, step))


def fraction_to_bf16(q: Fraction) -> np.uint16:
    """Round an exact rational once to bf16 (nearest, ties to even)."""
    if q == 0:
        return np.uint16(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    step = max(e, -126) - 7
    scaled = a / (Fraction(2) ** step)
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = np.float32(sign * math.ldexp(n, step))
    return np.uint16(v.view(np.uint32) >> np.uint32(16))


def _lsb_exponent(v: np.ndarray) -> np.ndarray:
    """Exponent of the lowest significant bit of bf16-valued entries (a lower bound for subnormals)."""
    _, e = np.frexp(v)
    return np.where(v != 0, e - 8, 10**6).astype(np.int64)


def _exact_dot(x: np.ndarray, w: np.ndarray):
    """x @ w for bf16-valued fp64 operands x [M, K], w [K, J]; returns (sum, exact mask).

    Every product of two bf16 values is exact in fp64 (8 + 8 significant
    bits).  The products are accumulated one index at a time.  If all products
    of an entry are multiples of 2^L and their magnitudes add up to less than
    2^(L+52), every partial sum is representable and the fp64 result is the
    exact sum; entries without that certificate are flagged.
    """
    acc = np.zeros((x.shape[0], w.shape[1]), dtype=np.float64)
    for c in range(x.shape[1]):
        acc += x[:, c:c + 1] * w[c:c + 1, :]
    lsb = _lsb_exponent(x).min(axis=1)[:, None] + _lsb_exponent(w).min(axis=0)[None, :]
    mag = np.abs(x) @ np.abs(w)
    exact = (mag == 0) | (mag < np.ldexp(1.0, np.minimum(lsb, 900) + 52))
    return acc, exact


def _fraction_dot(x_row: np.ndarray, w_col: np.ndarray) -> Fraction:
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x_row, w_col)), Fraction(0))


# ============================================================================ RoPE, eq. (1)
def rope_theta(D: int, base: float) -> np.ndarray:
    """theta_i = base^(-2(i-1)/D) for i = 1..D/2, decreasing with the channel index [FASB eq. (1)]."""
    i = np.arange(D // 2, dtype=np.float64)
    return base ** (-2.0 * i / D)


def rope_rotate(x, pos, base: float) -> np.ndarray:
    """R(m) x for rows x[..., D] at positions pos[...]: block-diagonal 2x2 rotations [FASB eq. (1)].

    Pair i = channels (2i, 2i+1) is rotated by angle m*theta_i:
    (a, b) -> (a cos - b sin, a sin + b cos).  fp64 throughout.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(D, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def rope_keys(k_pre_bits, base: float, pos=None) -> np.ndarray:
    """Post-RoPE key cache bf16(R(n) k_pre[n]) for rows at positions n (default 0..N-1)."""
    k = bf16_to_f64(k_pre_bits)
    if pos is None:
        pos = np.arange(k.shape[-2], dtype=np.int64)
    return f64_to_bf16(rope_rotate(k, pos, base))


# ============================================================================ indexer, eq. (4)
def index_project(x_bits, w_bits) -> np.ndarray:
    """bf16(exact x . W): the 16-d indexer projection of pre-RoPE rows [FASB eq. (4)].

    x_bits [..., D] bf16, w_bits [D, R] bf16 (stored D x R, the transpose of
    the r x d_h matrix of eq. (4)).  Returns bf16 bits [..., R].
    """
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    out = np.empty((x2.shape[0], w.shape[1]), dtype=np.uint16)
    for r0 in range(0, x2.shape[0], 1 << 16):          # row blocks only bound the memory
        xs = x2[r0:r0 + (1 << 16)]
        s, exact = _exact_dot(xs, w)
        blk = f64_to_bf16(s)
        for i, j in zip(*np.nonzero(~exact)):
            blk[i, j] = fraction_to_bf16(_fraction_dot(xs[i], w[:, j]))
        out[r0:r0 + xs.shape[0]] = blk
    return out.reshape(*lead, w.shape[1])


def indexer_logits(q_idx_bits, k_idx_bits) -> np.ndarray:
    """s_n = fp32(exact q_idx . K_idx[n]) for every cached row n [FASB eq. (4)]; float32 [N]."""
    q = bf16_to_f64(q_idx_bits).reshape(-1, 1)
    k = bf16_to_f64(k_idx_bits)
    s, exact = _exact_dot(k, q)
    out = s[:, 0].astype(np.float32)
    for i in np.nonzero(~exact[:, 0])[0]:
        out[i] = fraction_to_f32(_fraction_dot(k[i], q[:, 0]))
    return out


# ============================================================================ Top-P, eq. (5) + histogram
def topp_select(logits, p: float) -> dict:
    """Dynamic Top-P over softmax(logits) with the 256-bin histogram rule [FASB eq. (5); DR].

    Returns a dict with the selected positions ``sel`` (ascending), the
    boundary bin ``bstar``, the total mass ``Z``, ``need`` = p*Z and the
    relative ``margin`` of the closest mass decision (used by tests to
    recognise cases whose outcome hinges on rounding).
    """
    s = np.asarray(logits, dtype=np.float32)
    n = s.shape[0]
    if n == 0:
        return dict(sel=np.zeros(0, np.int64), bstar=-1, Z=0.0, need=0.0, margin=np.inf,
                    bins=np.zeros(0, np.int64), weights=np.zeros(0))
    if not np.all(np.isfinite(s)):
        raise ValueError("non-finite logit")
    s64 = s.astype(np.float64)
    cell = np.floor(s64 * CELLS_PER_UNIT).astype(np.int64)     # 8*s is exact in fp32
    M = s64.max()
    c = int(np.floor(M * CELLS_PER_UNIT))
    bins = np.minimum(c - cell, N_BINS - 1)
    w = np.exp(s64 - M)                                        # softmax numerators, max = 1
    if p >= 1.0:
        return dict(sel=np.arange(n, dtype=np.int64), bstar=N_BINS, Z=float(w.sum()),
                    need=float(w.sum()), margin=np.inf, bins=bins, weights=w)
    H = np.bincount(bins, weights=w, minlength=N_BINS)
    cum = np.cumsum(H)
    Z = float(cum[-1])
    need = p * Z
    bstar = int(np.searchsorted(cum, need, side="left"))      # first bin with cum >= need
    bstar = min(bstar, N_BINS - 1)
    before_bin = float(cum[bstar - 1]) if bstar > 0 else 0.0
    if bstar == N_BINS - 1:
        # Boundary in the clamp bin: its tokens lie 255 or more cells below the
        # top, so the bin carries no common weight scale to fill it by; the
        # reading takes it whole, i.e. every position.  (This needs a clamp
        # mass above (1 - p) Z, so p within N e^-31.75 of 1.)
        margin = min(abs(need - before_bin), abs(float(cum[bstar]) - need)) / Z
        return dict(sel=np.arange(n, dtype=np.int64), bstar=N_BINS, Z=Z, need=need, margin=margin, bins=bins,
                    weights=w, clamp_all=True)
    sure = np.nonzero(bins < bstar)[0]
    cand = np.nonzero(bins == bstar)[0]                        # ascending positions
    before_tok = before_bin + np.concatenate(([0.0], np.cumsum(w[cand])[:-1]))
    take = before_tok < need
    sel = np.sort(np.concatenate((sure, cand[take])))
    # closest mass decision, relative to Z
    m = [need - before_bin, float(cum[bstar]) - need]
    if take.any():
        m.append(need - float(before_tok[take][-1]))
    if (~take).any():
        m.append(float(before_tok[~take][0]) - need)
    margin = min(abs(x) for x in m) / Z
    return dict(sel=sel, bstar=bstar, Z=Z, need=need, margin=margin, bins=bins, weights=w)


def sorted_topp(logits, p: float) -> np.ndarray:
    """Textbook nucleus: the shortest prefix, by logit descending (ties by position), with mass >= p."""
    s64 = np.asarray(logits, dtype=np.float32).astype(np.float64)
    order = np.lexsort((np.arange(s64.size), -s64))
    w = np.exp(s64[order] - s64.max())
    if p >= 1.0:
        return np.sort(order)
    cum = np.cumsum(w)
    k = int(np.searchsorted(cum, p * cum[-1], side="left")) + 1
    return np.sort(order[:k])


def topk_select(logits, k: int) -> dict:
    """Fixed top-k on the same 256-bin histogram order [FASB sec. 2.3 / Table 1 (top-k vs top-p); DR].

    The k positions first in the order (bin ascending, position ascending),
    bins as in ``topp_select``.  Returns ``sel`` (ascending), ``bstar`` (the
    bin of the last position taken; N_BINS when every position is taken) and
    ``bins``.
    """
    s = np.asarray(logits, dtype=np.float32)
    n = s.shape[0]
    if k < 1:
        raise ValueError("k must be >= 1")
    if n == 0:
        return dict(sel=np.zeros(0, np.int64), bstar=-1, bins=np.zeros(0, np.int64))
    if not np.all(np.isfinite(s)):
        raise ValueError("non-finite logit")
    s64 = s.astype(np.float64)
    cell = np.floor(s64 * CELLS_PER_UNIT).astype(np.int64)
    c = int(np.floor(s64.max() * CELLS_PER_UNIT))
    bins = np.minimum(c - cell, N_BINS - 1)
    if k >= n:
        return dict(sel=np.arange(n, dtype=np.int64), bstar=N_BINS, bins=bins)
    order = np.lexsort((np.arange(n), bins))                   # bin, then position
    taken = order[:k]
    return dict(sel=np.sort(taken), bstar=int(bins[taken[-1]]), bins=bins)


def sorted_topk(logits, k: int) -> np.ndarray:
    """Textbook top-k: the k largest logits, ties by position; ascending positions."""
    s64 = np.asarray(logits, dtype=np.float32).astype(np.float64)
    order = np.lexsort((np.arange(s64.size), -s64))
    return np.sort(order[:k])


# ============================================================================ attention, eq. (5)
def attention(q_rot, k_rows, v_rows) -> np.ndarray:
    """sum_n softmax_n(q . k_n / sqrt(D)) v_n over the given rows [FASB eq. (5)]; fp64."""
    q = np.asarray(q_rot, dtype=np.float64)
    k = np.asarray(k_rows, dtype=np.float64)
    v = np.asarray(v_rows, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros(q.shape[-1])
    a = k @ q / math.sqrt(q.shape[-1])
    e = np.exp(a - a.max())
    return (e @ v) / e.sum()


def swa_positions(m: int, window: int, n_sink: int) -> np.ndarray:
    """Rows a local head reads at query position m: window m-W+1..m plus sinks 0..n_sink-1 [FASB sec. 3.2]."""
    lo = max(0, m - window + 1)
    rows = set(range(lo, m + 1))
    rows.update(range(min(n_sink, m + 1)))
    return np.array(sorted(rows), dtype=np.int64)


# ============================================================================ whole step
def query_positions(N: int, nq: int) -> np.ndarray:
    return np.arange(N - nq, N, dtype=np.int64)


def decode_step(q_pre, w_q, k_idx, k_cache, v_cache, head_mode, *, N, p, window, n_sink,
                rope_base, heads=None, batches=None, queries=None, want_logits=False, idx_group=1,
                top_k=0) -> dict:
    """One decode (nq = 1) or chunked-prefill (nq > 1) step of the layer.

    q_pre [B, Hq, nq, D] bf16; w_q [Hr, D, R] bf16; k_idx [B, Hi, >=N, R] bf16
    (indexer keys; retrieval head r reads head r // idx_group);
    k_cache / v_cache [B, Hkv, >=N, D] bf16
    (post-RoPE keys, values); head_mode [Hq] (1 retrieval, 0 local).
    Retrieval heads: eq. (4) scores, Top-P (or fixed top-k when top_k > 0),
    eq. (5) over the selected set.
    Local heads: eq. (5) over the sliding window plus sinks.
    ``heads``/``batches``/``queries`` restrict the work to a sample.
    Returns out[(b, h, i)] fp64 [D], sel[(b, r, i)], topp[(b, r, i)].
    """
    B, Hq, nq, D = q_pre.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    hm = np.asarray(head_mode)
    rheads = [int(h) for h in np.nonzero(hm)[0]]
    rindex = {h: r for r, h in enumerate(rheads)}
    pos = query_positions(N, nq)
    out, sel, topp, logits_out = {}, {}, {}, {}
    for b in (range(B) if batches is None else batches):
        for h in (range(Hq) if heads is None else heads):
            g = h // G
            for i in (range(nq) if queries is None else queries):
                m = int(pos[i])
                q_rot = rope_rotate(bf16_to_f64(q_pre[b, h, i]), m, rope_base)
                if hm[h]:
                    r = rindex[h]
                    q_idx = index_project(q_pre[b, h, i], w_q[r])
                    s = indexer_logits(q_idx, k_idx[b, r // idx_group, :m + 1])
                    t = topk_select(s, top_k) if top_k > 0 else topp_select(s, p)
                    rows = t["sel"]
                    sel[(b, r, i)] = rows
                    topp[(b, r, i)] = t
                    if want_logits:
                        logits_out[(b, r, i)] = s
                else:
                    rows = swa_positions(m, window, n_sink)
                out[(b, h, i)] = attention(q_rot, bf16_to_f64(k_cache[b, g, rows]),
                                           bf16_to_f64(v_cache[b, g, rows]))
    res = dict(out=out, sel=sel, topp=topp)
    if want_logits:
        res["logits"] = logits_out
    return res


def build_caches(wl, groups=None, heads=None):
    """Post-RoPE key cache and indexer-key cache of a generated workload (oracle's own arithmetic).

    Returns (k_cache [B,Hkv,N,D] bf16, k_idx [B,Hi,N,R] bf16).  Indexer-key
    head i serves retrieval heads i*ig .. i*ig+ig-1 (ig = spec.idx_group) and
    projects the keys of their KV group with W_k[i] (FASB eq. (4); ig > 1 is
    the shared-per-group variant).  ``groups`` / ``heads`` restrict which KV
    groups / retrieval heads are filled (others stay zero).
    """
    spec = wl.spec
    B, Hkv, N, D = wl.k_pre.shape
    G = spec.Hq // Hkv
    ig = getattr(spec, "idx_group", 1)
    rheads = [int(h) for h in np.nonzero(wl.head_mode)[0]]
    k_cache = np.zeros_like(wl.k_pre)
    k_idx = np.zeros((B, len(rheads) // ig, N, spec.R), dtype=np.uint16)
    pos = np.arange(N, dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            if groups is not None and g not in groups:
                continue
            k_cache[b, g] = rope_keys(wl.k_pre[b, g], spec.rope_theta, pos)
        for i in range(len(rheads) // ig):
            if heads is not None and not any(r // ig == i for r in heads):
                continue
            k_idx[b, i] = index_project(wl.k_pre[b, rheads[i * ig] // G], wl.w_k[i])
    return k_cache, k_idx
