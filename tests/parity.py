"""Parity checks between libkmip results and the fp64 oracle.

Selection (top-k index sets).  The GPU scores in fp32 (exact bf16 products,
fp32 accumulation); the oracle in fp64.  For query row (i, h) with oracle
scores s over its graph, k_eff = min(k, n_b), and the k-th / (k+1)-th largest
oracle scores s_k, s_k1, the tie band is

    delta = band_rel * max(|s_k|, |s_k1|) + 2 * eps,   band_rel = 1e-3,
    eps   = c * ||q_i|| * max_j ||k_j||,

eps bounding the error of one GPU score (Cauchy-Schwarz): c = d * 2^-23 for
bf16 inputs (fp32 accumulation of exact products), and for the fp32 entry
point's three-term bf16 split c = 3 * 2^-18 (dropped split terms) +
3d * 2^-23 (accumulation of 3d products).  Each computed score is off by at
most eps, so two keys can trade places across the boundary only when their
true scores are within 2 * eps.  A GPU set G is accepted iff it has exactly
k_eff distinct in-graph ids, padding -1 after them, and
min_{j in G} s_j >= max_{j not in G} s_j - delta.  When s_k - s_k1 > delta
this forces G to equal the oracle's set exactly.  The GPU order must be
non-increasing in oracle score up to 2*eps, the saved fp32 scores must match
the oracle scores of the same ids within eps (for the fp32 entry point,
which recomputes the saved scores in fp32 after selecting, within the plain
fp32 bound d * 2^-23 * ||q|| * max ||k||), and entries with bitwise-equal
GPU scores must be in ascending id order.  band_rel = 0 checks the selection
at the scores' own accuracy.

Values.  Outputs and gradients are compared row by row ((node, head)
d-vectors): max_c |x - ref| / max_c |ref| <= 2e-3, with the reference taken
from the oracle on the GPU's own index sets.  Rows whose reference is exactly
zero (keys no query selected) must be exactly zero.
"""
from __future__ import annotations

import numpy as np

import oracle.kmip_oracle as orc

REL_TOL = 2e-3
BAND_REL = 1e-3


def decode(w):
    """fp64 copies of a workload's inputs (bf16 bits through the oracle's own
    decoder; float32 values exactly)."""
    if getattr(w, "dtype", "bf16") == "f32":
        return tuple(np.asarray(x, dtype=np.float64) for x in (w.q, w.k, w.v))
    return (orc.bf16_bits_to_f64(w.q), orc.bf16_bits_to_f64(w.k), orc.bf16_bits_to_f64(w.v))


def eps_coef(d: int, split: bool = False) -> float:
    """c of the per-score error bound eps = c * ||q|| * max ||k||."""
    if split:
        return 3 * 2.0 ** -18 + 3 * d * 2.0 ** -23
    return d * 2.0 ** -23


def check_selection(gpu_idx, gpu_score, q, k, offsets, topk, rows, heads=None, *,
                    band_rel=BAND_REL, split=False):
    """Check GPU index/score rows (full [N][H][k] arrays) for the given nodes.

    split: the scores come from the fp32 entry point (three-term bf16 split).
    Returns a dict of statistics; raises AssertionError on the first failure.
    """
    n, H, d = q.shape
    coef = eps_coef(d, split)
    saved_coef = eps_coef(d, False)
    heads = range(H) if heads is None else heads
    ranges = orc.graph_ranges(offsets, n)
    starts = np.array([lo for lo, _ in ranges])
    stats = dict(rows=0, exact=0, in_band=0)
    rows = list(rows)
    graph_of = {}
    for i in rows:
        b = int(np.searchsorted(starts, i, side="right") - 1)
        while ranges[b][1] <= i:        # skip empty graphs sharing a start
            b += 1
        graph_of[i] = b
    for h in heads:
        kh = np.ascontiguousarray(k[:, h, :])
        knorm = np.linalg.norm(kh, axis=1)
        kmax_of = {}
        for i in rows:
            b = graph_of[i]
            lo, hi = ranges[b]
            if b not in kmax_of:
                kmax_of[b] = float(knorm[lo:hi].max())
            s = kh[lo:hi] @ q[i, h, :]
            nb = hi - lo
            kk = min(topk, nb)
            G = np.asarray(gpu_idx[i, h], dtype=np.int64)
            assert np.all(G[kk:] == -1), (i, h, "padding", G)
            assert np.all(np.isneginf(gpu_score[i, h, kk:])), (i, h, "pad score")
            g = G[:kk]
            assert np.all((g >= lo) & (g < hi)), (i, h, "out of graph", g, lo, hi)
            assert np.unique(g).size == kk, (i, h, "duplicates", g)
            loc = g - lo
            eps = coef * float(np.linalg.norm(q[i, h])) * kmax_of[b]
            inside = s[loc]
            mask = np.ones(nb, dtype=bool)
            mask[loc] = False
            outside_max = s[mask].max() if mask.any() else -np.inf
            if kk < nb:
                part = np.partition(s, [nb - kk - 1, nb - kk])
                s_k, s_k1 = part[nb - kk], part[nb - kk - 1]
            else:
                s_k, s_k1 = s.min(), -np.inf
            delta = band_rel * max(abs(s_k), abs(s_k1) if np.isfinite(s_k1) else 0.0) + 2 * eps
            assert inside.min() >= outside_max - delta, (
                i, h, "selection", inside.min(), outside_max, delta)
            ref_set = set(orc.select_topk_row(s, topk).tolist())
            if ref_set == set(loc.tolist()):
                stats["exact"] += 1
            else:
                stats["in_band"] += 1
            assert np.all(np.diff(inside) <= 2 * eps), (i, h, "order", inside)
            gs = np.asarray(gpu_score[i, h, :kk], dtype=np.float64)
            seps = saved_coef * float(np.linalg.norm(q[i, h])) * kmax_of[b]
            assert np.all(np.abs(gs - inside) <= seps + 1e-30), (i, h, "score", gs - inside, seps)
            if not split:
                # Equal saved scores are equal scan scores: ascending ids.
                # The fp32 entry point orders by its split-precision scan
                # scores but saves rescored fp32 values, which may tie where
                # the scan's did not; its tie rule is checked on inputs with
                # duplicate keys instead (tests/test_gpu_f32.py).
                eq = np.nonzero(np.diff(gs) == 0)[0]
                assert np.all(g[eq] < g[eq + 1]), (i, h, "tie order", g, gs)
            stats["rows"] += 1
    return stats


def row_rel_err(x, ref):
    """max over rows of max_c |x - ref| / max_c |ref|; rows with zero
    reference must match exactly (returns inf otherwise)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, x.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    scale = np.abs(ref).max(axis=1)
    diff = np.abs(x - ref).max(axis=1)
    zero = scale == 0
    if np.any(diff[zero] != 0):
        return np.inf
    if np.all(zero):
        return 0.0
    return float((diff[~zero] / scale[~zero]).max())


def assert_rows_close(x, ref, what, tol=REL_TOL):
    e = row_rel_err(x, ref)
    assert e <= tol, f"{what}: row-normalised error {e:.3e} > {tol:.1e}"
    return e
