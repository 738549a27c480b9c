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


def oracle_forward(q, k, v, offsets, topk, rows, workers=None):
    """The oracle's forward on the given rows: in this process for small row
    counts, over a pool of worker processes otherwise."""
    rows = np.asarray(list(rows) if not isinstance(rows, np.ndarray) else rows, dtype=np.int64)
    work = int(rows.size) * q.shape[1] * max(1, q.shape[0] // 1000)
    if workers == 1 or work < 200_000:
        return orc.kmip_forward(q, k, v, offsets, topk, rows=rows)
    from oracle.pool import forward_rows
    return forward_rows(q, k, v, offsets, topk, rows, workers=workers)


def check_selection(gpu_idx, gpu_score, q, k, offsets, topk, rows, heads=None, *,
                    band_rel=BAND_REL, split=False, ref=None, v=None, workers=None,
                    block=16384):
    """Check GPU index/score rows (full [N][H][k] arrays) for the given nodes.

    The oracle's own selection for those rows (``ref``, computed here when
    not given) decides every row whose GPU set equals it; the other rows are
    checked against the tie band on their full fp64 score rows.
    split: the scores come from the fp32 entry point (three-term bf16 split).
    Returns a dict of statistics; raises AssertionError on the first failure.
    """
    n, H, d = q.shape
    K = int(topk)
    coef = eps_coef(d, split)
    saved_coef = eps_coef(d, False)
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.asarray(list(rows) if not isinstance(rows, np.ndarray) else rows, dtype=np.int64)
    if ref is None:
        ref = oracle_forward(q, k, v if v is not None else k, offsets, K, rows, workers)
    off = (np.array([0, n], dtype=np.int64) if offsets is None or len(offsets) < 2
           else np.asarray(offsets, dtype=np.int64))
    b_of = np.searchsorted(off, rows, side="right") - 1          # skips empty graphs
    lo_r, hi_r = off[b_of], off[b_of + 1]
    kk_r = np.minimum(K, hi_r - lo_r)
    slot = np.arange(K)[None, :] < kk_r[:, None]                  # [R][K]
    stats = dict(rows=0, exact=0, in_band=0)
    for h in heads:
        kh = np.ascontiguousarray(k[:, h, :])
        knorm = np.linalg.norm(kh, axis=1)
        kmax_b = np.array([knorm[a:b].max() if b > a else 0.0 for a, b in zip(off[:-1], off[1:])])
        for a in range(0, rows.size, block):
            r = rows[a:a + block]
            sl = slot[a:a + block]
            lo, hi = lo_r[a:a + block, None], hi_r[a:a + block, None]
            G = np.asarray(gpu_idx[r, h], dtype=np.int64)
            GS = np.asarray(gpu_score[r, h], dtype=np.float64)
            bad = np.nonzero(np.any(~sl & (G != -1), axis=1))[0]
            assert bad.size == 0, (r[bad[0]], h, "padding", G[bad[0]])
            bad = np.nonzero(np.any(~sl & ~np.isneginf(GS), axis=1))[0]
            assert bad.size == 0, (r[bad[0]], h, "pad score", GS[bad[0]])
            bad = np.nonzero(np.any(sl & ((G < lo) | (G >= hi)), axis=1))[0]
            assert bad.size == 0, (r[bad[0]], h, "out of graph", G[bad[0]])
            Gs = np.sort(np.where(sl, G, -1 - np.arange(K)[None, :]), axis=1)
            bad = np.nonzero(np.any(np.diff(Gs, axis=1) == 0, axis=1))[0]
            assert bad.size == 0, (r[bad[0]], h, "duplicates", G[bad[0]])
            qr = q[r, h, :]
            inside = np.einsum("rkc,rc->rk", kh[np.where(sl, G, 0)], qr)
            inside = np.where(sl, inside, -np.inf)
            qn = np.linalg.norm(qr, axis=1) * kmax_b[b_of[a:a + block]]
            eps, seps = coef * qn, saved_coef * qn
            both = sl[:, 1:] & sl[:, :-1]
            dif = np.diff(np.where(sl, inside, 0.0), axis=1)
            bad = np.nonzero(np.any(both & (dif > 2 * eps[:, None]), axis=1))[0]
            assert bad.size == 0, (r[bad[0]], h, "order", inside[bad[0]])
            with np.errstate(invalid="ignore"):
                err = np.where(sl, np.abs(GS - inside), 0.0)
            bad = np.nonzero(np.any(err > seps[:, None] + 1e-30, axis=1))[0]
            assert bad.size == 0, (r[bad[0]], h, "score", err[bad[0]], seps[bad[0]])
            if not split:
                # Equal saved scores are equal scan scores: ascending ids.  The
                # fp32 entry point orders by its split-precision scan scores
                # but saves rescored fp32 values, which may tie where the
                # scan's did not; its tie rule is checked on inputs with
                # duplicate keys instead (tests/test_gpu_f32.py).
                tie = both & (np.diff(np.where(sl, GS, 0.0), axis=1) == 0)
                bad = np.nonzero(np.any(tie & (np.diff(G, axis=1) <= 0), axis=1))[0]
                assert bad.size == 0, (r[bad[0]], h, "tie order", G[bad[0]], GS[bad[0]])
            O = np.asarray(ref["idx"][a:a + block, h], dtype=np.int64)
            same = np.all(np.sort(np.where(sl, G, -1), axis=1)
                          == np.sort(np.where(sl, O, -1), axis=1), axis=1)
            stats["exact"] += int(same.sum())
            for u in np.nonzero(~same)[0]:
                i = int(r[u])
                glo, ghi = int(lo[u, 0]), int(hi[u, 0])
                s = kh[glo:ghi] @ q[i, h, :]
                nb, kk = ghi - glo, int(kk_r[a + u])
                loc = G[u, :kk] - glo
                mask = np.ones(nb, dtype=bool)
                mask[loc] = False
                outside_max = s[mask].max() if mask.any() else -np.inf
                if kk < nb:
                    part = np.partition(s, [nb - kk - 1, nb - kk])
                    s_k, s_k1 = part[nb - kk], part[nb - kk - 1]
                else:
                    s_k, s_k1 = s.min(), -np.inf
                delta = (band_rel * max(abs(s_k), abs(s_k1) if np.isfinite(s_k1) else 0.0)
                         + 2 * eps[u])
                assert s[loc].min() >= outside_max - delta, (
                    i, h, "selection", s[loc].min(), outside_max, delta)
                stats["in_band"] += 1
            stats["rows"] += int(r.size)
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
