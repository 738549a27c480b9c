"""The parity checker accepts the oracle's own results and rejects planted
errors (CPU only)."""
import numpy as np
import pytest

import oracle.kmip_oracle as orc
from tests.parity import check_selection, row_rel_err
from workloads import small_case, with_offsets


def _case():
    w = with_offsets("chk", [40, 7, 1, 60], heads=2, d=32, topk=9, law="iid", seed=5)
    q, k, v = (orc.bf16_bits_to_f64(x) for x in (w.q, w.k, w.v))
    fw = orc.kmip_forward(q, k, v, w.offsets, w.topk)
    idx = fw["idx"].astype(np.int32)
    score = fw["score"].astype(np.float32)
    return w, q, k, v, idx, score


def test_accepts_oracle():
    w, q, k, v, idx, score = _case()
    st = check_selection(idx, score, q, k, w.offsets, w.topk, range(w.n))
    assert st["rows"] == w.n * w.heads and st["in_band"] == 0


@pytest.mark.parametrize("mutation", ["swap_far", "duplicate", "padding", "order", "score"])
def test_rejects(mutation):
    w, q, k, v, idx, score = _case()
    idx = idx.copy()
    score = score.copy()
    i, h = 5, 1                         # a node of the first graph (40 nodes)
    if mutation == "swap_far":
        s = k[0:40, h] @ q[i, h]
        worst = int(np.argmin(s))
        idx[i, h, 3] = worst
        score[i, h, 3] = s[worst]
        order = np.argsort(-score[i, h, :9], kind="stable")
        idx[i, h, :9] = idx[i, h, order]
        score[i, h, :9] = score[i, h, order]
    elif mutation == "duplicate":
        idx[i, h, 4] = idx[i, h, 3]
    elif mutation == "padding":
        j = 41                          # node of the second graph (7 nodes, k=9)
        idx[j, 0, 8] = 40
    elif mutation == "order":
        idx[i, h, [0, 8]] = idx[i, h, [8, 0]]
        score[i, h, [0, 8]] = score[i, h, [8, 0]]
    elif mutation == "score":
        score[i, h, 2] *= 1.01
    with pytest.raises(AssertionError):
        check_selection(idx, score, q, k, w.offsets, w.topk, range(w.n))


def test_row_error():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((10, 2, 32))
    ref[3, 1] = 0.0
    x = ref.copy()
    assert row_rel_err(x, ref) == 0.0
    x[2, 0, 5] += 3e-3 * np.abs(ref[2, 0]).max()
    assert row_rel_err(x, ref) > 2e-3
    x = ref.copy()
    x[3, 1, 0] = 1e-30
    assert row_rel_err(x, ref) == np.inf


def test_small_case_generator_is_deterministic():
    a = small_case(100, 2, 32, 5, seed=3)
    b = small_case(100, 2, 32, 5, seed=3)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.dout, b.dout)


def test_accepts_swap_inside_tie_band():
    """A set that trades the k-th key for the (k+1)-th when their scores are
    within the band is accepted and counted as in-band; the same trade with
    the band closed is rejected."""
    w, q, k, v, idx, score = _case()
    idx, score = idx.copy(), score.copy()
    i, h = 5, 1
    s = k[0:40, h] @ q[i, h]
    order = np.lexsort((np.arange(40), -s))
    kth, nxt = order[8], order[9]
    k2 = k.copy()
    k2[nxt, h] = k[kth, h] + 1e-7 * (k[nxt, h] - k[kth, h])   # (k+1)-th just below k-th
    s2 = k2[0:40, h] @ q[i, h]
    assert 0 < s2[kth] - s2[nxt] < 1e-5
    idx[i, h, 8] = nxt
    score[i, h, 8] = s2[nxt]
    st = check_selection(idx, score, q, k2, w.offsets, w.topk, [i], heads=[h])
    assert st["in_band"] == 1
    with pytest.raises(AssertionError):
        _closed_band(idx, score, q, k2, w, i, h)


def _closed_band(idx, score, q, k, w, i, h):
    # zero relative band and a per-score error bound scaled to nothing
    import tests.parity as par
    saved = par.eps_coef
    par.eps_coef = lambda d, split=False: 0.0
    try:
        par.check_selection(idx, score, q, k, w.offsets, w.topk, [i], heads=[h], band_rel=0.0)
    finally:
        par.eps_coef = saved


def test_pool_matches_in_process_oracle():
    """The worker pool runs the same oracle function over row blocks."""
    from oracle.pool import forward_rows
    w = with_offsets("pool", [300, 5, 1, 420], heads=3, d=32, topk=7, law="clustered",
                     clusters=6, seed=8)
    q, k, v = (orc.bf16_bits_to_f64(x) for x in (w.q, w.k, w.v))
    rows = np.array([0, 3, 299, 300, 305, 306, 500, 725])
    a = orc.kmip_forward(q, k, v, w.offsets, w.topk, rows=rows)
    b = forward_rows(q, k, v, w.offsets, w.topk, rows, workers=2, block=3)
    for key in ("idx", "score", "out"):
        assert np.array_equal(a[key], b[key]), key
