"""GPU parity of the fp32 entry points (kmip_forward_f32 / kmip_backward_f32)
against the fp64 oracle evaluated on the same fp32 values.

The scan scores a three-term bf16 split of the fp32 inputs, so the selection
is checked at the scores' own accuracy: no relative tie band, only twice the
split's per-score error bound (tests/parity.py, eps_coef(split=True)).
"""
import numpy as np
import pytest

import oracle.kmip_oracle as orc
from tests.parity import assert_rows_close, check_selection, decode
from workloads import make_workload, small_case, with_offsets

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _forward_check(w, rows=None):
    from tests.gpu_util import np_, run_forward
    print(f"[case f32] {w.name} n={w.n} H={w.heads} d={w.d} k={w.topk} B={w.num_graphs}",
          flush=True)
    assert w.dtype == "f32"
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    idx_n, score_n, out_n = np_(idx), np_(score), np_(out)
    rows = range(w.n) if rows is None else rows
    st = check_selection(idx_n, score_n, q, k, w.offsets, w.topk, rows, band_rel=0.0,
                         split=True)
    rows = np.asarray(list(rows))
    ref = orc.attend_on_sets(q, k, v, idx_n[rows].astype(np.int64), rows=rows)
    assert_rows_close(out_n[rows], ref["out"], "out")
    return t, out, idx, score, st


def _backward_check(w, t, idx, score):
    from tests.gpu_util import np_, run_backward
    dq, dk, dv = run_backward(w, t, idx, score)
    q, k, v = decode(w)
    rq, rk, rv = orc.kmip_backward_on_sets(q, k, v, np_(idx).astype(np.int64),
                                           w.dout.astype(np.float64))
    assert_rows_close(np_(dq), rq, "dq")
    assert_rows_close(np_(dk), rk, "dk")
    assert_rows_close(np_(dv), rv, "dv")


@pytest.mark.parametrize("n,heads,d,topk", [
    (300, 2, 32, 15), (97, 1, 32, 15), (1000, 1, 64, 15), (517, 3, 64, 5),
    (33, 2, 32, 32), (260, 1, 32, 1), (130, 2, 32, 64), (400, 2, 64, 45),
])
def test_f32_single_graph_forward_backward(n, heads, d, topk):
    w = small_case(n, heads, d, topk, seed=3000 + n, dtype="f32")
    t, out, idx, score, st = _forward_check(w)
    _backward_check(w, t, idx, score)


@pytest.mark.parametrize("sizes,topk", [
    ([1, 3, 10, 17, 130, 257], 15),
    ([5, 0, 200, 1, 64, 0, 129], 8),
    ([2, 40, 3], 64),
    ([700, 50, 400], 45),
])
def test_f32_ragged_graphs(sizes, topk):
    w = with_offsets(f"f32_ragged_{len(sizes)}_{topk}", sizes, heads=2, d=32, topk=topk,
                     seed=sum(sizes) + topk + 1, dtype="f32")
    t, out, idx, score, st = _forward_check(w)
    _backward_check(w, t, idx, score)


@pytest.mark.parametrize("n,heads,d", [(16384, 2, 32), (8192, 4, 64)])
def test_f32_query_order_path(n, heads, d):
    """N*H >= 32768 takes the one-graph path with query grouping (the code
    is taken from the split rows' leading elements); sampled rows."""
    w = small_case(n, heads, d, 15, law="clustered", clusters=32, seed=n + d, dtype="f32")
    rows = np.random.default_rng(1).choice(n, size=600, replace=False)
    t, out, idx, score, st = _forward_check(w, rows=rows)
    assert st["rows"] == 600 * heads


def test_f32_batched_clustered_all_rows():
    """Batched graphs of a few thousand nodes, four heads, fp32 inputs
    (split-precision rows of width 96); every row, forward and backward."""
    w = with_offsets("f32_clustered_batch", [3000, 2500, 1, 3500], heads=4, d=32, topk=15,
                     law="clustered", clusters=40, seed=77, dtype="f32")
    t, out, idx, score, st = _forward_check(w)
    _backward_check(w, t, idx, score)


def test_f32_exact_ties_follow_ascending_id():
    from tests.gpu_util import np_, run_forward
    w = small_case(256, 2, 32, 6, seed=31, dtype="f32")
    w.k = np.ascontiguousarray(w.k[np.arange(256) % 8])   # 8 distinct keys, 32 copies each
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    fw = orc.kmip_forward(q, k, v, None, w.topk)
    assert np.array_equal(np_(idx), fw["idx"].astype(np.int32))


def test_f32_resolves_what_bf16_rounding_cannot():
    """Clustered queries and keys put many key scores within bf16 rounding of
    the k-th score.  On the same fp32 draws, the fp32 entry point selects the
    fp64 oracle's set in (nearly) every row, while rounding the inputs to bf16
    first changes the set in a visible fraction of rows."""
    from tests.gpu_util import np_, run_forward
    kw = dict(n=4096, heads=2, d=32, topk=15, law="clustered", clusters=4, sigma=0.05, seed=99)
    w32 = make_workload("near_ties_f32", dtype="f32", **kw)
    wbf = make_workload("near_ties_bf16", **kw)
    q, k, v = decode(w32)
    fw = orc.kmip_forward(q, k, v, None, kw["topk"])
    ref = np.sort(fw["idx"], axis=-1)
    _, _, i32, _ = run_forward(w32)
    _, _, ibf, _ = run_forward(wbf)
    same32 = (np.sort(np_(i32), axis=-1) == ref).all(-1).mean()
    samebf = (np.sort(np_(ibf), axis=-1) == ref).all(-1).mean()
    print(f"rows with the oracle's set: fp32 path {same32:.4f}, bf16-rounded {samebf:.4f}")
    assert same32 >= 0.995
    assert samebf < same32


@pytest.mark.parametrize("topk", [15, 45])
def test_f32_deterministic_repeat_pruned(topk):
    """2^16 nodes in fp32: the pruned selection over split rows (ball bounds
    through the high parts), whose heavy query blocks are listed through an
    atomic counter; k = 45 collects candidates from the pruned key blocks.
    Two calls give identical outputs and gradients, and the selection of a
    sample of rows matches the oracle."""
    from tests.gpu_util import np_, run_backward, run_forward, to_device
    w = small_case(65536, 2, 32, topk, law="clustered", clusters=64, seed=58, dtype="f32")
    print(f"[case f32] repeat {w.name} n={w.n} H={w.heads} k={w.topk}", flush=True)
    t = to_device(w)
    a = run_forward(w, t)
    b = run_forward(w, t)
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(np_(x), np_(y))
    ga = run_backward(w, t, a[2], a[3])
    gb = run_backward(w, t, a[2], a[3])
    for x, y in zip(ga, gb):
        assert np.array_equal(np_(x), np_(y))
    q, k, v = decode(w)
    rows = np.sort(np.random.default_rng(58).choice(w.n, 512, replace=False))
    check_selection(np_(a[2]), np_(a[3]), q, k, w.offsets, w.topk, rows, band_rel=0.0,
                    split=True)
