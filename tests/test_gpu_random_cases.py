"""Seeded random cases against the fp64 oracle: sizes, ragged batches, k,
d, input laws and the fp32 entry points drawn at random (every row, forward
and backward).  Complements the hand-picked cases with combinations nobody
chose, such as tight clusters with long lists or graphs smaller than k."""
import numpy as np
import pytest

import oracle.kmip_oracle as orc
from tests.parity import assert_rows_close, check_selection, decode
from workloads import make_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _draw(case):
    rng = np.random.default_rng(910_000 + case)
    d = int(rng.choice([32, 64]))
    heads = int(rng.choice([1, 2, 3, 4, 8]))
    topk = int(rng.choice([1, 3, 5, 8, 15, 16, 17, 32, 45, 64]))
    law = str(rng.choice(["iid", "clustered"]))
    dtype = str(rng.choice(["bf16", "bf16", "f32"]))
    clusters = int(rng.choice([4, 16, 64]))
    sigma = float(rng.choice([0.05, 0.3, 1.0]))
    if rng.random() < 0.5:
        kw = dict(n=int(rng.integers(1, 1200)))
    else:
        lo = int(rng.integers(1, 200))
        kw = dict(graph_sizes=(lo, lo + int(rng.integers(0, 500))),
                  num_graphs=int(rng.integers(2, 10)))
    return make_workload(f"random_{case}", heads=heads, d=d, topk=topk, law=law,
                         clusters=clusters if law == "clustered" else 0, sigma=sigma,
                         backward=True, seed=int(rng.integers(1 << 30)), dtype=dtype, **kw)


@pytest.mark.parametrize("case", range(40))
def test_random_case(case):
    from tests.gpu_util import np_, run_backward, run_forward
    w = _draw(case)
    print(f"[case] random {case}: n={w.n} B={w.num_graphs} H={w.heads} d={w.d} k={w.topk} "
          f"{w.meta['law']} C={w.meta['clusters']} sigma={w.meta['sigma']} {w.dtype}", flush=True)
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    idx_n = np_(idx)
    split = dict(band_rel=0.0, split=True) if w.dtype == "f32" else {}
    check_selection(idx_n, np_(score), q, k, w.offsets, w.topk, range(w.n), **split)
    ref = orc.attend_on_sets(q, k, v, idx_n.astype(np.int64))
    assert_rows_close(np_(out), ref["out"], "out")
    dq, dk, dv = run_backward(w, t, idx, score)
    rq, rk, rv = orc.kmip_backward_on_sets(q, k, v, idx_n.astype(np.int64),
                                           w.dout.astype(np.float64))
    assert_rows_close(np_(dq), rq, "dq")
    assert_rows_close(np_(dk), rk, "dk")
    assert_rows_close(np_(dv), rv, "dv")


def _draw_pruned(case):
    """One graph of 2^16 .. 2 * 10^5 nodes (the pruned selection's range):
    clustered inputs of random tightness and cluster count (some ranges
    stream, some query blocks split), or i.i.d. inputs (everything streams),
    with short and long lists."""
    rng = np.random.default_rng(930_000 + case)
    d = int(rng.choice([32, 64]))
    heads = int(rng.choice([1, 2, 4]))
    topk = int(rng.choice([1, 5, 8, 15, 16, 17, 32, 45, 64]))
    law = str(rng.choice(["clustered", "clustered", "clustered", "iid"]))
    clusters = int(rng.choice([16, 64, 256, 1024]))
    sigma = float(rng.choice([0.05, 0.3, 1.0]))
    n = int(rng.integers(1 << 16, 200_000))
    seed = int(rng.integers(1 << 30))
    # fp32 inputs at d = 32 prune on their 96-wide split rows
    dtype = "f32" if d == 32 and rng.random() < 0.3 else "bf16"
    return make_workload(f"random_pruned_{case}", n=n, heads=heads, d=d, topk=topk, law=law,
                         clusters=clusters if law == "clustered" else 0, sigma=sigma,
                         backward=True, seed=seed, dtype=dtype)


@pytest.mark.parametrize("case", range(24))
def test_random_case_pruned(case):
    """The pruned path on random shapes (bf16 rows, and fp32 inputs on their
    split rows): selection and output on 2048 seeded nodes x all heads, and
    dq on those rows, against the oracle."""
    from tests.gpu_util import np_, run_backward, run_forward
    w = _draw_pruned(case)
    print(f"[case] random pruned {case}: n={w.n} H={w.heads} d={w.d} k={w.topk} "
          f"{w.meta['law']} C={w.meta['clusters']} sigma={w.meta['sigma']} {w.dtype}", flush=True)
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    idx_n = np_(idx)
    rows = np.unique(np.concatenate(
        [[0, w.n - 1], np.random.default_rng(case).choice(w.n, 2048, replace=False)]))
    split = dict(band_rel=0.0, split=True) if w.dtype == "f32" else {}
    check_selection(idx_n, np_(score), q, k, w.offsets, w.topk, rows, **split)
    ref = orc.attend_on_sets(q, k, v, idx_n[rows].astype(np.int64), rows=rows)
    assert_rows_close(np_(out)[rows], ref["out"], "out")
    dq, _, _ = run_backward(w, t, idx, score)
    rq, _, _ = orc.kmip_backward_on_sets(q, k, v, idx_n[rows].astype(np.int64),
                                         w.dout.astype(np.float64), rows=rows)
    assert_rows_close(np_(dq)[rows], rq, "dq")
