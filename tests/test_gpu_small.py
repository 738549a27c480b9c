"""GPU parity on small seeded cases: every row against the fp64 oracle.

Sizes span several 128-query tiles and 32-key MFMA blocks with ragged tails,
every instantiated list length, d in {32, 64}, tiny and empty graphs,
graphs smaller than k, exact score ties, and the backward pass.
"""
import numpy as np
import pytest

import oracle.kmip_oracle as orc
from tests.parity import assert_rows_close, check_selection, decode
from workloads import small_case, with_offsets

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _forward_check(w, rows=None):
    from tests.gpu_util import np_, run_forward
    print(f"[case] {w.name} n={w.n} H={w.heads} d={w.d} k={w.topk} B={w.num_graphs}", flush=True)
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    idx_n, score_n, out_n = np_(idx), np_(score), np_(out)
    rows = range(w.n) if rows is None else rows
    st = check_selection(idx_n, score_n, q, k, w.offsets, w.topk, rows)
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
    return dq, dk, dv


@pytest.mark.parametrize("n,heads,d,topk", [
    (300, 2, 32, 15), (97, 1, 32, 15), (1000, 1, 64, 15), (517, 3, 64, 5),
    (33, 2, 32, 32), (260, 1, 32, 1), (130, 2, 32, 64),
])
def test_single_graph_forward_backward(n, heads, d, topk):
    w = small_case(n, heads, d, topk, seed=1000 + n)
    t, out, idx, score, st = _forward_check(w)
    _backward_check(w, t, idx, score)


@pytest.mark.parametrize("n,heads,law", [(300, 128, "clustered"), (20, 1664, "clustered"),
                                         (20, 1664, "iid")])
def test_query_order_with_few_nodes_per_head(n, heads, law):
    """N*H >= 32768 groups each head's queries by nearest pivot even when the
    head has few nodes: 32 pivots at node stride N/32 (300 nodes), or pivots
    clamped to the last node when N < 32 (20 nodes, repeated pivots).  With 8
    clusters over 20 nodes, nodes alone in their cluster have a self score
    ~30 above the rest: a softmax one-hot to ~1e-14 and gradients of that
    size, which the backward must still get to the row tolerance."""
    w = small_case(n, heads, 32, 15, law=law, clusters=8 if law == "clustered" else 0,
                   seed=77 + n)
    t, out, idx, score, st = _forward_check(w)
    assert st["rows"] == n * heads
    _backward_check(w, t, idx, score)


@pytest.mark.parametrize("n,heads,d,topk", [(8192, 4, 64, 15), (16384, 2, 32, 8),
                                          (12000, 3, 64, 45)])
def test_query_order_path_all_rows(n, heads, d, topk):
    """One graph with N*H >= 32768 (pivot query order) for bf16 rows of both
    widths and a long list: every query row against the oracle, then dq, dk
    and dv on every row."""
    w = small_case(n, heads, d, topk, law="clustered", clusters=48, seed=n + d + topk)
    t, out, idx, score, st = _forward_check(w)
    assert st["rows"] == n * heads
    _backward_check(w, t, idx, score)


@pytest.mark.parametrize("seed", [4242, 4243])
def test_extreme_softmax_ranges(seed):
    """Tight clusters in 64 dimensions: a node's own key scores ~80 above the
    rest of its selection, so those weights are ~e^-80 (below fp32's normal
    range) and some gradient rows are ~1e-36, or cancelling sums of tiny
    terms.  The backward recomputes the selected scores and their weights in
    fp64, which keeps such rows to 1e-4: the fp32 rounding of the per-pair
    (p, ds) carried to the key side.  Weights from the forward's fp32 scores
    measured 2e-4 on dk here."""
    from tests.gpu_util import np_, run_backward
    w = with_offsets(f"extreme_{seed}", list(np.random.default_rng(seed).integers(147, 276, 9)),
                     heads=3, d=64, topk=17, law="clustered", clusters=64, sigma=0.05,
                     seed=seed)
    t, out, idx, score, st = _forward_check(w)
    dq, dk, dv = run_backward(w, t, idx, score)
    q, k, v = decode(w)
    rq, rk, rv = orc.kmip_backward_on_sets(q, k, v, np_(idx).astype(np.int64),
                                           w.dout.astype(np.float64))
    for name, x, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert_rows_close(np_(x), ref, name, tol=1e-4)


@pytest.mark.parametrize("topk", [1, 2, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 45, 48, 63, 64])
def test_every_list_length(topk):
    w = small_case(400, 2, 32, topk, seed=2000 + topk)
    _forward_check(w)


def test_clustered_structure():
    w = small_case(3000, 4, 32, 15, law="clustered", clusters=16, seed=77)
    t, out, idx, score, st = _forward_check(w)
    _backward_check(w, t, idx, score)


@pytest.mark.parametrize("sizes,topk", [
    ([1, 3, 10, 17, 130, 257], 15),
    ([5, 0, 200, 1, 64, 0, 129], 8),
    ([2, 40, 3], 64),
    ([128, 128, 1], 15),
    ([700], 15),
])
def test_ragged_graphs(sizes, topk):
    w = with_offsets(f"ragged_{len(sizes)}_{topk}", sizes, heads=2, d=32, topk=topk,
                     law="iid", seed=sum(sizes) + topk)
    t, out, idx, score, st = _forward_check(w)
    _backward_check(w, t, idx, score)


@pytest.mark.parametrize("sizes,heads,d,topk", [
    ([3000, 1, 257, 4100, 0, 900, 2600], 4, 32, 15),
    ([2500, 5000, 900], 4, 64, 8),
    ([3000, 2200, 4000], 4, 32, 45),
])
def test_batched_clustered_all_rows(sizes, heads, d, topk):
    """Batched graphs of up to 5000 nodes, four heads, clustered rows (many
    sub-tiles per graph, partial last tiles, empty and one-node graphs),
    d = 32 and 64, short and long lists.  Every row, forward and backward."""
    w = with_offsets(f"clustered_batch_{len(sizes)}_{topk}", sizes, heads=heads, d=d,
                     topk=topk, law="clustered", clusters=48, seed=sum(sizes) + d + topk)
    t, out, idx, score, st = _forward_check(w)
    _backward_check(w, t, idx, score)


def test_single_node_graph_is_identity():
    from tests.gpu_util import np_, run_backward, run_forward
    w = with_offsets("singletons", [1, 1, 1, 1, 1], heads=2, d=64, topk=4, seed=9)
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    assert np.array_equal(np_(out), v.astype(np.float32))
    dq, dk, dv = run_backward(w, t, idx, score)
    assert not np_(dq).any() and not np_(dk).any()
    assert np.array_equal(np_(dv), w.dout)


def test_exact_ties_follow_ascending_id():
    """Duplicated key rows give bitwise-equal scores; the smaller node id wins."""
    from tests.gpu_util import np_, run_forward
    w = small_case(256, 2, 32, 6, seed=31)
    w.k = w.k[np.arange(256) % 8]                        # 8 distinct keys, 32 copies each
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    fw = orc.kmip_forward(q, k, v, None, w.topk)
    assert np.array_equal(np_(idx), fw["idx"].astype(np.int32))


@pytest.mark.parametrize("sizes,topk", [([1200], 45), ([700, 50, 400], 45), ([900], 32)])
def test_long_lists_with_overflowing_candidates(sizes, topk):
    """Lists longer than 16 go through per-row candidate arrays (128 per lane
    half).  Heavily duplicated keys tie at the k-th score, so rows whose best
    key has hundreds of copies overflow the arrays and are recomputed exactly;
    rows whose best keys are distinct do not.  Both must match the oracle,
    ties by ascending id."""
    from tests.gpu_util import np_, run_forward
    w = with_offsets(f"dup_{len(sizes)}_{topk}", sizes, heads=2, d=32, topk=topk,
                     law="iid", seed=sum(sizes) + topk)
    n = w.n
    dup = np.arange(n) < (2 * n) // 3
    w.k = w.k.copy()
    w.k[dup] = w.k[np.arange(n)[dup] % 2]                # two key rows, many copies
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    fw = orc.kmip_forward(q, k, v, w.offsets, w.topk)
    assert np.array_equal(np_(idx), fw["idx"].astype(np.int32))
    assert_rows_close(np_(out), fw["out"], "out")


def test_full_attention_limit():
    """k >= n_b: every key of the graph is kept, so the output is full softmax
    attention (oracle pinned to torch SDPA in fp64)."""
    w = with_offsets("full", [20, 33, 64], heads=2, d=32, topk=64, seed=4)
    _forward_check(w)


def _repeat(w):
    from tests.gpu_util import np_, run_backward, run_forward, to_device
    print(f"[case] repeat {w.name} n={w.n} H={w.heads} k={w.topk} B={w.num_graphs}", flush=True)
    t = to_device(w)
    a = run_forward(w, t)
    b = run_forward(w, t)
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(np_(x), np_(y))
    ga = run_backward(w, t, a[2], a[3])
    gb = run_backward(w, t, a[2], a[3])
    for x, y in zip(ga, gb):
        assert np.array_equal(np_(x), np_(y))


def test_deterministic_repeat():
    """Below the query-order threshold (N*H < 32768): node-order sub-tiles."""
    _repeat(small_case(2000, 4, 32, 15, law="clustered", clusters=8, seed=5))


@pytest.mark.parametrize("topk", [15, 45])
def test_deterministic_repeat_query_order(topk):
    """N*H >= 32768: the pivot query order, whose placement uses atomic
    counters, so the order inside a pivot group can change between calls;
    results must not."""
    _repeat(small_case(12288, 4, 32, topk, law="clustered", clusters=24, seed=55 + topk))


@pytest.mark.parametrize("topk", [15, 45])
def test_deterministic_repeat_pruned(topk):
    """2^16 nodes: the pruned selection, whose heavy query blocks are listed
    through an atomic counter (their order, and where their parts' lists
    go, change between calls); k = 45 collects candidates from the pruned
    key blocks.  Results must not change."""
    _repeat(small_case(65536, 2, 32, topk, law="clustered", clusters=64, seed=57))


def test_deterministic_repeat_batched():
    """Batched graphs: the ragged tile plan and 8-wavefront sub-tiles."""
    sizes = list(np.random.default_rng(56).integers(1, 2600, 23))
    _repeat(with_offsets("repeat_batched", sizes, heads=4, d=32, topk=15, law="clustered",
                         clusters=32, seed=57))


def test_gradient_identities_on_gpu_outputs():
    from tests.gpu_util import np_, run_backward, run_forward
    w = with_offsets("ident", [500, 300], heads=2, d=32, topk=15, seed=6)
    t, out, idx, score = run_forward(w)
    dq, dk, dv = (np_(x).astype(np.float64) for x in run_backward(w, t, idx, score))
    for lo, hi in orc.graph_ranges(w.offsets, w.n):
        sdo = w.dout[lo:hi].astype(np.float64).sum(0)
        assert np.allclose(dv[lo:hi].sum(0), sdo, atol=1e-3 * np.abs(sdo).max() + 1e-4)
        assert np.abs(dk[lo:hi].sum(0)).max() <= 1e-3 * np.abs(dk[lo:hi]).sum(0).max() + 1e-5


def _sample(n, m, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=m, replace=False)]))


@pytest.mark.parametrize("topk", [15, 45])
def test_exact_ties_on_the_pruned_path(topk):
    """One graph of 2^16 nodes (the pruned selection: keys scored in the
    query order, out of node order): 97 distinct key rows, each repeated
    ~676 times, give bitwise-equal scores, and the smaller node id must still
    win every tie, in the oracle's order, on 4096 sampled rows.  At k = 45
    the tied candidates overflow the rows' arrays, and the rank passes
    recompute those rows."""
    from tests.gpu_util import np_, run_forward
    from tests.parity import oracle_forward
    n = 65536
    w = small_case(n, 1, 32, topk, law="clustered", clusters=48, seed=131, backward=False)
    w.k = w.k[np.arange(n) % 97]
    print(f"[case] ties n={w.n} H={w.heads} d={w.d} k={w.topk}", flush=True)
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    rows = _sample(n, 4096, 5)
    ref = oracle_forward(q, k, v, None, w.topk, rows)
    assert np.array_equal(np_(idx)[rows], ref["idx"].astype(np.int32))


@pytest.mark.parametrize("d,topk", [(32, 8), (64, 8), (32, 45)])
def test_pruned_and_streaming_query_blocks_mixed(d, topk):
    """One graph of 2^16 nodes, half of them in tight clusters, half i.i.d.:
    the clustered query blocks' key blocks are mostly ruled out by their
    bounds, the i.i.d. ones (whose bounds leave most key blocks live) become
    heavy blocks split over several wavefronts; 4096 sampled rows against the
    oracle, forward and backward."""
    from workloads import f32_to_bf16_bits
    n, heads = 65536, 1
    w = small_case(n, heads, d, topk, law="clustered", clusters=32, seed=171 + d)
    rng = np.random.default_rng(5 + d)
    half = n // 2
    for name in ("q", "k"):
        x = getattr(w, name).copy()
        x[half:] = f32_to_bf16_bits(rng.standard_normal((n - half, heads, d), dtype=np.float32) * 1.4)
        setattr(w, name, x)
    rows = _sample(n, 4096, 7 + d)
    t, out, idx, score, st = _forward_check(w, rows=rows)
    assert st["rows"] == rows.size * heads
    from tests.gpu_util import np_, run_backward
    dq, dk, dv = run_backward(w, t, idx, score)
    q, k, v = decode(w)
    rq, _, _ = orc.kmip_backward_on_sets(q, k, v, np_(idx)[rows].astype(np.int64),
                                         w.dout.astype(np.float64), rows=rows)
    assert_rows_close(np_(dq)[rows], rq, "dq")


@pytest.mark.parametrize("topk", [15, 45])
def test_pruned_path_streams_inputs_without_cluster_structure(topk):
    """One graph of 2^16 i.i.d. nodes: nearly every key block stays live, so
    the range goes to the streaming pass; 2048 sampled rows against the
    oracle."""
    w = small_case(65536, 1, 32, topk, law="iid", seed=191, backward=False)
    rows = _sample(65536, 2048, 9)
    _forward_check(w, rows=rows)
