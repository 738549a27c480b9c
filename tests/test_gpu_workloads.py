"""GPU parity on the full-size workloads.

Every row, forward and backward, where the oracle can afford it:
  * N = 4096 (i.i.d.), N = 31623 and the 64-graph batch: every row forward;
  * the training workload (N = 10^5, k = 15) and the 64-graph batch: every
    row forward, and dq, dk, dv on every row against the oracle's backward
    on the GPU's own selection; both also repeated bitwise;
  * the fp32 entry points on the float32 draws of those two workloads: the
    same;
  * N = 10^5 with k in {5, 15, 45} and N = 5 * 10^5: 8192 seeded query nodes
    x all heads, each scored by the oracle against every key of the graph.
The oracle's selection runs over row blocks in a pool of host processes
(oracle/pool.py); its fixed-set steps are vectorised over rows.
"""
import numpy as np
import pytest

import oracle.kmip_oracle as orc
from tests.parity import BAND_REL, assert_rows_close, check_selection, decode
from workloads import get_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SAMPLE_NODES = 8192


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sample_rows(n, m, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(n, size=min(m, n), replace=False)
    return np.unique(np.concatenate([[0, n - 1], rows]))


def _forward(name, nrows, dtype="bf16"):
    from tests.gpu_util import np_, run_forward
    w = get_workload(name, dtype=dtype)
    print(f"[workload] {name} {dtype} n={w.n} H={w.heads} d={w.d} k={w.topk} "
          f"B={w.num_graphs}", flush=True)
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    rows = np.arange(w.n) if nrows is None else _sample_rows(w.n, nrows, w.meta["seed"])
    idx_n, score_n = np_(idx), np_(score)
    # fp32 inputs: the selection is checked at the split scores' own accuracy
    f32 = dtype == "f32"
    st = check_selection(idx_n, score_n, q, k, w.offsets, w.topk, rows, v=v,
                         band_rel=0.0 if f32 else BAND_REL, split=f32)
    assert st["rows"] == rows.size * w.heads
    ref = orc.attend_on_sets(q, k, v, idx_n[rows].astype(np.int64), rows=rows)
    assert_rows_close(np_(out)[rows], ref["out"], "out")
    print(f"[workload] {name} {dtype} rows checked {st}", flush=True)
    return w, t, out, idx, score, (q, k, v)


def _backward(w, t, idx, score, qkv):
    """dq, dk and dv on every row against the oracle's backward on the GPU's
    own selection; keys no query selected must be exact zeros."""
    from tests.gpu_util import np_, run_backward
    dq, dk, dv = (np_(x) for x in run_backward(w, t, idx, score))
    q, k, v = qkv
    idx_n = np_(idx).astype(np.int64)
    rq, rk, rv = orc.kmip_backward_on_sets(q, k, v, idx_n, w.dout.astype(np.float64))
    e = {n: assert_rows_close(x, r, n) for n, x, r in (("dq", dq, rq), ("dk", dk, rk),
                                                       ("dv", dv, rv))}
    for h in range(w.heads):
        sel = idx_n[:, h, :].ravel()
        deg = np.bincount(sel[sel >= 0], minlength=w.n)
        unselected = deg == 0
        assert not dk[unselected, h].any() and not dv[unselected, h].any()
        print(f"[workload] {w.name} head {h}: max in-degree {deg.max()}, "
              f"unselected keys {int(unselected.sum())}", flush=True)
    print(f"[workload] {w.name} backward row errors {e}", flush=True)
    return dq, dk, dv


def _repeat_bitwise(w, t, first, grads):
    """A second forward and backward on the same inputs give identical bits."""
    from tests.gpu_util import np_, run_backward, run_forward
    _, out, idx, score = run_forward(w, t)
    for name, a, b in (("out", first[0], out), ("idx", first[1], idx),
                       ("score", first[2], score)):
        assert np.array_equal(np_(a), np_(b)), name
    for name, a, b in zip(("dq", "dk", "dv"), grads,
                          run_backward(w, t, first[1], first[2])):
        assert np.array_equal(a, np_(b)), name


def test_iid_n4096_all_rows():
    _forward("iid_n4096_h1_d64_k15", None)


def test_clustered_n31623_all_rows():
    _forward("clustered_n31623_h4_d32_k15", None)


@pytest.mark.parametrize("k", [5, 15, 45])
def test_clustered_n100000_k_sweep(k):
    _forward(f"clustered_n100000_h4_d32_k{k}", SAMPLE_NODES)


def test_train_clustered_n100000_all_rows():
    w, t, out, idx, score, qkv = _forward("train_clustered_n100000_h4_d32_k15", None)
    grads = _backward(w, t, idx, score, qkv)
    _repeat_bitwise(w, t, (out, idx, score), grads)


def test_ragged64_all_rows():
    w, t, out, idx, score, qkv = _forward("ragged64_h4_d32_k15", None)
    grads = _backward(w, t, idx, score, qkv)
    _repeat_bitwise(w, t, (out, idx, score), grads)


@pytest.mark.parametrize("name", ["train_clustered_n100000_h4_d32_k15", "ragged64_h4_d32_k15"])
def test_f32_entry_points_full_size_all_rows(name):
    """The fp32 entry points on the float32 draws of the training and batched
    workloads (the bench's --precision fp32 runs)."""
    w, t, out, idx, score, qkv = _forward(name, None, dtype="f32")
    _backward(w, t, idx, score, qkv)


def test_pointcloud_n500000_linear_memory():
    from tests.gpu_util import np_, to_device
    from graph_transformer_sparse_amd import kmip
    w = get_workload("pointcloud_n500000_h4_d32_k15")
    print(f"[workload] {w.name} n={w.n}", flush=True)
    t = to_device(w)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    out, idx, score = kmip.forward(t["q"], t["k"], t["v"], w.topk, t["offsets"])
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    outputs = out.numel() * 4 + idx.numel() * 4 + score.numel() * 4
    ws = kmip.forward_workspace_bytes(w.n, w.heads, w.d, w.topk, w.num_graphs)
    # O(N * H * k): outputs plus workspace plus allocator rounding; one fp32
    # N x N score matrix per head would be 1 TB.
    assert peak <= outputs + ws + (64 << 20), (peak, outputs, ws)
    q, k, v = decode(w)
    rows = _sample_rows(w.n, SAMPLE_NODES, 6)
    idx_n, score_n = np_(idx), np_(score)
    st = check_selection(idx_n, score_n, q, k, w.offsets, w.topk, rows, v=v)
    assert st["rows"] == rows.size * w.heads
    ref = orc.attend_on_sets(q, k, v, idx_n[rows].astype(np.int64), rows=rows)
    assert_rows_close(np_(out)[rows], ref["out"], "out")
    print(f"[workload] {w.name} rows checked {st}", flush=True)
