"""GPU parity on the full-size benchmark workloads, on sampled rows.

Each sampled query row is still scored by the oracle against every key of its
graph; sampled keys for dk / dv sum over every query that selected them in
the GPU's own selection.  The sample always includes the first and last
node, the highest in-degree keys (hubs) and unselected keys (exact zeros).
"""
import numpy as np
import pytest

import oracle.kmip_oracle as orc
from tests.parity import BAND_REL, assert_rows_close, check_selection, decode
from workloads import get_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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
    print(f"[workload] {name} n={w.n} H={w.heads} d={w.d} k={w.topk} B={w.num_graphs}",
          flush=True)
    t, out, idx, score = run_forward(w)
    q, k, v = decode(w)
    rows = np.arange(w.n) if nrows is None else _sample_rows(w.n, nrows, w.meta["seed"])
    idx_n, score_n = np_(idx), np_(score)
    # fp32 inputs: the selection is checked at the split scores' own accuracy
    f32 = dtype == "f32"
    st = check_selection(idx_n, score_n, q, k, w.offsets, w.topk, rows,
                         band_rel=0.0 if f32 else BAND_REL, split=f32)
    ref = orc.attend_on_sets(q, k, v, idx_n[rows].astype(np.int64), rows=rows)
    assert_rows_close(np_(out)[rows], ref["out"], "out")
    print(f"[workload] {name} selection {st}", flush=True)
    return w, t, out, idx, score, (q, k, v), rows


def _backward(w, t, idx, score, qkv, rows, nkeys=48):
    from tests.gpu_util import np_, run_backward
    dq, dk, dv = (np_(x) for x in run_backward(w, t, idx, score))
    q, k, v = qkv
    idx_n = np_(idx).astype(np.int64)
    dout = w.dout.astype(np.float64)
    ref_dq = orc.dq_rows_on_sets(q, k, v, idx_n, dout, rows)
    assert_rows_close(dq[rows], ref_dq, "dq")
    for h in range(w.heads):
        sel = idx_n[:, h, :].ravel()
        deg = np.bincount(sel[sel >= 0], minlength=w.n)
        hubs = np.argsort(-deg, kind="stable")[:8]
        unselected = np.nonzero(deg == 0)[0][:8]
        rng = np.random.default_rng(h)
        picked = rng.choice(np.nonzero(deg > 0)[0], size=nkeys, replace=False)
        keys = np.unique(np.concatenate([hubs, unselected, picked]))
        rk, rv = orc.dkv_keys_on_sets(q, k, v, idx_n, dout, keys)
        assert_rows_close(dk[keys, h], rk[:, h], f"dk head {h}")
        assert_rows_close(dv[keys, h], rv[:, h], f"dv head {h}")
        assert not dk[unselected, h].any() and not dv[unselected, h].any()
        print(f"[workload] {w.name} head {h}: max in-degree {deg.max()}", flush=True)


def test_iid_n4096_all_rows():
    _forward("iid_n4096_h1_d64_k15", None)


def test_clustered_n31623():
    _forward("clustered_n31623_h4_d32_k15", 384)


@pytest.mark.parametrize("k", [5, 15, 45])
def test_clustered_n100000_k_sweep(k):
    _forward(f"clustered_n100000_h4_d32_k{k}", 192)


def test_train_clustered_n100000():
    w, t, out, idx, score, qkv, rows = _forward("train_clustered_n100000_h4_d32_k15", 192)
    _backward(w, t, idx, score, qkv, rows)


def test_ragged64():
    w, t, out, idx, score, qkv, rows = _forward("ragged64_h4_d32_k15", 1024)
    _backward(w, t, idx, score, qkv, rows)


@pytest.mark.parametrize("name,nrows", [("train_clustered_n100000_h4_d32_k15", 192),
                                        ("ragged64_h4_d32_k15", 512)])
def test_f32_entry_points_full_size(name, nrows):
    """The fp32 entry points on the float32 draws of the training and batched
    workloads (the bench's --precision fp32 runs)."""
    w, t, out, idx, score, qkv, rows = _forward(name, nrows, dtype="f32")
    _backward(w, t, idx, score, qkv, rows)


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
    rows = _sample_rows(w.n, 96, 6)
    idx_n, score_n = np_(idx), np_(score)
    check_selection(idx_n, score_n, q, k, w.offsets, w.topk, rows)
    ref = orc.attend_on_sets(q, k, v, idx_n[rows].astype(np.int64), rows=rows)
    assert_rows_close(np_(out)[rows], ref["out"], "out")
