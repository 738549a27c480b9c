"""kmip_forward_no_workspace (the library's per-GPU scratch array instead of a
caller workspace) against kmip_forward through the C ABI: two calls in a row,
the second with a smaller input and a different scratch layout, each equal
bit for bit to kmip_forward on the same inputs and within the oracle's
parity bar."""
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


def _call_both(w):
    from graph_transformer_sparse_amd import kmip
    from tests.gpu_util import to_device
    print(f"[case] no-workspace {w.name} n={w.n} H={w.heads} k={w.topk} B={w.num_graphs}",
          flush=True)
    t = to_device(w)
    a = kmip.forward(t["q"], t["k"], t["v"], w.topk, t["offsets"])
    b = kmip.forward_no_workspace(t["q"], t["k"], t["v"], w.topk, t["offsets"])
    torch.cuda.synchronize()
    return a, b


def _check(w, a, b):
    from tests.gpu_util import np_
    for name, x, y in zip(("out", "topk_idx", "topk_score"), a, b):
        assert np.array_equal(np_(x), np_(y)), name
    q, k, v = decode(w)
    idx = np_(b[1])
    check_selection(idx, np_(b[2]), q, k, w.offsets, w.topk, range(w.n), v=v)
    ref = orc.attend_on_sets(q, k, v, idx.astype(np.int64))
    assert_rows_close(np_(b[0]), ref["out"], "out")


def test_no_workspace_forward_matches_forward():
    from graph_transformer_sparse_amd import kmip
    # one graph on the pivot query order path (thresholds, order, counters)
    big = small_case(12288, 4, 32, 15, law="clustered", clusters=24, seed=71, backward=False)
    # then a smaller batch of graphs (thresholds and the ragged tile plan)
    small = with_offsets("noalloc_batched", [700, 1, 40, 1300, 9], heads=2, d=64, topk=8,
                         law="clustered", clusters=8, seed=72, backward=False)
    # (kmip_forward takes the pruned selection on the first case, whose
    # buffers the entry point without a workspace leaves out: the two paths
    # must still agree bit for bit)
    for w in (big, small):
        a, b = _call_both(w)
        _check(w, a, b)
    # a long list (per-row candidate arrays in the scratch), then the big case again
    longl = small_case(1500, 2, 32, 45, law="clustered", clusters=8, seed=73, backward=False)
    for w in (longl, big):
        a, b = _call_both(w)
        _check(w, a, b)


def test_no_workspace_forward_refuses_sizes_beyond_the_scratch():
    from graph_transformer_sparse_amd import kmip
    q = torch.zeros((100000, 4, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kmip.KmipError) as e:
        kmip.forward_no_workspace(q, q, q, 45)
    assert e.value.status == 3
