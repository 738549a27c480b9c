"""A captured k-MIP forward + backward (HIP-graph replay) against the fp64
oracle, and bit-identical to eager calls, with new inputs copied in and eager
work in between the replays."""
from __future__ import annotations

import numpy as np
import pytest

from workloads import small_case, with_offsets

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from graph_transformer_sparse_amd import kmip  # noqa: E402
from graph_transformer_sparse_amd.captured import CapturedKmip  # noqa: E402
import oracle.kmip_oracle as orc  # noqa: E402
from tests.gpu_util import bf16_tensor, np_  # noqa: E402
from tests.parity import assert_rows_close, check_selection, decode  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("sizes,topk", [([300], 15), ([100, 50, 200], 8), ([400], 32),
                                        ([16400], 15)])
def test_replays_match_eager(sizes, topk):
    heads, d = 2, 32
    base = with_offsets(f"cap_{len(sizes)}_{topk}", sizes, heads=heads, d=d, topk=topk,
                        law="clustered", clusters=8, seed=91 + topk)
    offs = torch.from_numpy(base.offsets).cuda() if base.num_graphs > 1 else None
    cap = CapturedKmip(base.n, heads, d, topk, offs, backward=True)
    for r in range(3):
        w = with_offsets(f"cap_{r}", sizes, heads=heads, d=d, topk=topk, law="clustered",
                         clusters=8, seed=500 + 7 * r + topk)
        q, k, v = (bf16_tensor(x) for x in (w.q, w.k, w.v))
        dout = torch.from_numpy(w.dout).cuda()
        for dst, src in ((cap.q, q), (cap.k, k), (cap.v, v), (cap.dout, dout)):
            dst.copy_(src)
        cap.replay()
        out, idx, score = kmip.forward(q, k, v, topk, offs)            # eager, same stream
        dq, dk, dv = kmip.backward(q, k, v, topk, idx, score, dout, offs)
        torch.cuda.synchronize()
        for a, b in ((cap.out, out), (cap.topk_idx, idx), (cap.topk_score, score),
                     (cap.dq, dq), (cap.dk, dk), (cap.dv, dv)):
            assert torch.equal(a, b), r
        # the replay's own results against the oracle
        qf, kf, vf = decode(w)
        ci = np_(cap.topk_idx)
        check_selection(ci, np_(cap.topk_score), qf, kf, w.offsets, topk, range(w.n))
        sets = ci.astype(np.int64)
        assert_rows_close(np_(cap.out), orc.attend_on_sets(qf, kf, vf, sets)["out"], "out")
        rq, rk, rv = orc.kmip_backward_on_sets(qf, kf, vf, sets, w.dout.astype(np.float64))
        for name, x, ref in (("dq", cap.dq, rq), ("dk", cap.dk, rk), ("dv", cap.dv, rv)):
            assert_rows_close(np_(x), ref, name)
