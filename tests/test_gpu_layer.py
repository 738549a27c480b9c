"""The autograd wrapper and the multi-head k-MIP layer on the GPU, against
fp64 references built from the oracle (attention on the GPU's own index sets,
so legitimate tie-band swaps are not counted as error)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle.kmip_oracle as orc
from tests.parity import assert_rows_close

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from graph_transformer_sparse_amd.layer import (GPSLayer, KMIPMultiheadAttention,  # noqa: E402
                                                kmip_attention)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16_round(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).to(torch.float64)


def _np(x):
    return x.detach().cpu().numpy()


@pytest.mark.parametrize("sizes,topk", [([700], 15), ([300, 1, 250], 8), ([500], 40)])
def test_autograd_function_matches_oracle(sizes, topk):
    g = torch.Generator().manual_seed(sum(sizes) + topk)
    n, heads, d = sum(sizes), 2, 32
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    q, k, v, G = (torch.randn((n, heads, d), generator=g) for _ in range(4))
    qg, kg, vg = (x.cuda().requires_grad_(True) for x in (q, k, v))
    go = torch.from_numpy(offs).cuda() if len(sizes) > 1 else None
    out, idx = kmip_attention(qg, kg, vg, topk, go)
    (out * G.cuda()).sum().backward()

    qr, kr, vr = (_np(_bf16_round(x)) for x in (q, k, v))
    sets = _np(idx).astype(np.int64)
    ref = orc.attend_on_sets(qr, kr, vr, sets)
    assert_rows_close(_np(out), ref["out"], "out")
    dq, dk, dv = orc.kmip_backward_on_sets(qr, kr, vr, sets, _np(G).astype(np.float64))
    assert_rows_close(_np(qg.grad), dq, "dq")
    assert_rows_close(_np(kg.grad), dk, "dk")
    assert_rows_close(_np(vg.grad), dv, "dv")


def _reference_layer(layer: KMIPMultiheadAttention, x: torch.Tensor, idx: np.ndarray):
    """The same layer in fp64 on the CPU: projections in torch, bf16 rounding
    of q, k, v with the gradient passed straight through (as the GPU's cast
    does), attention on the given index sets."""
    p = {n: t.detach().cpu().double().requires_grad_(True) for n, t in layer.named_parameters()}
    xd = x.detach().cpu().double()
    N, H, d = x.shape[0], layer.heads, layer.head_dim

    def proj(name):
        return xd @ p[f"{name}.weight"].T + p[f"{name}.bias"]

    def st_round(t):
        return t + (_bf16_round(t) - t).detach()

    q = st_round(proj("q_proj") * layer.scale).view(N, H, d)
    k = st_round(proj("k_proj")).view(N, H, d)
    v = st_round(proj("v_proj")).view(N, H, d)
    sel = torch.from_numpy(idx.astype(np.int64))               # [N, H, K], -1 padding
    valid = sel >= 0
    sc = sel.clamp(min=0)
    hh = torch.arange(H).view(1, H, 1).expand_as(sc)
    ksel, vsel = k[sc, hh], v[sc, hh]                          # [N, H, K, d]
    s = (q.unsqueeze(2) * ksel).sum(-1).masked_fill(~valid, float("-inf"))
    pr = torch.softmax(s, dim=-1)
    att = (pr.unsqueeze(-1) * vsel).sum(2).reshape(N, H * d)
    y = att @ p["out_proj.weight"].T + p["out_proj.bias"]
    return y, p


def test_multihead_layer_matches_fp64_reference():
    torch.manual_seed(7)
    N, C = 600, 48
    layer = KMIPMultiheadAttention(C, heads=4, head_dim=32, topk=15).cuda()
    x = torch.randn(N, C).cuda()
    y = layer(x)
    W = torch.randn(N, C).cuda()
    (y * W).sum().backward()
    idx = _np(layer.last_topk_idx)
    yr, p = _reference_layer(layer, x, idx)
    (yr * W.cpu().double()).sum().backward()
    assert_rows_close(_np(y), _np(yr), "layer output")
    for name, t in layer.named_parameters():
        g, gr = _np(t.grad).astype(np.float64), _np(p[name].grad)
        # The key bias shifts every score of a row equally, so its gradient is
        # exactly zero (the sum of dk over keys vanishes): measure errors on
        # the scale of the module's weight gradient.
        wscale = np.abs(_np(p[name.rsplit(".", 1)[0] + ".weight"].grad)).max()
        err = np.abs(g - gr).max() / max(np.abs(gr).max(), wscale)
        assert err <= 2e-3, (name, err)


def test_gps_layer_trains_one_step():
    torch.manual_seed(3)
    sizes = [300, 200, 100]
    offs = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32).cuda()
    N, C = sum(sizes), 64
    layer = GPSLayer(C, heads=2, head_dim=32, topk=8).cuda()
    opt = torch.optim.SGD(layer.parameters(), lr=1e-2)
    x = torch.randn(N, C).cuda()
    target = torch.randn(N, C).cuda()
    losses = []
    for _ in range(3):
        opt.zero_grad()
        loss = ((layer(x, offs) - target) ** 2).mean()
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    assert all(np.isfinite(losses))
    assert all(p.grad is not None and torch.isfinite(p.grad).all() for p in layer.parameters())
    idx = _np(layer.attn.last_topk_idx)
    lo = np.repeat(offs.cpu().numpy()[:-1], sizes)[:, None, None]
    hi = np.repeat(offs.cpu().numpy()[1:], sizes)[:, None, None]
    assert ((idx >= lo) & (idx < hi)).all()                   # keys stay inside the graph


def test_autograd_function_fp32_precision():
    """precision="fp32": the fp32 entry points, checked against the oracle on
    the unrounded values."""
    g = torch.Generator().manual_seed(11)
    n, heads, d, topk = 600, 2, 64, 15
    q, k, v, G = (torch.randn((n, heads, d), generator=g) for _ in range(4))
    qg, kg, vg = (x.cuda().requires_grad_(True) for x in (q, k, v))
    out, idx = kmip_attention(qg, kg, vg, topk, None, precision="fp32")
    (out * G.cuda()).sum().backward()
    qr, kr, vr = (_np(x).astype(np.float64) for x in (q, k, v))
    sets = _np(idx).astype(np.int64)
    ref = orc.attend_on_sets(qr, kr, vr, sets)
    assert_rows_close(_np(out), ref["out"], "out")
    dq, dk, dv = orc.kmip_backward_on_sets(qr, kr, vr, sets, _np(G).astype(np.float64))
    assert_rows_close(_np(qg.grad), dq, "dq")
    assert_rows_close(_np(kg.grad), dk, "dk")
    assert_rows_close(_np(vg.grad), dv, "dv")
