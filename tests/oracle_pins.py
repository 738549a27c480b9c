"""Pins that tie the fp64 oracle to facts fixed outside of it.

Each pin raises AssertionError when the oracle disagrees with:
  * a hand-worked closed-form example (tests/golden/hand_3nodes.json);
  * brute-force enumeration of every k-subset, in pure Python;
  * full softmax attention (torch's scaled_dot_product_attention in fp64,
    forward and autograd backward) when k >= n_b: the dense comparator of
    Appendix J, Table 12 of "k-Maximum Inner Product Attention for Graph
    Transformers ...", which k-MIP reduces to when every key is kept;
  * k = 1 (the argmax value row, zero dQ and dK);
  * permutation equivariance of graph layers, f(PH) = P f(H) (page "Graph
    Neural Networks (GNNs) ...", section 1, Architectural Foundations);
  * softmax rows summing to one; shifting every key by one vector;
  * exact fp64 scores of bf16 inputs (math.fsum of exact products);
  * gradient identities and an fp64 autograd re-derivation of the backward
    with the selection frozen, plus central finite differences;
  * linearity in V and block-diagonal batching.

The functions take the oracle module as an argument so that the mutation
tests can run them against oracles with planted mistakes.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _bf16_round(x):
    """Round float values to bf16-representable float64 values (RNE)."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ golden
def pin_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "hand_3nodes.json")))
    a = math.e / (math.e + 1.0)
    b = 1.0 / (math.e + 1.0)
    env = {"__builtins__": {}, "a": a, "b": b}

    def ev(m):
        return np.array([[eval(c, env) for c in row] for row in m], dtype=np.float64)

    q = np.array(g["q"], dtype=np.float64)[:, None, :]
    k = np.array(g["k"], dtype=np.float64)[:, None, :]
    v = np.array(g["v"], dtype=np.float64)[:, None, :]
    do = np.array(g["dout"], dtype=np.float64)[:, None, :]
    fw = orc.kmip_forward(q, k, v, None, g["topk"])
    assert np.array_equal(fw["idx"][:, 0, :], np.array(g["expect_idx"])), fw["idx"]
    assert np.allclose(fw["score"][:, 0, :], np.array(g["expect_score"]), atol=0, rtol=0)
    assert np.allclose(fw["out"][:, 0, :], ev(g["expect_out"]), atol=1e-14, rtol=0)
    dq, dk, dv = orc.kmip_backward_on_sets(q, k, v, fw["idx"], do)
    assert np.allclose(dq[:, 0, :], ev(g["expect_dq"]), atol=1e-14, rtol=0)
    assert np.allclose(dk[:, 0, :], ev(g["expect_dk"]), atol=1e-14, rtol=0)
    assert np.allclose(dv[:, 0, :], ev(g["expect_dv"]), atol=1e-14, rtol=0)


# ------------------------------------------------------------------ brute force
def _brute_row(qi, keys, vals, topk, scale):
    """Pure-Python enumeration of every subset of size min(topk, n)."""
    n = len(keys)
    kk = min(topk, n)
    s = [math.fsum(a * b for a, b in zip(qi, kj)) for kj in keys]
    winners = []
    for S in itertools.combinations(range(n), kk):
        inside = min(s[j] for j in S)
        outside = max((s[j] for j in range(n) if j not in S), default=-math.inf)
        if inside >= outside:
            winners.append(S)
    assert len(winners) == 1, "brute force expects distinct scores"
    S = sorted(winners[0], key=lambda j: (-s[j], j))
    m = max(s[j] for j in S)
    w = [math.exp(scale * (s[j] - m)) for j in S]
    Z = math.fsum(w)
    out = [math.fsum(w[t] * vals[S[t]][c] for t in range(kk)) / Z for c in range(len(vals[0]))]
    return S, out


def pin_bruteforce(orc, seed=11):
    rng = _rng(seed)
    for (sizes, heads, d, topk, scale) in [((7,), 2, 3, 1, 1.0), ((7,), 2, 3, 2, 1.0),
                                           ((8,), 1, 4, 3, 0.5), ((4, 6), 2, 3, 2, 1.0),
                                           ((3, 5), 1, 2, 4, 1.0)]:
        n = int(sum(sizes))
        offs = np.concatenate([[0], np.cumsum(sizes)])
        q = rng.standard_normal((n, heads, d))
        k = rng.standard_normal((n, heads, d))
        v = rng.standard_normal((n, heads, d))
        fw = orc.kmip_forward(q, k, v, offs, topk, scale=scale)
        for b in range(len(sizes)):
            lo, hi = int(offs[b]), int(offs[b + 1])
            for i in range(lo, hi):
                for h in range(heads):
                    keys = [list(k[j, h]) for j in range(lo, hi)]
                    vals = [list(v[j, h]) for j in range(lo, hi)]
                    S, out = _brute_row(list(q[i, h]), keys, vals, topk, scale)
                    kk = len(S)
                    got = list(fw["idx"][i, h, :kk] - lo)
                    assert got == S, (i, h, got, S)
                    assert all(fw["idx"][i, h, kk:] == -1)
                    assert np.allclose(fw["out"][i, h], out, atol=1e-12, rtol=0)


# ------------------------------------------------------------------ full attention
def _sdpa_graphs(q, k, v, offs, scale, dout=None):
    import torch
    import torch.nn.functional as F
    n, heads, d = q.shape
    out = np.zeros_like(q)
    grads = [np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)]
    for b in range(len(offs) - 1):
        lo, hi = int(offs[b]), int(offs[b + 1])
        tq = torch.tensor(q[lo:hi].transpose(1, 0, 2).copy(), dtype=torch.float64,
                          requires_grad=True)
        tk = torch.tensor(k[lo:hi].transpose(1, 0, 2).copy(), dtype=torch.float64,
                          requires_grad=True)
        tv = torch.tensor(v[lo:hi].transpose(1, 0, 2).copy(), dtype=torch.float64,
                          requires_grad=True)
        o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], scale=scale)[0]
        out[lo:hi] = o.detach().numpy().transpose(1, 0, 2)
        if dout is not None:
            td = torch.tensor(dout[lo:hi].transpose(1, 0, 2).copy(), dtype=torch.float64)
            (o * td).sum().backward()
            for g, t in zip(grads, (tq, tk, tv)):
                g[lo:hi] = t.grad.numpy().transpose(1, 0, 2)
    return out, grads


def pin_full_attention(orc, seed=12):
    rng = _rng(seed)
    for (sizes, heads, d, topk, scale) in [((9,), 2, 4, 9, 1.0), ((5, 7, 1), 2, 3, 16, 1.0),
                                           ((6, 4), 1, 8, 6, 0.37)]:
        n = int(sum(sizes))
        offs = np.concatenate([[0], np.cumsum(sizes)])
        q = rng.standard_normal((n, heads, d))
        k = rng.standard_normal((n, heads, d))
        v = rng.standard_normal((n, heads, d))
        do = rng.standard_normal((n, heads, d))
        fw = orc.kmip_forward(q, k, v, offs, topk, scale=scale)
        ref, (gq, gk, gv) = _sdpa_graphs(q, k, v, offs, scale, dout=do)
        assert np.allclose(fw["out"], ref, atol=1e-12, rtol=1e-12)
        dq, dk, dv = orc.kmip_backward_on_sets(q, k, v, fw["idx"], do, scale=scale)
        assert np.allclose(dq, gq, atol=1e-12, rtol=1e-10)
        assert np.allclose(dk, gk, atol=1e-12, rtol=1e-10)
        assert np.allclose(dv, gv, atol=1e-12, rtol=1e-10)


# ------------------------------------------------------------------ k = 1
def pin_k1(orc, seed=13):
    rng = _rng(seed)
    n, heads, d = 40, 3, 5
    offs = np.array([0, 17, 40])
    q, k, v, do = (rng.standard_normal((n, heads, d)) for _ in range(4))
    fw = orc.kmip_forward(q, k, v, offs, 1)
    dv_ref = np.zeros_like(v)
    for b in range(2):
        lo, hi = offs[b], offs[b + 1]
        for h in range(heads):
            s = q[lo:hi, h] @ k[lo:hi, h].T
            am = np.argmax(s, axis=1) + lo
            assert np.array_equal(fw["idx"][lo:hi, h, 0], am)
            assert np.array_equal(fw["out"][lo:hi, h], v[am, h])
            for i, j in zip(range(lo, hi), am):
                dv_ref[j, h] += do[i, h]
    dq, dk, dv = orc.kmip_backward_on_sets(q, k, v, fw["idx"], do)
    assert not dq.any() and not dk.any()
    assert np.allclose(dv, dv_ref, atol=1e-14, rtol=0)


# ------------------------------------------------------------------ equivariance
def pin_permutation(orc, seed=14):
    rng = _rng(seed)
    sizes = (13, 21)
    n, heads, d, topk = 34, 2, 6, 4
    offs = np.array([0, 13, 34])
    q, k, v = (rng.standard_normal((n, heads, d)) for _ in range(3))
    perm = np.concatenate([rng.permutation(13), 13 + rng.permutation(21)])
    fw = orc.kmip_forward(q, k, v, offs, topk)
    fp = orc.kmip_forward(q[perm], k[perm], v[perm], offs, topk)
    assert np.allclose(fp["out"], fw["out"][perm], atol=1e-13, rtol=0)
    # selected sets map through the permutation (scores are continuous: no ties)
    for i in range(n):
        for h in range(heads):
            a = set(perm[fp["idx"][i, h]].tolist())
            b = set(fw["idx"][perm[i], h].tolist())
            assert a == b
    assert sizes == (13, 21)


# ------------------------------------------------------------------ softmax rows
def pin_softmax_rows(orc, seed=15):
    rng = _rng(seed)
    n, heads, d, topk = 50, 2, 8, 7
    q, k, v = (rng.standard_normal((n, heads, d)) * 3 for _ in range(3))
    fw = orc.kmip_forward(q, k, v, None, topk)
    ev = orc.attend_on_sets(q, k, v, fw["idx"])
    p = ev["p"]
    assert np.all(p >= 0)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-14, rtol=0)
    assert np.all(np.diff(p, axis=-1) <= 1e-15)
    assert np.allclose(ev["out"], fw["out"], atol=1e-12, rtol=0)
    assert np.all(np.diff(fw["score"], axis=-1) <= 0)


# ------------------------------------------------------------------ key shift
def pin_key_shift(orc, seed=16):
    rng = _rng(seed)
    n, heads, d, topk = 45, 2, 6, 5
    q, k, v = (rng.standard_normal((n, heads, d)) for _ in range(3))
    c = rng.standard_normal((1, heads, d))
    fw = orc.kmip_forward(q, k, v, None, topk)
    fs = orc.kmip_forward(q, k + c, v, None, topk)
    assert np.array_equal(fw["idx"], fs["idx"])
    assert np.allclose(fw["out"], fs["out"], atol=1e-12, rtol=0)


# ------------------------------------------------------------------ score exactness
def pin_score_exact(orc, seed=17):
    """Scores of bf16 inputs equal math.fsum of the exact products; and the
    bit decoding matches float(bits << 16) read as an fp32."""
    import struct
    rng = _rng(seed)
    n, heads, d = 30, 2, 32
    bits = [((_bf16_round(rng.standard_normal((n, heads, d))).astype(np.float32)
              .view(np.uint32) >> 16).astype(np.uint16)) for _ in range(2)]
    q = orc.bf16_bits_to_f64(bits[0])
    k = orc.bf16_bits_to_f64(bits[1])
    for _ in range(20):
        i, j, h = rng.integers(n), rng.integers(n), rng.integers(heads)
        qi = [struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in bits[0][i, h]]
        kj = [struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in bits[1][j, h]]
        assert list(q[i, h]) == qi
        exact = math.fsum(a * b for a, b in zip(qi, kj))
        s = orc.scores_block(q[i:i + 1, h, :], k[j:j + 1, h, :])[0, 0]
        assert abs(s - exact) <= 1e-15 * math.fsum(abs(a * b) for a, b in zip(qi, kj))


# ------------------------------------------------------------------ gradients
def pin_grad_identities(orc, seed=18):
    rng = _rng(seed)
    n, heads, d, topk = 60, 2, 5, 6
    offs = np.array([0, 25, 60])
    q, k, v, do = (rng.standard_normal((n, heads, d)) for _ in range(4))
    fw = orc.kmip_forward(q, k, v, offs, topk)
    dq, dk, dv = orc.kmip_backward_on_sets(q, k, v, fw["idx"], do)
    for b in range(2):
        lo, hi = offs[b], offs[b + 1]
        assert np.allclose(dv[lo:hi].sum(0), do[lo:hi].sum(0), atol=1e-12, rtol=0)
        assert np.allclose(dk[lo:hi].sum(0), 0.0, atol=1e-12)
    unselected = np.setdiff1d(np.arange(n), np.unique(fw["idx"][:, 0, :]))
    assert unselected.size > 0
    assert not dk[unselected, 0].any() and not dv[unselected, 0].any()


def _torch_fixed_selection(q, k, v, idx, do, scale):
    """fp64 torch autograd of gather -> softmax -> weighted sum on fixed sets."""
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    n, heads, d = q.shape
    ix = torch.tensor(np.where(idx < 0, 0, idx), dtype=torch.long)      # [N][H][K]
    valid = torch.tensor(idx >= 0)
    hsel = torch.arange(heads)[None, :, None].expand_as(ix)
    ks = tk[ix, hsel]                                                   # [N][H][K][d]
    vs = tv[ix, hsel]
    s = (ks * tq[:, :, None, :]).sum(-1) * scale
    s = s.masked_fill(~valid, float("-inf"))
    p = torch.softmax(s, dim=-1)
    out = (p[..., None] * vs).sum(-2)
    (out * torch.tensor(do)).sum().backward()
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_backward_autograd(orc, seed=19):
    rng = _rng(seed)
    for (sizes, heads, d, topk, scale) in [((40,), 2, 6, 5, 1.0), ((9, 30, 2), 3, 4, 7, 0.6)]:
        n = int(sum(sizes))
        offs = np.concatenate([[0], np.cumsum(sizes)])
        q, k, v, do = (rng.standard_normal((n, heads, d)) for _ in range(4))
        fw = orc.kmip_forward(q, k, v, offs, topk, scale=scale)
        out, gq, gk, gv = _torch_fixed_selection(q, k, v, fw["idx"], do, scale)
        assert np.allclose(fw["out"], out, atol=1e-13, rtol=0)
        dq, dk, dv = orc.kmip_backward_on_sets(q, k, v, fw["idx"], do, scale=scale)
        assert np.allclose(dq, gq, atol=1e-12, rtol=0)
        assert np.allclose(dk, gk, atol=1e-12, rtol=0)
        assert np.allclose(dv, gv, atol=1e-12, rtol=0)
        # row-subset contributions add up to the full backward
        half = np.arange(n) % 2 == 0
        parts = [orc.kmip_backward_on_sets(q, k, v, fw["idx"][m], do, scale=scale,
                                           rows=np.nonzero(m)[0])
                 for m in (half, ~half)]
        assert np.allclose(parts[0][1] + parts[1][1], dk, atol=1e-13, rtol=0)
        assert np.allclose(parts[0][2] + parts[1][2], dv, atol=1e-13, rtol=0)
        assert np.allclose(parts[0][0], dq[half], atol=1e-13, rtol=0)
        assert np.allclose(parts[1][0], dq[~half], atol=1e-13, rtol=0)


def pin_finite_difference(orc, seed=20):
    """Central differences of L = sum(dO * out) with the selection frozen."""
    rng = _rng(seed)
    n, heads, d, topk = 12, 1, 3, 3
    q, k, v, do = (rng.standard_normal((n, heads, d)) for _ in range(4))
    fw = orc.kmip_forward(q, k, v, None, topk)
    idx = fw["idx"]
    dq, dk, dv = orc.kmip_backward_on_sets(q, k, v, idx, do)

    def loss(qq, kk, vv):
        return float((orc.attend_on_sets(qq, kk, vv, idx)["out"] * do).sum())

    h = 1e-6
    for arr, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for _ in range(6):
            i, c = rng.integers(n), rng.integers(d)
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][i, 0, c] += h
            args_m[which][i, 0, c] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[i, 0, c]) <= 1e-6 * max(1.0, abs(fd)), (which, i, c, fd, g[i, 0, c])


def pin_peaked_softmax_grads(orc, seed=23):
    """A selection whose best score leads the rest by ~30 (softmax one-hot to
    ~1e-14): dq against the definition evaluated in 60-digit decimal
    arithmetic, per-row relative 1e-9.  The gradient is ~1e-14 of its
    inputs here, so an evaluation that cancels in fp64 fails this pin."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    rng = _rng(seed)
    for gap in (30.0, 36.0):
        kk, d = 6, 4
        q = rng.standard_normal((kk + 1, 1, d))
        k = rng.standard_normal((kk + 1, 1, d))
        v = rng.standard_normal((kk + 1, 1, d))
        do = rng.standard_normal((kk + 1, 1, d))
        # key 0 scores gap above the others for query 0
        k[0, 0] = q[0, 0] * (gap / float(q[0, 0] @ q[0, 0]))
        idx = np.full((kk + 1, 1, kk), -1, dtype=np.int64)
        idx[0, 0] = np.arange(kk)
        dq, _, _ = orc.kmip_backward_on_sets(q, k, v, idx, do)
        D = lambda x: Decimal(repr(float(x)))
        s = [sum(D(k[j, 0, c]) * D(q[0, 0, c]) for c in range(d)) for j in range(kk)]
        smax = max(s)
        e = [(x - smax).exp() for x in s]
        z = sum(e)
        p = [x / z for x in e]
        dp = [sum(D(v[j, 0, c]) * D(do[0, 0, c]) for c in range(d)) for j in range(kk)]
        Dm = sum(pj * dpj for pj, dpj in zip(p, dp))
        ds = [pj * (dpj - Dm) for pj, dpj in zip(p, dp)]
        ref = np.array([float(sum(ds[j] * D(k[j, 0, c]) for j in range(kk))) for c in range(d)])
        assert np.max(np.abs(ref)) < 1e-9                       # the row is one-hot to ~1e-13
        err = np.max(np.abs(dq[0, 0] - ref)) / np.max(np.abs(ref))
        assert err <= 1e-9, (gap, err, dq[0, 0], ref)


# ------------------------------------------------------------------ linearity, batching
def pin_linearity(orc, seed=21):
    rng = _rng(seed)
    n, heads, d, topk = 30, 2, 4, 5
    q, k, v = (rng.standard_normal((n, heads, d)) for _ in range(3))
    fw = orc.kmip_forward(q, k, v, None, topk)
    f2 = orc.kmip_forward(q, k, 2.5 * v, None, topk)
    assert np.allclose(f2["out"], 2.5 * fw["out"], atol=1e-13, rtol=0)
    vc = np.broadcast_to(rng.standard_normal((1, heads, d)), v.shape).copy()
    fc = orc.kmip_forward(q, k, vc, None, topk)
    assert np.allclose(fc["out"], vc, atol=1e-14, rtol=0)


def pin_block_diagonal(orc, seed=22):
    rng = _rng(seed)
    sizes = (11, 3, 17)
    n, heads, d, topk = 31, 2, 4, 5
    offs = np.concatenate([[0], np.cumsum(sizes)])
    q, k, v = (rng.standard_normal((n, heads, d)) for _ in range(3))
    fb = orc.kmip_forward(q, k, v, offs, topk)
    for b in range(3):
        lo, hi = offs[b], offs[b + 1]
        fs = orc.kmip_forward(q[lo:hi], k[lo:hi], v[lo:hi], None, topk)
        sel = fs["idx"]
        assert np.array_equal(fb["idx"][lo:hi], np.where(sel >= 0, sel + lo, -1))
        assert np.array_equal(fb["out"][lo:hi], fs["out"])


ALL_PINS = [pin_golden, pin_bruteforce, pin_full_attention, pin_k1, pin_permutation,
            pin_softmax_rows, pin_key_shift, pin_score_exact, pin_grad_identities,
            pin_backward_autograd, pin_finite_difference, pin_peaked_softmax_grads,
            pin_linearity, pin_block_diagonal]
