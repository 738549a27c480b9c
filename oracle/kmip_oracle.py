"""Plain fp64 CPU oracle for k-Maximum-Inner-Product (k-MIP) attention.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
cpu_baseline leg import this module.  The GPU library never calls it, and
the two share no code: this file decodes, scores, selects and reduces on
its own with NumPy.

What it computes follows the page "k-Maximum Inner Product Attention for
Graph Transformers and the Expressive Power of GraphGPS" (De Schouwer,
Saez de Ocariz Borde, Dong), Abstract: for every query node the key nodes
with the k largest inner products <q_i, k_j> are selected by a top-k
operation, a softmax is taken over those k scores, and the output is the
softmax-weighted sum of the selected value rows.  The selection is exact, so
the oracle is that definition written out, in fp64, row block by row block
(never more than a block of scores is alive at once).

Readings where the page is silent (each is listed with its reason in the
design notes of the repository):
  * scores are the unscaled inner product; ``scale`` multiplies them before
    the softmax only (a positive scale never changes the selection);
  * heads are independent (own scores, selection and softmax per head);
  * the candidate keys of a query are all nodes of its own graph, itself
    included, so k >= n_b reproduces full softmax attention over the graph
    (the dense comparator of Appendix J, Table 12);
  * ties are broken by ascending node id: the selected set is the first
    k_eff keys in the order (score descending, node id ascending);
  * k_eff = min(k, n_b); unused slots hold index -1 and score -inf;
  * gradients flow through the selected entries only; the selection itself
    is piecewise constant and carries no gradient.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------- decoding
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bfloat16 -> float64: the 16 bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def graph_ranges(offsets, n: int):
    """[(lo, hi)] per graph; ``None`` or an empty batch means one graph of n."""
    if offsets is None or len(offsets) < 2:
        return [(0, n)]
    off = np.asarray(offsets, dtype=np.int64)
    return [(int(off[b]), int(off[b + 1])) for b in range(len(off) - 1)]


# ---------------------------------------------------------------- steps
def scores_block(q_rows: np.ndarray, k_graph: np.ndarray) -> np.ndarray:
    """s[r, j] = <q_r, k_j> in fp64 for a block of query rows of one head."""
    return q_rows @ k_graph.T


def select_topk_row(s: np.ndarray, topk: int) -> np.ndarray:
    """Local ids of the first min(topk, len(s)) keys under (-score, id)."""
    n = s.shape[0]
    kk = min(topk, n)
    if kk <= 0:
        return np.zeros(0, dtype=np.int64)
    if kk < n:
        t = np.partition(s, n - kk)[n - kk]          # kk-th largest value
        cand = np.nonzero(s >= t)[0]                 # every key that can be selected
    else:
        cand = np.arange(n)
    order = np.lexsort((cand, -s[cand]))             # primary -score, then id
    return cand[order[:kk]].astype(np.int64)


def softmax_selected(s_sel: np.ndarray, scale: float) -> np.ndarray:
    """Softmax of scale * s over the last axis.  Entries of -inf are slots
    that hold no key: they get weight 0, and a row with no key at all gets
    all zeros."""
    s_sel = np.asarray(s_sel, dtype=np.float64)
    if s_sel.size == 0:
        return s_sel.copy()
    m = s_sel.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isneginf(s_sel), 0.0, np.exp(scale * (s_sel - m)))
    z = w.sum(axis=-1, keepdims=True)
    return np.divide(w, z, out=np.zeros_like(w), where=z > 0)


# ---------------------------------------------------------------- forward
def kmip_forward(q, k, v, offsets, topk: int, scale: float = 1.0, rows=None,
                 block: int = 256):
    """k-MIP attention forward.

    q, k, v: float64 [N][H][d].  offsets: [B+1] graph offsets or None.
    rows: optional node ids to evaluate (all nodes when None); every such row
    is still scored against all keys of its graph.

    Returns dict with idx int64 [R][H][topk] (global ids, -1 padded),
    score float64 [R][H][topk] (-inf padded), out float64 [R][H][d].
    """
    n, heads, d = q.shape
    rng = graph_ranges(offsets, n)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    graph_of = np.empty(n, dtype=np.int64)
    for b, (lo, hi) in enumerate(rng):
        graph_of[lo:hi] = b
    R = rows.shape[0]
    idx = np.full((R, heads, topk), -1, dtype=np.int64)
    score = np.full((R, heads, topk), NEG_INF, dtype=np.float64)
    out = np.zeros((R, heads, d), dtype=np.float64)
    rg = graph_of[rows] if R else np.zeros(0, dtype=np.int64)
    for b, (lo, hi) in enumerate(rng):
        sel_pos = np.nonzero(rg == b)[0]
        if sel_pos.size == 0 or hi <= lo:
            continue
        for h in range(heads):
            kg = k[lo:hi, h, :]
            vg = v[lo:hi, h, :]
            for start in range(0, sel_pos.size, block):
                pos = sel_pos[start:start + block]
                s = scores_block(q[rows[pos], h, :], kg)
                for r, p in enumerate(pos):
                    loc = select_topk_row(s[r], topk)
                    kk = loc.size
                    ssel = s[r, loc]
                    w = softmax_selected(ssel, scale)
                    idx[p, h, :kk] = loc + lo
                    score[p, h, :kk] = ssel
                    out[p, h, :] = w @ vg[loc]
    return dict(idx=idx, score=score, out=out)


# ---------------------------------------------------------------- fixed sets
def _gather_selected(x, js, h):
    """Rows x[j, h] for a block of index rows js [R][K] (-1 slots give a
    placeholder row that the caller masks out)."""
    return x[np.where(js >= 0, js, 0), h, :]


def attend_on_sets(q, k, v, idx, rows=None, scale: float = 1.0, block: int = 8192):
    """Softmax-AV on given index sets (idx [R][H][topk], -1 = unused slot).

    Used to re-evaluate a selection produced elsewhere.  Returns dict with
    score [R][H][topk] (fp64 inner products, -inf on unused slots),
    p [R][H][topk] and out [R][H][d].
    """
    n, heads, d = q.shape
    idx = np.asarray(idx, dtype=np.int64)
    rows = np.arange(idx.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    R, _, K = idx.shape
    score = np.full((R, heads, K), NEG_INF)
    p = np.zeros((R, heads, K))
    out = np.zeros((R, heads, d))
    for h in range(heads):
        for a in range(0, R, block):
            js = idx[a:a + block, h, :]
            valid = js >= 0
            ks = _gather_selected(k, js, h)                          # [r][K][d]
            s = np.einsum("rkc,rc->rk", ks, q[rows[a:a + block], h, :])
            s = np.where(valid, s, NEG_INF)
            w = softmax_selected(s, scale)
            score[a:a + block, h] = s
            p[a:a + block, h] = w
            out[a:a + block, h] = np.einsum("rk,rkc->rc", w, _gather_selected(v, js, h))
    return dict(score=score, p=p, out=out)


def query_grads(q_rows, k_sel, v_sel, dout_rows, valid, scale: float):
    """Backward of a block of query rows with their selections fixed.

    q_rows, dout_rows [R][d]; k_sel, v_sel [R][K][d], the selected key and
    value rows (slots with valid == False hold no key).  Per row:
    s_j = q . k_j, p = softmax(scale s), dp_j = dO . v_j, D = sum_j p_j dp_j,
    ds_j = p_j (dp_j - D), dq = scale sum_j ds_j k_j.  Returns (p, ds, dq);
    p and ds are 0 on slots without a key.
    """
    s = np.where(valid, np.einsum("rkc,rc->rk", k_sel, q_rows), NEG_INF)
    p = softmax_selected(s, scale)
    dp = np.where(valid, np.einsum("rkc,rc->rk", v_sel, dout_rows), 0.0)
    # dp_j - D evaluated as (dp_j - dp_m) - sum_u p_u (dp_u - dp_m), m the
    # largest weight of the row: the same value, without the cancellation
    # that drops the small terms of p . dp when the softmax is nearly one-hot.
    m = np.argmax(p, axis=1)
    rel = np.where(valid, dp - np.take_along_axis(dp, m[:, None], axis=1), 0.0)
    ds = p * (rel - np.einsum("rk,rk->r", p, rel)[:, None])
    return p, ds, scale * np.einsum("rk,rkc->rc", ds, k_sel)


def kmip_backward_on_sets(q, k, v, idx, dout, scale: float = 1.0, rows=None,
                          block: int = 8192):
    """Gradients of L = sum(dout * out) with the selection idx held fixed.

    idx: int [R][H][topk] for the query nodes `rows` (every node when None).
    Returns dq [R][H][d] of those rows and the dk, dv contributions they make,
    [N][H][d] (with rows=None: the full gradients).  Keys selected by no
    query get exactly zero.
      dp_ij = dO_i . v_j,  D_i = sum_j p_ij dp_ij,  ds_ij = p_ij (dp_ij - D_i)
      dQ_i = scale sum_j ds_ij k_j,  dK_j = scale sum_i ds_ij q_i,
      dV_j = sum_i p_ij dO_i
    """
    n, heads, d = q.shape
    idx = np.asarray(idx, dtype=np.int64)
    rows = np.arange(idx.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    dq = np.zeros((R, heads, d))
    dk = np.zeros((n, heads, d))
    dv = np.zeros((n, heads, d))
    for h in range(heads):
        for a in range(0, R, block):
            js = idx[a:a + block, h, :]
            valid = js >= 0
            qr = q[rows[a:a + block], h, :]
            gr = dout[rows[a:a + block], h, :]
            p, ds, dq[a:a + block, h] = query_grads(qr, _gather_selected(k, js, h),
                                                    _gather_selected(v, js, h), gr, valid,
                                                    scale)
            r_of, t_of = np.nonzero(valid)
            np.add.at(dk[:, h, :], js[r_of, t_of], scale * ds[r_of, t_of, None] * qr[r_of])
            np.add.at(dv[:, h, :], js[r_of, t_of], p[r_of, t_of, None] * gr[r_of])
    return dq, dk, dv
