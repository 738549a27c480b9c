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
    """Softmax over the selected scores (a 1-D array, best first)."""
    if s_sel.size == 0:
        return s_sel.copy()
    m = s_sel.max()
    w = np.exp(scale * (s_sel - m))
    return w / w.sum()


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
def attend_on_sets(q, k, v, idx, rows=None, scale: float = 1.0):
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
    for r in range(R):
        i = rows[r]
        for h in range(heads):
            sel = idx[r, h]
            valid = sel >= 0
            js = sel[valid]
            if js.size == 0:
                continue
            s = k[js, h, :] @ q[i, h, :]
            w = softmax_selected(s, scale)
            score[r, h, valid] = s
            p[r, h, valid] = w
            out[r, h, :] = w @ v[js, h, :]
    return dict(score=score, p=p, out=out)


def query_grads(q_i, k_sel, v_sel, dout_i, scale: float):
    """Per-query backward with the selection fixed.

    k_sel, v_sel: the selected key / value rows (best first).  Returns
    (p, ds, dq_i):  p = softmax(scale s), dp_j = dO_i . v_j,
    D = sum_j p_j dp_j, ds_j = p_j (dp_j - D), dq_i = scale sum_j ds_j k_j.
    """
    s = k_sel @ q_i
    p = softmax_selected(s, scale)
    dp = v_sel @ dout_i
    # dp_j - D evaluated as (dp_j - dp_m) - sum_u p_u (dp_u - dp_m), m the
    # largest weight: the same value, without the cancellation that drops
    # the small terms of p . dp when the softmax is nearly one-hot.
    m = int(np.argmax(p))
    rel = dp - dp[m]
    ds = p * (rel - float(p @ rel))
    return p, ds, scale * (ds @ k_sel)


def kmip_backward_on_sets(q, k, v, idx, dout, scale: float = 1.0):
    """Gradients of L = sum(dout * out) with the selection idx held fixed.

    idx: int [N][H][topk] (every node is a query row).  Returns dq, dk, dv,
    float64 [N][H][d].  Keys selected by no query get exactly zero.
      dp_ij = dO_i . v_j,  D_i = sum_j p_ij dp_ij,  ds_ij = p_ij (dp_ij - D_i)
      dQ_i = scale sum_j ds_ij k_j,  dK_j = scale sum_i ds_ij q_i,
      dV_j = sum_i p_ij dO_i
    """
    n, heads, d = q.shape
    idx = np.asarray(idx, dtype=np.int64)
    dq = np.zeros((n, heads, d))
    dk = np.zeros((n, heads, d))
    dv = np.zeros((n, heads, d))
    for h in range(heads):
        for i in range(n):
            sel = idx[i, h]
            js = sel[sel >= 0]
            if js.size == 0:
                continue
            p, ds, dq[i, h, :] = query_grads(q[i, h, :], k[js, h, :], v[js, h, :],
                                             dout[i, h, :], scale)
            np.add.at(dk[:, h, :], js, scale * ds[:, None] * q[i, h, :][None, :])
            np.add.at(dv[:, h, :], js, p[:, None] * dout[i, h, :][None, :])
    return dq, dk, dv


def kmip_backward_rows(q, k, v, rows, idx_rows, dout, scale: float = 1.0):
    """Backward contributions of a subset of query rows (selection fixed).

    idx_rows: int [R][H][topk] for the node ids in rows.  Returns dq of those
    rows [R][H][d] and the dk, dv contributions they make ([N][H][d]); the
    full gradients are the sums of such contributions over all rows.
    """
    n, heads, d = q.shape
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, heads, d))
    dk = np.zeros((n, heads, d))
    dv = np.zeros((n, heads, d))
    for r, i in enumerate(rows):
        for h in range(heads):
            sel = idx_rows[r, h]
            js = sel[sel >= 0]
            if js.size == 0:
                continue
            p, ds, dq[r, h, :] = query_grads(q[i, h, :], k[js, h, :], v[js, h, :],
                                             dout[i, h, :], scale)
            np.add.at(dk[:, h, :], js, scale * ds[:, None] * q[i, h, :][None, :])
            np.add.at(dv[:, h, :], js, p[:, None] * dout[i, h, :][None, :])
    return dq, dk, dv


def kmip_backward(q, k, v, offsets, topk: int, dout, scale: float = 1.0):
    """Forward selection, then the fixed-selection gradients."""
    fw = kmip_forward(q, k, v, offsets, topk, scale=scale)
    return kmip_backward_on_sets(q, k, v, fw["idx"], dout, scale=scale)


# ---------------------------------------------------------------- sampled rows
def row_scores(q, k, offsets, i: int, h: int):
    """Full fp64 score row of query (i, h) over its graph, with the graph start."""
    n = q.shape[0]
    for lo, hi in graph_ranges(offsets, n):
        if lo <= i < hi:
            return k[lo:hi, h, :] @ q[i, h, :], lo
    raise IndexError(i)


def dq_rows_on_sets(q, k, v, idx, dout, rows, scale: float = 1.0):
    """dQ for the given node rows (idx [N][H][topk] over all nodes)."""
    heads, d = q.shape[1], q.shape[2]
    rows = np.asarray(rows, dtype=np.int64)
    res = np.zeros((rows.size, heads, d))
    for r, i in enumerate(rows):
        for h in range(heads):
            sel = idx[i, h]
            js = sel[sel >= 0]
            if js.size == 0:
                continue
            res[r, h, :] = query_grads(q[i, h, :], k[js, h, :], v[js, h, :],
                                       dout[i, h, :], scale)[2]
    return res


def dkv_keys_on_sets(q, k, v, idx, dout, keys, scale: float = 1.0):
    """dK and dV for the given key nodes, summing over every query that
    selected them in idx [N][H][topk]."""
    heads, d = q.shape[1], q.shape[2]
    keys = np.asarray(keys, dtype=np.int64)
    dk = np.zeros((keys.size, heads, d))
    dv = np.zeros((keys.size, heads, d))
    for h in range(heads):
        idx_h = idx[:, h, :]
        for r, j in enumerate(keys):
            qi, slot = np.nonzero(idx_h == j)
            for i, t in zip(qi, slot):
                sel = idx_h[i]
                js = sel[sel >= 0]
                p, ds, _ = query_grads(q[i, h, :], k[js, h, :], v[js, h, :],
                                       dout[i, h, :], scale)
                pos = int(np.nonzero(js == j)[0][0])
                dk[r, h, :] += scale * ds[pos] * q[i, h, :]
                dv[r, h, :] += p[pos] * dout[i, h, :]
    return dk, dv
