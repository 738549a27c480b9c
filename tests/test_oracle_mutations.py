"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each of them.  This is what makes the pins worth trusting:
a dropped term, a wrong sign, a wrong operand, an off-by-one or a reversed
tie rule must not pass silently."""
import numpy as np
import pytest

import oracle.kmip_oracle as orc
from tests.oracle_pins import ALL_PINS

_real = dict(select=orc.select_topk_row, softmax=orc.softmax_selected,
             ranges=orc.graph_ranges, grads=orc.query_grads, scores=orc.scores_block,
             decode=orc.bf16_bits_to_f64)


def _select_ties_desc(s, topk):
    n = s.shape[0]
    kk = min(topk, n)
    cand = np.arange(n)
    order = np.lexsort((-cand, -s[cand]))
    return cand[order[:kk]]


def _select_one_short(s, topk):
    return _real["select"](s, max(topk - 1, 1))


def _select_strict_candidates(s, topk):
    # keeps only keys strictly above the k-th value: drops tied keys
    n = s.shape[0]
    kk = min(topk, n)
    if kk < n:
        t = np.partition(s, n - kk)[n - kk]
        cand = np.nonzero(s > t)[0]
        if cand.size == 0:
            cand = np.nonzero(s >= t)[0]
    else:
        cand = np.arange(n)
    order = np.lexsort((cand, -s[cand]))
    return cand[order[:kk]]


def _softmax_unnormalised(s, scale):
    s = np.asarray(s, dtype=np.float64)
    m = s.max(axis=-1, keepdims=True)
    return np.where(np.isneginf(s), 0.0, np.exp(scale * (s - m)))


def _softmax_sign(s, scale):
    s = np.asarray(s, dtype=np.float64)
    m = s.max(axis=-1, keepdims=True)
    w = np.where(np.isneginf(s), 0.0, np.exp(-scale * (s - m)))
    return w / w.sum(axis=-1, keepdims=True)


def _softmax_noscale(s, scale):
    return _real["softmax"](s, 1.0)


def _ranges_drop_last(offsets, n):
    return [(lo, max(lo, hi - 1)) if hi - lo > 1 else (lo, hi)
            for lo, hi in _real["ranges"](offsets, n)]


def _grads_no_D(q_rows, k_sel, v_sel, dout_rows, valid, scale):
    s = np.where(valid, np.einsum("rkc,rc->rk", k_sel, q_rows), -np.inf)
    p = orc.softmax_selected(s, scale)
    ds = p * np.where(valid, np.einsum("rkc,rc->rk", v_sel, dout_rows), 0.0)
    return p, ds, scale * np.einsum("rk,rkc->rc", ds, k_sel)


def _grads_wrong_operand(q_rows, k_sel, v_sel, dout_rows, valid, scale):
    p, ds, _ = _real["grads"](q_rows, k_sel, v_sel, dout_rows, valid, scale)
    return p, ds, scale * np.einsum("rk,rkc->rc", ds, v_sel)


def _grads_sign(q_rows, k_sel, v_sel, dout_rows, valid, scale):
    p, ds, dq = _real["grads"](q_rows, k_sel, v_sel, dout_rows, valid, scale)
    return p, -ds, -dq


def _grads_no_scale(q_rows, k_sel, v_sel, dout_rows, valid, scale):
    p, ds, dq = _real["grads"](q_rows, k_sel, v_sel, dout_rows, valid, scale)
    return p, ds, dq / scale


def _grads_no_max_shift(q_rows, k_sel, v_sel, dout_rows, valid, scale):
    # D taken as the plain p . dp without the relative form: same value in
    # exact arithmetic, cancels on peaked rows
    s = np.where(valid, np.einsum("rkc,rc->rk", k_sel, q_rows), -np.inf)
    p = orc.softmax_selected(s, scale)
    dp = np.where(valid, np.einsum("rkc,rc->rk", v_sel, dout_rows), 0.0)
    ds = p * (dp - np.einsum("rk,rk->r", p, dp)[:, None])
    return p, ds, scale * np.einsum("rk,rkc->rc", ds, k_sel)


def _grads_dk_transposed(q_rows, k_sel, v_sel, dout_rows, valid, scale):
    # p and ds of the wrong slot order (reversed within each row)
    p, ds, dq = _real["grads"](q_rows, k_sel, v_sel, dout_rows, valid, scale)
    return p, ds[:, ::-1], dq


def _scores_reversed_keys(q_rows, k_graph):
    return q_rows @ k_graph[::-1].T


def _decode_shift15(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


MUTATIONS = {
    "select_ties_descending": ("select_topk_row", _select_ties_desc),
    "select_one_short": ("select_topk_row", _select_one_short),
    "select_drops_tied": ("select_topk_row", _select_strict_candidates),
    "softmax_unnormalised": ("softmax_selected", _softmax_unnormalised),
    "softmax_sign": ("softmax_selected", _softmax_sign),
    "softmax_ignores_scale": ("softmax_selected", _softmax_noscale),
    "graph_drops_last_key": ("graph_ranges", _ranges_drop_last),
    "grad_drops_D": ("query_grads", _grads_no_D),
    "grad_dq_uses_v": ("query_grads", _grads_wrong_operand),
    "grad_sign": ("query_grads", _grads_sign),
    "grad_dq_unscaled": ("query_grads", _grads_no_scale),
    "grad_cancelling_D": ("query_grads", _grads_no_max_shift),
    "grad_ds_slot_order": ("query_grads", _grads_dk_transposed),
    "scores_reversed_keys": ("scores_block", _scores_reversed_keys),
    "decode_shift15": ("bf16_bits_to_f64", _decode_shift15),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # an assertion, or a crash caused by the mutation
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {name}"
