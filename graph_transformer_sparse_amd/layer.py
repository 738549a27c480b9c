"""PyTorch autograd wrapper and a GraphGPS-style multi-head k-MIP attention
layer around libkmip.

Page "k-Maximum Inner Product Attention for Graph Transformers and the
Expressive Power of GraphGPS", Figure 1: a GPS layer adds a global attention
branch to a local message-passing branch, each with a residual connection,
followed by a feed-forward block.  k-MIP attention is the global branch: per
head, queries, keys and values are linear projections of the node features,
and each query attends to its k keys of largest inner product (Abstract).

Everything between the projections runs in libkmip: the top-k scan, the
softmax and the weighted sum, and the backward.  The projections,
normalisations and the feed-forward block are ordinary PyTorch modules.
"""
from __future__ import annotations

import math
from typing import Callable, Optional

import torch
from torch import nn

from . import kmip


class KMIPAttentionFunction(torch.autograd.Function):
    """out = kmip_attention(q, k, v) for q, k, v of shape [N, H, d].

    precision="bf16": q, k and v are rounded to bf16 (the bf16 entry points);
    their gradients are those of the rounded values (the cast passes
    gradients through unchanged).  precision="fp32": the fp32 entry points,
    whose scan scores a three-term bf16 split of the fp32 values (fp32-level
    scores at three times the matrix-core work).  The output and the
    gradients are fp32 (gradients are cast back to the input dtype).  The
    score is the unscaled inner product: fold a temperature such as 1/sqrt(d)
    into q.  The top-k selection is piecewise constant and carries no
    gradient.
    """

    @staticmethod
    def forward(ctx, q, k, v, topk: int, graph_offsets: Optional[torch.Tensor] = None,
                precision: str = "bf16"):
        if precision not in ("bf16", "fp32"):
            raise ValueError("precision must be 'bf16' or 'fp32'")
        dt = torch.float32 if precision == "fp32" else torch.bfloat16
        qb, kb, vb = (x.detach().to(dt).contiguous() for x in (q, k, v))
        out, idx, score = kmip.forward(qb, kb, vb, topk, graph_offsets)
        ctx.save_for_backward(qb, kb, vb, idx, score)
        ctx.topk = topk
        ctx.graph_offsets = graph_offsets
        ctx.dtypes = (q.dtype, k.dtype, v.dtype)
        ctx.mark_non_differentiable(idx)
        return out, idx

    @staticmethod
    def backward(ctx, dout, _didx):
        qb, kb, vb, idx, score = ctx.saved_tensors
        if dout is None:
            dout = torch.zeros(qb.shape, dtype=torch.float32, device=qb.device)
        dq, dk, dv = kmip.backward(qb, kb, vb, ctx.topk, idx, score,
                                   dout.to(torch.float32).contiguous(), ctx.graph_offsets)
        tq, tk, tv = ctx.dtypes
        return dq.to(tq), dk.to(tk), dv.to(tv), None, None, None


def kmip_attention(q, k, v, topk: int, graph_offsets: Optional[torch.Tensor] = None,
                   precision: str = "bf16"):
    """Differentiable k-MIP attention.  Returns (out [N, H, d] fp32,
    topk_idx [N, H, topk] int32, not differentiable)."""
    return KMIPAttentionFunction.apply(q, k, v, topk, graph_offsets, precision)


class KMIPMultiheadAttention(nn.Module):
    """Multi-head k-MIP attention over node features x [N, C].

    q = x W_q / sqrt(d), k = x W_k, v = x W_v (H heads of d channels each);
    per head, each node attends to the topk nodes of its graph with the
    largest q.k; the heads are concatenated and projected back to C channels.
    The 1/sqrt(d) temperature is folded into the query projection, since the
    kernels score the unscaled inner product.  precision selects the bf16 or
    the fp32 entry points (KMIPAttentionFunction).
    """

    def __init__(self, channels: int, heads: int, head_dim: int, topk: int,
                 bias: bool = True, precision: str = "bf16"):
        super().__init__()
        if head_dim not in (32, 64):
            raise ValueError("head_dim must be 32 or 64")
        self.heads, self.head_dim, self.topk = heads, head_dim, topk
        self.precision = precision
        inner = heads * head_dim
        self.q_proj = nn.Linear(channels, inner, bias=bias)
        self.k_proj = nn.Linear(channels, inner, bias=bias)
        self.v_proj = nn.Linear(channels, inner, bias=bias)
        self.out_proj = nn.Linear(inner, channels, bias=bias)
        self.scale = 1.0 / math.sqrt(head_dim)
        self.last_topk_idx: Optional[torch.Tensor] = None

    def forward(self, x: torch.Tensor, graph_offsets: Optional[torch.Tensor] = None):
        n = x.shape[0]
        shape = (n, self.heads, self.head_dim)
        q = (self.q_proj(x) * self.scale).view(shape)
        k = self.k_proj(x).view(shape)
        v = self.v_proj(x).view(shape)
        out, idx = kmip_attention(q, k, v, self.topk, graph_offsets, self.precision)
        self.last_topk_idx = idx
        return self.out_proj(out.reshape(n, self.heads * self.head_dim).to(x.dtype))


class GPSLayer(nn.Module):
    """One GraphGPS-style layer with k-MIP global attention (Figure 1):

        h = x + Dropout(Attn(x)) + Dropout(Local(x))
        y = h + Dropout(FFN(h))

    with a normalisation after each residual sum.  `local` is an optional
    message-passing module called as local(x, edge_index) -> [N, C]; without
    one the layer is the attention branch and the feed-forward block.
    """

    def __init__(self, channels: int, heads: int, head_dim: int, topk: int,
                 local: Optional[Callable] = None, dropout: float = 0.0,
                 ffn_mult: int = 2):
        super().__init__()
        self.attn = KMIPMultiheadAttention(channels, heads, head_dim, topk)
        self.local = local
        self.norm1 = nn.LayerNorm(channels)
        self.norm2 = nn.LayerNorm(channels)
        self.ffn = nn.Sequential(nn.Linear(channels, ffn_mult * channels), nn.ReLU(),
                                 nn.Linear(ffn_mult * channels, channels))
        self.drop = nn.Dropout(dropout)

    def forward(self, x: torch.Tensor, graph_offsets: Optional[torch.Tensor] = None,
                edge_index: Optional[torch.Tensor] = None):
        h = x + self.drop(self.attn(x, graph_offsets))
        if self.local is not None:
            h = h + self.drop(self.local(x, edge_index))
        h = self.norm1(h)
        return self.norm2(h + self.drop(self.ffn(h)))
