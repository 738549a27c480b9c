"""Seeded synthetic workloads for k-MIP attention.

This module only draws random inputs; it holds none of the attention
arithmetic.  It is shared by the tests, the benchmark and the smoke check so
that the CPU oracle and the GPU library see identical bytes.

Inputs are drawn in float32 from NumPy's PCG64 generator and rounded to
bfloat16 (round to nearest, ties to even) on the bit pattern.  Q, K and V are
returned as uint16 bf16 bit patterns laid out [N][H][d] (or, with
dtype="f32", as the float32 draws themselves); the upstream gradient is
float32 [N][H][d]; graph offsets are int32 [B+1].

The shapes stand in for the workloads of "k-Maximum Inner Product Attention
for Graph Transformers and the Expressive Power of GraphGPS": the controlled
random-graph runtime experiment (Appendix J, Tables 10-12), the large
City-Networks / point-cloud graphs (Table 13: 114k-569k nodes) and batched
small graphs (Tables 8-9).  No dataset item is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_BASE = 20260403


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


@dataclass
class Workload:
    name: str
    n: int
    heads: int
    d: int
    topk: int
    offsets: np.ndarray            # int32 [B+1]
    q: np.ndarray                  # uint16 bf16 bits [N][H][d] (float32 if dtype == "f32")
    k: np.ndarray
    v: np.ndarray
    dout: Optional[np.ndarray]     # float32 [N][H][d] or None (forward only)
    backward: bool
    meta: dict = field(default_factory=dict)
    dtype: str = "bf16"

    @property
    def num_graphs(self) -> int:
        return int(self.offsets.shape[0] - 1)

    def sum_nb2(self) -> int:
        nb = np.diff(self.offsets.astype(np.int64))
        return int((nb * nb).sum())


def _clustered_qk(rng, n, heads, d, clusters, sigma):
    assign = rng.integers(0, clusters, size=n)
    centres = rng.standard_normal((heads, clusters, d), dtype=np.float32)
    c = centres[:, assign, :].transpose(1, 0, 2)          # [N][H][d]
    qn = rng.standard_normal((n, heads, d), dtype=np.float32)
    q = c + np.float32(sigma) * qn
    del qn
    kn = rng.standard_normal((n, heads, d), dtype=np.float32)
    k = c + np.float32(sigma) * kn
    del kn, c
    return q, k


def make_workload(name: str, *, n: Optional[int] = None, heads: int, d: int, topk: int,
                  law: str = "iid", clusters: int = 0, sigma: float = 0.3,
                  graph_sizes: Optional[tuple] = None, num_graphs: int = 1,
                  backward: bool = False, seed: int = SEED_BASE,
                  dtype: str = "bf16") -> Workload:
    """Draw one workload.

    Draw order: graph sizes (ragged batches only), cluster assignments,
    centres [H][C][d], Q noise, K noise, V, then dO.
    law="iid": Q, K, V ~ N(0, 1).  law="clustered": a node takes one cluster
    for both its Q and K row; centres ~ N(0, 1) independently per head;
    Q = centre + sigma*noise, K = centre + sigma*independent noise.
    dtype="f32" keeps Q, K, V as float32 (same draws, no bf16 rounding).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if graph_sizes is not None:
        lo, hi = graph_sizes
        nb = rng.integers(lo, hi + 1, size=num_graphs).astype(np.int64)
        offsets = np.zeros(num_graphs + 1, dtype=np.int64)
        offsets[1:] = np.cumsum(nb)
        n = int(offsets[-1])
    else:
        assert n is not None
        offsets = np.array([0, n], dtype=np.int64)
    if law == "iid":
        q = rng.standard_normal((n, heads, d), dtype=np.float32)
        k = rng.standard_normal((n, heads, d), dtype=np.float32)
    elif law == "clustered":
        q, k = _clustered_qk(rng, n, heads, d, clusters, sigma)
    else:
        raise ValueError(law)
    v = rng.standard_normal((n, heads, d), dtype=np.float32)
    dout = rng.standard_normal((n, heads, d), dtype=np.float32) if backward else None
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return Workload(name=name, n=n, heads=heads, d=d, topk=topk,
                    offsets=offsets.astype(np.int32), q=q, k=k, v=v,
                    dout=dout, backward=backward,
                    meta=dict(law=law, clusters=clusters, sigma=sigma, seed=seed), dtype=dtype)


# The five workload families.  Ids fix the seeds (SEED_BASE + id).
WORKLOADS = {
    # 1 graph, i.i.d. Gaussian, small enough for an all-rows CPU check.
    "iid_n4096_h1_d64_k15": dict(n=4096, heads=1, d=64, topk=15, law="iid", id=1),
    # 1 graph, N = 10^4.5, 64 Gaussian clusters.
    "clustered_n31623_h4_d32_k15": dict(n=31623, heads=4, d=32, topk=15, law="clustered",
                                        clusters=64, id=2),
    # 1 graph, N = 10^5, 256 clusters, k sweep.
    "clustered_n100000_h4_d32_k5": dict(n=100000, heads=4, d=32, topk=5, law="clustered",
                                        clusters=256, id=3),
    "clustered_n100000_h4_d32_k15": dict(n=100000, heads=4, d=32, topk=15, law="clustered",
                                         clusters=256, id=3),
    "clustered_n100000_h4_d32_k45": dict(n=100000, heads=4, d=32, topk=45, law="clustered",
                                         clusters=256, id=3),
    # Training setting (forward + backward), N = 10^5.
    "train_clustered_n100000_h4_d32_k15": dict(n=100000, heads=4, d=32, topk=15,
                                               law="clustered", clusters=256, backward=True,
                                               id=4),
    # 64 ragged graphs of 500..5000 nodes, block-diagonal attention, training.
    "ragged64_h4_d32_k15": dict(graph_sizes=(500, 5000), num_graphs=64, heads=4, d=32,
                                topk=15, law="clustered", clusters=256, backward=True, id=5),
    # One point-cloud-like graph of 500k nodes, forward only.
    "pointcloud_n500000_h4_d32_k15": dict(n=500000, heads=4, d=32, topk=15,
                                          law="clustered", clusters=1024, id=6),
}


def get_workload(name: str, dtype: str = "bf16") -> Workload:
    spec = dict(WORKLOADS[name])
    wid = spec.pop("id")
    return make_workload(name, seed=SEED_BASE + wid, dtype=dtype, **spec)


def small_case(n: int, heads: int, d: int, topk: int, *, law: str = "iid", clusters: int = 0,
               graph_sizes=None, num_graphs: int = 1, backward: bool = True,
               seed: int = 12345, dtype: str = "bf16") -> Workload:
    """A small seeded case for parity tests (sizes chosen by the caller)."""
    if graph_sizes is not None:
        return make_workload(f"small_ragged_{seed}", heads=heads, d=d, topk=topk, law=law,
                             clusters=clusters, graph_sizes=graph_sizes,
                             num_graphs=num_graphs, backward=backward, seed=seed, dtype=dtype)
    return make_workload(f"small_{n}_{seed}", n=n, heads=heads, d=d, topk=topk, law=law,
                         clusters=clusters, backward=backward, seed=seed, dtype=dtype)


def with_offsets(name: str, sizes, heads: int, d: int, topk: int, *, law="iid",
                 clusters=0, sigma: float = 0.3, backward=True, seed=777,
                 dtype: str = "bf16") -> Workload:
    """A case with explicit graph sizes (edge cases: tiny graphs, n_b < k, ...)."""
    sizes = np.asarray(sizes, dtype=np.int64)
    offsets = np.zeros(len(sizes) + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(sizes)
    n = int(offsets[-1])
    w = make_workload(name, n=n, heads=heads, d=d, topk=topk, law=law, clusters=clusters,
                      sigma=sigma, backward=backward, seed=seed, dtype=dtype)
    w.offsets = offsets.astype(np.int32)
    return w
