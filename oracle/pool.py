"""Run the fp64 oracle's forward over row blocks in a pool of worker
processes.

TEST INFRASTRUCTURE, like the rest of oracle/: only the tests, the smoke
check and the benchmark's cpu_baseline leg use it.

The oracle scores every query row against every key of its graph and takes
an exact sort-based top-k per row, so checking every row of a 10^5-node graph
is ~10^11 fp64 multiply-adds plus 4 * 10^5 partial sorts.  Rows are
independent, so they are split into blocks and handed to worker processes,
one BLAS thread each.  The inputs are placed once in shared memory, which the
workers map read-only.  Workers are spawned (fresh interpreters that import
NumPy and the oracle only), never forked from a process that holds a GPU
context.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from multiprocessing import shared_memory

import numpy as np

_W = {}          # worker state: attached arrays


def host_workers() -> int:
    """Worker processes for the host's CPU share (at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _init(specs, offsets, topk, scale):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    shms = {}
    for name, (shm_name, shape) in specs.items():
        shm = shared_memory.SharedMemory(name=shm_name)
        shms[name] = shm
        _W[name] = np.ndarray(shape, dtype=np.float64, buffer=shm.buf)
    _W["_shm"] = shms
    _W["offsets"] = offsets
    _W["topk"] = topk
    _W["scale"] = scale


def _forward_block(rows):
    from oracle import kmip_oracle as orc
    fw = orc.kmip_forward(_W["q"], _W["k"], _W["v"], _W["offsets"], _W["topk"],
                          scale=_W["scale"], rows=rows)
    return fw["idx"], fw["score"], fw["out"]


def forward_rows(q, k, v, offsets, topk, rows=None, *, scale=1.0, workers=None,
                 block=None):
    """orc.kmip_forward(q, k, v, offsets, topk, rows=rows), computed in
    worker processes over blocks of rows.  Returns the same dict."""
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    workers = host_workers() if workers is None else workers
    if block is None:
        block = int(min(2048, max(64, -(-rows.size // (4 * workers)))))
    chunks = [rows[a:a + block] for a in range(0, rows.size, block)]
    offs = None if offsets is None else np.asarray(offsets, dtype=np.int64)
    shms = []
    try:
        specs = {}
        for name, arr in (("q", q), ("k", k), ("v", v)):
            shm = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
            shms.append(shm)
            np.ndarray(arr.shape, dtype=np.float64, buffer=shm.buf)[...] = arr
            specs[name] = (shm.name, arr.shape)
        ctx = mp.get_context("spawn")
        env_keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
        saved = {e: os.environ.get(e) for e in env_keys}
        for e in env_keys:
            os.environ[e] = "1"
        try:
            pool = ctx.Pool(workers, initializer=_init, initargs=(specs, offs, topk, scale))
        finally:
            for e, val in saved.items():
                if val is None:
                    os.environ.pop(e, None)
                else:
                    os.environ[e] = val
        with pool:
            parts = pool.map(_forward_block, chunks, chunksize=1)
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    H, d = q.shape[1], q.shape[2]
    if not parts:
        return dict(idx=np.zeros((0, H, topk), np.int64), score=np.zeros((0, H, topk)),
                    out=np.zeros((0, H, d)))
    return dict(idx=np.concatenate([p[0] for p in parts]),
                score=np.concatenate([p[1] for p in parts]),
                out=np.concatenate([p[2] for p in parts]))
