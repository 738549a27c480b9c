"""Benchmark: k-MIP attention forward + backward on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
top-k score scan, softmax + gather + AV, and the backward (query side,
selection transpose, key side).  The default workload is the training
setting at N = 10^5 nodes, H = 4 heads, d = 32, k = 15 with clustered
Gaussian Q/K (256 clusters) and i.i.d. V and dO.  Inputs are resident in HBM
before the timed region starts.

Prints one JSON line.  `roofline` is for the dominant kernel, the score scan
(one launch = its threshold and selection passes): algorithmic flops
2*d*H*sum_b n_b^2 per launch over its average duration, measured with events
on the stream it runs on, against the dense bf16 MFMA peak.  `traffic` is the
HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
summary (calibrated against a plain device copy), null once the scan sources
differ from the ones profiled.  `cpu_baseline` times the fp64 oracle on a
bounded sample of the same workload on the host cores.

With --precision fp32 the same workload runs through the fp32 entry points
(fp32 q, k, v; the scan scores three bf16 terms per product, so it does three
times the bf16 MFMA work); the forward is then timed as one phase and the
roofline counts the MFMA work of the split.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--precision bf16|fp32]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "queries/s and % bf16 MFMA peak, k-MIP fwd+bwd at N=10^5, H=4, d=32, k=15"
DEFAULT_WORKLOAD = "train_clustered_n100000_h4_d32_k15"
PEAK_BF16_TFLOPS = 2500.0         # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E


def gather_bytes_per_row(d, k):
    """idx + score + k gathered bf16 V rows + fp32 out."""
    return k * (8 + 2 * d) + 4 * d


def backward_bytes_per_row(d, k):
    """Query side (idx, score, K and V rows, (p, ds) write), selection
    transpose (3 x 4k + 4) and key side (pair id, (p, ds), q row, dO row),
    plus dO, dq, dk, dv."""
    return k * (40 + 10 * d) + 16 * d + 4


def scan_traffic(workload: str):
    """HBM bytes per score-scan launch from the committed rocprofv3 summary,
    or None when it was taken for another workload or the scan sources have
    changed since (the summary records their SHA-256)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_" + workload.replace("train_clustered_", "train_")
                        + ".md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        key, sep, val = line.strip().partition(": ")
        if sep:
            fields[key] = val
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "graph_transformer_sparse_amd", "csrc")
    for f in sorted(x for x in os.listdir(csrc) if x.startswith("kmip_scan")) + ["kmip_internal.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("workload") != workload or fields.get("scan_source_sha256") != h.hexdigest():
        return None
    return float(fields["score_topk_traffic_bytes_per_launch"])


def cpu_baseline(w, nodes: int, seed: int = 7):
    """Time the fp64 oracle (forward selection + softmax-AV, then the backward
    contributions of the same rows) on a seeded sample of query nodes."""
    import numpy as np
    import oracle.kmip_oracle as orc
    if getattr(w, "dtype", "bf16") == "f32":
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (w.q, w.k, w.v))
    else:
        q, k, v = (orc.bf16_bits_to_f64(x) for x in (w.q, w.k, w.v))
    dout = w.dout.astype(np.float64) if w.dout is not None else None
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(w.n, size=min(nodes, w.n), replace=False))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        pass
    t0 = time.perf_counter()
    fw = orc.kmip_forward(q, k, v, w.offsets, w.topk, rows=rows)
    if dout is not None:
        orc.kmip_backward_rows(q, k, v, rows, fw["idx"], dout)
    dt = time.perf_counter() - t0
    return dict(value=rows.size / dt, unit="query nodes/s", cores=threads or 1, kind="oracle",
                seconds=round(dt, 3),
                sample=f"{rows.size} seeded query nodes x {w.heads} heads of {w.name}, each "
                       f"scored against all {w.n if w.num_graphs == 1 else 'its graph'} keys; "
                       f"forward{' + backward' if dout is not None else ''} in fp64 NumPy")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The GPU's clocks settle over the first ~100 ms of sustained work.
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--precision", choices=("bf16", "fp32"), default="bf16")
    ap.add_argument("--cpu-nodes", type=int, default=16384,
                    help="query nodes in the CPU oracle sample (0 skips the CPU baseline)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy, whose byte "
                         "counters calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by query rows across GPUs; this benchmark times "
              "one MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from graph_transformer_sparse_amd import kmip
    from workloads import get_workload

    f32 = args.precision == "fp32"
    w = get_workload(args.workload, dtype="f32" if f32 else "bf16")
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    if f32:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (w.q, w.k, w.v))
    else:
        q, k, v = bf16(w.q), bf16(w.k), bf16(w.v)
    offs = torch.from_numpy(w.offsets).to(dev) if w.num_graphs > 1 else None
    N, H, d, K = w.n, w.heads, w.d, w.topk
    dout = torch.from_numpy(w.dout).to(dev) if w.backward else None
    out = torch.empty((N, H, d), dtype=torch.float32, device=dev)
    idx = torch.empty((N, H, K), dtype=torch.int32, device=dev)
    score = torch.empty((N, H, K), dtype=torch.float32, device=dev)
    fws = (kmip.forward_f32_workspace_bytes if f32 else kmip.forward_workspace_bytes)(
        N, H, d, K, w.num_graphs)
    fwork = torch.empty(max(fws, 1), dtype=torch.uint8, device=dev)
    if w.backward:
        dq, dk, dv = (torch.empty((N, H, d), dtype=torch.float32, device=dev) for _ in range(3))
        bws = kmip.backward_workspace_bytes(N, H, d, K, w.num_graphs)
        bwork = torch.empty(bws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if f32:
            # split rows, scan, fp32 rescoring and weighted sum: one call
            kmip.forward(q, k, v, K, offs, out=out, topk_idx=idx, topk_score=score,
                         workspace=fwork, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        else:
            kmip.score_topk(q, k, K, offs, topk_idx=idx, topk_score=score, workspace=fwork,
                            stream=stream)
            if ev is not None:
                ev[1].record(stream)
            kmip.gather_softmax_av(v, idx, score, out=out, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if w.backward:
            kmip.backward(q, k, v, K, idx, score, dout, offs, dq=dq, dk=dk, dv=dv,
                          workspace=bwork, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    scan_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    gather_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    bwd_ms = np.array([e[2].elapsed_time(e[3]) for e in events])
    ms_per_step = wall * 1e3 / args.steps
    flops = 2.0 * d * H * w.sum_nb2() * (3 if f32 else 1)   # MFMA work of the scan
    scan_tflops = flops / (scan_ms.mean() * 1e-3) / 1e12
    rows = N * H
    g_bytes = rows * gather_bytes_per_row(d, K)
    b_bytes = rows * backward_bytes_per_row(d, K)

    cpu = None
    if args.cpu_nodes > 0:
        cpu = cpu_baseline(w, args.cpu_nodes)

    res = {
        "metric": METRIC,
        "value": N / (ms_per_step * 1e-3),
        "unit": "query nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 (3-term bf16 split scan)" if f32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "N": N, "H": H, "d": d, "k": K,
                   "graphs": w.num_graphs, "law": w.meta["law"],
                   "clusters": w.meta["clusters"], "pass": "forward+backward"
                   if w.backward else "forward"},
        "roofline": {"bound": "mfma", "achieved": scan_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": scan_tflops / PEAK_BF16_TFLOPS,
                     "traffic": None if f32 else scan_traffic(w.name),
                     "kernel": "kmip_forward_f32 (split + scan + rescoring gather)" if f32
                     else "score_topk_kernel",
                     "algorithmic_flop_per_launch": flops,
                     "avg_launch_ms": float(scan_ms.mean())},
        "phases_ms": {("forward_f32" if f32 else "score_topk"): float(scan_ms.mean()),
                      "gather_softmax_av": None if f32 else float(gather_ms.mean()),
                      "backward": float(bwd_ms.mean()) if w.backward else None},
        "hbm_model": {
            "gather_GBps": None if f32 else g_bytes / (gather_ms.mean() * 1e-3) / 1e9,
            "gather_frac": None if f32 else
            g_bytes / (gather_ms.mean() * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "backward_GBps": (b_bytes / (bwd_ms.mean() * 1e-3) / 1e9) if w.backward else None,
            "backward_frac": (b_bytes / (bwd_ms.mean() * 1e-3) / 1e9 / PEAK_HBM_GBS)
            if w.backward else None,
        },
        "query_rows_per_s": rows / (ms_per_step * 1e-3),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
