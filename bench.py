"""Benchmark: k-MIP attention forward + backward on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
top-k score scan, softmax + gather + AV, and the backward (query side,
selection transpose, key side).  The default workload is the training
setting at N = 10^5 nodes, H = 4 heads, d = 32, k = 15 with clustered
Gaussian Q/K (256 clusters) and i.i.d. V and dO.  Inputs are resident in HBM
before the timed region starts.

Prints one JSON line:
  * `value`: query nodes per second over the timed steps (N / step time).
  * `roofline`: for the dominant kernel, the score scan (one
    kmip_score_topk launch: query order, threshold and selection passes):
    algorithmic flops 2*d*H*sum_b n_b^2 over its mean duration, measured with
    events on the stream it runs on, against the dense bf16 MFMA peak.
    `traffic` is the HBM bytes per launch from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (calibrated against a plain device copy),
    null once the library sources differ from the ones profiled.
  * `hbm`: the gather and the backward against the 8 TB/s HBM peak, from the
    same counters (bytes the kernels moved / their event time), next to
    the gathered-row byte model's rate (the model charges every gathered row
    to HBM, though repeated rows of hub keys come from L2 and the MALL, so
    the model rate is not a fraction of the HBM peak).
  * `timing`: median, min, mean and std of the step, and the step right
    after a 512 MB write that evicts the 256 MB MALL ("cold").
  * `configs`: bounded sub-records of the other workloads (forward and
    backward ms, query nodes/s, scan MFMA fraction), the fp32 entry points,
    and HIP-graph replay against eager calls at small N.
  * `measured_peaks`: a large bf16 GEMM and a device copy on this GPU.
  * `cpu_baseline`: the fp64 oracle on a bounded sample of the workload, over
    the host's cores (one worker process each).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--precision bf16|fp32] [--configs all|none]
"""
from __future__ import annotations

import argparse
import hashlib
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

# Other workloads reported as sub-records (forward-only ones time the forward).
SUB_WORKLOADS = ["iid_n4096_h1_d64_k15", "clustered_n31623_h4_d32_k15",
                 "clustered_n100000_h4_d32_k5", "clustered_n100000_h4_d32_k15",
                 "clustered_n100000_h4_d32_k45", "ragged64_h4_d32_k15",
                 "pointcloud_n500000_h4_d32_k15"]
SMALL_N = [100, 1000, 10000]


def gather_bytes_per_row(d, k):
    """idx + score + k gathered bf16 V rows + fp32 out."""
    return k * (8 + 2 * d) + 4 * d


def backward_bytes_per_row(d, k):
    """Query side (idx, score, K and V rows, (p, ds) write), selection
    transpose (3 x 4k + 4) and key side (pair id, (p, ds), q row, dO row),
    plus dO, dq, dk, dv."""
    return k * (40 + 10 * d) + 16 * d + 4


# ---------------------------------------------------------------- counters
def source_sha256():
    """Hash of the library sources, recorded in the traffic summaries."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "graph_transformer_sparse_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()


def counter_bytes(workload: str):
    """Per-phase HBM bytes per call from the committed rocprofv3 summary
    (profiles/traffic_<workload>.md), or None when there is none for this
    workload or the library sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        key, sep, val = line.strip().partition(": ")
        if sep:
            fields[key] = val
    if fields.get("workload") != workload or fields.get("source_sha256") != source_sha256():
        return None
    return {p: float(fields[f"{p}_bytes_per_call"]) for p in ("score_topk", "gather", "backward")
            if f"{p}_bytes_per_call" in fields}


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(w, nodes: int, seed: int = 7):
    """Time the fp64 oracle on a seeded sample of query nodes: the forward
    selection + softmax-AV over the host's cores, then the backward
    contributions of the same rows."""
    import numpy as np
    import oracle.kmip_oracle as orc
    from oracle.pool import cpu_model, forward_rows, host_workers
    if getattr(w, "dtype", "bf16") == "f32":
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (w.q, w.k, w.v))
    else:
        q, k, v = (orc.bf16_bits_to_f64(x) for x in (w.q, w.k, w.v))
    dout = w.dout.astype(np.float64) if w.dout is not None else None
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(w.n, size=min(nodes, w.n), replace=False))
    workers = host_workers()
    t0 = time.perf_counter()
    fw = forward_rows(q, k, v, w.offsets, w.topk, rows, workers=workers)
    t1 = time.perf_counter()
    if dout is not None:
        orc.kmip_backward_on_sets(q, k, v, fw["idx"], dout, rows=rows)
    t2 = time.perf_counter()
    return dict(value=rows.size / (t2 - t0), unit="query nodes/s", cores=workers,
                kind="oracle", cpu_model=cpu_model(), seconds=round(t2 - t0, 3),
                forward_seconds=round(t1 - t0, 3),
                sample=f"{rows.size} seeded query nodes x {w.heads} heads of {w.name}, each "
                       f"scored against all {w.n if w.num_graphs == 1 else 'its graph'} keys; "
                       f"fp64 NumPy forward over {workers} worker processes (one BLAS thread "
                       f"each){', then the backward of those rows in one process' if dout is not None else ''}")


# ---------------------------------------------------------------- GPU timing
class Path:
    """Device buffers for one workload and the calls of one step."""

    def __init__(self, w, f32=False):
        import numpy as np
        import torch
        from graph_transformer_sparse_amd import kmip
        self.w, self.f32, self.kmip = w, f32, kmip
        dev = torch.device("cuda", 0)
        if f32:
            q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (w.q, w.k, w.v))
        else:
            q, k, v = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
                torch.bfloat16).to(dev) for x in (w.q, w.k, w.v))
        self.q, self.k, self.v = q, k, v
        self.offs = torch.from_numpy(w.offsets).to(dev) if w.num_graphs > 1 else None
        N, H, d, K = w.n, w.heads, w.d, w.topk
        self.dout = torch.from_numpy(w.dout).to(dev) if w.backward else None
        self.out = torch.empty((N, H, d), dtype=torch.float32, device=dev)
        self.idx = torch.empty((N, H, K), dtype=torch.int32, device=dev)
        self.score = torch.empty((N, H, K), dtype=torch.float32, device=dev)
        fws = (kmip.forward_f32_workspace_bytes if f32 else kmip.forward_workspace_bytes)(
            N, H, d, K, w.num_graphs)
        self.fwork = torch.empty(max(fws, 1), dtype=torch.uint8, device=dev)
        if w.backward:
            self.dq, self.dk, self.dv = (torch.empty((N, H, d), dtype=torch.float32, device=dev)
                                         for _ in range(3))
            self.bwork = torch.empty(kmip.backward_workspace_bytes(N, H, d, K, w.num_graphs),
                                     dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)

    def step(self, ev=None):
        """Scan (+ gather), then the backward; events ev[0..3] bracket the
        scan, the gather and the backward on the kernels' stream."""
        km, s, w = self.kmip, self.stream, self.w
        if ev is not None:
            ev[0].record(s)
        if self.f32:
            km.forward(self.q, self.k, self.v, w.topk, self.offs, out=self.out,
                       topk_idx=self.idx, topk_score=self.score, workspace=self.fwork,
                       stream=s)
            if ev is not None:
                ev[1].record(s)
        else:
            km.score_topk(self.q, self.k, w.topk, self.offs, topk_idx=self.idx,
                          topk_score=self.score, workspace=self.fwork, stream=s)
            if ev is not None:
                ev[1].record(s)
            km.gather_softmax_av(self.v, self.idx, self.score, out=self.out, stream=s)
        if ev is not None:
            ev[2].record(s)
        if w.backward:
            km.backward(self.q, self.k, self.v, w.topk, self.idx, self.score, self.dout,
                        self.offs, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.bwork,
                        stream=s)
        if ev is not None:
            ev[3].record(s)

    def timed(self, steps, warmup):
        """Per-step phase times (ms) and the wall time of the timed steps."""
        import numpy as np
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ph = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]),
                        e[2].elapsed_time(e[3]), e[0].elapsed_time(e[3])] for e in events])
        return ph, wall

    def cold(self, reps=5):
        """Step time right after writing 512 MB (twice the MALL)."""
        import numpy as np
        import torch
        flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
        res = []
        for _ in range(reps):
            flush.fill_(1.0)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            self.step(ev)
            torch.cuda.synchronize()
            res.append(ev[0].elapsed_time(ev[3]))
        del flush
        return float(np.median(res))


def stats(x):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    return dict(median=float(np.median(x)), min=float(x.min()), mean=float(x.mean()),
                std=float(x.std()))


def scan_frac(w, scan_ms, f32=False):
    """Algorithmic flops of the scan (one d-term inner product per score, in
    either precision; the fp32 entry points compute each as three bf16
    products, and the pruned pass skips most of them) per second, against
    the bf16 dense MFMA peak the scan runs on."""
    flops = 2.0 * w.d * w.heads * w.sum_nb2()
    return flops / (scan_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS


def sub_record(name, f32=False, steps=10, warmup=5):
    """Bounded timing of one more workload."""
    import torch
    from workloads import get_workload
    w = get_workload(name, dtype="f32" if f32 else "bf16")
    p = Path(w, f32)
    ph, wall = p.timed(steps, warmup)
    rec = dict(workload=w.name, precision="fp32" if f32 else "bf16",
               pass_="forward+backward" if w.backward else "forward", N=w.n, graphs=w.num_graphs,
               k=w.topk, steps=steps, forward_ms=stats(ph[:, 0] + ph[:, 1]),
               scan_ms=stats(ph[:, 0]), backward_ms=stats(ph[:, 2]) if w.backward else None,
               ms_per_step=wall * 1e3 / steps,
               query_nodes_per_s=w.n / (wall / steps),
               scan_mfma_frac=scan_frac(w, float(ph[:, 0].mean()), f32),
               scan_flop=2.0 * w.d * w.heads * w.sum_nb2())
    rec["pass"] = rec.pop("pass_")
    if not f32:
        rows = w.n * w.heads
        rec["gather_model_GBps"] = rows * gather_bytes_per_row(w.d, w.topk) / (
            ph[:, 1].mean() * 1e-3) / 1e9
        if w.backward:
            rec["backward_model_GBps"] = rows * backward_bytes_per_row(w.d, w.topk) / (
                ph[:, 2].mean() * 1e-3) / 1e9
    del p
    torch.cuda.empty_cache()
    return rec


def small_n_latency(reps=50):
    """One forward + backward at small N: eager calls against the replay of a
    captured HIP graph (graph_transformer_sparse_amd.captured)."""
    import numpy as np
    import torch
    from graph_transformer_sparse_amd.captured import CapturedKmip
    from workloads import small_case
    res = []
    for n in SMALL_N:
        w = small_case(n, 4, 32, 15, law="iid", seed=4000 + n)
        p = Path(w)
        ph, wall = p.timed(reps, 10)
        cap = CapturedKmip(n, 4, 32, 15, None, backward=True)
        for dst, src in ((cap.q, p.q), (cap.k, p.k), (cap.v, p.v), (cap.dout, p.dout)):
            dst.copy_(src)
        for _ in range(10):
            cap.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            cap.replay()
        e1.record()
        torch.cuda.synchronize()
        res.append(dict(N=n, H=4, d=32, k=15, eager_ms=wall * 1e3 / reps,
                        eager_gpu_ms=float(np.median(ph[:, 3])),
                        captured_ms=e0.elapsed_time(e1) / reps))
    return res


def measured_peaks():
    """A large bf16 GEMM (library) and a device copy: what this GPU sustains
    against the spec peaks."""
    import torch
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2 * 8192 ** 3 * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    src = torch.ones(256 << 20, dtype=torch.float32, device="cuda")   # 1 GiB
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    bw = 2 * src.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return dict(bf16_gemm_TFLOPs=gemm, bf16_gemm_frac_of_spec=gemm / PEAK_BF16_TFLOPS,
                hbm_copy_GBps=bw, hbm_copy_frac_of_spec=bw / PEAK_HBM_GBS,
                how="torch.matmul 8192^3 bf16 (20 calls); 1 GiB device copy, read + write "
                    "bytes (10 calls)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The GPU's clocks settle over the first ~100 ms of sustained work.
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--precision", choices=("bf16", "fp32"), default="bf16")
    ap.add_argument("--configs", choices=("all", "none"), default="all",
                    help="also time the other workloads, the fp32 leg and small N")
    ap.add_argument("--cpu-nodes", type=int, default=32768,
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

    from workloads import get_workload

    f32 = args.precision == "fp32"
    w = get_workload(args.workload, dtype="f32" if f32 else "bf16")
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    path = Path(w, f32)
    ph, wall = path.timed(args.steps, args.warmup)
    scan_ms, gather_ms, bwd_ms, step_ms = ph[:, 0], ph[:, 1], ph[:, 2], ph[:, 3]
    ms_per_step = wall * 1e3 / args.steps
    N, H, d, K = w.n, w.heads, w.d, w.topk
    flops = 2.0 * d * H * w.sum_nb2()          # algorithmic: every score once
    scan_tflops = flops / (scan_ms.mean() * 1e-3) / 1e12
    rows = N * H
    g_model = rows * gather_bytes_per_row(d, K)
    b_model = rows * backward_bytes_per_row(d, K)
    cold_ms = path.cold() if args.configs == "all" else None
    del path
    torch.cuda.empty_cache()

    cnt = None if f32 else counter_bytes(w.name)
    hbm = {"gather_model_bytes": g_model,
           "gather_model_GBps": g_model / (gather_ms.mean() * 1e-3) / 1e9,
           "backward_model_bytes": b_model if w.backward else None,
           "backward_model_GBps": (b_model / (bwd_ms.mean() * 1e-3) / 1e9) if w.backward
           else None}
    for phase, t in (("gather", gather_ms), ("backward", bwd_ms)):
        b = None if cnt is None else cnt.get(phase)
        gbs = None if b is None or (phase == "backward" and not w.backward) else \
            b / (t.mean() * 1e-3) / 1e9
        hbm[f"{phase}_counter_bytes"] = b
        hbm[f"{phase}_counter_GBps"] = gbs
        hbm[f"{phase}_frac"] = None if gbs is None else gbs / PEAK_HBM_GBS
    hbm["note"] = ("frac = counter bytes (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated) / event "
                   "time / 8 TB/s; the model rate charges every gathered row to HBM and is not a "
                   "fraction of the HBM peak")

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
                     "traffic": None if cnt is None else cnt.get("score_topk"),
                     "kernel": "kmip_forward_f32 (split + scan + rescoring gather)" if f32
                     else "kmip_score_topk (query order, threshold and selection passes)",
                     "algorithmic_flop_per_launch": flops,
                     "avg_launch_ms": float(scan_ms.mean())},
        "phases_ms": {("forward_f32" if f32 else "score_topk"): float(scan_ms.mean()),
                      "gather_softmax_av": None if f32 else float(gather_ms.mean()),
                      "backward": float(bwd_ms.mean()) if w.backward else None},
        "hbm": hbm,
        "timing": {"step_ms": stats(step_ms), "cold_step_ms": cold_ms,
                   "how": "HIP events on the kernels' stream; cold = right after a 512 MB "
                          "device write (twice the 256 MB MALL)"},
        "query_rows_per_s": rows / (ms_per_step * 1e-3),
    }
    if args.configs == "all":
        subs = []
        for name in SUB_WORKLOADS:
            subs.append(sub_record(name))
        if not f32:
            subs.append(sub_record(DEFAULT_WORKLOAD, f32=True))
            subs.append(sub_record("ragged64_h4_d32_k15", f32=True))
        res["configs"] = subs
        res["small_n"] = small_n_latency()
        res["measured_peaks"] = measured_peaks()
    res["cpu_baseline"] = cpu_baseline(w, args.cpu_nodes) if args.cpu_nodes > 0 else None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
