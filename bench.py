"""Benchmark of the dynamically sparse int4 GEMV on one MI355X.

Workload: the Llama-3-8B-shaped down projection, K = 14336 inputs ->
N = 4096 outputs, int4 group-128 weights ~N(0, 0.02), activation
x = silu(g) * u with g, u ~N(0, 1), magnitude-thresholded at 50 % (the step),
with 70 % and 90 %, the dense int4 GEMV and the batched M = 1..16 union
variant measured beside it.  Synthetic, seeded data.

One step = one pass of the hot path on one activation vector:
threshold + compact (sgemv_gather_indices) then the sparse GEMV
(sgemv_run), reading the weights of the next of R packed copies whose total
exceeds 1 GiB so neither the L2 nor the 256 MB Infinity Cache can serve
them.  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` is microseconds per step (lower is better);
the effective HBM bandwidth of the sparse GEMV kernel and its fraction of
the 8 TB/s peak are in `roofline`, measured with HIP events around every
launch of that kernel on the stream it runs on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 1 << 30
K_DOWN, N_DOWN = 14336, 4096
KERNEL_SRC = os.path.join(ROOT, "activation_sparse_bit_amd", "csrc", "sgemv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_run_down14336_p50_traffic.json")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def run_bytes(A: int, Ag: int, N: int, M: int = 1) -> int:
    """Algorithmic bytes of one sparse GEMV launch: listed weight columns
    (N/2 bytes each), scale+zero of every touched group (4 bytes per output),
    the index list, the gathered activations and the output."""
    return A * N // 2 + Ag * N * 4 + A * 4 + M * A * 2 + M * N * 2


def gather_bytes(K: int, A: int, M: int = 1) -> int:
    return M * K * 2 + A * 4 + 4


def touched_groups(idx: np.ndarray) -> int:
    return int(np.unique(np.asarray(idx) // 128).size)


class Timer:
    """HIP-event timing of a sequence of launches on one stream."""

    def __init__(self, torch, n):
        self.torch = torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]

    def mean_ms(self, n):
        return float(np.mean([a.elapsed_time(b) for a, b in self.ev[:n]]))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="only the 50%% step (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy three times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; use --gpus 1"}))
        sys.exit(2)

    import torch

    import synth
    from activation_sparse_bit_amd import sgemv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---------------- inputs, resident in HBM ----------------
    q, s, z = synth.quantized_weights(0, N_DOWN, K_DOWN, 0.02)
    desc, blob = sgemv.sgemv_pack_layout(q, s, z)
    R = max(2, -(-ROTATE_BYTES // desc.total_bytes))
    blob_d = torch.from_numpy(blob).to(dev)
    copies = [blob_d] + [blob_d.clone() for _ in range(R - 1)]
    ws = torch.zeros(max(sgemv.sgemv_workspace_bytes(desc, 16), 256), dtype=torch.uint8, device=dev)

    x = synth.glu_activation(0, K_DOWN)
    xd = torch.from_numpy(x).to(dev)
    idx = torch.zeros(K_DOWN, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    y = torch.empty(N_DOWN, dtype=torch.float16, device=dev)

    def measure(p, steps, warmup, dense=False):
        t = synth.percentile_threshold(x, p)
        gath = Timer(torch, steps)
        runt = Timer(torch, steps)
        for i in range(warmup):
            if not dense:
                sgemv.sgemv_gather_indices(xd, [t], idx, cnt, stream=stream)
            sgemv.sgemv_run(desc, copies[i % R], xd, None if dense else idx, None if dense else cnt,
                            y, ws, stream=stream)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(steps):
            if not dense:
                gath.ev[i][0].record(stream)
                sgemv.sgemv_gather_indices(xd, [t], idx, cnt, stream=stream)
                gath.ev[i][1].record(stream)
            runt.ev[i][0].record(stream)
            sgemv.sgemv_run(desc, copies[i % R], xd, None if dense else idx, None if dense else cnt,
                            y, ws, stream=stream)
            runt.ev[i][1].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        total_ms = t0.elapsed_time(t1)
        if dense:
            A, Ag = K_DOWN, K_DOWN // 128
        else:
            c = int(cnt.item())
            lst = idx[:c].cpu().numpy()
            A, Ag = c, touched_groups(lst)
        run_ms = runt.mean_ms(steps)
        gat_ms = gath.mean_ms(steps) if not dense else 0.0
        rb = run_bytes(A, Ag, N_DOWN)
        return {
            "p": p, "active": A, "groups_touched": Ag,
            "us_per_step": total_ms * 1000.0 / steps,
            "us_run": run_ms * 1000.0, "us_gather": gat_ms * 1000.0,
            "run_bytes": rb, "run_GBps": rb / (run_ms * 1e-3) / 1e9,
            "run_frac_hbm_peak": rb / (run_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "gather_bytes": 0 if dense else gather_bytes(K_DOWN, A),
        }

    def measure_batched(M, steps, warmup):
        X = np.stack([synth.glu_activation(m, K_DOWN) for m in range(M)])
        ts = [synth.percentile_threshold(X[m], 0.7) for m in range(M)]
        Xd = torch.from_numpy(X).to(dev)
        Y = torch.empty((M, N_DOWN), dtype=torch.float16, device=dev)
        runt = Timer(torch, steps)
        for i in range(warmup):
            sgemv.sgemv_gather_indices(Xd, ts, idx, cnt, stream=stream)
            sgemv.sgemv_run_batched(desc, copies[i % R], Xd, ts, idx, cnt, Y, ws, stream=stream)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(steps):
            sgemv.sgemv_gather_indices(Xd, ts, idx, cnt, stream=stream)
            runt.ev[i][0].record(stream)
            sgemv.sgemv_run_batched(desc, copies[i % R], Xd, ts, idx, cnt, Y, ws, stream=stream)
            runt.ev[i][1].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        c = int(cnt.item())
        A, Ag = c, touched_groups(idx[:c].cpu().numpy())
        run_ms = runt.mean_ms(steps)
        rb = run_bytes(A, Ag, N_DOWN, M)
        return {"M": M, "active": A, "us_per_step": t0.elapsed_time(t1) * 1000.0 / steps,
                "us_run": run_ms * 1000.0, "run_GBps": rb / (run_ms * 1e-3) / 1e9}

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- the timed step: 50 % ----------------
    torch.cuda.synchronize()
    main_res = measure(0.5, args.steps, args.warmup)
    sweep = {"p50": main_res}
    batched = []
    if not args.quick:
        for p in (0.7, 0.9):
            sweep[f"p{int(p * 100)}"] = measure(p, args.steps, args.warmup)
        sweep["dense"] = measure(0.0, args.steps, args.warmup, dense=True)
        for M in (1, 2, 4, 8, 16):
            batched.append(measure_batched(M, max(20, args.steps // 4), max(5, args.warmup // 4)))
        dense_us = sweep["dense"]["us_run"]
        for k in ("p50", "p70", "p90"):
            sweep[k]["speedup_vs_dense_int4"] = dense_us / sweep[k]["us_per_step"]

    # ---------------- HBM traffic from committed counters ----------------
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256_16") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")

    # ---------------- CPU baseline: the oracle on the host ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t = synth.percentile_threshold(x, 0.5)
        n_calls, t_start = 0, time.perf_counter()
        while True:
            oracle.gemv_masked(q, s, z, x, t)
            n_calls += 1
            if time.perf_counter() - t_start > 10.0 or n_calls >= 50:
                break
        el = time.perf_counter() - t_start
        cpu = {"value": el / n_calls * 1e6, "unit": "us/call", "cores": 1, "kind": "oracle",
               "sample": f"{n_calls} full calls of the fp64 oracle (threshold, union, per-column "
                         f"dequantize and accumulate) on the 14336->4096 @50% input; "
                         f"single-threaded NumPy"}

    rb = main_res["run_GBps"]
    out = {
        "metric": "µs/call + effective HBM GB/s (% of peak), sparse int4 GEMV 14336→4096 @50/90%",
        "value": round(main_res["us_per_step"], 3),
        "unit": "us/call",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_res["us_per_step"] / 1000.0,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xfp16->fp32",
        "data": "synthetic (seeded Gaussian weights quantized to int4 g128; x = silu(g)*u)",
        "config": {"workload": "Llama-3-8B-shaped down_proj 14336->4096, batch 1, int4 g128, "
                               "50% magnitude sparsity (step = gather + sparse GEMV)",
                   "K": K_DOWN, "N": N_DOWN, "sparsity": 0.5, "weight_copies_rotated": R},
        "roofline": {"bound": "hbm", "kernel": "k_sp (sparse GEMV, M=1)",
                     "achieved": round(rb, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(rb / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": main_res["run_bytes"],
                     "avg_launch_us": round(main_res["us_run"], 3)},
        "cpu_baseline": cpu,
        "sweep": sweep,
        "batched_p70": batched,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
