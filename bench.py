"""Benchmark of the dynamically sparse int4 GEMV on one MI355X.

Workload: the Llama-3-8B-shaped down projection, K = 14336 inputs ->
N = 4096 outputs, int4 group-128 weights ~N(0, 0.02), activation
x = silu(g) * u with g, u ~N(0, 1), magnitude-thresholded at 50 % (the
step); 70 % and 90 %, the two-launch path (gather + run), the dense int4
GEMV, the batched M = 1..16 union variant, the Llama-3-8B decode layer, a
2048 x 2048 matrix and the Llama-3-70B MLP shapes (gate 8192 -> 28672, down
28672 -> 8192 at 50 % and 90 %) are measured beside it.  Synthetic, seeded
data.

One step = one pass of the hot path on one activation vector: threshold,
compact into the ascending list of active indices (written, with its
count) and the sparse GEMV over those columns - one launch of
sgemv_run_fused.  Every call reads the weights of the next of R packed
copies, R chosen so that at least 1 GiB of other weight bytes is read
between two uses of one copy, and a 1 GiB read of a scratch buffer precedes
every timed replay: neither the L2 nor the 256 MB Infinity Cache can serve
the weights, whatever the step count.  Inputs are resident in HBM before timing.

Prints one JSON line.  `value` is microseconds per step (lower is better).
`roofline` gives, for the step's kernel, the algorithmic bytes of one
launch divided by its average duration, against the 8 TB/s HBM peak and
against the read ceiling measured in the same process (a 2 GiB sequential
stream).  The K timed steps are one HIP graph replay (launches back to back,
as in a decode loop) bracketed by HIP events on the stream the kernels run
on; the warm-up steps are graph replays too, so that a kernel trace of the
run holds replayed dispatches only.
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
MFMA_FP16_PEAK_TFLOPS = 2500.0   # dense fp16 matrix-core peak of MI355X
ROTATE_BYTES = 1 << 30          # other weight bytes read between two uses of one copy
FLUSH_BYTES = 1 << 30           # scratch read before every timed replay
STREAM_BYTES = 2 << 30          # the sequential read ceiling's buffer
K_DOWN, N_DOWN = 14336, 4096
KERNEL_SRC = os.path.join(ROOT, "activation_sparse_bit_amd", "csrc", "sgemv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_fs_down14336_p50_traffic.json")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def gemv_bytes(A: int, Ag: int, N: int, M: int = 1) -> int:
    """Algorithmic bytes of the sparse GEMV over a given list: listed weight
    columns (N/2 bytes each), scale+zero of every touched group (4 bytes per
    output), the list, the gathered activations and the fp16 output."""
    return A * N // 2 + Ag * N * 4 + A * 4 + M * A * 2 + M * N * 2


def gather_bytes(K: int, A: int, M: int = 1) -> int:
    """Threshold + compact: the activations, the list and its count."""
    return M * K * 2 + A * 4 + 4


def fused_bytes(A: int, Ag: int, N: int, K: int, M: int = 1, with_list: bool = True, z4: bool = False,
                ng: bool = False) -> int:
    """One fused step: weight columns and metadata as above (2.5 instead of
    4 bytes per output and touched group with the compact metadata; with
    groups along N, 4 bytes per active column and 128 outputs), every
    activation once, the list and count (when written) and the output."""
    md = A * (N // 128) * 4 if ng else Ag * N * 5 // 2 if z4 else Ag * N * 4
    return A * N // 2 + md + M * K * 2 + (A * 4 + 4 if with_list else 0) + M * N * 2


def touched_groups(idx: np.ndarray) -> int:
    return int(np.unique(np.asarray(idx) // 128).size)


CPU_SCRIPT = r"""
import json, os, sys, time
sys.path.insert(0, sys.argv[1])
import numpy as np
import oracle, synth
K, N, runs, calls = 14336, 4096, int(sys.argv[2]), int(sys.argv[3])
q, s, z = synth.quantized_weights(0, N, K, 0.02)
x = synth.glu_activation(0, K)
t = synth.percentile_threshold(x, 0.5)
oracle.gemv_masked(q, s, z, x, t)            # warm-up call
per, cpu_wall = [], []
for r in range(runs):
    w0, c0 = time.perf_counter(), time.process_time()
    for _ in range(calls):
        oracle.active_indices(x, t)
        oracle.gemv_masked(q, s, z, x, t)
    w1, c1 = time.perf_counter(), time.process_time()
    per.append((w1 - w0) / calls)
    cpu_wall.append((c1 - c0) / (w1 - w0))
print(json.dumps({"per_call_s": per, "cpu_per_wall": cpu_wall}))
"""


def cpu_baseline(runs: int = 5, calls: int = 20) -> dict:
    """The fp64 oracle (threshold, compact, per-column dequantize and
    accumulate) on the step's input, in a child process whose OpenMP / BLAS
    thread counts are set to the host cores this process may use: `runs`
    runs of `calls` calls, the median of the runs' per-call times.  `cores`
    is the threads it actually kept busy (process CPU time over wall time,
    rounded): NumPy's element-wise work runs on one."""
    import subprocess
    n = len(os.sched_getaffinity(0))
    env = dict(os.environ)
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        env[k] = str(n)
    r = subprocess.run([sys.executable, "-c", CPU_SCRIPT, ROOT, str(runs), str(calls)], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, check=True)
    res = json.loads(r.stdout.strip().splitlines()[-1])
    per = sorted(res["per_call_s"])
    used = float(np.median(res["cpu_per_wall"]))
    return {"value": float(np.median(per)) * 1e6, "unit": "us/call", "cores": max(1, round(used)),
            "kind": "oracle",
            "sample": (f"median of {runs} runs x {calls} full calls of the fp64 oracle (threshold, compact, "
                       f"per-column dequantize and accumulate) on the 14336->4096 @50% input; "
                       f"OMP/OpenBLAS/MKL threads = {n} (host cores available); "
                       f"measured CPU/wall = {used:.2f}"),
            "runs_us_per_call": [p * 1e6 for p in res["per_call_s"]]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="only the timed step (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy three times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (there is no multi-GPU path); use --gpus 1"}))
        sys.exit(2)

    import torch

    import synth
    from activation_sparse_bit_amd import sgemv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def rotation(touched_bytes: int) -> int:
        """Copies needed so that at least ROTATE_BYTES of other weight bytes
        are read between two uses of one copy."""
        return max(2, 1 + -(-ROTATE_BYTES // max(1, touched_bytes)))

    # ---------------- inputs, resident in HBM ----------------
    q, s, z = synth.quantized_weights(0, N_DOWN, K_DOWN, 0.02)
    desc, blob = sgemv.sgemv_pack_layout(q, s, z)
    blob_d = torch.from_numpy(blob).to(dev)
    # the 90 % step touches the fewest bytes: enough copies for it serve every step
    x_probe = synth.glu_activation(0, K_DOWN)
    A90 = int(np.count_nonzero(np.abs(x_probe.astype(np.float32)) >= np.float32(synth.percentile_threshold(x_probe, 0.9))))
    R = rotation(fused_bytes(A90, K_DOWN // 128, N_DOWN, K_DOWN))
    copies = [blob_d] + [blob_d.clone() for _ in range(R - 1)]
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)

    def flush():
        """Read FLUSH_BYTES (a max reduction with ordinary loads): the L2 and
        the Infinity Cache then hold the flush buffer's lines, and no dirty
        data is left to be written back while the next kernels run.  (An
        int32 sum would first widen the buffer into a 2 GiB int64 copy, and
        the dirty lines of that copy slowed the replay right after it by
        ~5 %.)"""
        flush_buf.max()
    flush()                      # loads the reduction kernel now: its first call
    torch.cuda.synchronize()     # waits ~20 ms on the host, with the GPU idle
    ws = torch.zeros(max(sgemv.sgemv_workspace_bytes(desc, 16), 256), dtype=torch.uint8, device=dev)

    x = synth.glu_activation(0, K_DOWN)
    xd = torch.from_numpy(x).to(dev)
    idx = torch.zeros(K_DOWN, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    y = torch.empty(N_DOWN, dtype=torch.float16, device=dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def graph_time(launches, steps, warmup, spread=None, spread_replays=5):
        """Capture `steps` steps (each step calls every launch with the step
        number, on the current stream) in one HIP graph; replay it at least
        three times and until at least `warmup` steps have run (untimed; the
        first replays of a new graph ran slower than later ones), then
        synchronise, enqueue a read of the 1 GiB flush buffer and time one
        replay right behind it with HIP events on the replay stream, and
        synchronise again.  The flush keeps the weights out of every cache;
        enqueuing it just before the timed steps keeps the GPU busy up to
        them, as in a decode loop (after an idle wait for the host, the first
        timed steps ran up to 15 % slower).  Returns microseconds per step.  With a dict
        `spread`, `spread_replays` more replays after the timed one (each
        after a flush) fill it with the p10 / p50 / p90 of their microseconds
        per step.  A graph replay puts the launches back to back, as a decode
        loop does; eager Python launches would leave the GPU waiting for the
        host."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                for f in launches:
                    f(i)
        for _ in range(max(3, -(-warmup // steps))):   # upload and warm-up replays, untimed
            g.replay()
        torch.cuda.synchronize()
        flush()                  # enqueued right before the timed replay: cold weights, busy GPU
        t0, t1 = ev(), ev()
        cur = torch.cuda.current_stream()
        t0.record(cur)
        g.replay()
        t1.record(cur)
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1000.0 / steps
        if spread is not None:   # more replays, after the timed one, for the spread
            per = []
            for _ in range(spread_replays):
                flush()
                a, b = ev(), ev()
                a.record(cur)
                g.replay()
                b.record(cur)
                torch.cuda.synchronize()
                per.append(a.elapsed_time(b) * 1000.0 / steps)
            q = np.percentile(per, [10, 50, 90])
            spread.update({"p10": float(q[0]), "p50": float(q[1]), "p90": float(q[2]),
                           "replays": spread_replays, "steps_per_replay": steps})
        del g
        return us

    def eager_latency(launch, n=50):
        """Mean duration of single launches issued one at a time (events
        around each, GPU idle in between): the latency of one call."""
        ms = []
        for i in range(n):
            a, b = ev(), ev()
            cur = torch.cuda.current_stream()
            a.record(cur)
            launch(i)
            b.record(cur)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.mean(ms) * 1000.0)

    def cold_latency(launch, n=20):
        """Single calls with the caches cold: a 1 GiB scratch read before
        each (so neither L2 nor the Infinity Cache holds anything of the
        call), then HIP events around the call.  Returns p10/p50/p90 in
        microseconds."""
        ms = []
        for i in range(n + 2):
            flush()
            a, b = ev(), ev()
            cur = torch.cuda.current_stream()
            a.record(cur)
            launch(i)
            b.record(cur)
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(a.elapsed_time(b) * 1000.0)
        q = np.percentile(ms, [10, 50, 90])
        return {"p10": float(q[0]), "p50": float(q[1]), "p90": float(q[2]), "calls": n}

    def list_now():
        c = int(cnt.item())
        lst = idx[:c].cpu().numpy()
        return c, touched_groups(lst)

    def measure_fused(p, steps, warmup, with_list=True, latency=False, cold=False):
        t = synth.percentile_threshold(x, p)
        il, cl = (idx, cnt) if with_list else (None, None)
        f = lambda i: sgemv.sgemv_run_fused(desc, copies[i % R], xd, [t], y, ws, il, cl)
        spread = {} if latency else None
        us = graph_time([f], steps, warmup, spread=spread)
        sgemv.sgemv_run_fused(desc, copies[0], xd, [t], y, ws, idx, cnt)
        A, Ag = list_now()
        fb = fused_bytes(A, Ag, N_DOWN, K_DOWN, with_list=with_list)
        out = {"p": p, "active": A, "groups_touched": Ag, "us_per_step": us, "bytes": fb,
               "GBps": fb / (us * 1e-6) / 1e9, "frac_hbm_peak": fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        if latency:
            out["replay_spread_us_per_step"] = spread
            out["single_call_latency_us"] = eager_latency(f)
        if latency or cold:
            out["cold_single_call_us"] = cold_latency(f)
        return out

    def measure_fused_z4(ps, steps, warmup):
        """The step on the same matrix packed with compact metadata (layout
        version 2: fp16 scales, 4-bit zero-points)."""
        d2, b2 = sgemv.sgemv_pack_layout_z4(q, s, z)
        R2 = rotation(fused_bytes(A90, K_DOWN // 128, N_DOWN, K_DOWN, z4=True))
        bd = torch.from_numpy(b2).to(dev)
        cps = [bd] + [bd.clone() for _ in range(R2 - 1)]
        res = {}
        for p in ps:
            t = synth.percentile_threshold(x, p)
            us = graph_time([lambda i: sgemv.sgemv_run_fused(d2, cps[i % R2], xd, [t], y, ws, idx, cnt)],
                            steps, warmup)
            A, Ag = list_now()
            fb = fused_bytes(A, Ag, N_DOWN, K_DOWN, z4=True)
            res[f"fused_p{int(p * 100)}_z4"] = {"p": p, "active": A, "groups_touched": Ag, "us_per_step": us,
                                               "bytes": fb, "GBps": fb / (us * 1e-6) / 1e9,
                                               "frac_hbm_peak": fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        del cps, bd
        return res

    def measure_fused_ng(ps, steps, warmup):
        """The step on the same draw quantized with groups along N (layout
        version 3: one scale and zero-point per input column and 128
        outputs, read only with an active column)."""
        q3, s3, z3 = synth.quantized_weights_ng(0, N_DOWN, K_DOWN, 0.02)
        d3, b3 = sgemv.sgemv_pack_layout_ng(q3, s3, z3)
        R3 = rotation(fused_bytes(A90, K_DOWN // 128, N_DOWN, K_DOWN, ng=True))
        bd = torch.from_numpy(b3).to(dev)
        cps = [bd] + [bd.clone() for _ in range(R3 - 1)]
        res = {}
        for p in ps:
            t = synth.percentile_threshold(x, p)
            us = graph_time([lambda i: sgemv.sgemv_run_fused(d3, cps[i % R3], xd, [t], y, ws, idx, cnt)],
                            steps, warmup)
            A, Ag = list_now()
            fb = fused_bytes(A, Ag, N_DOWN, K_DOWN, ng=True)
            res[f"fused_p{int(p * 100)}_ng"] = {"p": p, "active": A, "groups_touched": Ag, "us_per_step": us,
                                               "bytes": fb, "GBps": fb / (us * 1e-6) / 1e9,
                                               "frac_hbm_peak": fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        del cps, bd
        return res

    def measure_split(p, steps, warmup, dense=False, cold=False):
        t = synth.percentile_threshold(x, p)
        gat = lambda i: sgemv.sgemv_gather_indices(xd, [t], idx, cnt)
        run = lambda i: sgemv.sgemv_run(desc, copies[i % R], xd, None if dense else idx,
                                        None if dense else cnt, y, ws)
        out = {"p": p}
        if dense:
            A, Ag = K_DOWN, K_DOWN // 128
            out["us_per_step"] = graph_time([run], steps, warmup)
            rb = K_DOWN * N_DOWN // 2 + Ag * N_DOWN * 4 + K_DOWN * 2 + N_DOWN * 2
            run_us = out["us_per_step"]
        else:
            out["us_per_step"] = graph_time([gat, run], steps, warmup)
            out["gather_us"] = graph_time([gat], steps, warmup)
            run_us = graph_time([run], steps, warmup)
            A, Ag = list_now()
            rb = gemv_bytes(A, Ag, N_DOWN)
            out["gather_bytes"] = gather_bytes(K_DOWN, A)
        if cold:
            out["cold_single_call_us"] = cold_latency(run)
        out.update({"active": A, "groups_touched": Ag, "run_us": run_us, "run_bytes": rb,
                    "run_GBps": rb / (run_us * 1e-6) / 1e9,
                    "run_frac_hbm_peak": rb / (run_us * 1e-6) / 1e9 / HBM_PEAK_GBPS})
        return out

    def measure_batched(M, steps, warmup):
        X = np.stack([synth.glu_activation(m, K_DOWN) for m in range(M)])
        ts = [synth.percentile_threshold(X[m], 0.7) for m in range(M)]
        Xd = torch.from_numpy(X).to(dev)
        Y = torch.empty((M, N_DOWN), dtype=torch.float16, device=dev)
        gat = lambda i: sgemv.sgemv_gather_indices(Xd, ts, idx, cnt)
        run = lambda i: sgemv.sgemv_run_batched(desc, copies[i % R], Xd, ts, idx, cnt, Y, ws)
        step_us = graph_time([gat, run], steps, warmup)
        run_us = graph_time([run], steps, warmup)
        A, Ag = list_now()
        rb = gemv_bytes(A, Ag, N_DOWN, M)
        res = {"M": M, "active_union": A, "us_per_step": step_us, "run_us": run_us,
               "run_GBps": rb / (run_us * 1e-6) / 1e9}
        # the fused call: one or two rows on the vector units, 3 to 16 on the matrix cores
        fus = graph_time(
            [lambda i: sgemv.sgemv_run_fused(desc, copies[i % R], Xd, ts, Y, ws, idx, cnt)], steps, warmup)
        fb = fused_bytes(A, Ag, N_DOWN, K_DOWN, M=M)
        flops = 2.0 * M * A * N_DOWN        # one multiply-add per row, union column and output
        res.update({"fused_us_per_step": fus, "fused_bytes": fb,
                    "fused_GBps": fb / (fus * 1e-6) / 1e9,
                    "fused_frac_hbm_peak": fb / (fus * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                    "fused_TFLOPs": flops / (fus * 1e-6) / 1e12,
                    "fused_frac_fp16_mfma_peak": flops / (fus * 1e-6) / 1e12 / MFMA_FP16_PEAK_TFLOPS})
        if M >= 3:    # the union's weight runs read alone, with the one-row grid
            lst = idx[:A].cpu().numpy().astype(np.int32)
            lus = listed_read_us(lst, K_DOWN, N_DOWN, copies, R, desc.w_off, steps, warmup)
            res.update({"union_listed_read_us": lus,
                        "union_listed_read_frac_hbm_peak": (A * N_DOWN // 2) / (lus * 1e-6) / 1e9 / HBM_PEAK_GBPS})
        if M == 16:   # the same call on the groups-along-N layout (version 3)
            q3, s3, z3 = synth.quantized_weights_ng(0, N_DOWN, K_DOWN, 0.02)
            d3, b3 = sgemv.sgemv_pack_layout_ng(q3, s3, z3)
            R3 = rotation(fused_bytes(A, Ag, N_DOWN, K_DOWN, M=M, ng=True))
            bd = torch.from_numpy(b3).to(dev)
            c3 = [bd] + [bd.clone() for _ in range(R3 - 1)]
            f3 = graph_time([lambda i: sgemv.sgemv_run_fused(d3, c3[i % R3], Xd, ts, Y, ws, idx, cnt)],
                            steps, warmup)
            fb3 = fused_bytes(A, Ag, N_DOWN, K_DOWN, M=M, ng=True)
            res.update({"fused_ng_us_per_step": f3, "fused_ng_bytes": fb3,
                        "fused_ng_frac_hbm_peak": fb3 / (f3 * 1e-6) / 1e9 / HBM_PEAK_GBPS})
            del c3, bd
        return res

    def measure_layer(steps, warmup):
        """Llama-3-8B-shaped decode layer at 50 % on every projection input:
        q/k/v and gate/up packed as one matrix each (4 fused launches), each
        projection on its own (7 fused launches), and the two-launch path
        (4 gathers + 7 runs)."""
        wl = synth.workload("layer-8b")
        P = {p.name: p for p in wl.projections}
        W = {n: synth.quantized_weights(P[n].weight_seed, P[n].N, P[n].K, P[n].sigma) for n in P}
        X = {k: synth.activation(*v) for k, v in wl.inputs.items()}
        T = {k: synth.percentile_threshold(v, 0.5) for k, v in X.items()}
        Xd = {k: torch.from_numpy(v).to(dev) for k, v in X.items()}
        groups = [("qkv", ("q", "k", "v"), "x_attn"), ("o", ("o",), "x_o"),
                  ("gate_up", ("gate", "up"), "x_mlp"), ("down", ("down",), "x_down")]
        fused = {g: sgemv.FusedProjections([(n, *W[n]) for n in names], device=dev, max_batch=1)
                 for g, names, _ in groups}
        single = {n: sgemv.PackedMatrix(*W[n], device=dev, max_batch=1) for n in P}
        touched = 0
        for g, names, xin in groups:
            A = int(np.count_nonzero(np.abs(X[xin].astype(np.float32)) >= np.float32(T[xin])))
            touched += fused_bytes(A, fused[g].K // 128, fused[g].N, fused[g].K)
        RL = rotation(touched)
        fcopies = {g: [f.matrix.blob] + [f.matrix.blob.clone() for _ in range(RL - 1)] for g, f in fused.items()}
        scopies = {n: [m.blob] + [m.blob.clone() for _ in range(RL - 1)] for n, m in single.items()}
        Y = {g: torch.empty(f.N, dtype=torch.float16, device=dev) for g, f in fused.items()}
        Ys = {n: torch.empty(m.N, dtype=torch.float16, device=dev) for n, m in single.items()}
        lidx = torch.zeros(14336, dtype=torch.int32, device=dev)
        lcnt = torch.zeros(1, dtype=torch.int32, device=dev)

        def fz(g, xin):
            f = fused[g]
            return lambda i: sgemv.sgemv_run_fused(f.matrix.desc, fcopies[g][i % RL], Xd[xin], [T[xin]], Y[g],
                                                   f.matrix.workspace, lidx, lcnt)

        def sz(n):
            m, xin = single[n], P[n].input_name
            return lambda i: sgemv.sgemv_run_fused(m.desc, scopies[n][i % RL], Xd[xin], [T[xin]], Ys[n],
                                                   m.workspace, lidx, lcnt)

        def gz(xin):
            return lambda i: sgemv.sgemv_gather_indices(Xd[xin], [T[xin]], lidx, lcnt)

        def rz(n):
            m, xin = single[n], P[n].input_name
            return lambda i: sgemv.sgemv_run(m.desc, scopies[n][i % RL], Xd[xin], lidx, lcnt, Ys[n], m.workspace)

        fused_us = graph_time([fz(g, xin) for g, _, xin in groups], steps, warmup)
        sep_us = graph_time([sz(n) for n in P], steps, warmup)
        split = []
        for g, names, xin in groups:
            split.append(gz(xin))
            split += [rz(n) for n in names]
        split_us = graph_time(split, steps, warmup)
        nbytes = 0
        for g, names, xin in groups:
            f = fused[g]
            A = int(np.count_nonzero(np.abs(X[xin].astype(np.float32)) >= np.float32(T[xin])))
            nbytes += fused_bytes(A, f.K // 128, f.N, f.K)
        del fcopies, scopies
        return {"projections_packed_by_input_us": fused_us, "launches": 4,
                "each_projection_fused_us": sep_us, "two_launch_path_us": split_us,
                "bytes": nbytes, "GBps": nbytes / (fused_us * 1e-6) / 1e9}

    def measure_shape(K, N, sigma, j, kind, ps, steps, warmup):
        """One matrix of another configuration: the fused step at each
        sparsity (list written) and the dense int4 GEMV, with their
        algorithmic bytes and the fraction of the HBM peak."""
        qq, ss, zz = synth.quantized_weights(j, N, K, sigma)
        dsc, bl = sgemv.sgemv_pack_layout(qq, ss, zz)
        del qq, ss, zz
        xv = synth.activation(kind, 0, K)
        pmax = max(ps)
        Amin = int(np.count_nonzero(np.abs(xv.astype(np.float32)) >= np.float32(synth.percentile_threshold(xv, pmax))))
        RR = rotation(fused_bytes(Amin, K // 128, N, K))
        bd = torch.from_numpy(bl).to(dev)
        cps = [bd] + [bd.clone() for _ in range(RR - 1)]
        w = torch.zeros(max(sgemv.sgemv_workspace_bytes(dsc, 1), 256), dtype=torch.uint8, device=dev)
        xdv = torch.from_numpy(xv).to(dev)
        iv = torch.zeros(K, dtype=torch.int32, device=dev)
        cv = torch.zeros(1, dtype=torch.int32, device=dev)
        yv = torch.empty(N, dtype=torch.float16, device=dev)
        res = {"K": K, "N": N, "weight_copies_rotated": RR}
        for pp in ps:
            t = synth.percentile_threshold(xv, pp)
            us = graph_time([lambda i: sgemv.sgemv_run_fused(dsc, cps[i % RR], xdv, [t], yv, w, iv, cv)],
                            steps, warmup)
            A = int(cv.item())
            Ag = touched_groups(iv[:A].cpu().numpy())
            fb = fused_bytes(A, Ag, N, K)
            res[f"fused_p{int(pp * 100)}"] = {"active": A, "groups_touched": Ag, "us_per_step": us, "bytes": fb,
                                             "GBps": fb / (us * 1e-6) / 1e9,
                                             "frac_hbm_peak": fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        dus = graph_time([lambda i: sgemv.sgemv_run(dsc, cps[i % RR], xdv, None, None, yv, w)], steps, warmup)
        db = K * N // 2 + (K // 128) * N * 4 + K * 2 + N * 2
        res["dense_int4"] = {"us_per_step": dus, "bytes": db, "GBps": db / (dus * 1e-6) / 1e9,
                             "frac_hbm_peak": db / (dus * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        for pp in ps:
            res[f"fused_p{int(pp * 100)}"]["speedup_vs_dense_int4"] = dus / res[f"fused_p{int(pp * 100)}"]["us_per_step"]
        # each call's own ceiling: the same weight runs read and nothing else
        for pp in ps + (0.0,):
            if pp > 0.0:
                t = synth.percentile_threshold(xv, pp)
                lst = np.flatnonzero(np.abs(xv.astype(np.float32)) >= np.float32(t)).astype(np.int32)
                r = res[f"fused_p{int(pp * 100)}"]
            else:
                lst, r = np.arange(K, dtype=np.int32), res["dense_int4"]
            lus = listed_read_us(lst, K, N, cps, RR, dsc.w_off, steps, warmup)
            r["listed_read_us"] = lus
            r["listed_read_frac_hbm_peak"] = (len(lst) * N // 2) / (lus * 1e-6) / 1e9 / HBM_PEAK_GBPS
            r["listed_read_over_call"] = lus / r["us_per_step"]
        del cps, bd
        torch.cuda.empty_cache()
        return res

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def stream_ceiling(reps=5):
        """Sequential read ceiling: a STREAM_BYTES buffer read with 16-byte
        non-temporal loads over the whole chip (measurement-only kernel),
        best of `reps` launches, each after the flush."""
        import ctypes
        bl = ctypes.CDLL(os.path.join(ROOT, "activation_sparse_bit_amd", "lib", "libsgemv_bench.so"))
        bl.sgemv_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        sink = torch.zeros(1024, dtype=torch.int32, device=dev)
        cur = torch.cuda.current_stream()
        best = 1e30
        for r in range(reps + 1):
            flush()
            a, b = ev(), ev()
            a.record(cur)
            if bl.sgemv_bench_stream_read(buf.data_ptr(), STREAM_BYTES, sink.data_ptr(), cur.cuda_stream) != 0:
                raise RuntimeError("sgemv_bench_stream_read failed")
            b.record(cur)
            torch.cuda.synchronize()
            if r:
                best = min(best, a.elapsed_time(b) * 1e-3)
        del buf
        return {"GBps": STREAM_BYTES / best / 1e9, "bytes": STREAM_BYTES, "us": best * 1e6,
                "kernel": "sequential 16-byte non-temporal loads, 4096 x 512 threads, best of %d" % reps}

    def listed_read_us(lst, K, N, cps, RR, w_off, steps, warmup):
        """Graph-timed microseconds per launch of the weight reads alone of a
        one-row call over the ascending list `lst`: for every half tile the
        128-byte run of each listed column, with the GEMV's lanes and grid of
        half tiles x 1024-column segments, and no activations, scales,
        arithmetic or sums (measurement-only kernel), over the same rotated
        copies `cps` as the call it bounds."""
        import ctypes
        bl = ctypes.CDLL(os.path.join(ROOT, "activation_sparse_bit_amd", "lib", "libsgemv_bench.so"))
        bl.sgemv_bench_listed_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        starts = np.searchsorted(lst, np.arange(0, K + 1, 128)).astype(np.int32)
        ld = torch.from_numpy(np.ascontiguousarray(lst, dtype=np.int32)).to(dev)
        sd = torch.from_numpy(starts).to(dev)
        sink = torch.zeros(1024, dtype=torch.int32, device=dev)

        def f(i):
            st = torch.cuda.current_stream().cuda_stream
            if bl.sgemv_bench_listed_read(cps[i % RR].data_ptr() + w_off, sd.data_ptr(), ld.data_ptr(),
                                          K, N, sink.data_ptr(), st) != 0:
                raise RuntimeError("sgemv_bench_listed_read failed")
        return graph_time([f], steps, warmup)

    def listed_read_ceiling(p, steps, warmup):
        """The step's weight reads alone (see listed_read_us)."""
        t = synth.percentile_threshold(x, p)
        lst = np.flatnonzero(np.abs(x.astype(np.float32)) >= np.float32(t)).astype(np.int32)
        us = listed_read_us(lst, K_DOWN, N_DOWN, copies, R, desc.w_off, steps, warmup)
        wb = len(lst) * N_DOWN // 2
        return {"p": p, "active": int(len(lst)), "us_per_launch": us, "weight_bytes": wb,
                "GBps": wb / (us * 1e-6) / 1e9}

    def settle(ms: float = 50.0):
        """Flushes and untimed fused steps for about `ms` milliseconds before the first
        measurement, so that it does not catch the GPU still raising its
        clocks (the first short replay of a fresh process ran up to 20 %
        slower than the same replay a moment later)."""
        t = synth.percentile_threshold(x, 0.5)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(100):
                sgemv.sgemv_run_fused(desc, copies[i % R], xd, [t], y, ws, idx, cnt)
        t_end = time.perf_counter() + ms * 1e-3
        while time.perf_counter() < t_end:
            flush()
            g.replay()
            torch.cuda.synchronize()
        del g

    # ---------------- the timed step: 50 %, fused, list written ----------------
    settle()
    main_res = measure_fused(0.5, args.steps, args.warmup, latency=not args.quick)
    ceiling = stream_ceiling()
    sweep = {"fused_p50": main_res}
    batched = []
    layer = None
    shapes = None
    if not args.quick:
        for p in (0.7, 0.9):
            sweep[f"fused_p{int(p * 100)}"] = measure_fused(p, args.steps, args.warmup, cold=True)
        sweep["fused_p50_no_list"] = measure_fused(0.5, args.steps, args.warmup, with_list=False)
        sweep.update(measure_fused_z4((0.5, 0.9), args.steps, args.warmup))
        sweep.update(measure_fused_ng((0.5, 0.9), args.steps, args.warmup))
        for p in (0.5, 0.7, 0.9):
            sweep[f"split_p{int(p * 100)}"] = measure_split(p, args.steps, args.warmup)
        sweep["dense_int4"] = measure_split(0.0, args.steps, args.warmup, dense=True, cold=True)
        for p in (0.5, 0.9):
            sweep[f"listed_read_p{int(p * 100)}"] = listed_read_ceiling(p, args.steps, args.warmup)
        dense_us = sweep["dense_int4"]["us_per_step"]
        # time against the active fraction (1 - p): least-squares line through
        # the 50 / 70 / 90 % steps; the intercept is the fixed cost of a step
        dens = np.array([1 - sweep[f"fused_p{q}"]["p"] for q in (50, 70, 90)])
        tus = np.array([sweep[f"fused_p{q}"]["us_per_step"] for q in (50, 70, 90)])
        slope, icpt = np.polyfit(dens, tus, 1)
        sweep["time_vs_active_fraction"] = {
            "points": [[float(a), float(b)] for a, b in zip(dens, tus)],
            "slope_us_per_unit": float(slope), "intercept_us": float(icpt),
            "p90_over_p50": float(tus[2] / tus[0]), "bytes_p90_over_p50":
                float(sweep["fused_p90"]["bytes"] / sweep["fused_p50"]["bytes"])}
        for k in ("fused_p50", "fused_p70", "fused_p90", "split_p50", "split_p70", "split_p90"):
            sweep[k]["speedup_vs_dense_int4"] = dense_us / sweep[k]["us_per_step"]
        for M in (1, 2, 4, 8, 16):
            batched.append(measure_batched(M, max(20, args.steps // 4), max(5, args.warmup // 4)))
        layer = measure_layer(max(20, args.steps // 4), max(5, args.warmup // 4))
        st, wu = max(20, args.steps // 2), max(5, args.warmup // 2)
        shapes = {
            "single_2048": measure_shape(2048, 2048, 0.02, 0, "plain", (0.5,), st, wu),
            "mlp70b_gate_8192_28672": measure_shape(8192, 28672, 0.015, 0, "plain", (0.5, 0.9), st, wu),
            "mlp70b_down_28672_8192": measure_shape(28672, 8192, 0.015, 2, "glu", (0.5, 0.9), st, wu),
        }

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
        cpu = cpu_baseline()

    kmean = main_res["us_per_step"]   # one launch per step
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
                               "50% magnitude sparsity; step = threshold + compact (list written) + "
                               "sparse GEMV in one launch",
                   "K": K_DOWN, "N": N_DOWN, "sparsity": 0.5, "weight_copies_rotated": R},
        "roofline": {"bound": "hbm", "kernel": "k_fs<1, 1, 8, false> (fused threshold + compact + sparse GEMV; layout version 1)",
                     "achieved": round(main_res["GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(main_res["frac_hbm_peak"], 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": main_res["bytes"],
                     "avg_launch_us": round(kmean, 3),
                     "ceiling_GBps": round(ceiling["GBps"], 1),
                     "frac_of_ceiling": round(main_res["GBps"] / ceiling["GBps"], 4),
                     "ceiling": ceiling},
        "cpu_baseline": cpu,
        "sweep": sweep,
        "batched_p70": batched,
        "layer_8b_p50": layer,
        "other_configs": shapes,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
