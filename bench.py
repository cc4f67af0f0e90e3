"""Benchmark of the stabilized parallel mLSTM forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full call of mlstm_parallel_fwd on one batch of synthetic
inputs that are resident in HBM before timing starts.  The default workload
is the ~125M-parameter xLSTM mLSTM layer (B=8, NH=4, T=2048, d=384, bf16
q/k/v), where the call is a single launch of the causal tile kernel that
scans its head's gates in its prologue (no workspace); longer sequences run
the gate scan and the tile kernel as two launches on a stream-ordered
workspace.  Prints ONE JSON line.

Metric: TFLOP/s with the causal work counted as 2 * T^2 * d per head.
The "roofline" object gives the dominant kernel's average duration from
HIP events on the stream it is launched on (on the default workload the
call's only kernel, so the events bracket the timed steps themselves),
against the bf16 dense MFMA peak; "staged" times the two-launch form of the
same pass.  The "cpu_baseline" object times the CPU oracle
(float64 NumPy) on a bounded sample of the same workload on this host.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU ("2.5 PFLOP/s")
PEAK_HBM_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "tiles_pairs_fused_xlstm125m_counters.json")
COPY_BYTES = 512 << 20
TILE_SRC = os.path.join(ROOT, "linear_recurrent_sequence_amd", "csrc", "tiles_pairs.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle-s", type=float, default=1.0,
                   help="seconds of untimed calls before the warmup steps: under sustained "
                        "load the GPU clock takes a few hundred ms to settle")
    p.add_argument("--workload", default="xlstm125m_layer")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-backward", action="store_true",
                   help="skip timing the backward pass")
    p.add_argument("--no-long-context", action="store_true",
                   help="skip the tile-skipping comparison on the 16K stress workload")
    p.add_argument("--no-wide", action="store_true",
                   help="skip the 1.3B-shaped layers (sub-heads of 512, true heads of 1024)")
    p.add_argument("--no-fp32", action="store_true",
                   help="skip the 125M-shaped layer with float32 inputs")
    p.add_argument("--cpu-budget-s", type=float, default=15.0,
                   help="approximate CPU seconds for the oracle sample")
    p.add_argument("--oracle-budget-s", type=float, default=6.0,
                   help="approximate CPU seconds of oracle per named workload")
    p.add_argument("--no-per-config", action="store_true",
                   help="skip the whole-call timing and oracle timing of every named workload")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 512 MiB float32 device copy (a torch neg kernel) "
                        "three times, the reference for rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return p.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counters_record():
    """The committed rocprofv3 counter record of the tile kernel, or None if
    absent or taken on a different kernel source."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("source_sha") == source_sha(TILE_SRC) else None


def traffic_from_counters(launch_bytes_key="bytes_per_launch"):
    """HBM bytes per launch of the tile kernel from committed rocprofv3 counter
    runs, or None if they are absent or were taken on a different kernel source."""
    rec = counters_record()
    return rec.get(launch_bytes_key) if rec else None


def cpu_baseline(x, budget_s):
    """Time the float64 oracle head by head until the budget is spent."""
    import numpy as np
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in info
                if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or blas
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    spec = x["spec"]
    B, NH, T, d = spec["B"], spec["NH"], spec["T"], spec["d"]
    done = 0
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(NH):
            sl = (slice(b, b + 1), slice(h, h + 1))
            oracle.forward_stabilized(x["q"][sl], x["k"][sl], x["v"][sl],
                                      x["igate"][sl], x["fgate"][sl])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    flops = 2.0 * T * T * d * done
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "host_cores": len(os.sched_getaffinity(0)), "blas": blas, "kind": "oracle",
            "sample": f"{done} of {B * NH} heads (full T={T}, d={d} each), float64 NumPy, "
                      f"{dt:.1f} s"}


def single_launch(spec):
    """Whether mlstm_parallel_fwd runs this workload as one kernel launch (the
    library's condition: bf16, d <= 512, T <= 2048 and divisible by 4)."""
    return (spec["dtype"] == "bf16" and spec["d"] <= 512 and spec["T"] <= 2048
            and spec["T"] % 4 == 0)


SCAN_MIN_BYTES_PER_POSITION = 16  # least traffic of the scan: f~, i~ in; m and one prefix term out


def scan_kernel_bytes(H, T):
    """The gate scan's own algorithmic bytes: f~, i~ in (8 B/position); m,
    R, C (float64), e out (24 B/position); two float64 bounds per 32 positions."""
    return H * T * (4 + 4 + 4 + 8 + 8 + 4) + 2 * H * (T // 32) * 8


NAMED = ("tiny_fp32", "small_bf16", "xlstm125m_layer", "xlstm1p3b_layer", "long_context_16k")


def per_config(torch, mlstm, workloads, dev, oracle_budget_s, with_oracle, calls=100,
               settle_s=0.5):
    """Every named workload: the whole mlstm_parallel_fwd call (median of
    ``calls`` calls, each between HIP events on its stream) and the CPU oracle
    (float64 NumPy) on the host, the full workload where it takes seconds,
    else a stated sample of heads."""
    import numpy as np
    out = []
    for name in NAMED:
        x = workloads.make(name, seed=0)
        spec = x["spec"]
        B, NH, T, d = spec["B"], spec["NH"], spec["T"], spec["d"]
        dt = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32
        q, k, v = (torch.from_numpy(x[n]).to(dev).to(dt).contiguous() for n in ("q", "k", "v"))
        ig = torch.from_numpy(x["igate"]).to(dev).contiguous()
        fg = torch.from_numpy(x["fgate"]).to(dev).contiguous()
        h = torch.empty_like(q)
        m = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
        n = torch.empty_like(m)
        # untimed calls until the clock has settled (the oracle timing of the
        # previous workload left the GPU idle), then 10 warm-up calls
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < settle_s:
            for _ in range(10):
                mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
            torch.cuda.synchronize()
        for _ in range(10):
            mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
        stream = torch.cuda.current_stream(dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(calls)]
        for a, b in evs:
            a.record(stream)
            mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
            b.record(stream)
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        med = us[len(us) // 2]
        flops = workloads.counted_flops(B, NH, T, d)
        rec = {"workload": name, "B": B, "NH": NH, "T": T, "d": d, "dtype": spec["dtype"],
               "call_median_us": round(med, 2), "call_min_us": round(us[0], 2),
               "counted_TFLOP/s": round(flops / (med * 1e-6) / 1e12, 3)}
        if with_oracle:
            rec["oracle"] = oracle_timing(x, oracle_budget_s)
            rec["oracle_over_gpu"] = round(rec["oracle"]["seconds_full"] / (med * 1e-6), 0)
        out.append(rec)
    return out


def oracle_timing(x, budget_s):
    """Seconds of the float64 oracle on this workload: heads one at a time
    until the whole workload is done or ``budget_s`` is spent; the full-time
    figure scales the measured heads to all of them (heads are equal work)."""
    import oracle
    spec = x["spec"]
    B, NH = spec["B"], spec["NH"]
    done = 0
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(NH):
            sl = (slice(b, b + 1), slice(h, h + 1))
            oracle.forward_stabilized(x["q"][sl], x["k"][sl], x["v"][sl],
                                      x["igate"][sl], x["fgate"][sl])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    return {"heads_timed": done, "heads": B * NH, "seconds": round(dt, 3),
            "seconds_full": round(dt * B * NH / done, 3),
            "sample": "all heads" if done == B * NH else f"{done} of {B * NH} heads, scaled"}


def long_context_skipping(torch, mlstm, workloads, dev, reps):
    """Stage-2 time on long_context_16k with and without decay-aware skipping."""
    x = workloads.make("long_context_16k", seed=0)
    spec = x["spec"]
    B, NH, T, d = spec["B"], spec["NH"], spec["T"], spec["d"]
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous()
               for n in ("q", "k", "v"))
    ig = torch.from_numpy(x["igate"]).to(dev).contiguous()
    fg = torch.from_numpy(x["fgate"]).to(dev).contiguous()
    ws = mlstm.alloc_workspace(B, NH, T, dev)
    m = mlstm.gate_scan(ig, fg, d, ws)
    h = torch.empty_like(q)
    n = torch.empty_like(m)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for kernel in ("mfma", "mfma_all_tiles"):
        mlstm.causal_tiles(q, k, v, m, ws, kernel=kernel, out=(h, n))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            mlstm.causal_tiles(q, k, v, m, ws, kernel=kernel, out=(h, n))
        e1.record(stream)
        torch.cuda.synchronize()
        out[kernel] = e0.elapsed_time(e1) / reps
    # the whole call (two-pass gate scan + tiles with skipping)
    m2 = torch.empty_like(m)
    for _ in range(3):
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m2, n))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m2, n))
    e1.record(stream)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / reps
    flops = workloads.counted_flops(B, NH, T, d)
    return {"workload": "long_context_16k", "B": B, "NH": NH, "T": T, "d": d,
            "call_ms": round(call_ms, 4),
            "tile_ms_skipping": round(out["mfma"], 4),
            "tile_ms_all_tiles": round(out["mfma_all_tiles"], 4),
            "counted_TFLOP/s_skipping": round(flops / (out["mfma"] * 1e-3) / 1e12, 1),
            "counted_TFLOP/s_all_tiles": round(flops / (out["mfma_all_tiles"] * 1e-3) / 1e12, 1),
            "speedup": round(out["mfma_all_tiles"] / out["mfma"], 2)}


def scan_at_size(torch, mlstm, dev, reps=20, warmup=5):
    """The gate scan alone at 2^26 positions (16384 heads of 4096), where it
    moves enough bytes to show its bandwidth (supplementary).  The untimed
    calls map the 1.6 GB of outputs and let the clock settle."""
    B, NH, T, d = 1024, 16, 4096, 384
    g = torch.Generator(device="cpu").manual_seed(0)
    ig = torch.randn((B, NH, T), generator=g).to(dev)
    fg = (3.0 + torch.randn((B, NH, T), generator=g)).to(dev)
    ws = mlstm.alloc_workspace(B, NH, T, dev)
    m = torch.empty_like(ig)
    for _ in range(warmup):
        mlstm.gate_scan(ig, fg, d, ws, m=m)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        mlstm.gate_scan(ig, fg, d, ws, m=m)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    H = B * NH
    nbytes = scan_kernel_bytes(H, T)
    sbytes = H * T * SCAN_MIN_BYTES_PER_POSITION
    return {"B": B, "NH": NH, "T": T, "positions": H * T, "avg_launch_ms": round(ms, 4),
            "kernel_bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes_16_per_position": sbytes,
            "GB/s_16_per_position": round(sbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_16_per_position": round(sbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def layer_timing(torch, mlstm, workloads, dev, name, reps=50, settle_s=0.5):
    """Whole call and tile kernel alone on another layer shape (default
    kernels), after settle_s seconds of untimed calls for the clock."""
    x = workloads.make(name, seed=0)
    spec = x["spec"]
    B, NH, T, d = spec["B"], spec["NH"], spec["T"], spec["d"]
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16).contiguous()
               for n in ("q", "k", "v"))
    ig = torch.from_numpy(x["igate"]).to(dev).contiguous()
    fg = torch.from_numpy(x["fgate"]).to(dev).contiguous()
    h = torch.empty_like(q)
    m = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    n = torch.empty_like(m)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle_s:
        for _ in range(5):
            mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
        torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
    e1.record(stream)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / reps
    ws = mlstm.alloc_workspace(B, NH, T, dev)
    mlstm.gate_scan(ig, fg, d, ws, m=m)
    e0.record(stream)
    for _ in range(reps):
        mlstm.causal_tiles(q, k, v, m, ws, out=(h, n))
    e1.record(stream)
    torch.cuda.synchronize()
    tile_ms = e0.elapsed_time(e1) / reps
    flops = workloads.counted_flops(B, NH, T, d)
    kernel = "tiles_wide" if d > 512 else ("tiles_pairs" if d <= 384 else "tiles_mfma")
    return {"workload": name, "B": B, "NH": NH, "T": T, "d": d, "kernel": kernel,
            "ms_per_call": round(call_ms, 4),
            "TFLOP/s": round(flops / (call_ms * 1e-3) / 1e12, 1),
            "tile_avg_launch_ms": round(tile_ms, 5),
            "tile_TFLOP/s": round(flops / (tile_ms * 1e-3) / 1e12, 1),
            "tile_frac": round(flops / (tile_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


PEAK_FP32_TFLOPS = 157.3  # MI355X dense float32 matrix (and vector) peak


def fp32_layer_timing(torch, mlstm, workloads, dev, reps=20):
    """The 125M-shaped layer (8 x 4 heads, T = 2048, d = 384) with float32
    inputs: whole call (one launch of the float32 matrix-core tile kernel,
    which scans the gates in its prologue), the two-launch form's tile kernel
    alone, and the float32 vector kernel on the same inputs."""
    spec = dict(B=8, NH=4, T=2048, d=384, dtype="fp32", igate=("normal", 0.0, 1.0),
                fgate=("normal", 3.0, 1.0), name="xlstm125m_layer_fp32")
    x = workloads.make(spec, seed=0)
    B, NH, T, d = 8, 4, 2048, 384
    q, k, v = (torch.from_numpy(x[n]).to(dev).contiguous() for n in ("q", "k", "v"))
    ig = torch.from_numpy(x["igate"]).to(dev).contiguous()
    fg = torch.from_numpy(x["fgate"]).to(dev).contiguous()
    h = torch.empty_like(q)
    m = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    n = torch.empty_like(m)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn, r, settle_s=0.3):
        # untimed calls until the clock has settled (the previous section may
        # have left the GPU idle or running another load)
        t_settle = time.perf_counter()
        while True:  # at least one untimed call
            fn()
            torch.cuda.synchronize()
            if time.perf_counter() - t_settle >= settle_s:
                break
        e0.record(stream)
        for _ in range(r):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / r

    call_ms = timed(lambda: mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n)), reps)
    ws = mlstm.alloc_workspace(B, NH, T, dev)
    mlstm.gate_scan(ig, fg, d, ws, m=m)
    tile_ms = timed(lambda: mlstm.causal_tiles(q, k, v, m, ws, out=(h, n)), reps)
    vec_ms = timed(lambda: mlstm.causal_tiles(q, k, v, m, ws, kernel="vector", out=(h, n)), 2,
                   settle_s=0.0)
    flops = workloads.counted_flops(B, NH, T, d)
    bwd = backward_timing(torch, mlstm, workloads, x, dev, reps=5)
    # the float32 vector passes of the backward on the same inputs
    os.environ["MLSTM_BWD_F32"] = "vector"
    try:
        bwd_vec = backward_timing(torch, mlstm, workloads, x, dev, reps=1)
    finally:
        del os.environ["MLSTM_BWD_F32"]
    return {"workload": spec["name"], "B": B, "NH": NH, "T": T, "d": d, "dtype": "f32",
            "kernel": "tiles_f32_kernel<384> (gate scan fused; output columns split over two "
                      "workgroups)",
            "ms_per_call": round(call_ms, 4),
            "TFLOP/s": round(flops / (call_ms * 1e-3) / 1e12, 2),
            "tile_avg_launch_ms": round(tile_ms, 4),
            "tile_TFLOP/s": round(flops / (tile_ms * 1e-3) / 1e12, 2),
            "peak_fp32": PEAK_FP32_TFLOPS,
            "tile_frac": round(flops / (tile_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4),
            "executed_frac": round(1.5 * flops / (tile_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4),
            "vector_kernel_ms": round(vec_ms, 3),
            "backward": bwd, "backward_vector_passes_ms": bwd_vec["ms_per_call"]}


def recurrent_decode(torch, mlstm, dev, B, NH, d, reps=50):
    """Time mlstm_recurrent_step (bf16 q/k/v, float32 state updated in place)."""
    g = torch.Generator(device="cpu").manual_seed(0)
    q, k, v = (torch.randn((B, NH, d), generator=g).to(dev).to(torch.bfloat16) for _ in range(3))
    ig = torch.randn((B, NH), generator=g).to(dev)
    fg = (3.0 + torch.randn((B, NH), generator=g)).to(dev)
    C, n, m = mlstm.recurrent_state(B, NH, d, dev)
    n2, m2 = torch.empty_like(n), torch.empty_like(m)
    states = [(C, n, m), (C, n2, m2)]
    for i in range(3):
        mlstm.recurrent_step(q, k, v, ig, fg, states[i % 2], out_state=states[(i + 1) % 2])
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        mlstm.recurrent_step(q, k, v, ig, fg, states[i % 2], out_state=states[(i + 1) % 2])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    H = B * NH
    # state read + written once, plus the step's vectors and scalars
    nbytes = H * (2 * d * d * 4 + 2 * d * 4 + 4 * d * 2 + 5 * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"B": B, "NH": NH, "d": d, "us_per_step": round(ms * 1e3, 2),
            "algorithmic_bytes": nbytes, "GB/s": round(gbs, 1),
            "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "state_MB": round(H * d * d * 4 / 1e6, 1)}


def backward_timing(torch, mlstm, workloads, x, dev, reps=20):
    """Time mlstm_parallel_bwd on the benchmarked layer (whole call: gate scan,
    per-row scalars, the three tile passes, the gate-gradient scan)."""
    spec = x["spec"]
    B, NH, T, d = spec["B"], spec["NH"], spec["T"], spec["d"]
    dt = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(dt).contiguous() for n in ("q", "k", "v"))
    ig = torch.from_numpy(x["igate"]).to(dev).contiguous()
    fg = torch.from_numpy(x["fgate"]).to(dev).contiguous()
    h, m, n, b = mlstm.parallel_fwd_train(q, k, v, ig, fg)
    dh = torch.randn(q.shape, generator=torch.Generator().manual_seed(1)).to(dev).to(dt)
    mfma = spec["dtype"] == "bf16" and d <= 512
    f32mm = spec["dtype"] == "fp32" and d % 32 == 0 and 32 <= d <= 384
    if not (mfma or f32mm):
        reps = 3
    for _ in range(2):
        mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        mlstm.parallel_bwd(q, k, v, ig, fg, h, m, n, b, dh)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    cf = workloads.counted_flops(B, NH, T, d)  # two causal contractions
    counted = 2.5 * cf  # five causal contractions: S, dh v^T, dQ, dK, dV
    # executed: on the matrix cores the keys pass alone forms S and dh v^T and
    # stores the operands of the dV and dQ passes, which only accumulate (5
    # contractions; 7 above d = 384, where the keys pass splits the output
    # columns over two workgroups that both form S and dh v^T).  The vector
    # passes recompute S and dh v^T once (7).  The float32 matrix-core passes
    # each form their own S (rows, keys, values) and dh v^T (rows, keys): 8
    executed = ((2.5 if d <= 384 else 3.5) if mfma else 4.0 if f32mm else 3.5) * cf
    peak = PEAK_BF16_TFLOPS if mfma else PEAK_FP32_TFLOPS
    return {"ms_per_call": round(ms, 4), "reps": reps,
            "kernels": "bf16 matrix-core passes (per-row scalars; dK, c and the stored dV and dQ "
                       "operands; dV; dQ)" if mfma
                       else "float32 matrix-core passes (per-row scalars; dQ, r; dK, c; dV)"
                       if f32mm else "float32 vector passes",
            "counted_flops": counted,
            "counted_TFLOP/s": round(counted / (ms * 1e-3) / 1e12, 2),
            "executed_TFLOP/s": round(executed / (ms * 1e-3) / 1e12, 2),
            "bound": "mfma" if (mfma or f32mm) else "alu", "peak": peak,
            "frac": round(counted / (ms * 1e-3) / 1e12 / peak, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from linear_recurrent_sequence_amd import mlstm, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = workloads.make(args.workload, seed=0)
    spec = x["spec"]
    B, NH, T, d = spec["B"], spec["NH"], spec["T"], spec["d"]
    dt = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(dt).contiguous() for n in ("q", "k", "v"))
    ig = torch.from_numpy(x["igate"]).to(dev).contiguous()
    fg = torch.from_numpy(x["fgate"]).to(dev).contiguous()
    h = torch.empty_like(q)
    m = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    n = torch.empty_like(m)
    flops = workloads.counted_flops(B, NH, T, d)

    # ---- whole-call throughput ----
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(20):
            mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
    torch.cuda.synchronize()
    # HIP events on the launch stream bracket the same timed steps: on a
    # single-launch workload their average is the dominant kernel's duration
    # over the timed region itself
    stream = torch.cuda.current_stream(dev)
    ev_t0 = torch.cuda.Event(enable_timing=True)
    ev_t1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev_t0.record(stream)
    for _ in range(args.steps):
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
    ev_t1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    value = flops / (ms * 1e-3) / 1e12
    timed_kernel_ms = ev_t0.elapsed_time(ev_t1) / args.steps

    # per-call durations: 100 calls, each between HIP events on the call's stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(100)]
    for a, b in evs:
        a.record(stream)
        mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
        b.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    per_call_rec = {"calls": len(per_call), "median_us": round(per_call[len(per_call) // 2], 2),
                    "min_us": round(per_call[0], 2),
                    "p90_us": round(per_call[int(0.9 * len(per_call))], 2),
                    "median_TFLOP/s": round(flops / (per_call[len(per_call) // 2] * 1e-6) / 1e12, 1)}

    # ---- dominant kernel alone: HIP events on the launch stream.  On a
    # single-launch workload the call is that kernel, and the timed steps
    # above are its launches, back to back.
    single = single_launch(spec)
    reps = max(args.steps, 20)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ws = mlstm.alloc_workspace(B, NH, T, dev)
    m_ws = torch.empty_like(m)
    mlstm.gate_scan(ig, fg, d, ws, m=m_ws)
    for _ in range(3):
        mlstm.causal_tiles(q, k, v, m_ws, ws, out=(h, n))
    e0.record(stream)
    for _ in range(reps):
        mlstm.causal_tiles(q, k, v, m_ws, ws, out=(h, n))
    e1.record(stream)
    torch.cuda.synchronize()
    staged_tile_ms = e0.elapsed_time(e1) / reps
    if single:
        tile_ms = timed_kernel_ms
        if d % 64 == 0 and d <= 192:
            kernel_name = f"tiles_pipe_kernel<{d}> (gate scan fused)"
        elif d <= 384:
            kernel_name = f"tiles_pairs_kernel<{(d + 63) // 64 * 64}, gate scan fused>"
        else:
            kernel_name = f"tiles_mfma_kernel<{(d + 31) // 32 * 32}, gate scan fused>"
    else:
        tile_ms = staged_tile_ms
        kernel_name = "causal tile kernel of the two-launch form"
    achieved = flops / (tile_ms * 1e-3) / 1e12

    # gate scan alone (HBM-bound in principle, latency-bound at these sizes)
    e0.record(stream)
    for _ in range(reps):
        mlstm.gate_scan(ig, fg, d, ws, m=m_ws)
    e1.record(stream)
    torch.cuda.synchronize()
    scan_ms = e0.elapsed_time(e1) / reps
    scan_bytes = scan_kernel_bytes(B * NH, T)
    scan_bytes16 = B * NH * T * SCAN_MIN_BYTES_PER_POSITION
    scan_large = scan_at_size(torch, mlstm, dev)

    # decay-aware tile skipping on the long-context stress workload: the same
    # call with skipping (default) and visiting every causal tile
    skip_rec = None
    if not args.no_long_context:
        skip_rec = long_context_skipping(torch, mlstm, workloads, dev, reps=10)

    wide = None
    if not args.no_wide:
        wide = [layer_timing(torch, mlstm, workloads, dev, name)
                for name in ("xlstm1p3b_layer", "xlstm1p3b_layer_d1024")]
        if not args.no_backward:
            # above d = 512 the backward runs the float32 vector passes in
            # head-dimension chunks (a correctness path): two calls
            xw = workloads.make("xlstm1p3b_layer_d1024", seed=0)
            wide[1]["backward"] = backward_timing(torch, mlstm, workloads, xw, dev, reps=2)

    f32 = None if args.no_fp32 else fp32_layer_timing(torch, mlstm, workloads, dev)

    # recurrent (generation) step on the same layer shape: the 8 x 4 heads'
    # state (19 MB) stays in the 256 MB last-level cache between steps; a
    # batch of 256 (604 MB of state) has to stream it from HBM
    rec = [recurrent_decode(torch, mlstm, dev, B, NH, d),
           recurrent_decode(torch, mlstm, dev, 256, NH, d, reps=20)]

    bwd = None if args.no_backward else backward_timing(torch, mlstm, workloads, x, dev)

    configs = None
    if not args.no_per_config:
        configs = per_config(torch, mlstm, workloads, dev, args.oracle_budget_s,
                             with_oracle=not args.no_cpu_baseline)

    # correctness spot check of the timed output (not part of the timing)
    mlstm.parallel_fwd(q, k, v, ig, fg, out=(h, m, n))
    torch.cuda.synchronize()
    finite = bool(torch.isfinite(h.float()).all().item())

    line = {
        "metric": "mLSTM parallel-forward TFLOP/s (causal, 2*T^2*d per head), 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec["dtype"] == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "NH": NH, "T": T, "d": d,
                   "heads": B * NH, "counted_flops": flops,
                   "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": {
            "bound": "mfma", "kernel": kernel_name, "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            # the committed counter record covers the 125M-shaped layer's kernel only
            "traffic": (traffic_from_counters()
                        if single and args.workload == "xlstm125m_layer" else None),
            "avg_launch_ms": round(tile_ms, 5),
        },
        "staged": {"gate_scan_avg_launch_ms": round(scan_ms, 5),
                   "tile_avg_launch_ms": round(staged_tile_ms, 5),
                   "tile_TFLOP/s": round(flops / (staged_tile_ms * 1e-3) / 1e12, 2)},
        "gate_scan": {"avg_launch_ms": round(scan_ms, 5),
                      "kernel_bytes": scan_bytes,
                      "GB/s": round(scan_bytes / (scan_ms * 1e-3) / 1e9, 1),
                      "frac_of_hbm": round(scan_bytes / (scan_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "bytes_16_per_position": scan_bytes16,
                      "GB/s_16_per_position": round(scan_bytes16 / (scan_ms * 1e-3) / 1e9, 1),
                      "at_2^26_positions": scan_large},
        "per_call": dict(per_call_rec, median_minus_kernel_us=round(
            per_call_rec["median_us"] - tile_ms * 1e3, 2)),
        "output_finite": finite,
    }
    if skip_rec is not None:
        line["tile_skipping"] = skip_rec
    if wide is not None:
        line["other_layers"] = wide
    if f32 is not None:
        line["fp32_layer"] = f32
    line["recurrent_step"] = rec
    if bwd is not None:
        line["backward"] = bwd
    if configs is not None:
        line["per_config"] = configs
    if args.copy_calibration:
        # reads and writes exactly COPY_BYTES each per launch
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = COPY_BYTES
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
