#!/usr/bin/env python3
"""Benchmark of the affine group-quantized qmv on one MI355X.

Metric: achieved HBM GB/s (and % of the 8 TB/s peak) and us/call of the 4-bit
qmv at M = 1 and at M = 13, on the 15360 x 3840 group-64 up-projection of a
12B-class dense model (random weights, synthetic bf16 activations).

A step is one qmv call (the whole hot path: activation staging, weight and
metadata streaming, decode, per-group dot and fold, reduction, output) over
one copy of the inputs.  Inputs rotate over enough copies (>= 1 GiB) that the
256 MB Infinity Cache cannot serve the weights, and are resident in HBM before
timing starts.  The K timed calls are captured once in a HIP graph on the
launch stream and replayed; HIP events on that stream bracket the replay, so
the per-call time is (event time) / K.

Algorithmic bytes per call = packed weights + scales + biases + activations +
outputs, each counted once:
    N*K*bits/8 + 2 * N*(K/gs)*2 + M*K*2 + M*N*2.

Prints one JSON line (the driver's contract) with extra objects:
    roofline        -- the dominant kernel against the HBM peak
    stream_ceiling  -- a load-and-discard kernel of the M = 1 launch shape over
                       the same byte count, with the same rotation: the share of
                       the peak any one-launch kernel of this size reaches
    m13             -- the same matrix at M = 13
    mxfp4           -- the mxfp4 mode (E2M1 codes, E8M0 scale per 32 values) on
                       the same shape at M = 1 and 13: us/call and GB/s of its
                       algorithmic bytes N*K/2 + N*K/32 + M*K*2 + M*N*2
    occupancy_17408x5120 -- resources per rows-per-wavefront on the 27B-class
                       up-projection (no launch)
    cpu_baseline    -- the CPU oracle on the machine's host cores (bounded sample),
                       and one of its calls on a single thread
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

METRIC = "achieved HBM GB/s (% of peak) and µs/call for 4-bit qmv at M=1 and M=13"
WORKLOAD = "up_4b_15360x3840"
PEAK_GBS = 8000.0           # MI355X HBM3E
# Vector-ALU peak of the dot products: 256 CUs x 64 lanes x 2.4 GHz, one
# v_dot2_f32_bf16 (2 multiply-adds = 4 flops) per lane per cycle.
PEAK_DOT_TFLOPS = 256 * 64 * 2.4e9 * 4 / 1e12
ROTATE_BYTES = 1 << 30      # >= 4x the 256 MB Infinity Cache
KERNEL_SOURCES = ("bit_quantized_gemv_amd/csrc/qmv_kernel.hpp",)
MX_KERNEL_SOURCES = ("bit_quantized_gemv_amd/csrc/qmv_kernel.hpp", "bit_quantized_gemv_amd/csrc/qmv_mx.hip")


def mx_bytes(N, K, M, y_bytes=2, x_bytes=2):
    """Algorithmic bytes of one mxfp4 call: E2M1 codes, one E8M0 byte per 32
    values, the activations (bf16 unless given), the output."""
    return N * K // 2 + N * (K // 32) + M * K * x_bytes + M * N * y_bytes


def alg_bytes(N, K, bits, gs, M, x_bytes=2, y_bytes=2, sb_bytes=2):
    return N * K * bits // 8 + 2 * N * (K // gs) * sb_bytes + M * K * x_bytes + M * N * y_bytes


def kernel_hash(sources=KERNEL_SOURCES) -> str:
    """Hash of the kernel source's code: comments and whitespace are dropped,
    so the counters stay attached to the code they were taken on."""
    import re
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def traffic_for(M: int, name="qmv_up_4b_15360x3840_traffic.json", sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash(sources):
        return None
    e = t.get("per_launch", {}).get(f"M{M}")
    return None if e is None else e.get("hbm_bytes")


def time_calls(launch, ncopies, M, steps, warmup, torch, replays=1):
    """Per-call microseconds: K calls captured in one HIP graph, replayed
    between HIP events on the capture/launch stream (the median of `replays`
    timed replays; one for the bench line, which times exactly K calls)."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i % ncopies, M, stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            launch((warmup + i) % ncopies, M, torch.cuda.current_stream())
    stream.synchronize()
    g.replay()                       # first replay uploads the graph
    stream.synchronize()
    times = []
    for _ in range(replays):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            start.record(stream)
            g.replay()
            end.record(stream)
        end.synchronize()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end))
    ms = sorted(times)[len(times) // 2]
    return ms * 1000.0 / steps, ms


def time_calls_eager(launch, ncopies, M, steps, torch):
    """Per-call microseconds with plain back-to-back launches (context only:
    includes host enqueue cost when the host is slower than the GPU)."""
    stream = torch.cuda.Stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for i in range(steps):
            launch(i % ncopies, M, stream)
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) * 1000.0 / steps


def cpu_baseline(p, budget_s: float):
    """The oracle as it stands, on all host cores, over whole M=1 problems of
    the bench workload, repeated until about budget_s seconds have passed."""
    from oracle import oracle
    orc = oracle.default()
    cores = len(os.sched_getaffinity(0))
    nbytes = alg_bytes(p.N, p.K, p.bits, p.gs, 1)
    t0 = time.perf_counter()
    orc.qmv(p.w_packed, p.scales, p.biases, p.x[:1], bits=p.bits, group_size=p.gs,
            sb_dtype=oracle.BF16, x_dtype=oracle.BF16, nthreads=cores)     # warm-up
    first = time.perf_counter() - t0
    reps = max(1, int(budget_s / max(first, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(reps):
        orc.qmv(p.w_packed, p.scales, p.biases, p.x[:1], bits=p.bits, group_size=p.gs,
                sb_dtype=oracle.BF16, x_dtype=oracle.BF16, nthreads=cores)
    dt = (time.perf_counter() - t0) / reps
    one = []
    for _ in range(3):
        t0 = time.perf_counter()
        orc.qmv(p.w_packed, p.scales, p.biases, p.x[:1], bits=p.bits, group_size=p.gs,
                sb_dtype=oracle.BF16, x_dtype=oracle.BF16, nthreads=1)
        one.append(time.perf_counter() - t0)
    one.sort()
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "us_per_call": round(dt * 1e6, 1),
            "sample": f"{reps} whole M=1 calls of {p.N}x{p.K} 4-bit g64 (fp64 accumulate, "
                      f"OpenMP over rows), after 1 warm-up call",
            "us_per_call_1thread": round(one[1] * 1e6, 1),
            "sample_1thread": "median of 3 whole M=1 calls on one thread",
            "cpu": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def workload_table(args, q, gen, torch, np, dev):
    """Every 12B/27B-class workload at M = 1, 2, 4, 8, 13: us per call (graph
    replay over rotating copies as in the bench line, median of three replays)
    and the default launch; then the mxfp4 mode on the four projection shapes,
    with bf16 and with fp32 activations."""
    for name in ("up_4b_15360x3840", "down_4b_3840x15360", "up_2b_15360x3840",
                 "up_4b_17408x5120", "down_4b_5120x17408"):
        p = gen.make_problem(name)
        N, K, bits, gs = p.N, p.K, p.bits, p.gs
        per_copy = alg_bytes(N, K, bits, gs, 13)
        nc = max(2, -(-ROTATE_BYTES // per_copy))
        base = [torch.from_numpy(p.w_packed.view(np.int32)).to(dev),
                torch.from_numpy(p.scales.view(np.int16)).view(torch.bfloat16).to(dev),
                torch.from_numpy(p.biases.view(np.int16)).view(torch.bfloat16).to(dev),
                torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).to(dev)]
        copies = [[t.clone() for t in base] + [torch.empty(13, N, dtype=torch.bfloat16, device=dev)]
                  for _ in range(nc)]

        def launch(i, M, stream):
            w, s, b, x, y = (t.data_ptr() for t in copies[i])
            st = q.affine_ptr(w, s, b, x, y, M, N, K, bits, gs, q.DT_BF16, q.DT_BF16, q.DT_BF16, 0,
                              stream.cuda_stream)
            if st != 0:
                raise q.QmvError(st, "qmv_affine_ex")

        for M in (1, 2, 4, 8, 13):
            us, _ = time_calls(launch, nc, M, args.steps, args.warmup, torch, replays=3)
            nb = alg_bytes(N, K, bits, gs, M)
            inf = q.kernel_info(M, N, K, bits, gs)
            print(json.dumps({"workload": name, "M": M, "us_per_call": round(us, 3),
                              "GB/s": round(nb / (us * 1e-6) / 1e9, 1),
                              "rows_per_wave": inf["rows_per_wave"], "wg_size": inf["wg_size"],
                              "grid": inf["grid"], "k_windows": inf["k_windows"]}), flush=True)
        del copies, base
        torch.cuda.empty_cache()
    # the mxfp4 mode on the same four projection shapes
    for N, K in ((15360, 3840), (3840, 15360), (17408, 5120), (5120, 17408)):
        pm = gen.make_mx_problem(N, K, "bf16", seed=4001)
        nc = max(2, -(-ROTATE_BYTES // mx_bytes(N, K, 13)))
        copies = [(torch.from_numpy(pm.w_packed.view(np.int32)).to(dev), torch.from_numpy(pm.scales).to(dev))
                  for _ in range(nc)]
        xbf = torch.from_numpy(pm.x.view(np.int16)).view(torch.bfloat16).to(dev)
        ym = torch.empty(13, N, dtype=torch.bfloat16, device=dev)
        for xm, x_dt, xb in ((xbf, q.DT_BF16, 2), (xbf.float(), q.DT_F32, 4)):
            def launch_mx(i, M, stream, xm=xm, x_dt=x_dt):
                st = q.mxfp4_ptr(copies[i][0].data_ptr(), copies[i][1].data_ptr(), xm.data_ptr(), ym.data_ptr(),
                                 M, N, K, x_dt, q.DT_BF16, stream.cuda_stream)
                if st != 0:
                    raise q.QmvError(st, "qmv_mxfp4")

            for M in (1, 2, 4, 8, 13):
                us, _ = time_calls(launch_mx, nc, M, args.steps, args.warmup, torch, replays=3)
                nb = mx_bytes(N, K, M, x_bytes=xb)
                print(json.dumps({"workload": f"mxfp4_{N}x{K}", "x": "f32" if xb == 4 else "bf16", "M": M,
                                  "us_per_call": round(us, 3), "GB/s": round(nb / (us * 1e-6) / 1e9, 1)}),
                      flush=True)
        del copies
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # timed calls per measurement, in one graph: 1000 spread the graph's own launch
    # cost (about 20 us per replay) to ~0.02 us per call (~0.1 us at 200)
    ap.add_argument("--steps", type=int, default=1000)
    # untimed calls before each measurement: 2000 (about 20 ms of GPU work) let the
    # clocks settle; with 20 the first measurements of a process ran up to 10% slower
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU-oracle baseline (0 = skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--table", action="store_true",
                    help="instead of the bench line, time every workload at M = 1, 2, 4, 8, 13 with "
                         "the library's default launch (one JSON line per case)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this qmv path has no multi-GPU part "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import bit_quantized_gemv_amd as q
    from inputs import gen

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.table:
        workload_table(args, q, gen, torch, np, dev)
        return
    wl = gen.WORKLOADS[WORKLOAD]
    p = gen.make_problem(WORKLOAD)
    N, K, bits, gs = p.N, p.K, p.bits, p.gs
    Mmax = 13

    w0 = torch.from_numpy(p.w_packed.view(np.int32)).to(dev)
    s0 = torch.from_numpy(p.scales.view(np.int16)).view(torch.bfloat16).to(dev)
    b0 = torch.from_numpy(p.biases.view(np.int16)).view(torch.bfloat16).to(dev)
    x0 = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).to(dev)
    per_copy = alg_bytes(N, K, bits, gs, Mmax)
    ncopies = max(2, -(-ROTATE_BYTES // per_copy))
    W = [w0.clone() for _ in range(ncopies)]
    S = [s0.clone() for _ in range(ncopies)]
    B = [b0.clone() for _ in range(ncopies)]
    X = [x0.clone() for _ in range(ncopies)]
    Y = [torch.empty(Mmax, N, dtype=torch.bfloat16, device=dev) for _ in range(ncopies)]
    ptrs = [(W[i].data_ptr(), S[i].data_ptr(), B[i].data_ptr(), X[i].data_ptr(), Y[i].data_ptr())
            for i in range(ncopies)]
    torch.cuda.synchronize()

    def launch(i, M, stream):
        w, s, b, x, y = ptrs[i]
        st = q.affine_ptr(w, s, b, x, y, M, N, K, bits, gs, q.DT_BF16, q.DT_BF16, q.DT_BF16, 0,
                          stream.cuda_stream)
        if st != 0:
            raise q.QmvError(st, "qmv_affine_ex")

    # correctness guard on the timed configuration: M=13 vector 0 == M=1 call
    launch(0, 1, torch.cuda.current_stream())
    y1 = Y[0][0].clone()
    launch(0, Mmax, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(Y[0][0], y1), "M-invariance violated on the bench workload"

    results = {}
    for M in (1, Mmax):
        us, total_ms = time_calls(launch, ncopies, M, args.steps, args.warmup, torch)
        us_eager = time_calls_eager(launch, ncopies, M, args.steps, torch)
        nb = alg_bytes(N, K, bits, gs, M)
        info = q.kernel_info(M, N, K, bits, gs)
        results[M] = dict(us=us, total_ms=total_ms, us_eager=us_eager, bytes=nb,
                          gbs=nb / (us * 1e-6) / 1e9, info=info)

    # streaming-read ceiling over the M=1 call's byte count, same rotation and timing
    nb1 = alg_bytes(N, K, bits, gs, 1)
    SB = [torch.randint(0, 256, (nb1,), dtype=torch.uint8, device=dev) for _ in range(ncopies)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def launch_stream(i, M, stream, checksum=False):
        st = q.stream_read_ptr(SB[i].data_ptr(), nb1, sink.data_ptr(), checksum, stream.cuda_stream)
        if st != 0:
            raise q.QmvError(st, "qmv_stream_read")

    launch_stream(0, 1, torch.cuda.current_stream(), checksum=True)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(SB[0].cpu().numpy().view(np.uint32)))
    assert (int(sink.item()) & 0xffffffff) == want, "stream-read checksum mismatch"
    us_stream, _ = time_calls(launch_stream, ncopies, 1, args.steps, args.warmup, torch)
    gbs_stream = nb1 / (us_stream * 1e-6) / 1e9
    del SB

    # mxfp4 mode on the same shape: M = 1 and 13, same rotation and graph timing
    pm = gen.make_mx_problem(N, K, "bf16", seed=4001)
    mw0 = torch.from_numpy(pm.w_packed.view(np.int32)).to(dev)
    ms0 = torch.from_numpy(pm.scales).to(dev)
    mx_copies = max(2, -(-ROTATE_BYTES // mx_bytes(N, K, Mmax)))
    MW = [mw0.clone() for _ in range(mx_copies)]
    MS = [ms0.clone() for _ in range(mx_copies)]

    def launch_mx(i, M, stream):
        st = q.mxfp4_ptr(MW[i].data_ptr(), MS[i].data_ptr(), X[i % ncopies].data_ptr(),
                         Y[i % ncopies].data_ptr(), M, N, K, q.DT_BF16, q.DT_BF16, stream.cuda_stream)
        if st != 0:
            raise q.QmvError(st, "qmv_mxfp4")

    mx = {"workload": f"mxfp4_{N}x{K}", "format": "E2M1 codes, E8M0 scale per 32 values, bf16 x and y"}
    for M in (1, Mmax):
        us_mx, _ = time_calls(launch_mx, mx_copies, M, args.steps, args.warmup, torch)
        nbm = mx_bytes(N, K, M)
        gbm = nbm / (us_mx * 1e-6) / 1e9
        mx[f"M{M}"] = {"us_per_call": round(us_mx, 3), "GB/s": round(gbm, 1),
                       "pct_of_hbm_peak": round(100 * gbm / PEAK_GBS, 2),
                       "alg_bytes_per_launch": nbm,
                       "roofline": {"bound": "hbm", "achieved": round(gbm, 1), "peak": PEAK_GBS,
                                    "unit": "GB/s", "frac": round(gbm / PEAK_GBS, 4),
                                    "traffic": traffic_for(M, "qmv_mx_15360x3840_traffic.json",
                                                           MX_KERNEL_SOURCES)}}
    del MW, MS

    occupancy = {}
    for M in (1, Mmax):
        for R in (1, 2, 3, 4):
            inf = q.kernel_info(M, 17408, 5120, 4, 64, rows_per_wave=R)
            occupancy[f"M{M}_R{R}"] = {k: inf[k] for k in ("vgprs", "lds_bytes", "waves_per_simd",
                                                          "grid", "k_windows")}

    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        c = torch.empty_like(a)
        c.copy_(a)
        torch.cuda.synchronize()

    r1, r13 = results[1], results[Mmax]
    flops13 = 2 * Mmax * N * K
    out = {
        "metric": METRIC,
        "value": round(r1["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r1["total_ms"] / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4*bf16->f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "N": N, "K": K, "bits": bits, "group_size": gs, "M": 1,
                   "x": "bf16", "scales_biases": "bf16", "y": "bf16", "accumulate": "f32",
                   "rotation_copies": ncopies, "rotation_bytes": ncopies * per_copy,
                   "timing": "HIP graph of K calls replayed between HIP events on the launch stream",
                   "seed": wl["seed"]},
        "us_per_call": round(r1["us"], 3),
        "pct_of_hbm_peak": round(100.0 * r1["gbs"] / PEAK_GBS, 2),
        "us_per_call_eager": round(r1["us_eager"], 3),
        "kernel": r1["info"],
        "roofline": {
            "bound": "hbm",
            "achieved": round(r1["gbs"], 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r1["gbs"] / PEAK_GBS, 4),
            "traffic": traffic_for(1),
            "alg_bytes_per_launch": r1["bytes"],
        },
        "stream_ceiling": {
            "bytes": nb1,
            "us_per_call": round(us_stream, 3),
            "GB/s": round(gbs_stream, 1),
            "frac_of_peak": round(gbs_stream / PEAK_GBS, 4),
            "qmv_frac_of_ceiling": round(r1["gbs"] / gbs_stream, 4),
        },
        "occupancy_17408x5120": occupancy,
        "mxfp4": mx,
        "m13": {
            "M": Mmax,
            "us_per_call": round(r13["us"], 3),
            "GB/s": round(r13["gbs"], 1),
            "pct_of_hbm_peak": round(100.0 * r13["gbs"] / PEAK_GBS, 2),
            "alg_bytes_per_launch": r13["bytes"],
            "us_per_call_eager": round(r13["us_eager"], 3),
            "valu_TFLOPs_dot": round(flops13 / (r13["us"] * 1e-6) / 1e12, 2),
            "roofline_alu": {
                "bound": "alu",
                "achieved": round(flops13 / (r13["us"] * 1e-6) / 1e12, 2),
                "peak": round(PEAK_DOT_TFLOPS, 1),
                "unit": "TFLOP/s",
                "frac": round(flops13 / (r13["us"] * 1e-6) / 1e12 / PEAK_DOT_TFLOPS, 4),
            },
            "traffic": traffic_for(Mmax),
            "kernel": r13["info"],
        },
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
