#!/usr/bin/env python3
"""Benchmark of the affine group-quantized qmv on one MI355X.

Metric: achieved HBM GB/s (and % of the 8 TB/s peak) and us/call of the 4-bit
qmv at M = 1 and at M = 13, on the 15360 x 3840 group-64 up-projection of a
12B-class dense model (random weights, synthetic bf16 activations).

A step is one qmv call (the whole hot path: activation staging, weight and
metadata streaming, decode, per-group dot and fold, reduction, output) over
one copy of the inputs.  Inputs rotate over enough copies (>= 1 GiB) that the
256 MB Infinity Cache cannot serve the weights, and are resident in HBM before
timing starts.  Before the first measurement the process runs untimed calls
for at least 30 ms of GPU time (clocks settle), then each measurement runs its
W warm-up calls and times graphs of K and of 2K calls on the launch stream
between HIP events (medians of alternating replays, at least 9 of each and
at least 20 ms of GPU time per graph size): the per-call time
is (T(2K) - T(K)) / K, the time of K whole calls without the fixed cost of a
graph replay.

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

Other modes (one JSON line per point instead of the bench line):
    --table          every 12B/27B-class workload at M = 1, 2, 4, 8, 13, and the
                     mxfp4 mode on the four projection shapes
    --sweep-rows     rows per wavefront 1-4 at M = 1, 4, 8, 13 on the 27B-class
                     shapes, with VGPRs, LDS, grid and wavefronts per SIMD
    --sweep-launch   the launch shape (rows per wavefront, wavefronts and row
                     blocks per workgroup) of the five workloads at M = 1 and 2
                     (--sweep-launch-m to choose), beside the library's launch
    --sweep-ceiling  the streaming-read ceiling over the launch shape, at the
                     4-bit and the 2-bit one-vector byte counts
    --timeline       per-wavefront timelines of the 4-bit projection shapes and
                     the 2-bit up-projection at M = 1 and 13 (stamped instance of
                     the same kernel), with cold and cache-hot activations
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
SETTLE_MS = 30.0            # untimed GPU work before the first measurement
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


def settle_clocks(launch, ncopies, torch, min_ms=SETTLE_MS):
    """Untimed calls until at least min_ms of GPU time has passed (clocks and
    power state settle before the first measurement of a process, whatever
    --warmup asks for)."""
    stream = torch.cuda.Stream()
    done_ms, calls = 0.0, 0
    while done_ms < min_ms and calls < 200000:
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            start.record(stream)
            for i in range(200):
                launch((calls + i) % ncopies, 1, stream)
            end.record(stream)
        end.synchronize()
        done_ms += start.elapsed_time(end)
        calls += 200
    return calls, done_ms


REPLAY_MS = 20.0            # GPU time each graph size is replayed for, at least
MIN_REPLAYS = 9


def time_calls(launch, ncopies, M, steps, warmup, torch, replays=None):
    """Per-call microseconds of `steps` calls, with the fixed cost of a graph
    replay cancelled.

    `warmup` untimed calls first; then two HIP graphs are captured on the
    launch stream, one of K = steps calls and one of 2K calls (inputs rotating
    over the copies), and replayed alternately between HIP events on that
    stream -- `replays` times, or by default at least MIN_REPLAYS times and
    until each size has run for REPLAY_MS (short graphs are replayed more
    often: their median is noisier).  A replay costs its kernels plus a fixed
    launch overhead (about 20 us here), so the difference of the median replay
    times, T(2K) - T(K), is the time of K whole calls with that overhead
    removed; the per-call time is that difference over K.  Returns (us per
    call, details)."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i % ncopies, M, stream)
    stream.synchronize()

    def capture(n, first):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                launch((first + i) % ncopies, M, torch.cuda.current_stream())
        return g

    g1 = capture(steps, warmup)
    g2 = capture(2 * steps, warmup + steps)
    for g in (g1, g2):               # the first replay uploads the graph
        g.replay()
    stream.synchronize()
    t1, t2 = [], []
    i = 0
    while (i < replays) if replays is not None else (i < MIN_REPLAYS or sum(t1) < REPLAY_MS):
        i += 1
        for g, ts in ((g1, t1), (g2, t2)):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                start.record(stream)
                g.replay()
                end.record(stream)
            end.synchronize()
            ts.append(start.elapsed_time(end))
    m1 = sorted(t1)[len(t1) // 2]
    m2 = sorted(t2)[len(t2) // 2]
    us = (m2 - m1) * 1000.0 / steps
    return us, {"graph_K_ms": round(m1, 4), "graph_2K_ms": round(m2, 4), "replays": len(t1),
                "us_per_call_graph_K": round(m1 * 1000.0 / steps, 3)}


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


def device_problem(p, torch, np, dev, ncopies, Mmax=13):
    """`ncopies` device copies of a generated problem (weights, scales, biases,
    13 activation vectors, output) as raw pointers, plus the tensors."""
    base = [torch.from_numpy(p.w_packed.view(np.int32)).to(dev),
            torch.from_numpy(p.scales.view(np.int16)).view(torch.bfloat16).to(dev),
            torch.from_numpy(p.biases.view(np.int16)).view(torch.bfloat16).to(dev),
            torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).to(dev)]
    copies = [[t.clone() for t in base] + [torch.empty(Mmax, p.N, dtype=torch.bfloat16, device=dev)]
              for _ in range(ncopies)]
    torch.cuda.synchronize()
    ptrs = [tuple(t.data_ptr() for t in c) for c in copies]
    return copies, ptrs


def affine_launcher(q, p, ptrs, R=0):
    N, K, bits, gs = p.N, p.K, p.bits, p.gs

    def launch(i, M, stream):
        w, s, b, x, y = ptrs[i]
        st = q.affine_ptr(w, s, b, x, y, M, N, K, bits, gs, q.DT_BF16, q.DT_BF16, q.DT_BF16, R,
                          stream.cuda_stream)
        if st != 0:
            raise q.QmvError(st, "qmv_affine_ex")
    return launch


def workload_table(args, q, gen, torch, np, dev):
    """Every 12B/27B-class workload at M = 1, 2, 4, 8, 13: us per call (the
    bench's timing: rotating copies, graphs of K and 2K calls) and the default
    launch; then the mxfp4 mode on the four projection shapes, with bf16 and
    with fp32 activations."""
    settled = False
    for name in ("up_4b_15360x3840", "down_4b_3840x15360", "up_2b_15360x3840",
                 "up_4b_17408x5120", "down_4b_5120x17408"):
        p = gen.make_problem(name)
        N, K, bits, gs = p.N, p.K, p.bits, p.gs
        nc = max(2, -(-ROTATE_BYTES // alg_bytes(N, K, bits, gs, 13)))
        copies, ptrs = device_problem(p, torch, np, dev, nc)
        launch = affine_launcher(q, p, ptrs)
        if not settled:
            settle_clocks(launch, nc, torch)
            settled = True
        for M in (1, 2, 4, 8, 13):
            us, _ = time_calls(launch, nc, M, args.steps, args.warmup, torch)
            nb = alg_bytes(N, K, bits, gs, M)
            inf = q.kernel_info(M, N, K, bits, gs)
            print(json.dumps({"workload": name, "M": M, "us_per_call": round(us, 3),
                              "GB/s": round(nb / (us * 1e-6) / 1e9, 1),
                              "rows_per_wave": inf["rows_per_wave"], "wg_size": inf["wg_size"],
                              "grid": inf["grid"], "k_windows": inf["k_windows"]}), flush=True)
        del copies
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
                us, _ = time_calls(launch_mx, nc, M, args.steps, args.warmup, torch)
                nb = mx_bytes(N, K, M, x_bytes=xb)
                print(json.dumps({"workload": f"mxfp4_{N}x{K}", "x": "f32" if xb == 4 else "bf16", "M": M,
                                  "us_per_call": round(us, 3), "GB/s": round(nb / (us * 1e-6) / 1e9, 1)}),
                      flush=True)
        del copies
        torch.cuda.empty_cache()


def sweep_rows(args, q, gen, torch, np, dev):
    """The 27B-class layer (17408 x 5120 and 5120 x 17408, 4-bit, group 64):
    every rows-per-wavefront R in {1, 2, 3, 4} at M in {1, 4, 8, 13}, timed as
    the bench line (the library's launch for that R), with the instance's
    VGPRs, LDS per workgroup, grid and wavefronts per SIMD.  One JSON line per
    point; `default` marks the R the library picks by itself."""
    settled = False
    for name in ("up_4b_17408x5120", "down_4b_5120x17408"):
        p = gen.make_problem(name)
        N, K, bits, gs = p.N, p.K, p.bits, p.gs
        nc = max(2, -(-ROTATE_BYTES // alg_bytes(N, K, bits, gs, 13)))
        copies, ptrs = device_problem(p, torch, np, dev, nc)
        if not settled:
            settle_clocks(affine_launcher(q, p, ptrs), nc, torch)
            settled = True
        for M in (1, 4, 8, 13):
            r_default = q.kernel_info(M, N, K, bits, gs)["rows_per_wave"]
            for R in (1, 2, 3, 4):
                us, det = time_calls(affine_launcher(q, p, ptrs, R), nc, M, args.steps, args.warmup, torch)
                inf = q.kernel_info(M, N, K, bits, gs, rows_per_wave=R)
                nb = alg_bytes(N, K, bits, gs, M)
                print(json.dumps({"sweep": "rows_per_wave", "workload": name, "M": M, "R": R,
                                  "default": R == r_default, "us_per_call": round(us, 3),
                                  "GB/s": round(nb / (us * 1e-6) / 1e9, 1),
                                  "vgprs": inf["vgprs"], "scratch_bytes": inf["scratch_bytes"],
                                  "lds_bytes": inf["lds_bytes"], "wg_size": inf["wg_size"],
                                  "grid": inf["grid"], "waves_per_simd": inf["waves_per_simd"],
                                  "k_windows": inf["k_windows"]}), flush=True)
        del copies
        torch.cuda.empty_cache()


def sweep_launch(args, q, gen, torch, np, dev):
    """The launch shape at few vectors (--sweep-launch-m, default 1 and 2) on
    the five projection workloads: rows per wavefront R, wavefronts per
    workgroup W in {4, 6, 8} and row blocks per workgroup in {1, 2, 3, 4}, each
    run through qmv_affine_shape (the library's kernels with that launch; the
    outputs equal the library's launch bit for bit, checked per point) and
    timed as the bench line, beside the library's own launch.  One JSON line
    per point; `default` marks the library's launch."""
    settled = False
    for name in ("up_4b_15360x3840", "down_4b_3840x15360", "up_2b_15360x3840",
                 "up_4b_17408x5120", "down_4b_5120x17408"):
        p = gen.make_problem(name)
        N, K, bits, gs = p.N, p.K, p.bits, p.gs
        nc = max(2, -(-ROTATE_BYTES // alg_bytes(N, K, bits, gs, 13)))
        copies, ptrs = device_problem(p, torch, np, dev, nc)
        lib_launch = affine_launcher(q, p, ptrs)
        if not settled:
            settle_clocks(lib_launch, nc, torch)
            settled = True
        for M in args.sweep_launch_m:
            nb = alg_bytes(N, K, bits, gs, M)
            lib_launch(0, M, torch.cuda.current_stream())
            torch.cuda.synchronize()
            ref = copies[0][4][:M].clone()
            us, _ = time_calls(lib_launch, nc, M, args.steps, args.warmup, torch)
            kinf = q.kernel_info(M, N, K, bits, gs)
            print(json.dumps({"sweep": "launch_shape", "workload": name, "M": M, "default": True,
                              "R": kinf["rows_per_wave"], "W": kinf["wg_size"] // 64, "grid": kinf["grid"],
                              "us_per_call": round(us, 3), "GB/s": round(nb / (us * 1e-6) / 1e9, 1)}),
                  flush=True)
            for R in ((1, 2, 3, 4) if bits == 4 else (1, 2)):
                for W in (4, 6, 8):
                    for per in (1, 2, 3, 4):
                        info = q.KernelInfo()

                        def launch(i, MM, stream, R=R, W=W, per=per, info=info):
                            w, s_, b, x, y = ptrs[i]
                            st = q.shape_ptr(w, s_, b, x, y, MM, N, K, bits, gs, q.DT_BF16, q.DT_BF16,
                                             q.DT_BF16, R, W, per, info, stream.cuda_stream)
                            if st != 0:
                                raise q.QmvError(st, "qmv_affine_shape")
                        copies[0][4].zero_()
                        try:
                            launch(0, M, torch.cuda.current_stream())
                        except q.QmvError as e:
                            print(json.dumps({"sweep": "launch_shape", "workload": name, "M": M, "R": R,
                                              "W": W, "row_blocks_per_wg": per, "error": str(e)}), flush=True)
                            continue
                        torch.cuda.synchronize()
                        if not torch.equal(copies[0][4][:M], ref):
                            raise RuntimeError(f"{name} M={M} R={R} W={W} per={per}: output differs")
                        us, _ = time_calls(launch, nc, M, args.steps, args.warmup, torch)
                        print(json.dumps({"sweep": "launch_shape", "workload": name, "M": M, "R": R, "W": W,
                                          "row_blocks_per_wg": per, "grid": info.grid,
                                          "vgprs": info.vgprs, "waves_per_simd": info.waves_per_simd,
                                          "lds_bytes": info.lds_bytes, "k_windows": info.k_windows,
                                          "us_per_call": round(us, 3),
                                          "GB/s": round(nb / (us * 1e-6) / 1e9, 1)}), flush=True)
        del copies
        torch.cuda.empty_cache()


def sweep_ceiling(args, q, gen, torch, np, dev):
    """The streaming-read ceiling over the one-vector byte counts of the bench
    line's workload (33,216,000 B) and of the 2-bit 15360 x 3840 workload
    (16,627,200 B), same rotation and timing, swept over the launch shape:
    workgroups per compute unit, wavefronts per workgroup, loads in flight per
    lane, and contiguous or interleaved spans.  One JSON line per shape, then
    the best shape of each byte count."""
    settled = False
    for name in (WORKLOAD, "up_2b_15360x3840"):
        p = gen.make_problem(name)
        nb = alg_bytes(p.N, p.K, p.bits, p.gs, 1)
        nc = max(2, -(-ROTATE_BYTES // nb))
        bufs = [torch.empty(nb, dtype=torch.uint8, device=dev).random_(0, 256) for _ in range(nc)]
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        shape = [4, 8, 4, 0]

        def launch(i, M, stream):
            st = q.stream_read_ex_ptr(bufs[i].data_ptr(), nb, sink.data_ptr(), *shape,
                                      stream=stream.cuda_stream)
            if st != 0:
                raise q.QmvError(st, "qmv_stream_read_ex")

        if not settled:
            settle_clocks(launch, nc, torch)
            settled = True
        best = None
        for wg in (1, 2, 4, 8, 16):
            for waves in (4, 8, 16):
                if wg * waves > 32 * 4:
                    continue
                for batch in (1, 2, 4, 8, 16):
                    for inter in (0, 1):
                        shape[:] = [wg, waves, batch, inter]
                        us, _ = time_calls(launch, nc, 1, args.steps, args.warmup, torch)
                        gbs = nb / (us * 1e-6) / 1e9
                        rec = {"sweep": "stream_ceiling", "workload": name, "bytes": nb, "wg_per_cu": wg,
                               "waves_per_wg": waves, "batch": batch, "interleave": inter,
                               "us_per_call": round(us, 3), "GB/s": round(gbs, 1),
                               "frac_of_peak": round(gbs / PEAK_GBS, 4)}
                        print(json.dumps(rec), flush=True)
                        if best is None or us < best["us_per_call"]:
                            best = rec
        print(json.dumps({**best, "sweep": "stream_ceiling_best"}), flush=True)
        del bufs
        torch.cuda.empty_cache()


def _pcts(v, np):
    """p10, p50, p90 and max of a sequence."""
    v = np.asarray(v, dtype=np.float64)
    return [float(np.percentile(v, 10)), float(np.percentile(v, 50)), float(np.percentile(v, 90)),
            float(v.max())]


def _timeline_stats(bufs, clock_khz, np):
    """Per-sample statistics of stamped launches (ns after the sample's earliest
    wavefront start), then the median over the samples."""
    ns_per_tick = 1e6 / clock_khz
    rows = []
    for b in bufs:
        a = b.cpu().numpy()
        t = (a[:, :3] - a[:, 0].min()).astype(np.float64) * ns_per_tick
        ids = a[:, 3]
        cu = (ids >> 32) * 256 + ((ids >> 8) & 0xFF)   # XCC, then HW_ID bits 8..15
        keys, inv, counts = np.unique(cu, return_inverse=True, return_counts=True)
        cu_end = np.full(len(keys), -np.inf)
        np.maximum.at(cu_end, inv, t[:, 2])
        rows.append({"start": _pcts(t[:, 0], np), "staged": _pcts(t[:, 1], np),
                     "end": _pcts(t[:, 2], np), "staging": _pcts(t[:, 1] - t[:, 0], np),
                     "after_staging": _pcts(t[:, 2] - t[:, 1], np), "cu_end": _pcts(cu_end, np),
                     "cus": len(keys), "waves_per_cu": [int(counts.min()), int(counts.max())]})

    def med(key):
        return [round(float(np.median([r[key][i] for r in rows])), 0) for i in range(4)]
    return {"ns_p10_p50_p90_max": {k: med(k) for k in ("start", "staged", "end", "staging",
                                                       "after_staging", "cu_end")},
            "cus": int(np.median([r["cus"] for r in rows])),
            "waves_per_cu": [int(np.median([r["waves_per_cu"][0] for r in rows])),
                             int(np.median([r["waves_per_cu"][1] for r in rows]))]}


def timeline(args, q, gen, torch, np, dev):
    """Per-wavefront timeline of the library's launch, from the stamped
    instance of the same kernel (qmv_affine_timeline): the 4-bit group-64
    projection shapes and the 2-bit group-128 up-projection at M = 1 and 13
    (--timeline-m to choose).  Each sample is one stamped call on a
    rotating copy, enqueued right after a few product calls on other copies
    (so the GPU is busy and the copy cold in the caches, as in the timed
    bench); per sample the stamps are taken relative to its earliest wavefront
    start, and the figures below are medians over the samples:
    p10 / p50 / p90 / max over the wavefronts of each event (start,
    activations staged, end; ns), of the staging time (staged - start) and of
    the time after staging (end - staged), and of the compute units' last
    wavefront end; the compute units used and the wavefronts per compute unit
    (min, max).  The product's and the stamped instance's us per call (bench
    timing) are printed beside them.  `x_hot` repeats the product timing and
    the stamps with every call reading one activation buffer (weights,
    scales and biases still rotate), as when x was just written by the
    previous operation: the difference is the cost of cold activations.  A
    call the library cuts into tiles of vectors (17408 x 5120 at 13 vectors)
    is stamped on its first tile's vectors.  One JSON line per point."""
    samples = max(5, min(args.steps, 50))
    settled = False
    for name in ("up_4b_15360x3840", "down_4b_3840x15360", "up_4b_17408x5120", "down_4b_5120x17408",
                 "up_2b_15360x3840"):
        p = gen.make_problem(name)
        N, K, bits, gs = p.N, p.K, p.bits, p.gs
        nc = max(2, -(-ROTATE_BYTES // alg_bytes(N, K, bits, gs, 13)))
        copies, ptrs = device_problem(p, torch, np, dev, nc)
        hot = [(w, s, b, ptrs[0][3], y) for (w, s, b, x, y) in ptrs]
        if not settled:
            settle_clocks(affine_launcher(q, p, ptrs), nc, torch)
            settled = True
        for M in args.timeline_m:
            # a call cut into tiles of vectors is stamped on its first tile
            info = q.TimelineInfo()
            while True:
                st = q.timeline_ptr(*ptrs[0][:5], M, N, K, bits, gs, q.DT_BF16, 0, None, 0, info)
                if st != 5 or M == 1:
                    break
                M -= 1
            if st != 0:
                raise q.QmvError(st, "qmv_affine_timeline")
            bufs = [torch.zeros((info.waves, q.STAMPS), dtype=torch.int64, device=dev)
                    for _ in range(samples)]

            def stamped_launcher(pp):
                def launch_stamped(i, M, stream, buf=None):
                    b = bufs[0] if buf is None else buf
                    st = q.timeline_ptr(*pp[i][:5], M, N, K, bits, gs, q.DT_BF16, 0, b.data_ptr(),
                                        b.numel(), info, stream.cuda_stream)
                    if st != 0:
                        raise q.QmvError(st, "qmv_affine_timeline")
                return launch_stamped

            def run(pp):
                launch, launch_stamped = affine_launcher(q, p, pp), stamped_launcher(pp)
                us, _ = time_calls(launch, nc, M, args.steps, args.warmup, torch)
                us_st, _ = time_calls(launch_stamped, nc, M, args.steps, args.warmup, torch)
                stream = torch.cuda.current_stream()
                c = 0
                for j in range(samples):
                    for _ in range(4):
                        launch(c % nc, M, stream)
                        c += 1
                    launch_stamped(c % nc, M, stream, bufs[j])
                    c += 1
                torch.cuda.synchronize()
                return us, us_st, _timeline_stats(bufs, info.clock_khz, np)

            us, us_st, cold = run(ptrs)
            us_hot, _, warm = run(hot)
            kinf = q.kernel_info(M, N, K, bits, gs)
            print(json.dumps({
                "timeline": name, "M": M, "rows_per_wave": kinf["rows_per_wave"], "grid": info.grid,
                "waves": info.waves, "samples": samples,
                "us_per_call": round(us, 3), "us_per_call_stamped": round(us_st, 3),
                "vgprs": [info.product_vgprs, info.vgprs],
                "blocks_per_cu": [info.product_blocks_per_cu, info.blocks_per_cu],
                **cold,
                "x_hot": {"us_per_call": round(us_hot, 3),
                          "ns_p10_p50_p90_max": warm["ns_p10_p50_p90_max"]}}), flush=True)
        del copies
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # K: calls per timed graph (graphs of K and 2K calls are timed; their
    # difference cancels the graph's fixed launch cost)
    ap.add_argument("--steps", type=int, default=200)
    # untimed calls before each measurement (after the process-wide clock settling)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU-oracle baseline (0 = skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (HBM counter calibration)")
    ap.add_argument("--table", action="store_true",
                    help="instead of the bench line, time every workload at M = 1, 2, 4, 8, 13 with "
                         "the library's default launch (one JSON line per case)")
    ap.add_argument("--sweep-rows", action="store_true",
                    help="instead of the bench line, time rows per wavefront 1-4 at M = 1, 4, 8, 13 on "
                         "the 27B-class shapes, with resources and occupancy per point")
    ap.add_argument("--sweep-launch", action="store_true",
                    help="time the launch shape (rows, wavefronts and row blocks per workgroup) at few vectors")
    ap.add_argument("--sweep-launch-m", type=lambda v: tuple(int(t) for t in v.split(",")), default=(1, 2),
                    help="vector counts of --sweep-launch (comma-separated)")
    ap.add_argument("--sweep-ceiling", action="store_true",
                    help="instead of the bench line, sweep the streaming-read ceiling's launch shape "
                         "over the 4-bit and 2-bit one-vector byte counts")
    ap.add_argument("--timeline", action="store_true",
                    help="instead of the bench line, per-wavefront timelines of the 4-bit projection "
                         "shapes at M = 1 and 13 (stamped instance of the same kernel)")
    ap.add_argument("--timeline-m", type=lambda v: tuple(int(t) for t in v.split(",")), default=(1, 13),
                    help="vector counts of --timeline, comma-separated (default 1,13)")
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
    if args.sweep_rows:
        sweep_rows(args, q, gen, torch, np, dev)
        return
    if args.sweep_launch:
        sweep_launch(args, q, gen, torch, np, dev)
        return
    if args.sweep_ceiling:
        sweep_ceiling(args, q, gen, torch, np, dev)
        return
    if args.timeline:
        timeline(args, q, gen, torch, np, dev)
        return
    wl = gen.WORKLOADS[WORKLOAD]
    p = gen.make_problem(WORKLOAD)
    N, K, bits, gs = p.N, p.K, p.bits, p.gs
    Mmax = 13
    per_copy = alg_bytes(N, K, bits, gs, Mmax)
    ncopies = max(2, -(-ROTATE_BYTES // per_copy))
    copies, ptrs = device_problem(p, torch, np, dev, ncopies)
    X = [c[3] for c in copies]
    Y = [c[4] for c in copies]
    launch = affine_launcher(q, p, ptrs)

    # correctness guard on the timed configuration: M=13 vector 0 == M=1 call
    launch(0, 1, torch.cuda.current_stream())
    y1 = Y[0][0].clone()
    launch(0, Mmax, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(Y[0][0], y1), "M-invariance violated on the bench workload"

    settle_calls, settle_ms = settle_clocks(launch, ncopies, torch)
    results = {}
    for M in (1, Mmax):
        us, det = time_calls(launch, ncopies, M, args.steps, args.warmup, torch)
        us_eager = time_calls_eager(launch, ncopies, M, args.steps, torch)
        nb = alg_bytes(N, K, bits, gs, M)
        info = q.kernel_info(M, N, K, bits, gs)
        results[M] = dict(us=us, det=det, us_eager=us_eager, bytes=nb,
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
    timing = (f"per call = (T(2K) - T(K)) / K: HIP graphs of K = {args.steps} and {2 * args.steps} calls "
              f"(inputs rotating over {ncopies} copies) replayed alternately {r1['det']['replays']} times each "
              f"(at least 9, and 20 ms of GPU time per size) between HIP events on the launch stream, "
              f"medians; {args.warmup} untimed calls before each "
              f"measurement, and {settle_calls} untimed calls ({settle_ms:.0f} ms of GPU time) before "
              f"the first")
    out = {
        "metric": METRIC,
        "value": round(r1["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r1["us"] / 1000.0, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4*bf16->f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "N": N, "K": K, "bits": bits, "group_size": gs, "M": 1,
                   "x": "bf16", "scales_biases": "bf16", "y": "bf16", "accumulate": "f32",
                   "rotation_copies": ncopies, "rotation_bytes": ncopies * per_copy,
                   "timing": timing, "seed": wl["seed"]},
        "us_per_call": round(r1["us"], 3),
        "pct_of_hbm_peak": round(100.0 * r1["gbs"] / PEAK_GBS, 2),
        "timing_detail": r1["det"],
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
            "shape": "4 workgroups of 8 wavefronts per CU, 4 loads in flight per lane",
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
            "timing_detail": r13["det"],
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
