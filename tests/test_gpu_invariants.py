"""GPU invariants of the fixed per-row order: each output vector of an M-vector
launch equals the 1-vector launch on that vector bit for bit, for every
workload and M; rows per wavefront never change the bits; repeated runs are
bit-identical; power-of-two scaling commutes exactly."""
import numpy as np
import pytest
import torch

import gpu_util as U
from inputs import gen

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


@pytest.mark.parametrize("name", list(gen.WORKLOADS))
def test_m_invariance(name):
    wl = gen.WORKLOADS[name]
    p = gen.make_problem(name)
    dev = U.to_dev(p)
    ones = [U.gpu(p, dev, 1, torch.float32, x=dev[3][m:m + 1]) for m in range(13)]
    for M in sorted(set(wl["Ms"]) | {2, 4, 5, 8, 10, 13}):
        U.say(f"M-invariance {name} M={M}")
        y = U.gpu(p, dev, M, torch.float32)
        for m in range(M):
            assert torch.equal(_bits(y[m]), _bits(ones[m][0])), f"{name}: M={M} vector {m}"
        y16 = U.gpu(p, dev, M, torch.bfloat16)
        for m in range(M):
            assert torch.equal(_bits(y16[m]), _bits(U.rne_bf16(ones[m][0])))


@pytest.mark.parametrize("name,gs", [
    ("up_4b_15360x3840", None), ("down_4b_3840x15360", None), ("up_2b_15360x3840", None),
    ("up_4b_17408x5120", None), ("down_4b_5120x17408", None),
    # 4-bit codes in groups of 128: four lanes per group (row groups of four at R = 4)
    ("up_4b_15360x3840", 128), ("down_4b_5120x17408", 128),
])
def test_rows_per_wave_invariance(name, gs):
    p = gen.make_problem(name, gs=gs)
    dev = U.to_dev(p)
    for M in (1, 2, 5, 13):
        U.say(f"R-invariance {name} gs={p.gs} M={M}")
        ys = [U.gpu(p, dev, M, torch.float32, R=R) for R in (1, 2, 3, 4)]
        for i in (1, 2, 3):
            assert torch.equal(_bits(ys[0]), _bits(ys[i])), f"R index {i}"


def test_run_to_run_determinism():
    p = gen.make_problem("up_4b_15360x3840")
    dev = U.to_dev(p)
    for M in (1, 13):
        U.say(f"determinism M={M}")
        y0 = U.gpu(p, dev, M, torch.float32)
        for _ in range(10):
            assert torch.equal(_bits(U.gpu(p, dev, M, torch.float32)), _bits(y0))


@pytest.mark.parametrize("name", ["up_4b_15360x3840", "up_2b_15360x3840", "tiny_4b_g64"])
def test_power_of_two_scaling_and_zero(name):
    p = gen.make_problem(name)
    dev = U.to_dev(p)
    w, s, b, x = dev
    U.say(f"scaling {name}")
    y = U.gpu(p, dev, 5, torch.float32)
    y2 = U.gpu(p, dev, 5, torch.float32, x=(x * 2).contiguous())
    assert torch.equal(_bits(y2), _bits(y * 2))
    z = U.gpu(p, dev, 3, torch.float32, x=torch.zeros_like(x))
    assert not bool(z.any())
    ys = U.gpu(p, (w, s * 2, b * 2, x), 4, torch.float32)
    assert torch.equal(_bits(ys), _bits(U.gpu(p, dev, 4, torch.float32) * 2))


def test_error_status_on_gpu():
    import bit_quantized_gemv_amd as q
    p = gen.make_problem("tiny_4b_g64")
    w, s, b, x = U.to_dev(p)
    # the binding refuses what it can check itself; statuses of the C ABI
    # surface as QmvError
    with pytest.raises(ValueError):
        q.affine(w, s, b, x[:13], bits=3, group_size=64)
    with pytest.raises(q.QmvError):
        q.affine(w, s, b, x[:5], bits=4, group_size=64, rows_per_wave=5)
    y = torch.empty(13, p.N, dtype=torch.float32, device=U.DEV)
    assert q.affine_ptr(w.data_ptr(), s.data_ptr(), b.data_ptr(), x.data_ptr(), y.data_ptr(), 13,
                        p.N, p.K, 3, 64, q.DT_F32, q.DT_F16, q.DT_F32, 0) == 2


@pytest.mark.parametrize("name", ["tiny_4b_g64", "up_4b_15360x3840", "up_2b_15360x3840"])
def test_more_than_one_tile_of_vectors(name):
    # M beyond one launch's 13 vectors runs as balanced tiles (14 -> 7 + 7,
    # 27 -> 9 x 3, 40 -> 10 x 4); every vector must still equal its one-vector call
    p = gen.make_problem(name)
    dev = U.to_dev(p)
    xs = gen.make_x(p.K, p.x_dtype, gen.WORKLOADS[name]["seed"], rows=40)
    xd = U.x_to_dev(xs, p.x_dtype)
    ones = [U.gpu(p, dev, 1, torch.float32, x=xd[m:m + 1]) for m in range(40)]
    for M in (14, 27, 40):
        U.say(f"tiles {name} M={M}")
        y = U.gpu(p, dev, M, torch.float32, x=xd)
        assert y.shape[0] == M
        for m in range(M):
            assert torch.equal(_bits(y[m]), _bits(ones[m][0])), f"{name}: M={M} vector {m}"
    if name == "tiny_4b_g64":
        U.check_parity(U.gpu(p, dev, 40, torch.float32, x=xd), U.ref(p, 40, x=xs), f"{name} M=40")


def test_long_k_vectors_cut_into_whole_k_tiles():
    # K = 6144 (three full wave steps): 13 vectors' activations do not fit LDS
    # whole; with 17408 rows each workgroup walks several row blocks, so the
    # call runs as two whole-K launches (7 + 6 vectors) instead of one
    # K-windowed launch
    assert U.q.kernel_info(13, 17408, 6144, 4, 64)["k_windows"] == 1
    # few rows: one row block per workgroup, so windowing is kept
    assert U.q.kernel_info(13, 256, 6144, 4, 64)["k_windows"] > 1
    # K = 5120 ends half-way through its third wave step: a vector's slot holds
    # the row's 160 chunks and one zero chunk (10,944 bytes, not three padded
    # steps' 13,056), so 13 vectors fit one whole-K launch
    info = U.q.kernel_info(13, 17408, 5120, 4, 64)
    assert info["k_windows"] == 1 and info["lds_bytes"] >= 13 * 10944, info
    # vectors still equal their one-vector calls through the tiled launches
    p = gen.make_problem(N=17408, K=6144, bits=4, gs=64, sb="bf16", x_dtype="bf16", seed=61)
    dev = U.to_dev(p)
    U.say("whole-K tiles 17408x6144 M=13")
    y = U.gpu(p, dev, 13, torch.float32)
    for m in (0, 6, 7, 12):
        one = U.gpu(p, dev, 1, torch.float32, x=dev[3][m:m + 1])
        assert torch.equal(_bits(y[m]), _bits(one[0])), f"vector {m}"


@pytest.mark.parametrize("M,N,K,bits,gs,R,grid", [
    (1, 15360, 3840, 4, 64, 4, 240),     # bench shape: four rows, one workgroup of two row blocks per CU
    (13, 15360, 3840, 4, 64, 4, 240),    # bench shape at 13 vectors: four rows
    (1, 5120, 17408, 4, 64, 3, 214),     # 5120 rows: three rows spread over 214 CUs
    (13, 5120, 17408, 4, 64, 3, 214),
    (1, 17408, 5120, 4, 64, 3, 242),     # 17408 rows: three rows, one workgroup of three blocks per CU
    (1, 15360, 3840, 2, 128, 2, 480),    # 2 bits: two rows
])
def test_launch_shape_choices(M, N, K, bits, gs, R, grid):
    # the planner's documented choices on an MI355X (256 CUs)
    import torch as _t
    if _t.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("launch-shape choices are documented for 256 compute units")
    info = U.q.kernel_info(M, N, K, bits, gs)
    assert (info["rows_per_wave"], info["grid"]) == (R, grid), info


def test_graph_capture_replays_match_eager():
    # The calls can be captured in a HIP graph (one kernel launch per tile, no
    # allocation, no memset): every replay, with eager work and new inputs in
    # between, equals the eager call on the same inputs.
    p = gen.make_problem("up_4b_15360x3840")
    w, s, b, x = U.to_dev(p)
    xs = gen.make_x(p.K, p.x_dtype, 77, rows=3 * 13)
    xall = U.x_to_dev(xs, p.x_dtype)
    xin = x[:13].clone()
    y_graph = torch.empty(13, p.N, dtype=torch.float32, device=x.device)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        U.q.affine(w, s, b, xin, bits=p.bits, group_size=p.gs, out=y_graph)      # warm-up
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        U.q.affine(w, s, b, xin, bits=p.bits, group_size=p.gs, out=y_graph,
                   stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i in range(3):
        U.say(f"graph replay {i}")
        xin.copy_(xall[13 * i:13 * (i + 1)])
        eager = U.gpu(p, (w, s, b, xall[13 * i:13 * (i + 1)]), 13, torch.float32)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y_graph), _bits(eager)), f"replay {i}"


def test_lds_limit_kept_across_shapes():
    # One kernel instance serves shapes with different LDS sizes above the
    # 64 KiB default (fp32 activations, 4 vectors: two and three wave steps of
    # K staged whole).  Planning the smaller one after the larger one must not
    # lower the limit the larger one's launch needs.
    infos = [U.q.kernel_info(4, 512, K, 4, 64, x_dt=U.q.DT_F32) for K in (6144, 4096)]
    assert infos[0]["lds_bytes"] > infos[1]["lds_bytes"] > 65536, infos
    assert infos[0]["k_windows"] == infos[1]["k_windows"] == 1
    for K in (6144, 4096, 6144):
        p = gen.make_problem(N=512, K=K, bits=4, gs=64, sb="bf16", x_dtype="f32", seed=K)
        dev = U.to_dev(p)
        U.say(f"LDS limit K={K}")
        y = U.gpu(p, dev, 4, torch.float32)
        U.check_parity(y, U.ref(p, 4), f"K={K}")


def test_concurrent_calls_from_host_threads():
    # Calls from several host threads, each on its own stream, with shapes and
    # M that the first call of each thread still has to plan: every result
    # equals the same call made alone.
    import threading
    probs = [gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb="bf16", x_dtype="bf16", seed=N + K)
             for N, K, bits, gs in ((300, 2560, 4, 64), (517, 1536, 4, 128), (260, 4096, 2, 128), (129, 1024, 2, 64))]
    devs = [U.to_dev(p) for p in probs]
    Ms = (1, 3, 7, 13)
    jobs = [(i, M) for i in range(len(probs)) for M in Ms]
    out = {}
    errors = []

    def worker(t):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for k in range(3):
                    for j, (i, M) in enumerate(jobs):
                        if (j + t) % 4 == 0:
                            w, s, b, x = devs[i]
                            y = U.q.affine(w, s, b, x[:M], bits=probs[i].bits, group_size=probs[i].gs,
                                           out_dtype=torch.float32)
                            out[(t, k, i, M)] = y
            st.synchronize()
        except Exception as e:  # noqa: BLE001
            errors.append(repr(e))

    U.say("concurrent host threads")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for (t, k, i, M), y in out.items():
        w, s, b, x = devs[i]
        alone = U.gpu(probs[i], devs[i], M, torch.float32)
        assert torch.equal(_bits(y), _bits(alone)), (t, k, i, M)
    assert len(out) == 3 * len(jobs)
