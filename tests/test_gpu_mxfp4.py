"""GPU parity of the mxfp4 mode through the C ABI against the oracle: small
shapes over wave-step tails and ragged row blocks, the longest K, tiles of
vectors, the up-projection workload, exact read-out, bf16 rounding, fp32
activations, and every output vector against the one-vector call bit for
bit."""
import numpy as np
import pytest
import torch

import gpu_util as U
from inputs import gen
from oracle import oracle

pytestmark = pytest.mark.gpu


def _dev(p):
    w = torch.from_numpy(p.w_packed.view(np.int32)).to(U.DEV)
    s = torch.from_numpy(p.scales).to(U.DEV)
    return w, s


def _x(p, rows, x_dtype="bf16"):
    xs = gen.make_x(p.K, x_dtype, 7 + p.N, rows=rows)
    return xs, U.x_to_dev(xs, x_dtype)


def _ref(p, xs, x_dtype="bf16"):
    return oracle.default().qmv_mxfp4(p.w_packed, p.scales, xs, x_dtype=oracle.DT[x_dtype], nthreads=16)


def _bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


CASES = [  # N, K, Ms
    (67, 2080, (1, 3, 13)),      # 65 chunks: one full wave step and a 1-chunk tail
    (1, 32, (1, 2)),             # one block, one row
    (130, 4096, (2, 13)),        # two full wave steps
    (33, 544, (1, 5, 27)),       # 27 vectors: three tiles
    (200, 32768, (1, 4)),        # long K: two vectors per launch
    (5, 65536, (1, 3)),          # the longest K
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}_K{c[1]}")
def test_mx_small_vs_oracle(case):
    N, K, Ms = case
    p = gen.make_mx_problem(N, K, "bf16", seed=N + K)
    w, s = _dev(p)
    xs, xd = _x(p, max(Ms))
    for M in Ms:
        U.say(f"mxfp4 N={N} K={K} M={M}")
        y = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.float32)
        torch.cuda.synchronize()
        U.check_parity(y, _ref(p, xs[:M]), f"mxfp4 N={N} K={K} M={M}")
        y16 = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(y16.view(torch.int16), U.rne_bf16(y).view(torch.int16))
        for m in range(M):
            one = U.q.mxfp4(w, s, xd[m:m + 1], out_dtype=torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(_bits(y[m]), _bits(one[0])), f"M={M} vector {m}"


def test_mx_workload_up_15360x3840():
    p = gen.make_mx_problem(15360, 3840, "bf16", seed=4001)
    w, s = _dev(p)
    xs, xd = _x(p, 13)
    for M in (1, 13):
        U.say(f"mxfp4 15360x3840 M={M}")
        y = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.float32)
        torch.cuda.synchronize()
        U.check_parity(y, _ref(p, xs[:M]), f"mxfp4 15360x3840 M={M}")


def test_mx_readout_exact():
    # scale 1 (E = 127) and x = e_k: y[m][n] is the E2M1 value of q[n][k_m] exactly
    import json, os
    table = np.array(json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_e2m1.json")))["e2m1"])
    N, K = 37, 4096
    p = gen.make_mx_problem(N, K, "bf16", seed=9, keep_q=True)
    p.scales[:] = 127
    w, s = _dev(p)
    ks = [0, 1, 31, 32, 63, 64, 2047, 2048, 4000, 4095]
    x = np.zeros((len(ks), K), dtype=np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    xd = torch.from_numpy(x).to(torch.bfloat16).to(U.DEV)
    U.say("mxfp4 read-out")
    y = U.q.mxfp4(w, s, xd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), table[p.q[:, ks].T].astype(np.float32))


def _random_cases(n=60, seed=4242, n_hi=321, seed0=6000):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = 32 * int(rng.integers(1, 257))
        N = int(rng.integers(1, n_hi))
        M = int(rng.choice([1, 2, 3, 4, 5, 7, 9, 13, 14, 20, 27]))
        out.append((N, K, M, seed0 + i))
    return out


# 60 shapes with up to 320 rows and 20 with one to three rows (held to the
# a-priori bound where their few outputs cancel below 2e-5)
@pytest.mark.parametrize("case", _random_cases() + _random_cases(20, 4243, 4, 6500),
                         ids=lambda c: f"N{c[0]}_K{c[1]}_M{c[2]}")
def test_mx_random_shape_vs_oracle(case):
    # seeded random shapes (ragged N, K from one block up, M up to 27) against
    # the oracle, bf16 rounding and the one-vector calls of the first and last vector
    N, K, M, seed = case
    p = gen.make_mx_problem(N, K, "bf16", seed=seed)
    w, s = _dev(p)
    xs, xd = _x(p, max(M, 13))
    U.say(f"mxfp4 random N={N} K={K} M={M}")
    y = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.float32)
    y16 = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    mag = oracle.default().qmv_mxfp4_mag(p.scales, xs[:M], x_dtype=oracle.BF16)
    U.check_parity(y, _ref(p, xs[:M]), f"mxfp4 N={N} K={K} M={M}", mag=mag,
                   depth=U.mx_depth(K, "bf16"))
    assert torch.equal(y16.view(torch.int16), U.rne_bf16(y).view(torch.int16))
    for m in sorted({0, M - 1}):
        one = U.q.mxfp4(w, s, xd[m:m + 1], out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y[m]), _bits(one[0])), f"vector {m}"


F32_CASES = [  # N, K, Ms: fp32 activations (four vectors per launch)
    (67, 2080, (1, 4, 5, 13)),   # wave-step tail; 5 and 13 vectors: balanced tiles
    (300, 4096, (2, 3)),         # ragged row blocks
    (200, 32768, (1, 4)),        # long K: one vector whole, four in K windows
    (5, 65536, (1, 3)),          # the longest K: K windows even for one vector
    (15360, 3840, (1, 13)),      # the up-projection shape
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: f"N{c[0]}_K{c[1]}")
def test_mx_f32_x_vs_oracle(case):
    N, K, Ms = case
    p = gen.make_mx_problem(N, K, "f32", seed=N + K + 1)
    w, s = _dev(p)
    xs, xd = _x(p, max(Ms), "f32")
    for M in Ms:
        U.say(f"mxfp4 fp32 x N={N} K={K} M={M}")
        y = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.float32)
        y16 = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        U.check_parity(y, _ref(p, xs[:M], "f32"), f"mxfp4 fp32 x N={N} K={K} M={M}")
        assert torch.equal(y16.view(torch.int16), U.rne_bf16(y).view(torch.int16))
        for m in sorted({0, M // 2, M - 1}):
            one = U.q.mxfp4(w, s, xd[m:m + 1], out_dtype=torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(_bits(y[m]), _bits(one[0])), f"M={M} vector {m}"


def _random_f32_cases(n=30, seed=4343):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = 32 * int(rng.integers(1, 513))
        N = int(rng.integers(1, 321))
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 13]))
        out.append((N, K, M, 7000 + i))
    return out


@pytest.mark.parametrize("case", _random_f32_cases(), ids=lambda c: f"N{c[0]}_K{c[1]}_M{c[2]}")
def test_mx_f32_x_random_shape_vs_oracle(case):
    # seeded random shapes with fp32 activations (K up to 16384, M up to 13)
    N, K, M, seed = case
    p = gen.make_mx_problem(N, K, "f32", seed=seed)
    w, s = _dev(p)
    xs, xd = _x(p, 13, "f32")
    U.say(f"mxfp4 fp32 x random N={N} K={K} M={M}")
    y = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.float32)
    torch.cuda.synchronize()
    mag = oracle.default().qmv_mxfp4_mag(p.scales, xs[:M], x_dtype=oracle.F32)
    U.check_parity(y, _ref(p, xs[:M], "f32"), f"mxfp4 fp32 x N={N} K={K} M={M}", mag=mag,
                   depth=U.mx_depth(K, "f32"))
    one = U.q.mxfp4(w, s, xd[M - 1:M], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y[M - 1]), _bits(one[0])), f"vector {M - 1}"


def test_mx_graph_capture_replays_match_eager():
    # mxfp4 calls captured in one HIP graph (bf16 x at M = 1 and 13, fp32 x at
    # M = 5: two tiles): every replay, with new inputs and eager calls in
    # between, equals the eager calls on the same inputs bit for bit.
    p = gen.make_mx_problem(15360, 3840, "bf16", seed=4101)
    w, s = _dev(p)
    xs_b, xall_b = _x(p, 3 * 13)
    xall_f = U.x_to_dev(gen.make_x(p.K, "f32", 4102, rows=3 * 5), "f32")
    xin_b = xall_b[:13].clone()
    xin_f = xall_f[:5].clone()
    outs = [torch.empty(1, p.N, dtype=torch.float32, device=U.DEV),
            torch.empty(13, p.N, dtype=torch.bfloat16, device=U.DEV),
            torch.empty(5, p.N, dtype=torch.float32, device=U.DEV)]

    def calls(stream):
        U.q.mxfp4(w, s, xin_b[:1], out=outs[0], stream=stream)
        U.q.mxfp4(w, s, xin_b, out=outs[1], stream=stream)
        U.q.mxfp4(w, s, xin_f, out=outs[2], stream=stream)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        calls(stream)                                                   # warm-up
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i in range(3):
        U.say(f"mxfp4 graph replay {i}")
        xb = xall_b[13 * i:13 * (i + 1)]
        xf = xall_f[5 * i:5 * (i + 1)]
        xin_b.copy_(xb)
        xin_f.copy_(xf)
        eager = [U.q.mxfp4(w, s, xb[:1], out_dtype=torch.float32),
                 U.q.mxfp4(w, s, xb, out_dtype=torch.bfloat16),
                 U.q.mxfp4(w, s, xf, out_dtype=torch.float32)]
        g.replay()
        torch.cuda.synchronize()
        for j in range(3):
            assert torch.equal(_bits(outs[j]), _bits(eager[j])), f"replay {i} call {j}"


def test_mx_special_scale_exponents():
    """E8M0 scales at the ends of the range: one block per row at E = 0 (the
    subnormal 2^-127), 1, 2, 253 or 254 (that block's codes zero but one 0.5,
    on an activation below 1 in magnitude, so the row stays finite); rows
    whose every block is at E = 0..2, of which rows 15..19 hold two E = 0
    blocks of one such 0.5 code each and nothing else (results below 2^-126,
    which must not flush to zero); and rows with one E = 255 block, whose
    outputs must be NaN for every vector while every other row stays finite.
    Held to the a-priori bound of the fp32 evaluation plus one subnormal
    spacing per rounding."""
    N, K, M = 48, 256, 3
    p = gen.make_mx_problem(N, K, "bf16", seed=77, keep_q=True)
    xs, xd = _x(p, M)
    xf = gen.bf16_bits_to_f32(xs)
    rng = np.random.default_rng(78)
    q, e = p.q.copy(), p.scales.copy()
    nb = K // 32
    for n, E in enumerate((0, 1, 2, 253, 254) * 3):           # rows 0..14: one special block
        blk = n % nb
        e[n, blk] = E
        if E >= 253:
            ks = [k for k in range(32 * blk, 32 * blk + 32) if np.all(np.abs(xf[:, k]) < 1.0)]
            q[n, 32 * blk:32 * blk + 32] = 0
            q[n, ks[n % len(ks)]] = 1                            # E2M1 code 1 = 0.5
    e[15:24] = rng.integers(0, 3, size=(9, nb))                  # rows 15..23: every block tiny
    for n in range(15, 20):                                      # rows 15..19: subnormal results
        q[n] = 0
        for blk in (n % nb, (n + 3) % nb):
            e[n, blk] = 0
            ks = [k for k in range(32 * blk, 32 * blk + 32) if np.all(np.abs(xf[:, k]) < 1.0)]
            q[n, ks[n % len(ks)]] = 1
    nan_rows = [24, 31, 47]
    for n in nan_rows:
        e[n, n % nb] = 255
    p.w_packed = gen.pack(q, 4)
    p.scales = e
    w, s = _dev(p)
    U.say("mxfp4 special scale exponents")
    y = U.q.mxfp4(w, s, xd[:M], out_dtype=torch.float32)
    torch.cuda.synchronize()
    g = y.cpu().numpy().astype(np.float64)
    is_nan = np.isnan(g)
    assert np.array_equal(is_nan.any(axis=0), np.isin(np.arange(N), nan_rows)), np.nonzero(is_nan.any(axis=0))
    assert is_nan[:, nan_rows].all()
    ok = np.setdiff1d(np.arange(N), nan_rows)
    assert np.isfinite(g[:, ok]).all()
    want = _ref(p, xs[:M])
    mag = oracle.default().qmv_mxfp4_mag(p.scales, xs[:M], x_dtype=oracle.DT["bf16"])
    d = U.mx_depth(K, "bf16")
    bound = U.gamma(d) * mag[:, ok] + d * 2.0 ** -149
    over = np.abs(g[:, ok] - want[:, ok]) > bound
    assert not over.any(), [(int(m), int(ok[n])) for m, n in zip(*np.nonzero(over))][:8]
    # rows 15..19 are subnormal results (two terms below 2^-127 each), not flushed to zero
    tiny = g[:, 15:20]
    assert np.all(np.abs(tiny) < 2.0 ** -126) and np.all(tiny != 0.0)
    for m in range(M):
        one = U.q.mxfp4(w, s, xd[m:m + 1], out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y[m]), _bits(one[0])), f"vector {m}"
