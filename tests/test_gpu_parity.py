"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small shapes span several wave steps, ragged step tails, ragged row blocks,
K windows, single-group rows, N = 1, both code widths, both group sizes and all
dtypes, compared element by element with the full oracle.  The full-size
workloads are compared on every row of every vector, in the launch
configuration the bench times.  The exact-integer and read-out cases must
match bit for bit.
"""
import numpy as np
import pytest
import torch

import gpu_util as U
from inputs import gen
from oracle import oracle

pytestmark = pytest.mark.gpu

SMALL = [  # N, K, bits, gs, sb, x, Ms
    (67, 2560, 4, 64, "bf16", "bf16", (1, 3, 13)),    # 80 chunks: 1.25 wave steps
    (67, 6400, 4, 64, "bf16", "bf16", (2, 13)),       # K windows at M = 13
    (33, 512, 4, 128, "f16", "bf16", (1, 5)),
    (130, 4608, 2, 128, "bf16", "bf16", (1, 5, 13)),  # 72 chunks
    (45, 1024, 2, 64, "f16", "bf16", (2, 9)),
    (256, 512, 4, 64, "f16", "f32", (1, 4)),          # the tiny workload's shape
    (61, 2560, 2, 64, "bf16", "f32", (1, 7)),
    (29, 1536, 4, 128, "bf16", "f32", (13,)),
    (1, 128, 4, 64, "bf16", "bf16", (1, 13)),          # N = 1
    (5, 64, 4, 64, "f16", "bf16", (1, 2)),             # one group per row
    (3, 128, 2, 128, "bf16", "f32", (1, 3)),
    (200, 8192, 2, 64, "bf16", "bf16", (6,)),          # 2 full wave steps at 2 bits
    (8, 1 << 20, 4, 128, "bf16", "bf16", (1, 13)),      # the largest K: 512 wave steps, hundreds of K windows
    (96, 131072, 2, 64, "f16", "bf16", (2, 13)),        # long K at 2 bits: many windows, restaged per window
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"N{c[0]}_K{c[1]}_b{c[2]}_g{c[3]}_{c[4]}_{c[5]}")
def test_small_vs_oracle(case):
    N, K, bits, gs, sb, xdt, Ms = case
    p = gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype=xdt, seed=N * 7 + K)
    dev = U.to_dev(p)
    for M in Ms:
        U.say(f"case N={N} K={K} bits={bits} gs={gs} sb={sb} x={xdt} M={M}")
        want = U.ref(p, M)
        y32 = U.gpu(p, dev, M, torch.float32)
        U.check_parity(y32, want, f"M={M}")
        y16 = U.gpu(p, dev, M, torch.bfloat16)
        assert torch.equal(y16.view(torch.int16), U.rne_bf16(y32).view(torch.int16))


@pytest.mark.parametrize("N,K,bits,gs,sb", [
    (67, 2560, 4, 128, "bf16"),     # four lanes per group; 67 rows: a ragged row group
    (130, 1536, 4, 128, "f16"),
    (61, 2560, 4, 64, "bf16"),      # two lanes per group
    (45, 4608, 2, 128, "bf16"),
])
def test_every_rows_per_wave_vs_oracle(N, K, bits, gs, sb):
    # every row blocking (1-4 rows per wavefront; 2-bit codes up to 2) against the
    # oracle, and bit-identical to each other, at M = 1 .. 13 with bf16 activations
    p = gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype="bf16", seed=N * 5 + K)
    dev = U.to_dev(p)
    Rs = (1, 2, 3, 4) if bits == 4 else (1, 2)
    for M in (1, 2, 3, 4, 8, 13):
        want = U.ref(p, M)
        ys = []
        for R in Rs:
            U.say(f"rows per wave N={N} K={K} bits={bits} gs={gs} M={M} R={R}")
            ys.append(U.gpu(p, dev, M, torch.float32, R=R))
        U.check_parity(ys[0], want, f"M={M}")
        for R, y in zip(Rs[1:], ys[1:]):
            assert torch.equal(y.view(torch.int32), ys[0].view(torch.int32)), f"M={M} R={R}"


WORKLOADS = [n for n in gen.WORKLOADS if n != "tiny_4b_g64"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_vs_oracle_every_row(name):
    """Each full-size workload at M = 1 and every M it names, in the launch the
    bench times (the library's default), element by element against the full
    oracle: every row of every vector, normwise and under the a-priori bound.
    The bf16 output equals the RNE of the fp32 output and lies within one bf16
    ulp of the exact value (plus the fp32 tolerance, for outputs near zero)."""
    wl = gen.WORKLOADS[name]
    p = gen.make_problem(name)
    dev = U.to_dev(p)
    Ms = sorted(set((1,) + tuple(wl["Ms"])))
    U.say(f"workload {name}: oracle over {max(Ms)} vectors")
    want_all = U.ref(p, max(Ms), nthreads=16)        # vectors 0..M-1 are shared by every M
    mag_all = U.affine_mag(p, max(Ms))
    depth = U.affine_depth(p.K, p.bits, p.gs, p.x_dtype)
    for M in Ms:
        U.say(f"workload {name} M={M}")
        y32 = U.gpu(p, dev, M, torch.float32)
        U.check_parity(y32, want_all[:M], f"{name} M={M}", mag=mag_all[:M], depth=depth)
        y16 = U.gpu(p, dev, M, torch.bfloat16)
        assert torch.equal(y16.view(torch.int16), U.rne_bf16(y32).view(torch.int16))
        U.check_bf16_output(y16, want_all[:M], f"{name} M={M}")


def test_tiny_workload_full():
    p = gen.make_problem("tiny_4b_g64")
    dev = U.to_dev(p)
    U.say("workload tiny_4b_g64 M=1")
    U.check_parity(U.gpu(p, dev, 1, torch.float32), U.ref(p, 1), "tiny")


def _exact_integer_problem(N, K, bits, gs, sb, xdt, seed):
    """x in {-2..2}, scale = 2^-3, bias = -zp * 2^-3: every partial sum is an
    exact multiple of 2^-3 far below 2^24, so any fp32 order gives the exact
    value."""
    p = gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype=xdt, seed=seed)
    G = K // gs
    zp = 8 if bits == 4 else 2
    tdt = torch.float16 if sb == "f16" else torch.bfloat16
    p.scales = torch.full((N, G), 0.125, dtype=tdt).view(torch.int16).numpy().view(np.uint16).copy()
    p.biases = torch.full((N, G), -zp * 0.125, dtype=tdt).view(torch.int16).numpy().view(np.uint16).copy()
    xi = np.random.default_rng(seed).integers(-2, 3, size=(13, K)).astype(np.float32)
    p.x = xi if xdt == "f32" else torch.from_numpy(xi).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    return p


@pytest.mark.parametrize("case", [
    (15360, 3840, 4, 64, "bf16", "bf16"), (3840, 15360, 4, 64, "bf16", "bf16"),
    (15360, 3840, 2, 128, "bf16", "bf16"), (17408, 5120, 4, 64, "bf16", "bf16"),
    (5120, 17408, 4, 64, "bf16", "bf16"), (77, 2560, 4, 128, "f16", "f32"),
    (91, 4608, 2, 64, "f16", "bf16"),
], ids=lambda c: f"N{c[0]}_K{c[1]}_b{c[2]}_g{c[3]}_{c[5]}")
def test_exact_integer_bit_exact(case):
    """Every row of every vector bit for bit, at M = 1 and 13 (the full-size
    projection shapes included)."""
    N, K, bits, gs, sb, xdt = case
    p = _exact_integer_problem(N, K, bits, gs, sb, xdt, seed=N + K)
    dev = U.to_dev(p)
    want = U.ref(p, 13, nthreads=16)
    for M in (1, 13):
        U.say(f"exact-integer N={N} K={K} bits={bits} gs={gs} M={M}")
        y = U.gpu(p, dev, M, torch.float32).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, want[:M])


@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 128), (2, 64), (2, 128)])
def test_readout_e_k(bits, gs):
    """scale 1, bias 0, x = e_k: y[m][n] = q[n][k_m] exactly, with q the
    generator's codes before packing."""
    N, K = 37, 8192
    wp, _, _, qc = gen.make_weights(N, K, bits, gs, "bf16", seed=5 + bits + gs, keep_q=True)
    G = K // gs
    ks = [0, 1, 31, 32, 63, 64, 2047, 2048, 4095, 4096, 6000, 8190, 8191]
    x = np.zeros((13, K), dtype=np.float32)
    x[np.arange(13), ks] = 1.0
    w = torch.from_numpy(wp.view(np.int32)).to(U.DEV)
    one = torch.ones(N, G, dtype=torch.bfloat16, device=U.DEV)
    zero = torch.zeros(N, G, dtype=torch.bfloat16, device=U.DEV)
    import bit_quantized_gemv_amd as q
    for xdt in ("bf16", "f32"):
        U.say(f"read-out bits={bits} gs={gs} x={xdt}")
        xd = U.x_to_dev(x if xdt == "f32" else torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), xdt)
        y = q.affine(w, one, zero, xd, bits=bits, group_size=gs, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), qc[:, ks].T.astype(np.float32))


def test_subnormal_fp16_scales():
    """fp16 parameters convert exactly, subnormals included."""
    N, K = 64, 1024
    p = gen.make_problem(N=N, K=K, bits=4, gs=64, sb="f16", x_dtype="f32", seed=3)
    p.scales = p.scales.copy()
    p.scales[:, ::3] = np.arange(1, 1 + p.scales[:, ::3].size, dtype=np.uint16).reshape(p.scales[:, ::3].shape) % 1023 + 1
    dev = U.to_dev(p)
    U.say("fp16 subnormal scales")
    U.check_parity(U.gpu(p, dev, 3), U.ref(p, 3), "subnormal scales")
