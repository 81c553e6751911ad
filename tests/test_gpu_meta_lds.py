"""GPU tests of the whole-K instances that keep each wavefront's scales and
biases in LDS (rows per wavefront a multiple of the lanes per group): parity
with the oracle, bit identity with the one-row instance (which loads them per
unit), and the fallback to per-unit loads where the copies do not fit.  The
cases cover odd group counts (rows that start 2 bytes into a 16-byte piece),
rows past N in the last row block, fewer rows than one wavefront holds, many
row blocks per workgroup, fp16 scales and fp32 activations."""
import pytest
import torch

import gpu_util as U
from inputs import gen

pytestmark = pytest.mark.gpu

CASES = [
    # N, K, bits, gs, sb, x, rows per wavefront, M values, copies in LDS
    (1000, 1984, 4, 64, "bf16", "bf16", 2, (1, 2, 3), 1),    # 31 groups per row
    (777, 2240, 4, 64, "f16", "bf16", 4, (1, 5, 13), 1),     # 35 groups, fp16 scales
    (300, 1152, 4, 128, "bf16", "f32", 4, (1, 2, 9), 1),     # four lanes per group, fp32 activations
    (513, 2176, 2, 128, "bf16", "bf16", 2, (1, 3), 1),       # 2-bit codes, 17 groups
    (3, 640, 4, 64, "bf16", "bf16", 4, (1, 2), 1),           # fewer rows than one wavefront's
    (1, 640, 4, 64, "f16", "bf16", 2, (1,), 1),
    (100000, 256, 4, 64, "bf16", "bf16", 2, (1, 2), 1),      # many row blocks per workgroup
    (3840, 15360, 4, 64, "bf16", "bf16", 4, (1, 2), 0),      # 4 x 240 groups: per-unit loads, one window
]


def _bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16)


@pytest.mark.parametrize("N,K,bits,gs,sb,xdt,R,Ms,meta", CASES)
def test_meta_lds_parity_and_identity(N, K, bits, gs, sb, xdt, R, Ms, meta):
    p = gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype=xdt, seed=N + K + R)
    dev = U.to_dev(p)
    x_dt = U.q.DT_F32 if xdt == "f32" else U.q.DT_BF16
    sb_dt = U.q.DT_F16 if sb == "f16" else U.q.DT_BF16
    for M in Ms:
        label = f"N={N} K={K} bits={bits} gs={gs} sb={sb} x={xdt} R={R} M={M}"
        U.say(label)
        info = U.q.kernel_info(M, N, K, bits, gs, x_dt=x_dt, sb_dt=sb_dt, rows_per_wave=R)
        assert info["meta_lds"] == meta and info["k_windows"] == 1, info
        y = U.gpu(p, dev, M, torch.float32, R=R)
        U.check_parity(y, U.ref(p, M), label)
        # one row per wavefront loads the scales and biases per unit; the
        # per-row arithmetic is the same, so the bits are too
        y1 = U.gpu(p, dev, M, torch.float32, R=1)
        assert U.q.kernel_info(M, N, K, bits, gs, x_dt=x_dt, sb_dt=sb_dt, rows_per_wave=1)["meta_lds"] == 0
        assert torch.equal(_bits(y), _bits(y1)), label
        if M > 1:
            for m in (0, M - 1):
                one = U.gpu(p, dev, 1, torch.float32, R=R, x=dev[3][m:m + 1])
                assert torch.equal(_bits(y[m]), _bits(one[0])), f"{label}: vector {m}"


def test_meta_lds_on_the_bench_shapes():
    # the planner's choices on the 12B-class projections hold the copies
    for M, N, K in ((1, 15360, 3840), (2, 15360, 3840), (13, 15360, 3840), (1, 3840, 15360)):
        info = U.q.kernel_info(M, N, K, 4, 64)
        assert info["meta_lds"] == 1, (M, N, K, info)
