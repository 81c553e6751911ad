"""The C ABI on the GPU: qmv_affine (the bf16 entry point) called directly
through ctypes, against qmv_affine_ex and the oracle; the binding's argument
checks raising before anything is launched; the mxfp4 mode's special
E8M0 scale bytes (0, 1, 2, 253, 254 and NaN) against the oracle; and the
launch with a given shape (qmv_affine_shape) bit for bit against the
library's own launch."""
import ctypes

import numpy as np
import pytest
import torch

import gpu_util as U
from inputs import gen
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,M", [("up_4b_15360x3840", 1), ("up_4b_15360x3840", 13),
                                    ("up_2b_15360x3840", 5)])
def test_qmv_affine_entry_point(name, M):
    """qmv_affine(w, s, b, x, y, M, N, K, bits, gs, stream) with bf16 x, scales,
    biases and y: bit-identical to qmv_affine_ex with the same dtypes and the
    library's row blocking, and within one bf16 ulp (plus the fp32 tolerance)
    of the exact value on every row."""
    p = gen.make_problem(name)
    w, s, b, x = U.to_dev(p)
    y = torch.full((M, p.N), -1.0, dtype=torch.bfloat16, device=U.DEV)
    y_ex = torch.full((M, p.N), -1.0, dtype=torch.bfloat16, device=U.DEV)
    L = U.q.lib()
    stream = torch.cuda.current_stream().cuda_stream
    U.say(f"qmv_affine {name} M={M}")
    st = L.qmv_affine(w.data_ptr(), s.data_ptr(), b.data_ptr(), x.data_ptr(), y.data_ptr(),
                      M, p.N, p.K, p.bits, p.gs, ctypes.c_void_p(stream))
    assert st == 0, U.q.status_string(st)
    st = U.q.affine_ptr(w.data_ptr(), s.data_ptr(), b.data_ptr(), x.data_ptr(), y_ex.data_ptr(),
                        M, p.N, p.K, p.bits, p.gs, U.q.DT_BF16, U.q.DT_BF16, U.q.DT_BF16, 0, stream)
    assert st == 0, U.q.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ex.view(torch.int16))
    U.check_bf16_output(y, U.ref(p, M, nthreads=16), f"qmv_affine {name} M={M}")


def test_qmv_affine_rejects_before_launch():
    """Validation errors from qmv_affine leave y untouched (nothing launched)."""
    p = gen.make_problem(N=64, K=512, bits=4, gs=64, sb="bf16", x_dtype="bf16", seed=1)
    w, s, b, x = U.to_dev(p)
    y = torch.full((1, 64), 7.0, dtype=torch.bfloat16, device=U.DEV)
    L = U.q.lib()
    assert L.qmv_affine(w.data_ptr(), s.data_ptr(), b.data_ptr(), x.data_ptr(), y.data_ptr(),
                        1, 64, 512, 3, 64, None) == 2
    assert L.qmv_affine(w.data_ptr(), s.data_ptr(), b.data_ptr(), x.data_ptr(), y.data_ptr(),
                        0, 64, 512, 4, 64, None) == 5
    torch.cuda.synchronize()
    assert bool((y.float() == 7.0).all())


@pytest.mark.parametrize("what", ["w", "scales", "biases", "gs", "out"])
def test_binding_shape_errors_launch_nothing(what):
    """Device tensors of the wrong shape raise ValueError in the binding, and
    the output tensor passed in is left as it was."""
    p = gen.make_problem(N=64, K=512, bits=4, gs=64, sb="bf16", x_dtype="bf16", seed=2)
    w, s, b, x = U.to_dev(p)
    out = torch.full((1, 64), 3.0, dtype=torch.float32, device=U.DEV)
    kw = dict(bits=4, group_size=64, out=out)
    if what == "w":
        w = w[:, :32].contiguous()
    elif what == "scales":
        s = s[:, :4].contiguous()
    elif what == "biases":
        b = b[:32].contiguous()
    elif what == "gs":
        kw["group_size"] = 128
    elif what == "out":
        kw["out"] = torch.empty((1, 63), dtype=torch.float32, device=U.DEV)
    with pytest.raises(ValueError):
        U.q.affine(w, s, b, x[:1], **kw)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())


def _mx_call(w, s, x):
    y = U.q.mxfp4(w, s, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def test_mxfp4_special_scale_bytes():
    """E8M0 bytes 0 (the subnormal 2^-127), 1, 2, 253, 254 and 255 (NaN).
    Rows 0-15 take only E in {0, 1, 2}, rows 16-31 only E in {253, 254}, rows
    32-63 the usual range, and row 40 one NaN block.  With N(0,1) activations
    the small-scale rows are compared (their outputs lie near the bottom of
    the fp32 range, subnormal steps included); with activations scaled by
    2^-124 the large-scale rows are (finite, near 2^3).  NaN appears in row 40
    and nowhere else."""
    N, K = 64, 256
    p = gen.make_mx_problem(N, K, "bf16", seed=31)
    rng = np.random.default_rng(31)
    sc = p.scales.copy()
    sc[0:16] = rng.choice([0, 1, 2], size=(16, K // 32))
    sc[16:32] = rng.choice([253, 254], size=(16, K // 32))
    sc[40, 3] = 255
    w = torch.from_numpy(p.w_packed.view(np.int32)).to(U.DEV)
    s = torch.from_numpy(sc).to(U.DEV)
    x64 = np.random.default_rng(32).standard_normal((3, K))
    # |x| >= 1/4 keeps x * 2^-124 a normal bf16 (>= 2^-126)
    x64 = np.sign(x64) * np.maximum(np.abs(x64), 0.25)
    orc = oracle.default()
    keep = np.ones(N, dtype=bool)
    keep[40] = False
    for scale, rows, finite in ((1.0, slice(0, 16), keep & (np.arange(N) >= 32) | (np.arange(N) < 16)),
                                (2.0 ** -124, slice(16, 32), keep)):
        xb = torch.from_numpy(x64 * scale).to(torch.bfloat16)
        xs = xb.view(torch.int16).numpy().view(np.uint16).copy()
        want = orc.qmv_mxfp4(p.w_packed, sc, xs, x_dtype=oracle.BF16)
        mag = orc.qmv_mxfp4_mag(sc, xs, x_dtype=oracle.BF16)
        U.say(f"mxfp4 special scales, x scaled by {scale:g}")
        got = _mx_call(w, s, xb.to(U.DEV))
        assert np.isnan(got[:, 40]).all() and np.isnan(want[:, 40]).all()
        # with unscaled x the 2^126..2^127 rows overflow (inf, or NaN where
        # lanes of opposite sign meet); every other row is finite
        assert np.isfinite(got[:, finite]).all()
        sub = got[:, rows]
        ref = want[:, rows]
        # normwise over the rows of this scale class, and the a-priori bound;
        # fp32 subnormal steps add at most 2^-150 absolute per rounding
        for m in range(3):
            err = np.abs(sub[m] - ref[m])
            assert np.max(err) <= 2e-5 * np.max(np.abs(ref[m])), (scale, m)
            assert np.all(err <= U.gamma(U.mx_depth(K, "bf16")) * mag[m, rows] + 64 * 2.0 ** -150), (scale, m)


@pytest.mark.parametrize("spec,M", [((1000, 1984, 4), 1), ((1000, 1984, 4), 5), ((777, 2176, 2), 3),
                                    ("up_4b_15360x3840", 1), ("down_4b_3840x15360", 13)])
def test_shape_launch_matches_the_library(spec, M):
    """qmv_affine_shape with a given rows per wavefront, workgroup size and row
    blocks per workgroup writes the bits qmv_affine_ex writes: the per-row
    arithmetic does not depend on the launch shape."""
    if isinstance(spec, str):
        p = gen.make_problem(spec)
    else:
        N, K, bits = spec
        p = gen.make_problem(N=N, K=K, bits=bits, gs=64 if bits == 4 else 128, sb="bf16", x_dtype="bf16",
                             seed=N + K)
    w, s, b, x = U.to_dev(p)
    xm = x[:M].contiguous()
    y = U.q.affine(w, s, b, xm, bits=p.bits, group_size=p.gs, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Rs = (1, 2, 3, 4) if p.bits == 4 else (1, 2)
    for R in Rs:
        for Wv in (3, 8):
            for per in (1, 3):
                U.say(f"shape launch {spec} M={M} R={R} W={Wv} per={per}")
                out = torch.full((M, p.N), float("nan"), dtype=torch.float32, device=U.DEV)
                info = U.q.KernelInfo()
                st = U.q.shape_ptr(w.data_ptr(), s.data_ptr(), b.data_ptr(), xm.data_ptr(), out.data_ptr(),
                                   M, p.N, p.K, p.bits, p.gs, U.q.DT_BF16, U.q.DT_BF16, U.q.DT_F32,
                                   R, Wv, per, info, torch.cuda.current_stream().cuda_stream)
                torch.cuda.synchronize()
                assert st == 0, (R, Wv, per, st)
                assert info.wg_size == 64 * Wv and info.rows_per_wave == R
                n_rb = -(-p.N // (Wv * R))
                assert info.grid == -(-n_rb // per)
                assert torch.equal(out.view(torch.int32), y.view(torch.int32)), (R, Wv, per)
