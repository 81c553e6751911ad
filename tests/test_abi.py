"""The C ABI library loads, exports every function include/qmv.h declares, and
rejects bad arguments on the host before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmv_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from bit_quantized_gemv_amd import qmv
    if not os.path.exists(qmv.library_path()):
        from bit_quantized_gemv_amd import build
        build.build()
    return qmv.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == ["qmv_affine", "qmv_affine_ex", "qmv_affine_shape", "qmv_affine_timeline",
                                    "qmv_kernel_info", "qmv_mxfp4", "qmv_status_string",
                                    "qmv_stream_read", "qmv_stream_read_ex"]


def test_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    from bit_quantized_gemv_amd import qmv
    names = ["QMV_OK", "QMV_E_NULL", "QMV_E_BITS", "QMV_E_GROUP", "QMV_E_SHAPE", "QMV_E_M_RANGE",
             "QMV_E_ALIGN", "QMV_E_DTYPE", "QMV_E_ROWS", "QMV_E_ALIAS", "QMV_E_LAUNCH"]
    for i, n in enumerate(names):
        assert qmv.status_string(i) == n
    assert qmv.status_string(99) == "QMV_E_UNKNOWN"
    hdr = open(HEADER).read()
    for i, n in enumerate(names):
        assert re.search(rf"\b{n}\s*=\s*{i}\b", hdr), n


# fake, 16-byte aligned, far-apart addresses: validation fails before any use
A = 1 << 20
S = 1 << 40
W, SC, BI, X, Y = A, A + S, A + 2 * S, A + 3 * S, A + 4 * S
GOOD = dict(M=1, N=256, K=512, bits=4, gs=64, xdt=2, sdt=2, ydt=2, R=0)


def call(L, w=W, s=SC, b=BI, x=X, y=Y, **kw):
    a = dict(GOOD)
    a.update(kw)
    return L.qmv_affine_ex(w, s, b, x, y, a["M"], a["N"], a["K"], a["bits"], a["gs"],
                           a["xdt"], a["sdt"], a["ydt"], a["R"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(w=0), 1), (dict(s=0), 1), (dict(b=0), 1), (dict(x=0), 1), (dict(y=0), 1),
    (dict(bits=3), 2), (dict(bits=8), 2), (dict(bits=1), 2),
    (dict(gs=32), 3), (dict(gs=256), 3),
    (dict(N=0), 4), (dict(N=-5), 4), (dict(K=0), 4), (dict(K=96), 4), (dict(K=32), 4),
    (dict(K=(1 << 20) + 64), 4),
    (dict(M=0), 5), (dict(M=65537), 5), (dict(M=-1), 5),
    (dict(w=W + 8), 6), (dict(s=SC + 4), 6), (dict(b=BI + 2), 6), (dict(x=X + 8), 6),
    (dict(y=Y + 1), 6), (dict(y=Y + 2, ydt=0), 6),
    (dict(xdt=1), 7), (dict(xdt=5), 7), (dict(sdt=0), 7), (dict(ydt=1), 7),
    (dict(R=5), 8), (dict(R=8), 8), (dict(R=-1), 8),
    (dict(y=X), 9), (dict(y=W + 64), 9), (dict(y=SC - 16), 9),
])
def test_rejects_bad_arguments(L, kw, code):
    assert call(L, **kw) == code


def test_kernel_info_validates(L):
    from bit_quantized_gemv_amd import qmv
    info = qmv.KernelInfo()
    # (M, N, K, bits, gs, x_dt, sb_dt, y_dt, R, out)
    assert L.qmv_kernel_info(1, 256, 512, 3, 64, 2, 2, 2, 0, ctypes.byref(info)) == 2
    assert L.qmv_kernel_info(65537, 256, 512, 4, 64, 2, 2, 2, 0, ctypes.byref(info)) == 5
    assert L.qmv_kernel_info(1, 256, 512, 4, 64, 2, 2, 2, 0, None) == 1
    assert L.qmv_kernel_info(1, 256, 512, 4, 64, 2, 0, 2, 0, ctypes.byref(info)) == 7   # sb_dt f32
    assert L.qmv_kernel_info(1, 256, 512, 4, 64, 2, 2, 1, 0, ctypes.byref(info)) == 7   # y_dt f16
    assert L.qmv_kernel_info(1, 256, 512, 4, 64, 2, 2, 2, 5, ctypes.byref(info)) == 8


def test_timeline_validates(L):
    # the stamped launch: pure host checks, in the header's order, before any HIP call
    from bit_quantized_gemv_amd import qmv
    info = qmv.TimelineInfo()
    ST = A + 5 * S

    def tl(w=W, s=SC, b=BI, x=X, y=Y, M=1, N=256, K=512, bits=4, gs=64, ydt=2, R=0, st=ST, n=1 << 20,
           inf=info):
        return L.qmv_affine_timeline(w, s, b, x, y, M, N, K, bits, gs, ydt, R, st, n,
                                     None if inf is None else ctypes.byref(inf), None)
    assert tl(inf=None) == 1                       # QMV_E_NULL: info is required
    assert tl(w=0) == 1
    assert tl(K=96) == 4                           # not a multiple of the group size 64
    assert tl(bits=3) == 2 and tl(gs=32) == 3
    assert tl(bits=4, gs=128) == 3 and tl(bits=2, gs=64) == 3   # only 4-bit g64 and 2-bit g128 are stamped
    assert tl(M=0) == 5 and tl(M=14) == 5          # one launch of at most 13 vectors
    assert tl(x=X + 8) == 6
    assert tl(ydt=1) == 7
    assert tl(R=5) == 8
    assert tl(y=X) == 9
    assert tl(st=ST + 4) == 6                      # stamps 8-byte aligned
    assert tl(n=0) == 4                            # an empty stamps buffer
    assert tl(st=Y) == 9 and tl(st=W + 8) == 9     # stamps overlap y / the weights
    # the checks end here: the next step asks the runtime for the device
    # (QMV_E_LAUNCH without a GPU)


def test_shape_launch_validates(L):
    # the launch with a given shape: host checks before any HIP call
    def sh(w=W, s=SC, b=BI, x=X, y=Y, M=1, N=256, K=512, bits=4, gs=64, R=2, Wv=8, per=1):
        return L.qmv_affine_shape(w, s, b, x, y, M, N, K, bits, gs, 2, 2, 2, R, Wv, per, None, None)
    assert sh(R=0) == 8                            # QMV_E_ROWS: the rows per wavefront are given
    assert sh(R=5) == 8
    assert sh(bits=2, gs=128, R=3) == 8            # no three-row 2-bit instances
    assert sh(w=0) == 1
    assert sh(K=96) == 4
    assert sh(Wv=0) == 4 and sh(Wv=9) == 4         # at most eight wavefronts per workgroup
    assert sh(per=0) == 4
    assert sh(y=X) == 9
    # the checks end here: the next step asks the runtime for the device


def _tensors(N=4, K=512, bits=4, gs=64, M=1):
    import torch
    w = torch.zeros(N, K * bits // 32, dtype=torch.int32)
    s = torch.zeros(N, K // gs, dtype=torch.bfloat16)
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    return w, s, s.clone(), x


@pytest.mark.parametrize("what", ["w_cols", "w_rows", "scales", "biases", "bits", "gs", "K",
                                  "dtype_mix", "x_3d"])
def test_binding_checks_shapes_before_the_call(what):
    """Wrong shapes raise in the binding, before anything reaches the C ABI
    (which sees only pointers): the checks run before the device check, so
    CPU tensors show it."""
    import torch
    from bit_quantized_gemv_amd import qmv
    w, s, b, x = _tensors()
    kw = dict(bits=4, group_size=64)
    if what == "w_cols":
        w = w[:, :-4].contiguous()
    elif what == "w_rows":        # scales and biases for 5 rows, w for 4
        s, b = torch.zeros(5, 8, dtype=torch.bfloat16), torch.zeros(5, 8, dtype=torch.bfloat16)
    elif what == "scales":
        s = torch.zeros(4, 4, dtype=torch.bfloat16)
    elif what == "biases":
        b = torch.zeros(4, 16, dtype=torch.bfloat16)
    elif what == "bits":
        kw["bits"] = 2            # w holds 4-bit rows: K would be 1024, x says 512
    elif what == "gs":
        kw["group_size"] = 128    # scales hold 8 groups, 128 would need 4
    elif what == "K":
        x = torch.zeros(1, 480, dtype=torch.bfloat16)
    elif what == "dtype_mix":
        b = b.half()
    elif what == "x_3d":
        x = x.view(1, 1, 512)
    err = TypeError if what == "dtype_mix" else ValueError
    with pytest.raises(err) as ei:
        qmv.affine(w, s, b, x, **kw)
    assert "CUDA" not in str(ei.value), str(ei.value)


@pytest.mark.parametrize("what", ["w_cols", "scales_rows", "scales_cols", "K"])
def test_mxfp4_binding_checks_shapes_before_the_call(what):
    import torch
    from bit_quantized_gemv_amd import qmv
    w = torch.zeros(4, 64, dtype=torch.int32)
    s = torch.zeros(4, 16, dtype=torch.uint8)
    x = torch.zeros(1, 512, dtype=torch.bfloat16)
    if what == "w_cols":
        w = torch.zeros(4, 60, dtype=torch.int32)
    elif what == "scales_rows":
        s = torch.zeros(3, 16, dtype=torch.uint8)
    elif what == "scales_cols":
        s = torch.zeros(4, 15, dtype=torch.uint8)
    elif what == "K":
        x = torch.zeros(1, 500, dtype=torch.bfloat16)
    with pytest.raises(ValueError) as ei:
        qmv.mxfp4(w, s, x)
    assert "CUDA" not in str(ei.value), str(ei.value)


def test_binding_refuses_cpu_tensors():
    import torch
    from bit_quantized_gemv_amd import qmv
    w = torch.zeros(4, 64, dtype=torch.int32)
    s = torch.zeros(4, 8, dtype=torch.bfloat16)
    x = torch.zeros(1, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qmv.affine(w, s, s, x, bits=4, group_size=64)


def test_stream_read_validates(L):
    # argument errors return before any HIP call
    P = ctypes.c_void_p
    L.qmv_stream_read.argtypes = [P, ctypes.c_longlong, P, ctypes.c_int, P]
    assert L.qmv_stream_read(None, 1024, 4096, 0, None) == 1          # QMV_E_NULL
    assert L.qmv_stream_read(4096, 1024, None, 0, None) == 1
    assert L.qmv_stream_read(4096, 1000, 8192, 0, None) == 4          # QMV_E_SHAPE: not whole 16-byte chunks
    assert L.qmv_stream_read(4096, 0, 8192, 0, None) == 4
    assert L.qmv_stream_read(4104, 1024, 8192, 0, None) == 6          # QMV_E_ALIGN
    assert L.qmv_stream_read(4096, 1024, 8194, 0, None) == 6
    I = ctypes.c_int
    L.qmv_stream_read_ex.argtypes = [P, ctypes.c_longlong, P, I, I, I, I, I, P]
    for shape in ((0, 8, 4, 0), (33, 8, 4, 0), (4, 0, 4, 0), (4, 17, 4, 0), (4, 8, 3, 0),
                  (4, 8, 32, 0), (4, 8, 4, 2)):
        assert L.qmv_stream_read_ex(4096, 1024, 8192, 0, *shape, None) == 4, shape
    assert L.qmv_stream_read_ex(None, 1024, 8192, 0, 4, 8, 4, 0, None) == 1


def test_mxfp4_validates(L):
    # argument errors of the mxfp4 mode return before any HIP call; every call
    # here fails validation, so none reaches a launch
    P, I = ctypes.c_void_p, ctypes.c_int
    L.qmv_mxfp4.argtypes = [P, P, P, P, I, I, I, I, I, P]
    w, s, x, y = 1 << 20, 1 << 24, 1 << 28, 1 << 32
    F32, F16, BF16 = 0, 1, 2
    call = lambda **k: L.qmv_mxfp4(k.get("w", w), k.get("s", s), k.get("x", x), k.get("y", y),
                                   k.get("M", 1), k.get("N", 8), k.get("K", 64), k.get("xdt", BF16),
                                   k.get("dt", BF16), None)
    assert call(w=None) == 1 and call(s=None) == 1 and call(x=None) == 1 and call(y=None) == 1
    assert call(M=0) == 5 and call(M=65537) == 5                        # QMV_E_M_RANGE
    assert call(K=48) == 4 and call(K=16) == 4 and call(K=65536 + 32) == 4 and call(N=0) == 4
    assert call(dt=F16) == 7 and call(xdt=F16) == 7 and call(xdt=5) == 7  # QMV_E_DTYPE
    assert call(w=w + 8) == 6 and call(x=x + 8) == 6 and call(y=y + 2, dt=F32) == 6
    assert call(y=w + 64) == 9                                          # QMV_E_ALIAS
    # one fp32 vector of K = 64 spans 256 bytes (bf16: 128)
    assert call(y=x + 192, M=1, K=64, xdt=F32) == 9
    # scales need no alignment: the call gets past the alignment checks to the alias check
    assert call(s=s + 1, y=w + 64) == 9
