"""ctypes binding of the qmv C ABI (include/qmv.h).

Argument marshalling only: every step of the product runs in the HIP kernels of
lib/libqmv.so.  If the library has not been built this module raises -- there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "lib", "libqmv.so")

DT_F32, DT_F16, DT_BF16 = 0, 1, 2
MAX_M = 65536     # vectors per call
TILE_M = 13       # vectors per kernel launch


class QmvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class KernelInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("vgprs", "scratch_bytes", "lds_bytes", "wg_size",
                                             "grid", "waves_per_simd", "rows_per_wave",
                                             "k_windows", "prefetch_units", "meta_lds")]


STAMPS = 4        # values per wavefront written by the stamped launch


class TimelineInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("waves", "wg_size", "grid", "clock_khz",
                                             "blocks_per_cu", "product_blocks_per_cu",
                                             "vgprs", "product_vgprs")]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library {_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.qmv_affine.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
        L.qmv_affine.restype = I
        L.qmv_affine_ex.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, P]
        L.qmv_affine_ex.restype = I
        L.qmv_kernel_info.argtypes = [I, I, I, I, I, I, I, I, I, ctypes.POINTER(KernelInfo)]
        L.qmv_kernel_info.restype = I
        L.qmv_status_string.argtypes = [I]
        L.qmv_status_string.restype = ctypes.c_char_p
        L.qmv_stream_read.argtypes = [P, ctypes.c_longlong, P, I, P]
        L.qmv_stream_read.restype = I
        L.qmv_stream_read_ex.argtypes = [P, ctypes.c_longlong, P, I, I, I, I, I, P]
        L.qmv_stream_read_ex.restype = I
        L.qmv_mxfp4.argtypes = [P, P, P, P, I, I, I, I, I, P]
        L.qmv_mxfp4.restype = I
        L.qmv_affine_timeline.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, ctypes.c_longlong,
                                          ctypes.POINTER(TimelineInfo), P]
        L.qmv_affine_timeline.restype = I
        L.qmv_affine_shape.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, I,
                                       ctypes.POINTER(KernelInfo), P]
        L.qmv_affine_shape.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qmv_status_string(status).decode()


def affine_ptr(w, s, b, x, y, M, N, K, bits, group_size, x_dt=DT_BF16, sb_dt=DT_BF16,
               y_dt=DT_BF16, rows_per_wave=0, stream=0) -> int:
    """Raw C-ABI call with integer device pointers; returns the status code."""
    return lib().qmv_affine_ex(w, s, b, x, y, M, N, K, bits, group_size, x_dt, sb_dt, y_dt,
                               rows_per_wave, stream)


def stream_read_ptr(buf, nbytes, out, checksum=False, stream=0) -> int:
    """Raw C-ABI call of the streaming-read ceiling kernel (a measurement aid):
    reads the nbytes at device pointer buf; with checksum, XORs their XOR into
    the uint32 at out."""
    return lib().qmv_stream_read(buf, nbytes, out, 1 if checksum else 0, stream)


def stream_read_ex_ptr(buf, nbytes, out, wg_per_cu, waves_per_wg, batch, interleave=0,
                      checksum=False, stream=0) -> int:
    """The streaming-read ceiling kernel with an explicit launch shape."""
    return lib().qmv_stream_read_ex(buf, nbytes, out, 1 if checksum else 0, wg_per_cu,
                                    waves_per_wg, batch, interleave, stream)


def mxfp4_ptr(w, s, x, y, M, N, K, x_dt=DT_BF16, y_dt=DT_BF16, stream=0) -> int:
    """Raw C-ABI call of the mxfp4 mode with integer device pointers; returns
    the status code."""
    return lib().qmv_mxfp4(w, s, x, y, M, N, K, x_dt, y_dt, stream)


def mxfp4(w, scales, x, *, out=None, out_dtype=None, stream=None):
    """y[M][N] of the mxfp4 mode on the current (or given) torch stream.

    w: int32/uint32 [N][K/8] packed E2M1 codes (field 0 in the low bits);
    scales: uint8 [N][K/32] E8M0 block scales; x: bf16 or fp32 [M][K] (or [K]); out:
    optional fp32/bf16 [M][N] tensor, else allocated with out_dtype (default
    bf16).  Shapes, dtypes and devices are checked here (ValueError /
    TypeError) before the call: the C ABI sees only pointers.
    """
    import torch
    squeeze = x.dim() == 1
    if squeeze:
        x = x.unsqueeze(0)
    if w.dtype not in (torch.int32, torch.uint32):
        raise TypeError("w must be int32 or uint32 packed words")
    if scales.dtype != torch.uint8:
        raise TypeError("scales must be uint8 (E8M0)")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be bf16 or fp32")
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x must be [M][K] (or [K]) and w [N][K/8]")
    M, K = x.shape
    N = w.shape[0]
    if K % 32 != 0:
        raise ValueError(f"K = {K} is not a multiple of 32")
    _expect(w, (N, K // 8), "w")
    _expect(scales, (N, K // 32), "scales")
    _check_tensors(((w, "w"), (scales, "scales"), (x, "x")))
    out = _out_for(out, out_dtype, M, N, x, torch)
    st = torch.cuda.current_stream(x.device) if stream is None else stream
    status = mxfp4_ptr(w.data_ptr(), scales.data_ptr(), x.data_ptr(), out.data_ptr(), M, N, K,
                       _dt_of(x, "x"), _dt_of(out, "out"), st.cuda_stream)
    if status != 0:
        raise QmvError(status, "qmv_mxfp4")
    return out[0] if squeeze else out


def _dt_of(t, what):
    import torch
    if t.dtype == torch.float32:
        return DT_F32
    if t.dtype == torch.float16:
        return DT_F16
    if t.dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError(f"{what}: unsupported dtype {t.dtype}")


def affine(w, scales, biases, x, *, bits: int, group_size: int, out=None, out_dtype=None,
           rows_per_wave: int = 0, stream=None):
    """y[M][N] = qmv(x) on the current (or given) torch stream.

    w: int32/uint32 [N][K*bits/32] packed codes (field 0 in the low bits);
    scales, biases: fp16 or bf16 [N][K/group_size]; x: fp32 or bf16 [M][K]
    (or [K]); out: optional fp32/bf16 [M][N] tensor, else allocated with
    out_dtype (default bf16).  Shapes, dtypes and devices are checked here
    (ValueError / TypeError) before the call: the C ABI sees only pointers.
    """
    import torch
    squeeze = x.dim() == 1
    if squeeze:
        x = x.unsqueeze(0)
    if w.dtype not in (torch.int32, torch.uint32):
        raise TypeError("w must be int32 or uint32 packed words")
    if scales.dtype != biases.dtype:
        raise TypeError("scales and biases must share a dtype")
    if bits not in (2, 4):
        raise ValueError(f"bits must be 2 or 4, got {bits}")
    if group_size not in (64, 128):
        raise ValueError(f"group_size must be 64 or 128, got {group_size}")
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x must be [M][K] (or [K]) and w [N][K*bits/32]")
    M, K = x.shape
    N = w.shape[0]
    if K % group_size != 0:
        raise ValueError(f"K = {K} is not a multiple of group_size = {group_size}")
    _expect(w, (N, K * bits // 32), "w")
    _expect(scales, (N, K // group_size), "scales")
    _expect(biases, (N, K // group_size), "biases")
    _check_tensors(((w, "w"), (scales, "scales"), (biases, "biases"), (x, "x")))
    out = _out_for(out, out_dtype, M, N, x, torch)
    st = torch.cuda.current_stream(x.device) if stream is None else stream
    status = affine_ptr(w.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(),
                        out.data_ptr(), M, N, K, bits, group_size, _dt_of(x, "x"),
                        _dt_of(scales, "scales"), _dt_of(out, "out"), rows_per_wave,
                        st.cuda_stream)
    if status != 0:
        raise QmvError(status, "qmv_affine_ex")
    return out[0] if squeeze else out


def shape_ptr(w, s, b, x, y, M, N, K, bits, group_size, x_dt, sb_dt, y_dt, rows_per_wave,
              waves_per_wg, row_blocks_per_wg, info=None, stream=0) -> int:
    """Raw C-ABI call of one launch with its launch shape given (a measurement
    aid for sweeping it); info, if given, is a KernelInfo filled by the call."""
    return lib().qmv_affine_shape(w, s, b, x, y, M, N, K, bits, group_size, x_dt, sb_dt, y_dt,
                                  rows_per_wave, waves_per_wg, row_blocks_per_wg,
                                  None if info is None else ctypes.byref(info), stream)


def timeline_ptr(w, s, b, x, y, M, N, K, bits, group_size, y_dt, rows_per_wave, stamps,
                 stamps_len, info, stream=0) -> int:
    """Raw C-ABI call of the stamped launch (a measurement aid); info is a
    TimelineInfo filled by the call; stamps may be 0 (no launch)."""
    return lib().qmv_affine_timeline(w, s, b, x, y, M, N, K, bits, group_size, y_dt,
                                     rows_per_wave, stamps, stamps_len, ctypes.byref(info), stream)


def timeline(w, scales, biases, x, *, bits: int = 4, group_size: int = 64, rows_per_wave: int = 0,
             out=None, out_dtype=None, stream=None):
    """The one launch `affine` makes for bf16 activations and bf16
    scales/biases with 4-bit codes in groups of 64 or 2-bit codes in groups of
    128, run with per-wavefront stamps (a measurement aid).  Returns (y,
    stamps, info): y as `affine` returns it;
    stamps an int64 [waves][STAMPS] tensor on the device (start, activations
    staged, end -- in ticks of info["clock_khz"] per ms -- and
    (XCC id << 32) | HW_ID); info the launch's fields (TimelineInfo).
    """
    import torch
    if (bits, group_size) not in ((4, 64), (2, 128)):
        raise ValueError("the stamped launch takes 4-bit codes in groups of 64 or 2-bit in groups of 128")
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x must be [M][K] and w [N][K*bits/32]")
    if x.dtype != torch.bfloat16 or scales.dtype != torch.bfloat16 or biases.dtype != torch.bfloat16:
        raise TypeError("the stamped launch takes bf16 activations, scales and biases")
    if w.dtype not in (torch.int32, torch.uint32):
        raise TypeError("w must be int32 or uint32 packed words")
    M, K = x.shape
    N = w.shape[0]
    if K % group_size != 0:
        raise ValueError(f"K = {K} is not a multiple of {group_size}")
    _expect(w, (N, K * bits // 32), "w")
    _expect(scales, (N, K // group_size), "scales")
    _expect(biases, (N, K // group_size), "biases")
    _check_tensors(((w, "w"), (scales, "scales"), (biases, "biases"), (x, "x")))
    out = _out_for(out, out_dtype, M, N, x, torch)
    info = TimelineInfo()
    args = (w.data_ptr(), scales.data_ptr(), biases.data_ptr(), x.data_ptr(), out.data_ptr(),
            M, N, K, bits, group_size, _dt_of(out, "out"), rows_per_wave)
    status = timeline_ptr(*args, None, 0, info)
    if status != 0:
        raise QmvError(status, "qmv_affine_timeline")
    stamps = torch.zeros((info.waves, STAMPS), dtype=torch.int64, device=x.device)
    st = torch.cuda.current_stream(x.device) if stream is None else stream
    status = timeline_ptr(*args, stamps.data_ptr(), stamps.numel(), info, st.cuda_stream)
    if status != 0:
        raise QmvError(status, "qmv_affine_timeline")
    return out, stamps, {n: getattr(info, n) for n, _ in TimelineInfo._fields_}


def _check_tensors(named):
    """Every tensor on one HIP device and contiguous."""
    dev = None
    for t, n in named:
        if not t.is_cuda:
            raise ValueError(f"{n} must be a CUDA (HIP) tensor")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{n} is on {t.device}, the other inputs on {dev}")


def _expect(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _out_for(out, out_dtype, M, N, x, torch):
    if out is None:
        return torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=x.device)
    if not out.is_cuda or out.device != x.device:
        raise ValueError("out must be on the inputs' device")
    if not out.is_contiguous() or tuple(out.shape) != (M, N):
        raise ValueError("out must be a contiguous [M][N] tensor")
    return out


def kernel_info(M, N, K, bits, group_size, x_dt=DT_BF16, sb_dt=DT_BF16, y_dt=DT_BF16,
                rows_per_wave=0) -> dict:
    info = KernelInfo()
    status = lib().qmv_kernel_info(M, N, K, bits, group_size, x_dt, sb_dt, y_dt, rows_per_wave,
                                   ctypes.byref(info))
    if status != 0:
        raise QmvError(status, "qmv_kernel_info")
    return {n: getattr(info, n) for n, _ in KernelInfo._fields_}
