"""Python access to the plain C oracle of the affine group-quantized qmv (and
of its mxfp4 mode).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the cpu_baseline leg of bench.py.  The GPU package never imports this module.

The oracle itself is ``qmv_oracle.c`` (fp64 accumulation, grouped form of the
affine-dequantized product; see that file's header for the passages it
follows).  This module only compiles it with the host C compiler and marshals
numpy arrays into it.  ``Oracle(path)`` can load any build of that source,
which lets a test compile a copy with a planted mistake and check that the
pins reject it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmv_oracle.c")
LIB = os.path.join(HERE, "liborc.so")

F32, F16, BF16 = 0, 1, 2
DT = {"f32": F32, "f16": F16, "bf16": BF16}


def compile_source(src: str, out: str) -> str:
    """gcc -O3 -fopenmp, no intrinsics."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O3", "-fopenmp", "-std=c99", "-fPIC", "-shared",
                           "-Wall", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        compile_source(SRC, LIB)
    return LIB


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    def __init__(self, path: str = LIB):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.orc_qmv_affine.argtypes = [P, P, P, I, P, I, P, I, I, I, I, I, I]
        L.orc_qmv_affine.restype = I
        L.orc_qmv_affine_at.argtypes = [P, P, P, I, P, I, P, P, I, P, I, I, I, I, I]
        L.orc_qmv_affine_at.restype = I
        L.orc_unpack_row.argtypes = [P, I, I, P]
        L.orc_unpack_row.restype = None
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16_rne.restype = ctypes.c_uint16
        L.orc_round_outputs.argtypes = [P, ctypes.c_size_t, P, P]
        L.orc_round_outputs.restype = None
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = I
        L.orc_qmv_mxfp4.argtypes = [P, P, P, I, P, I, I, I, I]
        L.orc_qmv_mxfp4.restype = I
        L.orc_e2m1_to_f64.argtypes = [ctypes.c_uint]
        L.orc_e2m1_to_f64.restype = ctypes.c_double
        L.orc_e8m0_to_f64.argtypes = [ctypes.c_uint]
        L.orc_e8m0_to_f64.restype = ctypes.c_double
        L.orc_qmv_affine_mag.argtypes = [P, P, I, P, I, P, I, I, I, I, I, I]
        L.orc_qmv_affine_mag.restype = I
        L.orc_qmv_mxfp4_mag.argtypes = [P, P, I, P, I, I, I, I]
        L.orc_qmv_mxfp4_mag.restype = I
        self.L = L

    def qmv(self, w_packed, scales, biases, x, *, bits, group_size, sb_dtype, x_dtype,
            nthreads: int = 0) -> np.ndarray:
        """y_ref[M][N] (float64).

        w_packed: uint32 [N][K*bits/32]; scales/biases: uint16 bit patterns
        [N][K/gs] of sb_dtype (F16 or BF16); x: float32 [M][K] (x_dtype F32) or
        uint16 bf16 bit patterns [M][K] (x_dtype BF16).
        """
        w_packed = np.ascontiguousarray(w_packed, dtype=np.uint32)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
        biases = np.ascontiguousarray(biases, dtype=np.uint16)
        x = np.ascontiguousarray(x, dtype=np.float32 if x_dtype == F32 else np.uint16)
        N = w_packed.shape[0]
        M, K = x.shape
        assert w_packed.shape[1] * (32 // bits) == K
        y = np.zeros((M, N), dtype=np.float64)
        rc = self.L.orc_qmv_affine(_ptr(w_packed), _ptr(scales), _ptr(biases), sb_dtype,
                                   _ptr(x), x_dtype, _ptr(y), M, N, K, bits, group_size,
                                   nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the shape (code {rc})")
        return y

    def qmv_at(self, w_packed, scales, biases, x, ms, ns, *, bits, group_size, sb_dtype,
               x_dtype, nthreads: int = 0) -> np.ndarray:
        """y_ref[ms[i]][ns[i]] (float64) for sampled index pairs."""
        w_packed = np.ascontiguousarray(w_packed, dtype=np.uint32)
        x = np.ascontiguousarray(x, dtype=np.float32 if x_dtype == F32 else np.uint16)
        ms = np.ascontiguousarray(ms, dtype=np.int32)
        ns = np.ascontiguousarray(ns, dtype=np.int32)
        N = w_packed.shape[0]
        K = x.shape[1]
        assert int(ms.max(initial=0)) < x.shape[0]
        out = np.zeros(ms.shape[0], dtype=np.float64)
        rc = self.L.orc_qmv_affine_at(_ptr(w_packed), _ptr(scales), _ptr(biases), sb_dtype,
                                      _ptr(x), x_dtype, _ptr(ms), _ptr(ns), int(ms.shape[0]),
                                      _ptr(out), N, K, bits, group_size, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the request (code {rc})")
        return out

    def qmv_mag(self, scales, biases, x, *, bits, group_size, sb_dtype, x_dtype,
                nthreads: int = 0) -> np.ndarray:
        """mag[M][N] (float64): the sum of the magnitudes of each output's terms,
        sum_g (2^(bits+2)|scale| + |bias|) * sum_{k in g} |x[m][k]|, for the
        a-priori bound |y - y_ref| <= gamma_d * mag of an fp32 evaluation."""
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
        biases = np.ascontiguousarray(biases, dtype=np.uint16)
        x = np.ascontiguousarray(x, dtype=np.float32 if x_dtype == F32 else np.uint16)
        N = scales.shape[0]
        M, K = x.shape
        assert scales.shape[1] * group_size == K and biases.shape == scales.shape
        mag = np.zeros((M, N), dtype=np.float64)
        rc = self.L.orc_qmv_affine_mag(_ptr(scales), _ptr(biases), sb_dtype, _ptr(x), x_dtype,
                                       _ptr(mag), M, N, K, bits, group_size, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the shape (code {rc})")
        return mag

    def qmv_mxfp4_mag(self, scales, x, *, x_dtype, nthreads: int = 0) -> np.ndarray:
        """mag[M][N] (float64) of the mxfp4 mode: sum_b 2^(E-127) * 6 * sum_{k in b} |x[m][k]|."""
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        x = np.ascontiguousarray(x, dtype=np.float32 if x_dtype == F32 else np.uint16)
        N = scales.shape[0]
        M, K = x.shape
        assert scales.shape[1] * 32 == K
        mag = np.zeros((M, N), dtype=np.float64)
        rc = self.L.orc_qmv_mxfp4_mag(_ptr(scales), _ptr(x), x_dtype, _ptr(mag), M, N, K, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the shape (code {rc})")
        return mag

    def qmv_mxfp4(self, w_packed, scales, x, *, x_dtype, nthreads: int = 0) -> np.ndarray:
        """y_ref[M][N] (float64) of the mxfp4 mode.

        w_packed: uint32 [N][K/8] (E2M1 codes, field 0 low); scales: uint8
        [N][K/32] (E8M0); x: float32 [M][K] (x_dtype F32) or uint16 bf16 bit
        patterns [M][K] (x_dtype BF16).
        """
        w_packed = np.ascontiguousarray(w_packed, dtype=np.uint32)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        x = np.ascontiguousarray(x, dtype=np.float32 if x_dtype == F32 else np.uint16)
        N = w_packed.shape[0]
        M, K = x.shape
        assert w_packed.shape[1] * 8 == K and scales.shape == (N, K // 32)
        y = np.zeros((M, N), dtype=np.float64)
        rc = self.L.orc_qmv_mxfp4(_ptr(w_packed), _ptr(scales), _ptr(x), x_dtype, _ptr(y),
                                  M, N, K, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the shape (code {rc})")
        return y

    def e2m1_to_f64(self, c: int) -> float:
        return self.L.orc_e2m1_to_f64(c)

    def e8m0_to_f64(self, e: int) -> float:
        return self.L.orc_e8m0_to_f64(e)

    def unpack_row(self, row, K: int, bits: int) -> np.ndarray:
        row = np.ascontiguousarray(row, dtype=np.uint32)
        q = np.zeros(K, dtype=np.uint8)
        self.L.orc_unpack_row(_ptr(row), K, bits, _ptr(q))
        return q

    def f16_to_f64(self, h: int) -> float:
        return self.L.orc_f16_to_f64(h)

    def bf16_to_f64(self, h: int) -> float:
        return self.L.orc_bf16_to_f64(h)

    def f32_to_bf16(self, f: float) -> int:
        return self.L.orc_f32_to_bf16_rne(f)

    def round_outputs(self, y):
        """(fp32 RNE of y, bf16 RNE of that fp32 as uint16 bit patterns)."""
        y = np.ascontiguousarray(y, dtype=np.float64)
        y32 = np.zeros(y.shape, dtype=np.float32)
        y16 = np.zeros(y.shape, dtype=np.uint16)
        self.L.orc_round_outputs(_ptr(y), y.size, _ptr(y32), _ptr(y16))
        return y32, y16

    def max_threads(self) -> int:
        return self.L.orc_max_threads()


_default = None


def default() -> Oracle:
    """The oracle built from qmv_oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build(force=True)
        _default = Oracle(LIB)
    return _default
