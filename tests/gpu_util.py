"""Helpers shared by the GPU tests: device copies of generated problems, calls
through the C ABI, and the oracle comparison of the parity bar."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import bit_quantized_gemv_amd as q
from inputs import gen
from oracle import oracle

DEV = "cuda:0"
TOL = 2e-5   # max |y - y_ref| / max |y_ref| per output vector, fp32 output


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(p: gen.Problem):
    w = torch.from_numpy(p.w_packed.view(np.int32)).to(DEV)
    sdt = torch.float16 if p.sb == "f16" else torch.bfloat16
    s = torch.from_numpy(p.scales.view(np.int16)).view(sdt).to(DEV)
    b = torch.from_numpy(p.biases.view(np.int16)).view(sdt).to(DEV)
    if p.x_dtype == "f32":
        x = torch.from_numpy(p.x).to(DEV)
    else:
        x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return w, s, b, x


def x_to_dev(xnp: np.ndarray, x_dtype: str):
    if x_dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(xnp, dtype=np.float32)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(xnp, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def gpu(p: gen.Problem, dev, M: int, out_dtype=torch.float32, R: int = 0, x=None):
    w, s, b, xd = dev
    xx = (xd if x is None else x)[:M].contiguous()
    y = q.affine(w, s, b, xx, bits=p.bits, group_size=p.gs, out_dtype=out_dtype, rows_per_wave=R)
    torch.cuda.synchronize()
    return y


def ref(p: gen.Problem, M: int, x=None, nthreads: int = 0):
    xx = (p.x if x is None else x)[:M]
    return oracle.default().qmv(p.w_packed, p.scales, p.biases, xx, bits=p.bits,
                                group_size=p.gs, sb_dtype=oracle.DT[p.sb],
                                x_dtype=oracle.DT[p.x_dtype], nthreads=nthreads)


def ref_rows(p: gen.Problem, M: int, rows: np.ndarray):
    ms = np.repeat(np.arange(M, dtype=np.int32), rows.size)
    ns = np.tile(rows.astype(np.int32), M)
    v = oracle.default().qmv_at(p.w_packed, p.scales, p.biases, p.x[:M], ms, ns, bits=p.bits,
                                group_size=p.gs, sb_dtype=oracle.DT[p.sb],
                                x_dtype=oracle.DT[p.x_dtype])
    return v.reshape(M, rows.size)


def check_parity(got: torch.Tensor, want: np.ndarray, what: str, tol: float = TOL):
    """Element by element: |y - y_ref| <= tol * max|y_ref| for every element of
    each output vector (the normwise reading of the 2e-5 bar)."""
    g = got.float().cpu().numpy().astype(np.float64)
    assert g.shape == want.shape, (g.shape, want.shape)
    worst = 0.0
    for m in range(want.shape[0]):
        den = float(np.max(np.abs(want[m])))
        err = float(np.max(np.abs(g[m] - want[m])))
        rel = err / den if den > 0 else err
        worst = max(worst, rel)
        assert np.all(np.isfinite(g[m])), f"{what}: non-finite output in vector {m}"
        assert rel <= tol, f"{what}: vector {m} normwise error {rel:.3e} > {tol:g}"
    log = os.environ.get("QMV_PARITY_LOG")
    if log:                          # optional record of the errors seen, one line per check
        with open(log, "a") as f:
            f.write(f"{what}\t{worst:.3e}\n")
    return worst


def rne_bf16(t: torch.Tensor) -> torch.Tensor:
    return t.float().to(torch.bfloat16)
