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


U32 = 2.0 ** -24          # unit roundoff of fp32


def gamma(d: int) -> float:
    """gamma_d = d*u / (1 - d*u): the relative bound of d successive fp32 roundings."""
    return d * U32 / (1 - d * U32)


def affine_depth(K: int, bits: int, gs: int, x_dtype: str) -> int:
    """Most fp32 roundings any term of one output goes through in the library's
    fixed order (counted generously): the chunk's dot chain (two roundings per
    bf16 dot2 step, one per fp32 fma), the group sum S (at most 16), the
    combine of a group's lanes (at most 2), the two fmas of the group's fold,
    the fold's accumulator over a lane's later groups (two per wave step), and
    the six levels of the 64-lane tree."""
    chain = 2 * (64 // bits) if x_dtype == "bf16" else 128 // bits
    nsteps = -(-(K * bits // 128) // 64)
    return chain + 16 + 2 + 2 + 2 * nsteps + 6


def mx_depth(K: int, x_dtype: str) -> int:
    """The same count for the mxfp4 mode: a block's chain (16 bf16 dot2 steps at
    two roundings, or 32 fmas), its fold, the accumulator over a lane's later
    blocks (one per wave step) and the 64-lane tree."""
    chain = 32
    nsteps = -(-(K // 32) // 64)
    return chain + 1 + nsteps + 6


def affine_mag(p: gen.Problem, M: int, x=None) -> np.ndarray:
    xx = (p.x if x is None else x)[:M]
    return oracle.default().qmv_mag(p.scales, p.biases, xx, bits=p.bits, group_size=p.gs,
                                    sb_dtype=oracle.DT[p.sb], x_dtype=oracle.DT[p.x_dtype])


def check_parity(got: torch.Tensor, want: np.ndarray, what: str, tol: float = TOL,
                 mag: np.ndarray | None = None, depth: int | None = None):
    """The parity bar, per output vector m:

    * normwise: |y - y_ref| <= tol * max|y_ref| for every element; and, when
      the oracle's term magnitudes `mag` and the rounding depth are given,
    * a priori: |y - y_ref| <= gamma_depth * mag for every element -- the
      rounding-error bound of any fp32 evaluation with at most `depth`
      roundings per term, which holds whatever the conditioning.

    A vector of at most three outputs whose values cancel far below their
    terms may miss the normwise bar (no fp32 order avoids it); it passes if it
    meets the a-priori bound.  Every other vector must meet the normwise bar."""
    g = got.float().cpu().numpy().astype(np.float64)
    assert g.shape == want.shape, (g.shape, want.shape)
    bound = None if mag is None else gamma(depth) * mag
    worst = 0.0
    for m in range(want.shape[0]):
        den = float(np.max(np.abs(want[m])))
        diff = np.abs(g[m] - want[m])
        err = float(np.max(diff))
        rel = err / den if den > 0 else err
        assert np.all(np.isfinite(g[m])), f"{what}: non-finite output in vector {m}"
        if bound is not None:
            over = diff > bound[m]
            assert not over.any(), (f"{what}: vector {m} exceeds the a-priori bound at "
                                    f"n = {int(np.argmax(over))}")
        if rel > tol and bound is not None and want.shape[1] <= 3:
            continue                    # ill-conditioned few-row vector, within the bound
        worst = max(worst, rel)
        assert rel <= tol, f"{what}: vector {m} normwise error {rel:.3e} > {tol:g}"
    log = os.environ.get("QMV_PARITY_LOG")
    if log:                          # optional record of the errors seen, one line per check
        with open(log, "a") as f:
            f.write(f"{what}\t{worst:.3e}\n")
    return worst


def check_bf16_output(y16: torch.Tensor, want: np.ndarray, what: str, tol: float = TOL):
    """A bf16 output against the exact value: it is the round-to-nearest-even of
    an fp32 result within tol * max|y_ref| of y_ref, so per element
    |y16 - y_ref| <= ulp_bf16(y_ref) + 1.01 * tol * max|y_ref| (half an ulp of
    the rounding, doubled for a result that lands in the next binade, and
    2^-8 of the fp32 error for one that lands further up).  Where that
    error is below half an ulp this means one bf16 ulp of RNE_bf16(y_ref); for
    outputs near zero it admits the fp32 error the parity bar allows."""
    g = y16.float().cpu().numpy().astype(np.float64)
    assert g.shape == want.shape, (g.shape, want.shape)
    a = np.abs(want)
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -133)))
    ulp = np.exp2(np.maximum(e, -126.0) - 7.0)
    for m in range(want.shape[0]):
        lim = ulp[m] + 1.01 * tol * float(np.max(a[m]))
        over = np.abs(g[m] - want[m]) > lim
        assert not over.any(), f"{what}: bf16 vector {m} off at n = {int(np.argmax(over))}"


def rne_bf16(t: torch.Tensor) -> torch.Tensor:
    return t.float().to(torch.bfloat16)
