"""The parity bar on ill-conditioned outputs.

Vectors of one to three rows can cancel: their outputs are far below the
magnitude of the terms they sum, and no fp32 evaluation order meets a
normwise 2e-5 bar on them (the grouped and dequantized forms are equal in
real arithmetic only: mlxcel issue "an order-preserving streamed qmv would give
MTP the fast kernel and byte-identity together", section "Correction to the
obvious sketch").  Such vectors are held to the a-priori rounding-error bound
gamma_d * mag instead, with mag the oracle's term magnitudes; every vector of
four or more rows stays on the normwise bar.

The cancelling inputs are built, not searched for: x is drawn at random and
projected in fp64 onto the orthogonal complement of the (dense, dequantized)
weight rows, then rounded to the activation dtype, so y_ref is of the order of
that rounding.  Each case asserts that it really cancels, that the kernel
meets the a-priori bound on it, and that every vector equals its one-vector
call bit for bit.
"""
import numpy as np
import pytest
import torch

import gpu_util as U
from inputs import gen
from oracle import oracle

pytestmark = pytest.mark.gpu


def _f64(bits16: np.ndarray, dt: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits16).view(np.int16))
    return t.view(torch.float16 if dt == "f16" else torch.bfloat16).double().numpy()


def _store(x64: np.ndarray, x_dtype: str) -> np.ndarray:
    if x_dtype == "f32":
        return x64.astype(np.float32)
    return torch.from_numpy(x64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _project_out(W: np.ndarray, M: int, K: int, seed: int) -> np.ndarray:
    """M random vectors with the row space of W (fp64, [N][K]) removed."""
    r = np.random.default_rng(seed).standard_normal((M, K))
    Q, _ = np.linalg.qr(W.T)                       # orthonormal basis of the rows
    return r - (r @ Q) @ Q.T


AFFINE = [  # N, K, bits, gs, sb, x
    (1, 3840, 4, 64, "bf16", "bf16"),
    (2, 4096, 2, 128, "bf16", "bf16"),
    (3, 2560, 4, 128, "f16", "f32"),
    (1, 64, 4, 64, "f16", "bf16"),
    (3, 8192, 2, 64, "f16", "f32"),
]


@pytest.mark.parametrize("case", AFFINE, ids=lambda c: f"N{c[0]}_K{c[1]}_b{c[2]}_g{c[3]}_{c[5]}")
def test_affine_cancelling_rows(case):
    N, K, bits, gs, sb, xdt = case
    p = gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype=xdt, seed=700 + N + K, keep_q=True)
    W = np.repeat(_f64(p.scales, sb), gs, axis=1) * p.q + np.repeat(_f64(p.biases, sb), gs, axis=1)
    M = 5
    p.x = _store(_project_out(W, M, K, seed=K + N), xdt)
    want = U.ref(p, M)
    mag = U.affine_mag(p, M)
    assert np.max(np.abs(want)) < 1e-3 * np.min(np.max(mag, axis=1)), "the case does not cancel"
    dev = U.to_dev(p)
    U.say(f"cancelling affine N={N} K={K} bits={bits} gs={gs} x={xdt}")
    y = U.gpu(p, dev, M, torch.float32)
    U.check_parity(y, want, f"cancelling N={N} K={K}", mag=mag,
                   depth=U.affine_depth(K, bits, gs, xdt))
    for m in range(M):
        one = U.gpu(p, dev, 1, torch.float32, x=dev[3][m:m + 1])
        assert torch.equal(y[m].view(torch.int32), one[0].view(torch.int32)), f"vector {m}"


@pytest.mark.parametrize("N,K,xdt", [(1, 3840, "bf16"), (3, 1024, "f32"), (2, 32, "bf16")])
def test_mxfp4_cancelling_rows(N, K, xdt):
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    p = gen.make_mx_problem(N, K, xdt, seed=800 + N + K, keep_q=True)
    W = table[p.q] * np.repeat(np.ldexp(1.0, p.scales.astype(np.int64) - 127), 32, axis=1)
    M = 4
    xs = _store(_project_out(W, M, K, seed=K + 3 * N), xdt)
    ref = oracle.default().qmv_mxfp4(p.w_packed, p.scales, xs, x_dtype=oracle.DT[xdt])
    mag = oracle.default().qmv_mxfp4_mag(p.scales, xs, x_dtype=oracle.DT[xdt])
    assert np.max(np.abs(ref)) < 1e-3 * np.min(np.max(mag, axis=1)), "the case does not cancel"
    w = torch.from_numpy(p.w_packed.view(np.int32)).to(U.DEV)
    s = torch.from_numpy(p.scales).to(U.DEV)
    xd = U.x_to_dev(xs, xdt)
    U.say(f"cancelling mxfp4 N={N} K={K} x={xdt}")
    y = U.q.mxfp4(w, s, xd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    U.check_parity(y, ref, f"cancelling mxfp4 N={N} K={K}", mag=mag, depth=U.mx_depth(K, xdt))
    for m in range(M):
        one = U.q.mxfp4(w, s, xd[m:m + 1], out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y[m].view(torch.int32), one[0].view(torch.int32)), f"vector {m}"


def test_a_priori_bound_is_tight_enough_to_fail():
    """The a-priori check has teeth: one planted error (on the CPU copy of a
    GPU result) of a few times the bound is rejected."""
    p = gen.make_problem(N=2, K=1024, bits=4, gs=64, sb="bf16", x_dtype="bf16", seed=5)
    dev = U.to_dev(p)
    want = U.ref(p, 2)
    mag = U.affine_mag(p, 2)
    depth = U.affine_depth(p.K, p.bits, p.gs, p.x_dtype)
    y = U.gpu(p, dev, 2, torch.float32).cpu()
    U.check_parity(y, want, "unplanted", mag=mag, depth=depth)
    bad = y.clone()
    bad[1, 0] += float(4 * U.gamma(depth) * mag[1, 0])
    with pytest.raises(AssertionError):
        U.check_parity(bad, want, "planted", mag=mag, depth=depth)
