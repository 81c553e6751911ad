"""Seeded synthetic inputs for the affine group-quantized qmv.

This module is shared by the oracle side (tests, cpu_baseline) and the GPU side
(tests, bench, smoke).  It holds the data recipe and the storage encoding only
-- none of the product's arithmetic: no unpacking, no dot products, no folds.

Recipe (the shapes and distributions of the workloads measured on the pages,
with random weights in place of trained checkpoints):

* q ~ uniform integers in [0, 2^bits), packed 32/bits per uint32 word with
  field j of the word in bits [bits*j, bits*(j+1)) -- field 0 in the low bits;
* scale = |N(0, 0.02)| rounded (round-to-nearest-even) to the parameter dtype;
* bias  = -c * scale + N(0, 0.002), computed in fp32 from the already rounded
  scale and then rounded to the parameter dtype; c = 8 at 4 bits, 1.5 at 2 bits
  (the zero point of the unsigned code range);
* x ~ N(0, 1), drawn once as 13 rows and rounded to the activation dtype; an
  M-vector launch uses rows 0..M-1, so every M shares the M=1 vector.

Draw order on one ``torch.Generator('cpu')`` seeded with ``seed``: q, scale,
bias noise.  x comes from a second generator seeded with ``seed + 500``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

MAX_M = 13

# Workloads: name -> shape and dtypes.  Sizes are those of the MLP projections
# of a 12B-class dense model (15360 x 3840 and its transpose) and of a
# 27B-class layer (17408 x 5120 and its transpose), plus a tiny case.
WORKLOADS = {
    "tiny_4b_g64":       dict(N=256,   K=512,   bits=4, gs=64,  sb="f16",  x="f32",  y="f32",  seed=1000, Ms=(1,)),
    "up_4b_15360x3840":  dict(N=15360, K=3840,  bits=4, gs=64,  sb="bf16", x="bf16", y="bf16", seed=1001, Ms=(1, 2, 5, 10, 13)),
    "down_4b_3840x15360": dict(N=3840, K=15360, bits=4, gs=64,  sb="bf16", x="bf16", y="bf16", seed=1102, Ms=(2, 5, 10, 13)),
    "up_2b_15360x3840":  dict(N=15360, K=3840,  bits=2, gs=128, sb="bf16", x="bf16", y="bf16", seed=1003, Ms=(1, 5)),
    "up_4b_17408x5120":  dict(N=17408, K=5120,  bits=4, gs=64,  sb="bf16", x="bf16", y="bf16", seed=1004, Ms=(1, 4, 8, 13)),
    "down_4b_5120x17408": dict(N=5120, K=17408, bits=4, gs=64,  sb="bf16", x="bf16", y="bf16", seed=1104, Ms=(1, 4, 8, 13)),
}

_TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Problem:
    N: int
    K: int
    bits: int
    gs: int
    sb: str              # "f16" | "bf16"
    x_dtype: str         # "f32" | "bf16"
    w_packed: np.ndarray  # uint32 [N][K*bits/32]
    scales: np.ndarray    # uint16 bit patterns [N][K/gs]
    biases: np.ndarray    # uint16 bit patterns [N][K/gs]
    x: np.ndarray         # float32 [13][K] or uint16 bf16 bit patterns [13][K]
    q: np.ndarray | None = field(default=None, repr=False)  # uint8 [N][K] codes (optional)


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Encode integer codes q[N][K] (0 <= q < 2^bits) into uint32 words, field j
    of each word in bits [bits*j, bits*(j+1))."""
    pf = 32 // bits
    N, K = q.shape
    assert K % pf == 0
    qq = q.reshape(N, K // pf, pf).astype(np.uint32)
    w = np.zeros((N, K // pf), dtype=np.uint32)
    for j in range(pf):
        w |= qq[:, :, j] << np.uint32(bits * j)
    return w


def _bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def make_weights(N: int, K: int, bits: int, gs: int, sb: str, seed: int, keep_q: bool = False):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randint(0, 1 << bits, (N, K), generator=g, dtype=torch.uint8)
    G = K // gs
    scale = (torch.randn(N, G, generator=g) * 0.02).abs().to(_TORCH_DT[sb])
    eps = torch.randn(N, G, generator=g) * 0.002
    c = 8.0 if bits == 4 else 1.5
    bias = (-c * scale.float() + eps).to(_TORCH_DT[sb])
    qn = q.numpy()
    w = pack(qn, bits)
    return w, _bits16(scale), _bits16(bias), (qn if keep_q else None)


@dataclass
class MxProblem:
    """The mxfp4 mode: E2M1 codes packed 8 per uint32 (field 0 low), one E8M0
    scale byte per block of 32 along K."""
    N: int
    K: int
    x_dtype: str
    w_packed: np.ndarray  # uint32 [N][K/8]
    scales: np.ndarray    # uint8 [N][K/32]
    x: np.ndarray         # float32 [13][K] or uint16 bf16 bit patterns [13][K]
    q: np.ndarray | None = field(default=None, repr=False)  # uint8 [N][K] codes (optional)


def make_mx_problem(N: int, K: int, x_dtype: str = "bf16", seed: int = 0, keep_q: bool = False,
                    e_lo: int = 116, e_hi: int = 124) -> MxProblem:
    """Uniform random E2M1 codes (both signs, every magnitude) and block scale
    exponents uniform in [e_lo, e_hi] -- 2^-11 .. 2^-3 around 127, the scales
    a 0.02-wide weight distribution gets when its block maximum maps near the
    E2M1 maximum of 6."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randint(0, 16, (N, K), generator=g, dtype=torch.uint8).numpy()
    e = torch.randint(e_lo, e_hi + 1, (N, K // 32), generator=g, dtype=torch.int32).numpy().astype(np.uint8)
    return MxProblem(N=N, K=K, x_dtype=x_dtype, w_packed=pack(q, 4), scales=e,
                     x=make_x(K, x_dtype, seed), q=(q if keep_q else None))


def make_x(K: int, x_dtype: str, seed: int, rows: int = MAX_M) -> np.ndarray:
    g = torch.Generator("cpu").manual_seed(seed + 500)
    x = torch.randn(rows, K, generator=g)
    if x_dtype == "f32":
        return x.numpy().astype(np.float32)
    return _bits16(x.to(_TORCH_DT[x_dtype]))


def make_problem(name: str | None = None, *, N=None, K=None, bits=None, gs=None, sb=None,
                 x_dtype=None, seed=None, keep_q: bool = False) -> Problem:
    """A named workload (see WORKLOADS) or an explicit shape."""
    if name is not None:
        w = WORKLOADS[name]
        N = w["N"] if N is None else N
        K = w["K"] if K is None else K
        bits = w["bits"] if bits is None else bits
        gs = w["gs"] if gs is None else gs
        sb = w["sb"] if sb is None else sb
        x_dtype = w["x"] if x_dtype is None else x_dtype
        seed = w["seed"] if seed is None else seed
    wp, s, b, q = make_weights(N, K, bits, gs, sb, seed, keep_q)
    x = make_x(K, x_dtype, seed)
    return Problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype=x_dtype, w_packed=wp,
                   scales=s, biases=b, x=x, q=q)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact): a storage conversion, used to
    hand bf16 data to code that wants float32 arrays."""
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)
