"""Pins of the CPU oracle: checks against what the pages and the mathematics fix,
each independent of the oracle's own code.

Each pin takes an ``Oracle`` and raises AssertionError when it disagrees.  The
normal suite runs them on the real oracle (test_oracle_pins.py); a mutation
suite runs them on copies of the oracle with planted mistakes and requires
that every mistake is caught (test_oracle_mutations.py).

Independent means: decoding here goes through numpy's bit unpacking (or the
float-floor chain of the 2-bit PR), storage conversions through numpy/torch,
dense products through numpy matmul or exact integer arithmetic -- never
through the oracle's shift-and-mask, its conversions or its grouped loop.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from inputs import gen
from oracle.oracle import F16, F32, BF16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers ---

def decode_unpackbits(w_packed: np.ndarray, bits: int) -> np.ndarray:
    """Codes q[N][K] from packed words via numpy's little-endian bit unpacking:
    bit i of the row's bit string is bit (i mod 32) of word i // 32, and field k
    is bits [bits*k, bits*(k+1)) of that string, lowest bit first."""
    w = np.ascontiguousarray(w_packed, dtype="<u4")
    N = w.shape[0]
    bitstr = np.unpackbits(w.view(np.uint8).reshape(N, -1), axis=1, bitorder="little")
    K = bitstr.shape[1] // bits
    fb = bitstr.reshape(N, K, bits).astype(np.int64)
    return (fb * (1 << np.arange(bits, dtype=np.int64))).sum(axis=2)


def f16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(u, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(u, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).double().numpy()


def sb_to_f64(u, sb):
    return f16_bits_to_f64(u) if sb == "f16" else bf16_bits_to_f64(u)


def x_to_f64(x, x_dtype):
    return x.astype(np.float64) if x_dtype == "f32" else bf16_bits_to_f64(x)


def f64_to_bits(v: np.ndarray, dt: str) -> np.ndarray:
    """Exact storage of values known to be representable (asserted)."""
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    t = torch.from_numpy(np.asarray(v, dtype=np.float64)).to(tdt)
    assert np.array_equal(t.double().numpy(), np.asarray(v, dtype=np.float64)), "not exact"
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normwise(a: np.ndarray, ref: np.ndarray) -> float:
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(a - ref)) / den) if den > 0 else float(np.max(np.abs(a)))


def run(orc, p: gen.Problem, x=None, M=None):
    x = p.x if x is None else x
    if M is not None:
        x = x[:M]
    return orc.qmv(p.w_packed, p.scales, p.biases, x, bits=p.bits, group_size=p.gs,
                   sb_dtype=F16 if p.sb == "f16" else BF16,
                   x_dtype=F32 if p.x_dtype == "f32" else BF16)


SHAPES = [  # (N, K, bits, gs, sb, x_dtype) -- small, several groups, odd N
    (37, 384, 4, 64, "f16", "f32"),
    (19, 256, 4, 128, "bf16", "bf16"),
    (23, 512, 2, 64, "bf16", "f32"),
    (17, 384, 2, 128, "f16", "bf16"),
]


# ------------------------------------------------------------------- pins ---

def pin_codec_golden(orc):
    """Hand-derived words (tests/golden/codec_words.json) decode to their fields."""
    with open(os.path.join(GOLDEN, "codec_words.json")) as f:
        spec = json.load(f)
    for e in spec["words"]:
        bits = e["bits"]
        w = np.array([int(e["word"], 16)], dtype=np.uint32)
        got = orc.unpack_row(w, 32 // bits, bits)
        assert list(got) == e["fields"], (e, list(got))


def pin_2bit_float_floor_exhaustive(orc):
    """All 256 byte values, at every byte position of a word: the oracle's 2-bit
    fields equal the float-floor chain of llama.cpp PR 'PQ2_0 and Q2_0 mat-vec
    dot in exact float' (section 'How'): u = b/256, g_k = floor(4^k u) exact in
    fp32, fields 3, 2, 1, 0 = g1, g2-4g1, g3-4g2, b-4g3.  The chain is also
    checked to reject the base-3 digit order (g1 read as field 0), so the
    comparison has teeth."""
    b = np.arange(256, dtype=np.float32)
    u = b / np.float32(256.0)
    g1 = np.floor(np.float32(4.0) * u)
    g2 = np.floor(np.float32(16.0) * u)
    g3 = np.floor(np.float32(64.0) * u)
    chain = np.stack([b - 4 * g3, g3 - 4 * g2, g2 - 4 * g1, g1], axis=1).astype(np.int64)
    wrong = chain[:, ::-1]
    assert np.count_nonzero(np.any(chain != wrong, axis=1)) > 0
    for pos in range(4):
        words = (np.arange(256, dtype=np.uint32) << np.uint32(8 * pos)).astype(np.uint32)
        for v in range(256):
            f = orc.unpack_row(words[v:v + 1], 16, 2)
            assert np.array_equal(f[4 * pos:4 * pos + 4].astype(np.int64), chain[v]), (pos, v)
            others = np.delete(f, np.arange(4 * pos, 4 * pos + 4))
            assert not others.any(), (pos, v)
    # the collapse identity of the same section, exact on integer activations
    rng = np.random.default_rng(7)
    y = rng.integers(-50, 50, size=(256, 4)).astype(np.float64)
    lhs = (chain * y).sum(axis=1)
    rhs = g1 * (y[:, 3] - 4 * y[:, 2]) + g2 * (y[:, 2] - 4 * y[:, 1]) \
        + g3 * (y[:, 1] - 4 * y[:, 0]) + b.astype(np.float64) * y[:, 0]
    assert np.array_equal(lhs, rhs)


def pin_4bit_nibbles_exhaustive(orc):
    """All 256 byte values at every byte position: low nibble = field 2p, high
    nibble = field 2p+1, checked two independent ways -- numpy bit unpacking,
    and the masked-bits form of the 'Correction' section (mask 0xf << 4j, then
    divide by 16^j in floating point)."""
    for pos in range(4):
        words = (np.arange(256, dtype=np.uint32) << np.uint32(8 * pos)).astype(np.uint32)
        ref = decode_unpackbits(words.reshape(256, 1), 4)
        for v in range(256):
            f = orc.unpack_row(words[v:v + 1], 8, 4).astype(np.int64)
            assert np.array_equal(f, ref[v]), (pos, v)
            masked = [float(int(words[v]) & (0xF << (4 * j))) / float(16 ** j) for j in range(8)]
            assert np.array_equal(f, np.array(masked, dtype=np.int64)), (pos, v)


def pin_readout(orc):
    """scale = 1, bias = 0, x = e_k for every k: y[k][n] = q[n][k] exactly, where
    q are the generator's codes before packing (a round trip through the
    packing and the whole product)."""
    for bits, gs in ((4, 64), (4, 128), (2, 64), (2, 128)):
        N, K = 13, 256
        wp, _, _, q = gen.make_weights(N, K, bits, gs, "f16", seed=77 + bits + gs, keep_q=True)
        G = K // gs
        one = np.full((N, G), 0x3C00, dtype=np.uint16)
        zero = np.zeros((N, G), dtype=np.uint16)
        x = np.eye(K, dtype=np.float32)
        y = orc.qmv(wp, one, zero, x, bits=bits, group_size=gs, sb_dtype=F16, x_dtype=F32)
        assert np.array_equal(y, q.T.astype(np.float64)), (bits, gs)


def _golden_case(c):
    bits, gs, N, K, M = c["bits"], c["group_size"], c["N"], c["K"], c["M"]
    rows = []
    for r in c["w_rows"]:
        rows.append([int(h, 16) for h in r["words"]] * r["repeat"])
    wp = np.array(rows, dtype=np.uint32)
    sb = c["sb_dtype"]
    s = np.array([[int(h, 16) for h in row] for row in c[f"scales_{sb}_bits"]], dtype=np.uint16)
    b = np.array([[int(h, 16) for h in row] for row in c[f"biases_{sb}_bits"]], dtype=np.uint16)
    assert np.array_equal(sb_to_f64(s, sb), np.array(c["scales_values"]))
    assert np.array_equal(sb_to_f64(b, sb), np.array(c["biases_values"]))
    k = np.arange(K)
    if c["name"].startswith("4bit"):
        xs = np.stack([(k % 2 == 0).astype(np.float64), (k % 16 == 3).astype(np.float64)])
    else:
        xs = np.where(k % 4 == 1, 1.0, np.where(k % 4 == 3, 2.0, 0.0))[None, :]
    if c["x_dtype"] == "f32":
        x = xs.astype(np.float32)
        xdt = F32
    else:
        x = f64_to_bits(xs, "bf16")
        xdt = BF16
    return wp, s, b, x, xdt, bits, gs, sb


def pin_worked_examples(orc):
    """Hand-worked results of tests/golden/worked_examples.json."""
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        spec = json.load(f)
    for c in spec["cases"]:
        wp, s, b, x, xdt, bits, gs, sb = _golden_case(c)
        y = orc.qmv(wp, s, b, x, bits=bits, group_size=gs,
                    sb_dtype=F16 if sb == "f16" else BF16, x_dtype=xdt)
        assert np.array_equal(y, np.array(c["y"], dtype=np.float64)), (c["name"], y)


def pin_bruteforce_dequant(orc):
    """The grouped oracle equals dequantize-then-dot (dense W = scale*q + bias,
    then a numpy matmul, all fp64) on small shapes: the two forms are equal in
    real arithmetic (mlxcel issue, 'Correction' section), so in fp64 they agree
    to rounding."""
    for (N, K, bits, gs, sb, xdt) in SHAPES:
        p = gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype=xdt, seed=4242 + N)
        q = decode_unpackbits(p.w_packed, bits).astype(np.float64)
        s = np.repeat(sb_to_f64(p.scales, sb), gs, axis=1)
        bb = np.repeat(sb_to_f64(p.biases, sb), gs, axis=1)
        W = s * q + bb
        x = x_to_f64(p.x[:5], xdt)
        ref = x @ W.T
        y = run(orc, p, M=5)
        assert normwise(y, ref) <= 1e-12, (N, K, bits, gs, normwise(y, ref))


def pin_closed_forms(orc):
    """Special cases with closed forms, and the exact-integer case."""
    for (N, K, bits, gs, sb, xdt) in SHAPES:
        p = gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype=xdt, seed=99 + K)
        G = K // gs
        sdt, xdc = (F16 if sb == "f16" else BF16), (F32 if xdt == "f32" else BF16)
        xv = x_to_f64(p.x[:3], xdt)
        S = xv.reshape(3, G, gs).sum(axis=2)                           # [3][G]
        # x = 0 -> y = 0
        y0 = orc.qmv(p.w_packed, p.scales, p.biases, np.zeros_like(p.x[:2]), bits=bits,
                     group_size=gs, sb_dtype=sdt, x_dtype=xdc)
        assert not y0.any()
        # scale = 0 -> y = sum_g bias * S_g
        ys = orc.qmv(p.w_packed, np.zeros_like(p.scales), p.biases, p.x[:3], bits=bits,
                     group_size=gs, sb_dtype=sdt, x_dtype=xdc)
        ref = S @ sb_to_f64(p.biases, sb).T
        assert normwise(ys, ref) <= 1e-12
        # bias = 0 and every code = c -> y = sum_g scale * c * S_g
        c = (1 << bits) - 2
        qc = np.full((N, K), c, dtype=np.uint8)
        wc = gen.pack(qc, bits)
        yc = orc.qmv(wc, p.scales, np.zeros_like(p.biases), p.x[:3], bits=bits,
                     group_size=gs, sb_dtype=sdt, x_dtype=xdc)
        ref = c * (S @ sb_to_f64(p.scales, sb).T)
        assert normwise(yc, ref) <= 1e-12
        # y(2x) = 2 y(x) exactly (a power of two commutes with every rounding)
        if xdt == "f32":
            x2 = (p.x[:3] * np.float32(2.0)).astype(np.float32)
        else:
            x2 = f64_to_bits(2.0 * xv, "bf16")
        ya = orc.qmv(p.w_packed, p.scales, p.biases, p.x[:3], bits=bits, group_size=gs,
                     sb_dtype=sdt, x_dtype=xdc)
        yb = orc.qmv(p.w_packed, p.scales, p.biases, x2, bits=bits, group_size=gs,
                     sb_dtype=sdt, x_dtype=xdc)
        assert np.array_equal(yb, 2.0 * ya)
        # exact-integer case: x in {-2..2}, scale = 2^-j, bias = -zp * 2^-j;
        # y = 2^-j * sum_k (q - zp) x exactly, checked in int64 arithmetic
        rng = np.random.default_rng(K + N)
        xi = rng.integers(-2, 3, size=(3, K))
        j = 3
        zp = 8 if bits == 4 else 2
        s_bits = f64_to_bits(np.full((N, G), 2.0 ** -j), sb)
        b_bits = f64_to_bits(np.full((N, G), -zp * 2.0 ** -j), sb)
        xin = xi.astype(np.float32) if xdt == "f32" else f64_to_bits(xi.astype(np.float64), "bf16")
        yi = orc.qmv(p.w_packed, s_bits, b_bits, xin, bits=bits, group_size=gs,
                     sb_dtype=sdt, x_dtype=xdc)
        qi = decode_unpackbits(p.w_packed, bits)
        exact = (xi @ (qi - zp).T).astype(np.float64) * 2.0 ** -j
        assert np.array_equal(yi, exact)


def pin_conversions(orc):
    """Storage conversions against numpy/torch over every 16-bit pattern, and
    fp32 -> bf16 round-to-nearest-even against torch (ties included)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref16 = f16_bits_to_f64(allb)
    refbf = bf16_bits_to_f64(allb)
    for h in range(0, 65536, 1):
        a = orc.f16_to_f64(h)
        r = ref16[h]
        assert (np.isnan(a) and np.isnan(r)) or a == r, ("f16", h, a, r)
    for h in range(0, 65536, 1):
        a = orc.bf16_to_f64(h)
        r = refbf[h]
        assert (np.isnan(a) and np.isnan(r)) or a == r, ("bf16", h, a, r)
    rng = np.random.default_rng(3)
    f = rng.standard_normal(20000).astype(np.float32)
    u = f.view(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    for arr in (f, ties, f * np.float32(1e30), f * np.float32(1e-38)):
        want = torch.from_numpy(arr.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        _, got = orc.round_outputs(arr.astype(np.float64))
        # round_outputs rounds f64 -> f32 first; arr is already f32, so exact
        assert np.array_equal(got, want)


def pin_sampled_matches_full(orc):
    """The sampled entry point returns the full result's entries."""
    p = gen.make_problem(N=41, K=256, bits=4, gs=64, sb="bf16", x_dtype="bf16", seed=5)
    y = run(orc, p, M=4)
    ms = np.array([0, 3, 1, 2, 3], dtype=np.int32)
    ns = np.array([0, 40, 17, 5, 0], dtype=np.int32)
    z = orc.qmv_at(p.w_packed, p.scales, p.biases, p.x[:4], ms, ns, bits=4, group_size=64,
                   sb_dtype=BF16, x_dtype=BF16)
    assert np.array_equal(z, y[ms, ns])


def pin_magnitude(orc):
    """The term magnitude of the a-priori error bound.  Closed form on x = +-e_k:
    mag[k][n] = 2^(bits+2)|scale[n][g(k)]| + |bias[n][g(k)]| exactly (the signs
    of x, scales and biases must not matter); mag(2x) = 2 mag(x) exactly; and
    mag dominates every output's terms: mag >= |x| @ |W|^T with W = scale*q + bias
    dequantized densely by numpy (so it also dominates |y|)."""
    for (N, K, bits, gs, sb, xdt) in SHAPES:
        p = gen.make_problem(N=N, K=K, bits=bits, gs=gs, sb=sb, x_dtype=xdt, seed=313 + K)
        G = K // gs
        sdt, xdc = (F16 if sb == "f16" else BF16), (F32 if xdt == "f32" else BF16)
        s64 = sb_to_f64(p.scales, sb)
        flip = (np.arange(N * G).reshape(N, G) % 3) == 0
        sc = f64_to_bits(np.where(flip, -s64, s64), sb)          # some negative scales
        sv, bv = sb_to_f64(sc, sb), sb_to_f64(p.biases, sb)
        ks = np.arange(0, K, max(1, K // 24))
        e = np.zeros((ks.size, K), dtype=np.float64)
        e[np.arange(ks.size), ks] = np.where(np.arange(ks.size) % 2 == 0, 1.0, -1.0)
        xe = e.astype(np.float32) if xdt == "f32" else f64_to_bits(e, "bf16")
        mag = orc.qmv_mag(sc, p.biases, xe, bits=bits, group_size=gs, sb_dtype=sdt, x_dtype=xdc)
        want = (2.0 ** (bits + 2)) * np.abs(sv[:, ks // gs]).T + np.abs(bv[:, ks // gs]).T
        assert np.array_equal(mag, want), (N, K, bits, gs)
        xv = x_to_f64(p.x[:4], xdt)
        m1 = orc.qmv_mag(sc, p.biases, p.x[:4], bits=bits, group_size=gs, sb_dtype=sdt, x_dtype=xdc)
        x2 = (p.x[:4] * np.float32(2.0)).astype(np.float32) if xdt == "f32" else f64_to_bits(2.0 * xv, "bf16")
        m2 = orc.qmv_mag(sc, p.biases, x2, bits=bits, group_size=gs, sb_dtype=sdt, x_dtype=xdc)
        assert np.array_equal(m2, 2.0 * m1)
        q = decode_unpackbits(p.w_packed, bits).astype(np.float64)
        W = np.repeat(sv, gs, axis=1) * q + np.repeat(bv, gs, axis=1)
        assert np.all(m1 >= np.abs(xv) @ np.abs(W).T * (1 - 1e-12)), (N, K, bits, gs)


def pin_round_outputs(orc):
    """fp64 -> fp32 -> bf16 rounding of the outputs.  fp64 values off the fp32
    grid, and exact fp32 midpoints (ties), round to nearest even: the expected
    fp32 is picked by comparing distances in exact fp64 arithmetic, the tie by
    the even significand; the bf16 step then matches torch on that fp32."""
    rng = np.random.default_rng(21)
    base = (rng.standard_normal(4000) * np.exp2(rng.integers(-60, 60, 4000))).astype(np.float32)
    lo = base.astype(np.float64)
    hi = np.nextafter(base, np.float32(np.inf)).astype(np.float64)
    frac = rng.random(4000)
    frac[:1000] = 0.5                                            # exact midpoints
    v = lo + (hi - lo) * frac                                    # exact in fp64 for a midpoint
    mid = lo + (hi - lo) * 0.5
    even_lo = (base.view(np.uint32) & np.uint32(1)) == 0
    pick_lo = (v < mid) | ((v == mid) & even_lo)
    want32 = np.where(pick_lo, base, np.nextafter(base, np.float32(np.inf))).astype(np.float32)
    got32, got16 = orc.round_outputs(v)
    assert np.array_equal(got32.view(np.uint32), want32.view(np.uint32))
    want16 = torch.from_numpy(want32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got16, want16)


# ------------------------------------------------------------- mxfp4 mode ---

def _mx_golden():
    with open(os.path.join(GOLDEN, "mxfp4_e2m1.json")) as f:
        return json.load(f)


def pin_mx_codes_golden(orc):
    """Every E2M1 code and sample E8M0 scales against hand-worked values."""
    gd = _mx_golden()
    for c, v in enumerate(gd["e2m1"]):
        got = orc.e2m1_to_f64(c)
        assert got == v and np.signbit(got) == np.signbit(v), (c, got, v)
    for e, v in gd["e8m0"]:
        assert orc.e8m0_to_f64(e) == v, (e, orc.e8m0_to_f64(e), v)
    assert np.isnan(orc.e8m0_to_f64(gd["e8m0_nan"]))


def _mx_dense(p):
    """Dequantized weights from numpy bit unpacking, the golden code table and
    ldexp of the scale bytes: W[n][k] = 2^(E[n][k/32] - 127) * e2m1(q[n][k])."""
    table = np.array(_mx_golden()["e2m1"], dtype=np.float64)
    q = decode_unpackbits(p.w_packed, 4)
    sc = np.ldexp(1.0, p.scales.astype(np.int64) - 127)
    return table[q] * np.repeat(sc, 32, axis=1)


def pin_mx_bruteforce(orc):
    """Dequantize-then-dot (numpy matmul over the dense weights) equals the
    oracle's blocked form to fp64 rounding, on several tiny shapes."""
    for N, K, xdt, seed in ((7, 96, "bf16", 1), (5, 32, "f32", 2), (11, 256, "bf16", 3)):
        p = gen.make_mx_problem(N, K, xdt, seed, e_lo=100, e_hi=140)
        x64 = x_to_f64(p.x[:3], xdt)
        want = x64 @ _mx_dense(p).T
        got = orc.qmv_mxfp4(p.w_packed, p.scales, p.x[:3], x_dtype=F32 if xdt == "f32" else BF16)
        assert normwise(got, want) <= 1e-12, (N, K, normwise(got, want))


def pin_mx_readout(orc):
    """Scale 1 (E = 127) and x = e_k read one code value back exactly; a
    scale byte one higher doubles it exactly."""
    table = np.array(_mx_golden()["e2m1"], dtype=np.float64)
    p = gen.make_mx_problem(9, 128, "f32", 4, keep_q=True)
    ks = [0, 1, 7, 8, 31, 32, 63, 64, 100, 127]
    x = np.zeros((len(ks), 128), dtype=np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    for E, mult in ((127, 1.0), (128, 2.0)):
        sc = np.full(p.scales.shape, E, dtype=np.uint8)
        y = orc.qmv_mxfp4(p.w_packed, sc, x, x_dtype=F32)
        assert np.array_equal(y, mult * table[p.q[:, ks].T]), E


def pin_mx_magnitude(orc):
    """The mxfp4 term magnitude: on x = +-e_k it is 6 * 2^(E-127) exactly; a row
    with a NaN scale (E = 255) in any block is NaN for every vector (NaN * 0 is
    NaN, as in the product itself); mag(2x) = 2 mag(x), and it dominates
    |x| @ |W|^T for the dense dequantized weights."""
    p = gen.make_mx_problem(6, 128, "f32", 8, e_lo=0, e_hi=254)
    sc = p.scales.copy()
    sc[2, 1] = 255
    ks = np.array([0, 5, 31, 32, 70, 127])
    x = np.zeros((ks.size, 128), dtype=np.float32)
    x[np.arange(ks.size), ks] = np.where(np.arange(ks.size) % 2 == 0, 1.0, -1.0)
    mag = orc.qmv_mxfp4_mag(sc, x, x_dtype=F32)
    want = 6.0 * np.ldexp(1.0, sc[:, ks // 32].astype(np.int64) - 127).T
    want[:, 2] = np.nan
    assert np.array_equal(mag, want, equal_nan=True)
    p = gen.make_mx_problem(9, 256, "bf16", 9, e_lo=100, e_hi=140)
    xv = x_to_f64(p.x[:3], "bf16")
    m1 = orc.qmv_mxfp4_mag(p.scales, p.x[:3], x_dtype=BF16)
    m2 = orc.qmv_mxfp4_mag(p.scales, f64_to_bits(2.0 * xv, "bf16"), x_dtype=BF16)
    assert np.array_equal(m2, 2.0 * m1)
    assert np.all(m1 >= np.abs(xv) @ np.abs(_mx_dense(p)).T * (1 - 1e-12))


ALL_PINS = [pin_codec_golden, pin_2bit_float_floor_exhaustive, pin_4bit_nibbles_exhaustive,
            pin_readout, pin_worked_examples, pin_bruteforce_dequant, pin_closed_forms,
            pin_conversions, pin_sampled_matches_full, pin_magnitude, pin_round_outputs,
            pin_mx_codes_golden, pin_mx_bruteforce, pin_mx_readout, pin_mx_magnitude]
