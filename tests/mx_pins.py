"""Pins for the MXFP4 part of the CPU oracle (the OCP Microscaling Formats
(MX) Specification v1.0 format: 32-element blocks, E8M0 shared scale, E2M1
elements).  Each pin is written independently of the oracle's code: hand
derived values under ``tests/golden/`` (each file cites the specification
section it follows), closed forms, a differently written rounding, and a
brute-force GEMM.

Every function takes an ``oracle.Oracle`` instance and raises
AssertionError on a mismatch; ``tests/test_mx_oracle.py`` runs them on the
real oracle and on builds with planted mistakes.
"""
import math
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.split("#", 1)[0].strip()
            if ln:
                yield ln


def _bits(vals):
    return synth.bf16_bits(np.asarray(vals, np.float32))


def pin_mx_scale_values(o):
    """E8M0 (section 5.4): code c is 2^(c - 127); 255 is NaN."""
    for c in range(255):
        assert o.mx_scale_value(c) == math.ldexp(1.0, c - 127), c
    assert math.isnan(o.mx_scale_value(255))


def pin_mx_scale_codes(o):
    """Shared exponent of section 6.3, hand-derived (golden file)."""
    for ln in _rows("mx_scale_codes.txt"):
        amax, _, code = ln.split()
        assert o.mx_scale_code(float(amax)) == int(code), (amax, o.mx_scale_code(float(amax)), code)


def pin_mx_e2m1_worked(o):
    """Element rounding, hand-derived ties and saturation (golden file)."""
    for ln in _rows("mx_e2m1_values.txt"):
        v, nib = ln.split()
        assert o.mx_e2m1_nibble(float(v)) == int(nib), (v, o.mx_e2m1_nibble(float(v)), nib)
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for n in range(16):
        assert o.mx_e2m1_value(n) == (-grid[n & 7] if n & 8 else grid[n & 7]), n


def _rne_e2m1_binary(v):
    """Round-to-nearest-even on E2M1's binary significand, written from the
    format: below 2 the spacing is 0.5 (subnormal 0.5 and the binade [1, 2)),
    in the binade [2^e, 2^(e+1)) with e >= 1 it is 2^(e-1); the integer
    multiple of the spacing is rounded half to even, then saturation at 6."""
    a = abs(v)
    step = 0.5 if a < 2 else 2.0 ** (math.floor(math.log2(a)) - 1)
    r = np.rint(a / step) * step  # numpy rint rounds halves to even
    r = min(float(r), 6.0)
    mag = [0, 0.5, 1, 1.5, 2, 3, 4, 6].index(r)
    return mag | (8 if math.copysign(1.0, v) < 0 else 0)


def pin_mx_e2m1_sweep(o):
    """Every multiple of 1/256 in [-8, 8], every grid midpoint and its
    neighbours: the oracle agrees with the binary round-to-nearest-even."""
    vals = [k / 256.0 for k in range(-2048, 2049)]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for m in mids:
        for s in (-1.0, 1.0):
            vals += [s * m, s * np.nextafter(m, 0.0), s * np.nextafter(m, 10.0)]
    vals += [-0.0, 6.0, np.nextafter(6.0, 10.0), 1e30]
    for v in vals:
        assert o.mx_e2m1_nibble(v) == _rne_e2m1_binary(v), (v, o.mx_e2m1_nibble(v), _rne_e2m1_binary(v))


def pin_mx_crafted_blocks(o):
    """Blocks with hand-derived scale codes and bytes (golden file)."""
    for ln in _rows("mx_crafted_blocks.txt"):
        name, elems, code, hexbytes = [p.strip() for p in ln.split("|")]
        x = np.zeros(32, np.float32)
        ev = [float(t) for t in elems.split()]
        x[:len(ev)] = ev
        bits = _bits(x)
        assert np.array_equal(synth.bf16_values(bits), x), f"block {name} is not bf16-exact"
        q, c = o.mx_quantize_block(bits)
        want = bytes.fromhex(hexbytes.replace(" ", ""))
        assert c == int(code), (name, c, code)
        assert bytes(q) == want, (name, bytes(q).hex(), want.hex())


def pin_mx_roundtrip(o):
    """Properties of section 6.3 on seeded blocks of many magnitudes: a block
    with a scale code above 0 has its largest element at 4 or 6 (max |V| / X
    lies in [4, 8)); dequantizing and quantizing again reproduces the bytes;
    every element is within 2 X of its input (X when not saturated)."""
    rng = np.random.default_rng(1234)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    bits = _bits(x)
    xv = synth.bf16_values(bits).astype(np.float64)
    q, sc = o.mx_quantize(bits)
    xh = o.mx_dequantize(q, sc)
    X = np.repeat(np.exp2(sc.astype(np.float64) - 127), 32, axis=1)
    err = np.abs(xv - xh)
    assert np.all(err <= 2 * X), "error above 2 X"
    unsat = np.abs(xv) <= 6 * X
    assert np.all(err[unsat] <= X[unsat]), "error above X where not saturated"
    blocks = np.abs(xh).reshape(64, 8, 32).max(axis=2) / np.exp2(sc.astype(np.float64) - 127)
    assert np.all(np.isin(blocks[sc > 0], (4.0, 6.0))), "block maximum not at 4 or 6"
    hb = _bits(xh.astype(np.float32))
    assert np.array_equal(synth.bf16_values(hb).astype(np.float64), xh), "dequantized values not bf16"
    q2, sc2 = o.mx_quantize(hb)
    assert np.array_equal(q, q2) and np.array_equal(sc, sc2), "quantize(dequantize(q)) != q"


def pin_mx_linear(o):
    """The GEMM against a brute-force product of the dequantized operands
    (rows of A times rows of W), and the all-ones closed form: A all 1
    (scale 2^-2, elements 4) and W all 2 (scale 2^-1, elements 4) give
    y = 2 K everywhere."""
    rng = np.random.default_rng(77)
    M, N, K = 5, 7, 96
    a = _bits(rng.standard_normal((M, K)).astype(np.float32))
    w = _bits((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    aq, asc = o.mx_quantize(a)
    wq, wsc = o.mx_quantize(w)
    A, W = o.mx_dequantize(aq, asc), o.mx_dequantize(wq, wsc)
    y = o.mx_linear(aq, asc, wq, wsc, threads=2)
    ref = np.array([[sum(A[m, k] * W[n, k] for k in range(K)) for n in range(N)] for m in range(M)])
    assert np.allclose(y, ref, rtol=1e-12, atol=0), np.abs(y - ref).max()
    ones = _bits(np.ones((3, 64), np.float32))
    twos = _bits(np.full((4, 64), 2.0, np.float32))
    oq, osc = o.mx_quantize(ones)
    tq, tsc = o.mx_quantize(twos)
    assert np.all(osc == 125) and np.all(tsc == 126)
    assert np.all(o.mx_linear(oq, osc, tq, tsc, threads=1) == 128.0)


MX_PINS = [pin_mx_scale_values, pin_mx_scale_codes, pin_mx_e2m1_worked, pin_mx_e2m1_sweep,
           pin_mx_crafted_blocks, pin_mx_roundtrip, pin_mx_linear]
