"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, each written independently of the oracle's own code.

Every function takes an ``oracle.Oracle`` instance and raises AssertionError
on a mismatch.  ``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` runs them on builds with planted mistakes
and expects at least one to fail for each mistake.
"""
import math
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.split("#", 1)[0].strip()
            if ln:
                yield ln


def bf16_round(vals):
    return synth.bf16_values(synth.bf16_bits(np.asarray(vals, np.float32)))


# -------------------------------------------------------------- E4M3 scale
def pin_e4m3_worked(o):
    """Worked values printed on NVFP4-1.1_APPROACH_PART_2.md."""
    for ln in _lines("e4m3_worked_values.txt"):
        kind, inp, code, dec = ln.split()
        if kind == "encode":
            got = o.e4m3_encode(float(inp))
            assert got == int(code, 16), (inp, hex(got), code)
            assert o.e4m3_value(got) == float(dec), (inp, o.e4m3_value(got), dec)
        else:
            v = o.e4m3_value(int(inp, 16))
            if dec == "nan":
                assert math.isnan(v), (inp, v)
            else:
                assert v == float(dec), (inp, v, dec)


def pin_e4m3_decode_vs_torch(o):
    """All 256 codes against torch.float8_e4m3fn (an independent library
    decoder of the same OCP format)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = o.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), (hex(c), v)
        else:
            assert v == ref[c], (hex(c), v, ref[c])


def _e4m3_grid():
    """All non-negative finite E4M3 magnitudes, from torch's decoder."""
    ref = torch.arange(0x7f, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    return ref.to(torch.float64).numpy()


def _sweep_values():
    """fp32 test values for the encoder: a strided sweep of [0, 2^10) plus,
    around every midpoint of two neighbouring E4M3 values, the midpoint and
    its fp32 neighbours."""
    rng = np.random.Generator(np.random.PCG64(12345))
    top = np.float32(1024.0).view(np.uint32)
    bits = np.arange(0, top, 503, dtype=np.uint32)
    vals = [bits.view(np.float32)]
    vals.append(rng.uniform(0, 2.0 ** -5, 200_000).astype(np.float32))
    grid = _e4m3_grid()
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, np.float32([448.0, 456.0, 464.0, 472.0, 480.0, 500.0, 1000.0])])
    vals += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))]
    vals.append(grid.astype(np.float32))
    return np.concatenate(vals).astype(np.float32)


def _pages_encode(v):
    """The pages' E4M3 procedure (NVFP4-1.1_APPROACH_PART_2.md): clamp at 448;
    subnormals round v * 512 to nearest even; normals take the floor of log2
    as exponent, round (norm - 1) * 8 to nearest even and carry a mantissa of
    8 into the exponent; exponent 15 with mantissa 7 is guarded to 448."""
    v = np.asarray(v, np.float64)
    out = np.zeros(v.shape, np.int64)
    sat = v >= 448.0
    sub = (~sat) & (v < 2.0 ** -6)
    nor = (~sat) & (~sub)
    out[sat] = 0x7E
    m = np.rint(v[sub] * 512.0).astype(np.int64)       # m == 8 is exponent 1, mantissa 0
    out[sub] = m
    vn = v[nor]
    ef = np.floor(np.log2(vn)).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    ef = np.where(np.ldexp(1.0, ef) > vn, ef - 1, ef)
    ef = np.where(np.ldexp(1.0, ef + 1) <= vn, ef + 1, ef)
    norm = vn / np.ldexp(1.0, ef)
    mant = np.rint((norm - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    mant[carry] = 0
    ef[carry] += 1
    exp = ef + 7
    nan_guard = (exp == 15) & (mant == 7)
    mant[nan_guard] = 6
    out[nor] = (exp << 3) | mant
    return out


_SWEEP = {}


def _encoded_sweep(o):
    """The sweep values and the oracle's codes for them (cached per build)."""
    if o.path not in _SWEEP:
        v = _sweep_values()
        _SWEEP[o.path] = (v, o.e4m3_encode_array(v))
    return _SWEEP[o.path]


def pin_e4m3_encode_vs_pages_procedure(o):
    v, got = _encoded_sweep(o)
    got = got.astype(np.int64)
    ref = _pages_encode(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, ("encode mismatches", bad.size, v[bad[:5]], got[bad[:5]], ref[bad[:5]])
    assert not np.any(got == 0x7F)


def pin_e4m3_encode_vs_torch(o):
    """torch's fp32 -> float8_e4m3fn cast rounds to nearest even; below 448
    it is an independent encoder (saturation is checked by the pages' pins)."""
    v, got = _encoded_sweep(o)
    keep = v < 448.0
    v, got = v[keep], got[keep]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, ("encode vs torch", bad.size, v[bad[:5]], got[bad[:5]], ref[bad[:5]])


def pin_e4m3_roundtrip(o):
    for c in range(0x7F):
        assert o.e4m3_encode(o.e4m3_value(c)) == c, hex(c)


# -------------------------------------------------------------- E2M1 element
def _e2m1_magnitude(idx):
    """OCP E2M1: exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
    subnormal (m * 0.5)."""
    e, m = idx >> 1, idx & 1
    return m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)


def pin_e2m1_worked(o):
    for ln in _lines("e2m1_worked_values.txt"):
        kind, inp, exp = ln.split()
        if kind == "nibble":
            assert o.e2m1_nibble(float(inp), False) == int(exp), (inp, o.e2m1_nibble(float(inp), False))
        elif kind == "halfup":
            hs = int(float(inp) * 2 + 0.5)
            assert o.step_to_idx(hs) == int(exp)
            assert o.e2m1_nibble(float(inp), False) != int(exp)
        else:
            assert o.step_to_idx(int(inp)) == int(exp)
    # clamp at 6 (|s| beyond the largest magnitude encodes as 6)
    for s in (6.0, 6.3, 7.0, 1e6, 3e38):
        assert o.e2m1_nibble(s, False) == 7
        assert o.e2m1_nibble(-s, True) == 15


def pin_e2m1_grid(o):
    """Nibble values follow the E2M1 definition; the half-step table maps
    each exactly representable half step to itself and the others to the
    nearest magnitude with ties to the even index."""
    mags = [_e2m1_magnitude(i) for i in range(8)]
    for n in range(16):
        want = mags[n & 7] * (-1 if n & 8 else 1)
        assert o.e2m1_value(n) == want, (n, o.e2m1_value(n), want)
    for hs in range(13):
        v = hs / 2
        d = [abs(m - v) for m in mags]
        best = min(d)
        cands = [i for i in range(8) if d[i] == best]
        want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        assert o.step_to_idx(hs) == want, (hs, o.step_to_idx(hs), want)
    # a value of the form k/4 with k odd is a first-stage tie: half to even
    for k in range(1, 48, 2):
        s = k / 4.0
        hs_even = int(round(s * 2))          # Python round: half to even
        assert o.e2m1_nibble(s, False) == o.step_to_idx(min(hs_even, 12)), s


# -------------------------------------------------------------- blocks
def pin_crafted_blocks(o):
    for ln in _lines("crafted_blocks.txt"):
        name, g, vals, sf, qb = [p.strip() for p in ln.split("|")]
        xs = bf16_round([float(t) for t in vals.split()])
        q, s = o.quantize_block(xs, float(g))
        assert s == int(sf, 16), (name, hex(s), sf)
        want = bytes(int(t, 16) for t in qb.split())
        assert bytes(q) == want, (name, bytes(q).hex(), want.hex())


def _random_blocks(seed, n, scale_spread=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((n, 16)).astype(np.float32)
    if scale_spread:
        x *= np.float32(2.0) ** rng.integers(-12, 12, size=(n, 1)).astype(np.float32)
    return bf16_round(x)


def pin_global_scale(o):
    """The dynamic global scale puts the block holding amax exactly on the
    E4M3 maximum 448 (0x7e) and no block above it."""
    for seed in range(20):
        xb = _random_blocks(seed, 64)
        bits = synth.bf16_bits(xb)
        g = o.global_scale(bits)
        q, sf = o.quantize(bits.reshape(4, 256), g)
        blk_max = np.abs(xb).max(axis=1)
        top = int(np.argmax(blk_max))
        assert sf.reshape(-1)[top] == 0x7E, (seed, hex(sf.reshape(-1)[top]))
        assert sf.max() <= 0x7E
    z = np.zeros((2, 32), np.uint16)
    assert o.global_scale(z) == np.float32(1.0)


def pin_quantize_invariants(o):
    """Over 500 random trials at the pages' test shapes (M=1,N=16; M=1,N=64;
    M=8,N=64): for blocks with a normal scale the largest element encodes to
    index 7 (6 / (1 + 1/16) > 5.5), quantize(dequantize(q)) == q with the same
    global scale, and |x - x_hat| <= 1.25 * sfd * g (the two-stage worst case
    at s = 5.25) plus fp32 rounding."""
    rng = np.random.Generator(np.random.PCG64(77))
    shapes = [(1, 16), (1, 64), (8, 64)]
    for trial in range(500):
        M, N = shapes[trial % 3]
        x = rng.standard_normal((M, N)).astype(np.float32)
        x *= np.float32(2.0) ** rng.integers(-6, 6, size=(M, N // 16, 1)).repeat(16, 2).reshape(M, N).astype(np.float32)
        bits = synth.bf16_bits(x)
        xv = synth.bf16_values(bits)
        g = o.global_scale(bits)
        q, sf = o.quantize(bits, g)
        xh = o.dequantize(q, sf, g)
        sfd = np.array([o.e4m3_value(c) for c in sf.reshape(-1)]).reshape(M, N // 16)
        err = np.abs(xv - xh).reshape(M, N // 16, 16).max(axis=2)
        assert np.all(err <= 1.25 * sfd * g * (1 + 2.0 ** -20) + 1e-30), trial
        normal = sf >= 0x08
        nib = np.stack([q & 15, q >> 4], -1).reshape(M, N)
        xb = np.abs(xv).reshape(M, N // 16, 16)
        top = np.argmax(xb, axis=2)
        top_nib = np.take_along_axis(nib.reshape(M, N // 16, 16), top[..., None], 2)[..., 0]
        assert np.all((top_nib[normal] & 7) == 7), trial
        q2, sf2 = o.quantize(synth.bf16_bits(xh), g)
        assert np.array_equal(sf2[normal], sf[normal]), trial
        qn = q.reshape(M, N // 16, 8)[normal]
        q2n = q2.reshape(M, N // 16, 8)[normal]
        assert np.array_equal(qn, q2n), trial


def pin_dequant_exhaustive(o):
    """16 nibbles x every non-NaN scale byte: x_hat = f32(f32(e2m1 * sfd) * g),
    with e2m1 from the format definition and sfd from torch's decoder."""
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    sfd = torch.tensor(codes, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    M = len(codes)
    q = np.tile(np.array([0x10 * (2 * i + 1) + 2 * i for i in range(8)], np.uint8), (M, 1))
    q = np.concatenate([q, q], axis=1)                         # 32 elements per row
    nib = np.stack([q & 15, q >> 4], -1).reshape(M, 32)
    sf = np.stack([np.array(codes, np.uint8)] * 2, 1)
    vals = np.array([_e2m1_magnitude(n & 7) * (-1 if n & 8 else 1) for n in range(16)], np.float32)
    for g in (1.0, 0.0078125, 3.0e-3, 17.25):
        g32 = np.float32(g)
        want = (vals[nib] * np.repeat(sfd[:, None], 32, 1)).astype(np.float32) * g32
        got = o.dequantize(q, sf, g32)
        assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32)), g
        got16 = o.dequantize(q, sf, g32, "bf16")
        want16 = synth.bf16_bits(want)
        assert np.array_equal(got16, want16), g


# -------------------------------------------------------------- GEMM / MoE
def _oracle_weights(o, cfg):
    E, I, H = cfg.E, cfg.I, cfg.H
    w = dict(w1q=np.zeros((E, 2 * I, H // 2), np.uint8), w1sf=np.zeros((E, 2 * I, H // 16), np.uint8),
             w1gs=np.zeros(E, np.float32), w2q=np.zeros((E, H, I // 2), np.uint8),
             w2sf=np.zeros((E, H, I // 16), np.uint8), w2gs=np.zeros(E, np.float32))
    for e in range(E):
        a, b = synth.expert_weights(cfg, e)
        a, b = synth.torch_bits(a), synth.torch_bits(b)
        w["w1gs"][e] = o.global_scale(a)
        w["w1q"][e], w["w1sf"][e] = o.quantize(a, w["w1gs"][e])
        w["w2gs"][e] = o.global_scale(b)
        w["w2q"][e], w["w2sf"][e] = o.quantize(b, w["w2gs"][e])
    return w


def pin_moe_all_ones(o):
    """All-ones activations and weights (the pages' all-ones GEMM idea): every
    block scale is 0x7e and every element encodes to 6, so each operand
    dequantizes to 2688 before its global scale; with a2_gs = c/2688,
    y = I * 2688^2 * f32(a2_gs * g_w2) * sum(w)."""
    T, H, I, E, k = 4, 64, 32, 2, 2
    one = np.full((T, H), 0x3F80, np.uint16)
    ids = np.array([[0, 1], [1, 0], [0, 1], [1, 0]], np.int32)
    wts = np.array([[0.25, 0.75], [0.5, 0.5], [1.0, 0.0], [0.125, 0.875]], np.float32)
    w1 = np.full((2 * I, H), 0x3F80, np.uint16)
    w2 = np.full((H, I), 0x3F80, np.uint16)
    g1 = o.global_scale(w1)
    g2 = o.global_scale(w2)
    q1, s1 = o.quantize(w1, g1)
    q2, s2 = o.quantize(w2, g2)
    assert np.all(s1 == 0x7E) and np.all(q1 == 0x77)
    gx = np.float32(1.0) / np.float32(2688.0)
    assert o.global_scale(one) == gx
    alpha1 = np.float32(gx * g1)
    h = H * 2688.0 * 2688.0 * float(alpha1)
    c = h / (1 + math.exp(-h)) * h
    c_bf = float(bf16_round([c])[0])
    a2 = np.float32(c_bf) / np.float32(2688.0)
    out = o.moe_tokens(one, ids, wts, np.stack([q1] * E), np.stack([s1] * E), np.float32([g1] * E),
                       np.stack([q2] * E), np.stack([s2] * E), np.float32([g2] * E), a2,
                       want_pairs=True)
    assert np.all(out["a2_sf"] == 0x7E) and np.all(out["a2_q"] == 0x77)
    alpha2 = float(np.float32(a2 * g2))
    for t in range(T):
        want = I * 2688.0 * 2688.0 * alpha2 * float(wts[t].astype(np.float64).sum())
        assert np.allclose(out["y"][t], np.float32(want), rtol=1e-6, atol=0), (t, out["y"][t][0], want)


def pin_moe_dense(o):
    cfg = synth.TINY
    w = _oracle_weights(o, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    out = o.moe_tokens(x, ids, wts, w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"],
                       cfg.a2_gs, want_pairs=True)
    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.topk
    gx = o.global_scale(x)
    xq, xsf = o.quantize(x, gx)
    xa = o.dequantize(xq, xsf, 1.0).astype(np.float64)
    assert out["x_gs"] == gx
    w1a = [o.dequantize(w["w1q"][e], w["w1sf"][e], 1.0).astype(np.float64) for e in range(cfg.E)]
    w2a = [o.dequantize(w["w2q"][e], w["w2sf"][e], 1.0).astype(np.float64) for e in range(cfg.E)]
    c_or = synth.bf16_values(out["c"]).astype(np.float64)
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            h = (w1a[e] @ xa[t]) * float(np.float32(gx * w["w1gs"][e]))
            hh = h.reshape(I // 8, 2, 8)
            gate, up = hh[:, 0, :].reshape(-1), hh[:, 1, :].reshape(-1)
            c = gate / (1.0 + np.exp(-gate)) * up
            # oracle c is c rounded once to bf16: within half a bf16 ulp
            assert np.all(np.abs(c_or[t, j] - c) <= np.abs(c) * 2.0 ** -8 + 1e-30), (t, j)
            # the MoE's internal requantization is the (pinned) tensor quantizer
            cq, csf = o.quantize(out["c"][t, j][None, :], cfg.a2_gs)
            assert np.array_equal(cq[0], out["a2_q"][t, j]) and np.array_equal(csf[0], out["a2_sf"][t, j])
            a2 = o.dequantize(cq, csf, 1.0).astype(np.float64)[0]
            oo = (w2a[e] @ a2) * float(np.float32(np.float32(cfg.a2_gs) * w["w2gs"][e]))
            y[t] += float(wts[t, j]) * oo
    err = np.linalg.norm(out["y"] - y) / np.linalg.norm(y)
    assert err < 1e-6, err


def pin_moe_dynamic_all_ones(o):
    """The all-ones case with the dynamic L1-output scale: c is the same
    constant in every pair, so g2 = bf16(c) / 2688 exactly (the scale the
    static all-ones pin supplies by hand) and y has the same closed form."""
    T, H, I, E, k = 4, 64, 32, 2, 2
    one = np.full((T, H), 0x3F80, np.uint16)
    ids = np.array([[0, 1], [1, 0], [0, 1], [1, -1]], np.int32)
    wts = np.array([[0.25, 0.75], [0.5, 0.5], [1.0, 0.0], [0.125, 0.875]], np.float32)
    w1 = np.full((2 * I, H), 0x3F80, np.uint16)
    w2 = np.full((H, I), 0x3F80, np.uint16)
    g1, g2w = o.global_scale(w1), o.global_scale(w2)
    q1, s1 = o.quantize(w1, g1)
    q2, s2 = o.quantize(w2, g2w)
    gx = np.float32(1.0) / np.float32(2688.0)
    h = H * 2688.0 * 2688.0 * float(np.float32(gx * g1))
    c_bf = float(bf16_round([h / (1 + math.exp(-h)) * h])[0])
    out = o.moe_tokens_dynamic(one, ids, wts, np.stack([q1] * E), np.stack([s1] * E),
                               np.float32([g1] * E), np.stack([q2] * E), np.stack([s2] * E),
                               np.float32([g2w] * E))
    assert out["a2_gs"] == np.float32(c_bf) / np.float32(2688.0)
    alpha2 = float(np.float32(out["a2_gs"] * g2w))
    for t in range(T):
        valid = ids[t] >= 0
        want = I * 2688.0 * 2688.0 * alpha2 * float(wts[t][valid].astype(np.float64).sum())
        assert np.allclose(out["y"][t], np.float32(want), rtol=1e-6, atol=0), (t, out["y"][t][0], want)


def pin_moe_dynamic_dense(o):
    """Dynamic L1-output scale on the tiny workload with two skipped pairs:
    g2 is the largest bf16-rounded SwiGLU value of the valid pairs (brute
    force, fp64 matmuls) / 2688, and y follows with g2 as the scale."""
    cfg = synth.TINY
    w = _oracle_weights(o, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    ids = ids.copy()
    ids[3, 0], ids[5, 1] = -1, cfg.E
    out = o.moe_tokens_dynamic(x, ids, wts, w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"],
                               w["w2gs"])
    T, H, I, k = cfg.T, cfg.H, cfg.I, cfg.topk
    gx = o.global_scale(x)
    xq, xsf = o.quantize(x, gx)
    xa = o.dequantize(xq, xsf, 1.0).astype(np.float64)
    w1a = [o.dequantize(w["w1q"][e], w["w1sf"][e], 1.0).astype(np.float64) for e in range(cfg.E)]
    w2a = [o.dequantize(w["w2q"][e], w["w2sf"][e], 1.0).astype(np.float64) for e in range(cfg.E)]
    cs = {}
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if not 0 <= e < cfg.E:
                continue
            hh = ((w1a[e] @ xa[t]) * float(np.float32(gx * w["w1gs"][e]))).reshape(I // 8, 2, 8)
            gate, up = hh[:, 0, :].reshape(-1), hh[:, 1, :].reshape(-1)
            cs[t, j] = synth.bf16_bits((gate / (1.0 + np.exp(-gate)) * up).astype(np.float32))
    amax = max(float(np.abs(synth.bf16_values(c)).max()) for c in cs.values())
    g2 = np.float32(np.float32(amax) / np.float32(2688.0))
    assert out["a2_gs"] == g2, (out["a2_gs"], g2)
    y = np.zeros((T, H))
    for (t, j), c in cs.items():
        e = ids[t, j]
        cq, csf = o.quantize(c[None, :], g2)
        a2 = o.dequantize(cq, csf, 1.0).astype(np.float64)[0]
        y[t] += float(wts[t, j]) * (w2a[e] @ a2) * float(np.float32(g2 * w["w2gs"][e]))
    err = np.linalg.norm(out["y"] - y) / np.linalg.norm(y)
    assert err < 1e-6, err


def pin_linear_bruteforce(o):
    """Dense linear on a tiny shape against triple loops over values decoded
    here from the bytes: nibbles by the E2M1 definition, scale bytes by
    torch's float8_e4m3fn (both independent of the oracle's decoders)."""
    rng = np.random.Generator(np.random.PCG64(9))
    M, K, N = 3, 48, 5
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    gw = o.global_scale(w)
    wq, wsf = o.quantize(w, gw)
    y, gx = o.linear(x, wq, wsf, gw)
    assert gx == o.global_scale(x)
    xq, xsf = o.quantize(x, gx)
    sfdec = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()

    def value(q, sf, r, k):
        nib = (int(q[r, k // 2]) >> (4 * (k % 2))) & 15
        mag = _e2m1_magnitude(nib & 7)
        return (-mag if nib & 8 else mag) * float(sfdec[sf[r, k // 16]])

    alpha = float(np.float32(gx * gw))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += value(xq, xsf, m, k) * value(wq, wsf, n, k)
            want = acc * alpha
            assert abs(float(y[m, n]) - want) <= abs(want) * 2.0 ** -23 + 1e-30, (m, n, y[m, n], want)
    # rows and columns subsets are the same numbers
    ys, _ = o.linear(x, wq, wsf, gw, rows=[2, 0], cols=[4, 1])
    assert np.array_equal(ys, y[[2, 0]][:, [4, 1]])


def pin_linear_all_ones(o):
    """All-ones x and W: every operand dequantizes to 2688 before its global
    scale, so y = K * 2688^2 * f32(g_x * g_w) = K * f32(1/2688 * 1/2688) * 2688^2."""
    M, K, N = 2, 64, 3
    one_x = np.full((M, K), 0x3F80, np.uint16)
    one_w = np.full((N, K), 0x3F80, np.uint16)
    gw = o.global_scale(one_w)
    wq, wsf = o.quantize(one_w, gw)
    y, gx = o.linear(one_x, wq, wsf, gw)
    want = K * 2688.0 * 2688.0 * float(np.float32(gx * gw))
    assert np.all(y == np.float32(want)), (y, want)


def pin_l1_rows_dense(o):
    """Single-expert L1 + SwiGLU rows against a dense fp64 matmul."""
    rng = np.random.Generator(np.random.PCG64(5))
    M, K, I = 24, 128, 64
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wn = synth.bf16_bits((rng.standard_normal((2 * I, K)) * 0.02).astype(np.float32))
    wi = synth.interleave_gate_up(wn)
    gx, gw = o.global_scale(x), o.global_scale(wi)
    xq, xsf = o.quantize(x, gx)
    wq, wsf = o.quantize(wi, gw)
    rows = np.array([0, 5, 23, 7], np.int64)
    c, h = o.l1_swiglu_rows(xq, xsf, gx, wq, wsf, gw, rows, want_h=True)
    xa = o.dequantize(xq, xsf, 1.0).astype(np.float64)
    # undo the interleave by construction: natural order = gate rows, then up rows
    wa = o.dequantize(wq, wsf, 1.0).astype(np.float64)
    hr = xa[rows] @ wa.T * float(np.float32(gx * gw))
    assert np.allclose(h, hr, rtol=1e-12, atol=1e-12)
    hh = hr.reshape(len(rows), I // 8, 2, 8)
    gate, up = hh[:, :, 0, :].reshape(len(rows), I), hh[:, :, 1, :].reshape(len(rows), I)
    cr = gate / (1 + np.exp(-gate)) * up
    cv = synth.bf16_values(c)
    assert np.all(np.abs(cv - cr) <= np.abs(cr) * 2.0 ** -8 + 1e-30)


# cheapest first (the mutation tests stop at the first failing pin)
ALL_PINS = [
    pin_e4m3_worked, pin_e4m3_decode_vs_torch, pin_e4m3_roundtrip, pin_e2m1_worked,
    pin_e2m1_grid, pin_crafted_blocks, pin_global_scale, pin_dequant_exhaustive,
    pin_moe_all_ones, pin_moe_dynamic_all_ones, pin_l1_rows_dense, pin_moe_dense,
    pin_moe_dynamic_dense, pin_linear_all_ones, pin_linear_bruteforce, pin_quantize_invariants,
    pin_e4m3_encode_vs_pages_procedure, pin_e4m3_encode_vs_torch,
]
