"""GPU parity: nvfp4_quantize / nvfp4_dequantize through the C ABI against the
CPU oracle, bit-exact on every byte (scale bytes, packed nibbles, global
scale, dequantized values)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_bf16, dev_f32, host, host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import quantization_nvfp4_quantize_amd as nv
    assert torch.cuda.is_available()
    return nv


def _gpu_quant(nv, bits, g=None):
    x = dev_bf16(bits)
    q, sf, gs = nv.quantize(x, None if g is None else dev_f32(g))
    torch.cuda.synchronize()
    return host(q), host(sf), host(gs)[0]


def _check(nv, orc, bits, g=None, what=""):
    qg, sfg, gsg = _gpu_quant(nv, bits, g)
    g_or = orc.global_scale(bits) if g is None else np.float32(g)
    assert gsg.view(np.uint32) == np.float32(g_or).view(np.uint32), (what, gsg, g_or)
    q, sf = orc.quantize(bits, g_or)
    bad_sf = np.nonzero(sfg != sf)
    assert bad_sf[0].size == 0, (what, "scale mismatches", bad_sf[0].size, sfg[bad_sf][:8], sf[bad_sf][:8])
    bad_q = np.nonzero(qg != q)
    assert bad_q[0].size == 0, (what, "nibble mismatches", bad_q[0].size, qg[bad_q][:8], q[bad_q][:8])
    return qg, sfg, gsg


def test_quantize_500_trials(nv, orc):
    """The pages' method: 500 random trials at M=1,N=16; M=1,N=64; M=8,N=64
    (0 mismatches of scale bytes and nibbles)."""
    rng = np.random.Generator(np.random.PCG64(2024))
    shapes = [(1, 16), (1, 64), (8, 64)]
    for t in range(500):
        M, N = shapes[t % 3]
        x = rng.standard_normal((M, N)).astype(np.float32)
        if t % 5 == 0:
            x *= np.float32(10.0) ** rng.integers(-4, 4, size=(M, N)).astype(np.float32)
        _check(nv, orc, synth.bf16_bits(x), what=f"trial {t}")


def test_quantize_crafted_blocks(nv, orc):
    import pins
    for ln in pins._lines("crafted_blocks.txt"):
        name, g, vals, sf, qb = [p.strip() for p in ln.split("|")]
        bits = synth.bf16_bits(np.array([float(v) for v in vals.split()], np.float32))[None, :]
        q, s, _ = _check(nv, orc, bits, g=float(g), what=name)
        assert s[0, 0] == int(sf, 16)
        assert bytes(q[0]) == bytes(int(t, 16) for t in qb.split())


def test_quantize_exhaustive_bf16(nv, orc):
    """Every finite bf16 value v in the block [M*, v, 0, ...] with M* = 3.0,
    and alone in its block, under two global scales."""
    v = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (v & 0x7F80) != 0x7F80
    v = v[finite]
    blocks = np.zeros((v.size, 16), np.uint16)
    blocks[:, 0] = synth.bf16_bits(np.float32([3.0]))[0]
    blocks[:, 1] = v
    alone = np.zeros((v.size, 16), np.uint16)
    alone[:, 5] = v
    for g in (1.0, 2.0 ** -6):
        _check(nv, orc, blocks.reshape(-1, 64), g=g, what=f"with M*, g={g}")
        _check(nv, orc, alone.reshape(-1, 64), g=g, what=f"alone, g={g}")
    _check(nv, orc, alone.reshape(-1, 64), what="alone, dynamic g")


@pytest.mark.parametrize("M,K", [(0, 16), (1, 16), (3, 48), (5, 272), (7, 7168), (33, 2048)])
def test_quantize_shapes(nv, orc, M, K):
    rng = np.random.Generator(np.random.PCG64(M * 1000 + K))
    bits = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    _check(nv, orc, bits, what=f"{M}x{K}")
    _check(nv, orc, bits, g=0.0123, what=f"{M}x{K} supplied g")


def test_quantize_zero_and_extreme_scales(nv, orc):
    z = np.zeros((4, 64), np.uint16)
    _, _, g = _check(nv, orc, z, what="all zero")
    assert g == np.float32(1.0)
    rng = np.random.Generator(np.random.PCG64(9))
    bits = synth.bf16_bits(rng.standard_normal((4, 256)).astype(np.float32))
    for g in (1e-30, 1e-10, 1.0, 1e10, 1e30):
        _check(nv, orc, bits, g=g, what=f"g={g}")
    # the smallest magnitudes inside the supported range (g > 2^-117)
    tiny = synth.bf16_bits(rng.standard_normal((4, 256)).astype(np.float32) * np.float32(1e-30))
    _check(nv, orc, tiny, what="amax ~1e-30")


def test_quantize_config_q_full(nv, orc):
    """The 8192 x 7168 workload (N(0,1), 1% outliers x100, 1% tiny blocks),
    compared in full."""
    bits = synth.quant_tensor()
    _check(nv, orc, bits, what="8192x7168 dynamic g")


def test_quantize_deterministic(nv):
    bits = synth.quant_tensor(512, 7168, seed=3)
    a = _gpu_quant(nv, bits)
    b = _gpu_quant(nv, bits)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_dequantize_exhaustive(nv, orc):
    """16 nibbles x every non-NaN scale byte, bf16 and fp32 outputs."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    M = codes.size
    q = np.tile(np.array([0x10 * ((2 * i + 1) & 15) + 2 * i for i in range(8)], np.uint8), (M, 2))
    sf = np.stack([codes, codes], 1)
    for g in (1.0, 3.0e-3, 17.25):
        for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            ref = orc.dequantize(q, sf, g, dt)
            out = nv.dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(sf).cuda(), dev_f32(g), tdt)
            torch.cuda.synchronize()
            got = host_bits(out) if dt == "bf16" else host(out)
            if dt == "f32":
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (g, dt)
            else:
                assert np.array_equal(got, ref), (g, dt)


def test_dequantize_config_q(nv, orc):
    bits = synth.quant_tensor(1024, 7168, seed=5)
    g = orc.global_scale(bits)
    q, sf = orc.quantize(bits, g)
    for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        ref = orc.dequantize(q, sf, g, dt)
        out = nv.dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(sf).cuda(), dev_f32(g), tdt)
        torch.cuda.synchronize()
        got = host_bits(out) if dt == "bf16" else host(out).view(np.uint32)
        want = ref if dt == "bf16" else ref.view(np.uint32)
        assert np.array_equal(got, want), dt


def test_roundtrip_on_gpu(nv, orc):
    """quantize(dequantize(q)) == q on the GPU for normal-scale blocks."""
    bits = synth.quant_tensor(256, 7168, seed=6)
    x = dev_bf16(bits)
    q, sf, gs = nv.quantize(x)
    xh = nv.dequantize(q, sf, gs, torch.bfloat16)
    q2, sf2, _ = nv.quantize(xh, gs)
    torch.cuda.synchronize()
    sfh, sf2h = host(sf), host(sf2)
    normal = sfh >= 0x08
    assert np.array_equal(sfh[normal], sf2h[normal])
    qh = host(q).reshape(sfh.shape[0], -1, 8)
    q2h = host(q2).reshape(sfh.shape[0], -1, 8)
    assert np.array_equal(qh[normal], q2h[normal])


def test_quantize_rejects_bad_args(nv):
    x = torch.zeros((4, 24), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(nv.Nvfp4Error):
        nv.quantize(x)


# ------------------------------------------------------------------ E4M3 sweep
# The block-scale encoder (fp32 -> E4M3, nearest with ties to the even code,
# saturating at 448) driven through nvfp4_quantize at chosen values.  The
# pages' worked values (NVFP4-1.1_APPROACH_PART_2.md, FP8 E4M3 fixes: 0.001 ->
# 0x01, 250 -> 0x78 by the mantissa carry, 448 -> 0x7e, no 0x7f) sit among the
# targets; the expected bytes are the oracle's.
def _bits_of(v):
    return np.array([np.float32(v)], np.float32).view(np.uint32).astype(np.int64)[0]


def _from_bits(b):
    return np.array([b], np.uint32).view(np.float32)[0]


def _e4m3_magnitudes():
    """Magnitudes of the codes 0x00..0x7e, decoded by torch's float8_e4m3fn."""
    return torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def _scale_targets():
    """Block-scale values bsf to drive the encoder with: every midpoint of
    two neighbouring codes and its fp32 neighbours (+-1, +-2 ulp), every code
    value +-1 ulp, the saturation range [448, 481] around the 464 tie, and
    the pages' worked values."""
    vals = _e4m3_magnitudes()
    mids, out = [], []
    for c in range(0x7E):
        mid = np.float32((np.float64(vals[c]) + np.float64(vals[c + 1])) / 2)
        assert np.float64(mid) == (np.float64(vals[c]) + np.float64(vals[c + 1])) / 2
        mids.append(mid)
        out += [_from_bits(_bits_of(mid) + d) for d in (-2, -1, 0, 1, 2)]
    for c in range(1, 0x7F):
        out += [_from_bits(_bits_of(vals[c]) + d) for d in (-1, 1)]
    for v in (448, 450, 455.5, 456, 460, 463.75, 464, 464.25, 470, 479.5, 480, 481, 500, 1e4, 3e38,
              0.001, 240, 248, 250, 256, 2.0 ** -10, 2.0 ** -11, 1e-30):
        out += [_from_bits(_bits_of(v) + d) for d in (-1, 0, 1)]
    return np.unique(np.array(out, np.float32)), np.array(mids, np.float32)


def _g_with_reciprocal(E):
    """A global scale g > 2^-117 whose fp32 reciprocal f32(1/g) is exactly E."""
    E = np.float32(E)
    b = _bits_of(np.float32(1.0) / E)
    for d in range(8):
        for s in (1, -1):
            g = _from_bits(b + s * d)
            if np.isfinite(g) and g > 2.0 ** -117 and np.float32(1.0) / g == E:
                return g
    return None


def _bf16_exact(v):
    return float(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).float()) == v


def _block_for(v):
    """(bmax, g) with bmax a bf16 value and f32(f32(bmax / 6) * f32(1 / g))
    == v exactly: bmax = 6 c 2^k makes bmax / 6 = c 2^k exact, E = 1 / g is
    searched next to v / (c 2^k), and g next to 1 / E."""
    v = np.float32(v)
    for c in (1.0, 1.5, 1.25, 1.75, 1.125, 1.375, 1.625, 1.875):
        k = int(np.floor(np.log2(np.float64(v) / c)))
        for kk in (k, k - 1, k + 1, k - 20, k + 20):
            b = 6.0 * c * 2.0 ** kk
            if not (1e-37 < b < 3e38) or not _bf16_exact(b):
                continue
            bmax = np.float32(b)
            q = np.float32(bmax / np.float32(6.0))
            if np.float64(q) != b / 6.0:
                continue
            base = _bits_of(np.float32(np.float64(v) / np.float64(q)))
            for d in range(-3, 4):
                E = _from_bits(base + d)
                if not np.isfinite(E) or E <= 0 or np.float32(q * E) != v:
                    continue
                g = _g_with_reciprocal(E)
                if g is not None and np.float32(q * (np.float32(1.0) / g)) == v:
                    return float(bmax), g
    return None


def test_e4m3_encoder_sweep(nv, orc):
    """Blocks whose scale product lands exactly on every E4M3 midpoint (ties
    to the even code), on its fp32 neighbours, on every code +-1 ulp, across
    the saturation range and on the pages' worked values: scale bytes and
    nibbles bit-exact against the oracle."""
    targets, mids = _scale_targets()
    rng = np.random.Generator(np.random.PCG64(77))
    jobs = []
    for v in targets:
        sol = _block_for(v)
        if sol is None:
            continue
        bmax, g = sol
        blk = np.float32(bmax) * rng.uniform(-1.0, 1.0, size=16).astype(np.float32)
        blk[rng.integers(16)] = np.float32(bmax) * (1 if rng.integers(2) else -1)
        bits = synth.bf16_bits(blk)[None, :]
        assert np.abs(synth.bf16_values(bits)).max() == np.float32(bmax)
        q, sf, _ = nv.quantize(dev_bf16(bits), dev_f32(g))
        jobs.append((v, g, bits, q, sf))
    solved = np.array([j[0] for j in jobs], np.float32)
    # every midpoint and its +-1 ulp neighbours is driven, and almost all else
    for m in mids:
        for d in (-1, 0, 1):
            assert _from_bits(_bits_of(m) + d) in solved, (m, d)
    assert solved.size >= 0.99 * targets.size, (solved.size, targets.size)
    torch.cuda.synchronize()
    codes = {}
    for v, g, bits, q, sf in jobs:
        oq, osf = orc.quantize(bits, g)
        assert host(sf)[0, 0] == osf[0, 0], (float(v), float(g), host(sf)[0, 0], osf[0, 0])
        assert np.array_equal(host(q), oq), (float(v), float(g))
        codes[float(v)] = int(osf[0, 0])
    # the pages' worked values, reached through the whole quantizer
    assert codes[float(np.float32(0.001))] == 0x01
    assert codes[250.0] == 0x78 and codes[248.0] == 0x78 and codes[240.0] == 0x77
    assert codes[448.0] == 0x7E and codes[464.0] == 0x7E and codes[480.0] == 0x7E
    assert 0x7F not in codes.values()
    print(f"E4M3 encoder: {solved.size} of {targets.size} target scales driven, all equal to the oracle")


@pytest.mark.parametrize("g", [0.3, 1.0 / 3.7, 0.0123, 7.77, 3.14159e-3, 2.0 ** -20 * 1.37])
def test_e4m3_encoder_dense_bf16_maxima(nv, orc, g):
    """Every finite bf16 block maximum (in [bmax, bmax/2, -bmax/3, 0, ...]
    blocks) under irregular supplied global scales: the products bsf fall
    densely across the whole E4M3 range, not on a power-of-two grid."""
    v = np.arange(0, 1 << 15, dtype=np.uint32).astype(np.uint16)
    v = v[(v & 0x7F80) != 0x7F80]
    vals = synth.bf16_values(v)
    blocks = np.zeros((v.size, 16), np.float32)
    blocks[:, 0] = vals
    blocks[:, 1] = vals / 2
    blocks[:, 2] = -vals / 3
    blocks[:, 7] = vals * np.float32(0.77)
    bits = synth.bf16_bits(blocks)
    bits[:, 0] = v
    _check(nv, orc, bits.reshape(-1, 128), g=g, what=f"dense maxima, g={g}")


@pytest.mark.parametrize("E,R,C", [(1, 2, 64), (3, 4, 128), (2, 256, 448), (1, 0, 64)])
def test_pair_scales_layout(nv, E, R, C):
    """nvfp4_pair_scales moves byte c of row r to (r / 2) 2C + 128 (c / 64) +
    64 (r % 2) + c % 64 (the rows of all matrices taken in order): checked
    byte for byte against that formula applied with numpy, the layout's
    definition (a forward-mapping roundtrip, like the pages' scale-factor
    remap verifier in DEBUG_LOG.md, "Current State")."""
    rng = np.random.default_rng(1000 * E + R + C)
    sf = rng.integers(0, 256, size=(E, R, C), dtype=np.uint8)
    out = host(nv.pair_scales(torch.from_numpy(sf).cuda()))
    torch.cuda.synchronize()
    flat = sf.reshape(-1, C)
    r = np.arange(flat.shape[0])[:, None]
    c = np.arange(C)[None, :]
    idx = (r // 2) * 2 * C + 128 * (c // 64) + 64 * (r % 2) + c % 64
    ref = np.zeros(flat.size, np.uint8)
    ref[idx.ravel()] = flat.ravel()
    assert np.unique(idx).size == flat.size  # a permutation
    assert np.array_equal(out.reshape(-1), ref)
