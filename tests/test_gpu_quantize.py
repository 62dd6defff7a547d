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
