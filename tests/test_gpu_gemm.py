"""GPU parity of the single-expert L1 stage (nvfp4_gemm_swiglu_quant): NVFP4
GEMM + SwiGLU + compact bf16 + fused NVFP4, against the CPU oracle.

Gates: compact bf16 SwiGLU output within relative Frobenius error 1e-3 and
cosine >= 0.9999 of the oracle's; the fused NVFP4 bytes (nibbles and scale
bytes) equal, bit for bit, the oracle's quantization of the GPU's own bf16
output under the same supplied global scale, on every compared row.  The
scale bytes that differ from the oracle's quantization of its own bf16 output
(where the two GEMMs' bf16 roundings differ) are counted and reported."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import cosine, dev_bf16, dev_f32, host, host_bits, rel_fro

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import quantization_nvfp4_quantize_amd as nv
    return nv


def _problem(M, K, I, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    wn = synth.bf16_bits((rng.standard_normal((2 * I, K)) * 0.02).astype(np.float32))
    return x, synth.interleave_gate_up(wn)


def _run(nv, orc, x, w, out_gs, rows=None, expand_a=True):
    M, K = x.shape
    N2 = w.shape[0]
    xq, xsf, xg = nv.quantize(dev_bf16(x))
    wq, wsf, wg = nv.quantize(dev_bf16(w))
    c, cq, csf = nv.gemm_swiglu_quant(xq, xsf, xg, wq, wsf, wg, dev_f32(out_gs), expand_a=expand_a)
    torch.cuda.synchronize()
    gx, gw = orc.global_scale(x), orc.global_scale(w)
    oq, osf = orc.quantize(x, gx)
    owq, owsf = orc.quantize(w, gw)
    assert np.array_equal(host(xq), oq) and np.array_equal(host(wq), owq)
    if rows is None:
        rows = np.arange(M)
    c_or, _ = orc.l1_swiglu_rows(oq, osf, gx, owq, owsf, gw, rows)
    return dict(c=host_bits(c)[rows], cq=host(cq)[rows], csf=host(csf)[rows], c_or=c_or, rows=rows)


def _gate(r, orc, out_gs, tol=1e-3):
    cg = synth.bf16_values(r["c"])
    co = synth.bf16_values(r["c_or"])
    err, cos = rel_fro(cg, co), cosine(cg, co)
    assert err <= tol and cos >= 0.9999, (err, cos)
    # the fused NVFP4 bytes == the oracle's quantization of the GPU's own bf16
    # output under the same supplied scale, nibbles and scale bytes
    gq, gsf = orc.quantize(r["c"], out_gs)
    bad = np.nonzero(r["csf"] != gsf)
    assert bad[0].size == 0, ("scale bytes", bad[0].size, r["csf"][bad][:8], gsf[bad][:8])
    bad = np.nonzero(r["cq"] != gq)
    assert bad[0].size == 0, ("nibbles", bad[0].size, r["cq"][bad][:8], gq[bad][:8])
    # against the oracle's quantization of its own bf16 output: scale bytes
    # may differ only in blocks whose bf16 values differ
    _, osf = orc.quantize(r["c_or"], out_gs)
    same = (r["c"].reshape(len(r["rows"]), -1, 16) == r["c_or"].reshape(len(r["rows"]), -1, 16)).all(-1)
    assert np.array_equal(r["csf"][same], osf[same])
    return err, cos, float((r["csf"] != osf).mean())


# expand_a: the activations expanded to f16 in a workspace first, or (False)
# read as NVFP4 and dequantized into LDS inside the GEMM
@pytest.mark.parametrize("expand_a", [True, False])
@pytest.mark.parametrize("M,K,I", [(1, 64, 128), (300, 512, 256), (517, 256, 384), (40, 1216, 128)])
def test_l1_stage_small(nv, orc, M, K, I, expand_a):
    x, w = _problem(M, K, I, seed=M + K + I)
    out_gs = np.float32(4.0 / 2688.0) * np.float32(np.sqrt(K / 256.0))
    r = _run(nv, orc, x, w, out_gs, expand_a=expand_a)
    err, cos, flip = _gate(r, orc, out_gs)
    print(f"M{M} K{K} I{I}: rel_fro {err:.3e} cos {cos:.7f} scale-byte flips {flip:.2e}")


def test_l1_stage_all_ones(nv, orc):
    """All-ones operands (the pages' all-ones GEMM check): every operand
    dequantizes to 2688 * g, so h = K * 2688^2 * f32(gx * gw) exactly in fp32
    and c = silu(h) * h rounded to bf16."""
    M, K, I = 256, 512, 128
    x = np.full((M, K), 0x3F80, np.uint16)
    w = np.full((2 * I, K), 0x3F80, np.uint16)
    r = _run(nv, orc, x, w, np.float32(1.0))
    assert np.array_equal(r["c"], r["c_or"])
    g = np.float32(np.float32(1.0) / np.float32(2688.0))
    h = np.float32(K * 2688.0 * 2688.0) * np.float32(g * g)
    want = synth.bf16_bits(np.float32([h / (1 + np.exp(-h)) * h]))[0]
    assert np.all(r["c"] == want)


@pytest.mark.parametrize("expand_a", [True, False])
def test_l1_stage_expert_config_sampled(nv, orc, expand_a):
    """The single-expert workload M4096 K7168 N 2x2048, run in full on the
    GPU, compared on 128 sampled rows (every tile edge included)."""
    x, w1 = synth.expert_problem()
    w = synth.torch_bits(w1)
    # every 256-row tile boundary (rows 256 t - 1, 256 t, 256 t + 1) plus a
    # seeded spread of interior rows: 128 rows in all
    edges = np.array([r for t in range(17) for r in (256 * t - 1, 256 * t, 256 * t + 1) if 0 <= r < 4096])
    rng = np.random.Generator(np.random.PCG64(41))
    inner = rng.choice(np.setdiff1d(np.arange(4096), edges), size=128 - edges.size, replace=False)
    rows = np.sort(np.concatenate([edges, inner]))
    r = _run(nv, orc, x, w, np.float32(synth.EXPERT_A2_GS), rows=rows, expand_a=expand_a)
    err, cos, flip = _gate(r, orc, np.float32(synth.EXPERT_A2_GS))
    print(f"expert config: rel_fro {err:.3e} cos {cos:.7f} scale-byte flips {flip:.2e}")


def test_l1_stage_paths_identical(nv):
    """Both activation paths feed the same exact f16 values to the same MFMA
    sequence: every output byte is identical."""
    x, w = _problem(700, 1024, 256, seed=9)
    xq, xsf, xg = nv.quantize(dev_bf16(x))
    wq, wsf, wg = nv.quantize(dev_bf16(w))
    og = dev_f32(0.01)
    a = nv.gemm_swiglu_quant(xq, xsf, xg, wq, wsf, wg, og, expand_a=True)
    b = nv.gemm_swiglu_quant(xq, xsf, xg, wq, wsf, wg, og, expand_a=False)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(a[0]), host_bits(b[0]))
    assert all(np.array_equal(host(u), host(v)) for u, v in zip(a[1:], b[1:]))


def test_l1_stage_deterministic(nv):
    x, w = _problem(512, 1024, 256, seed=3)
    xq, xsf, xg = nv.quantize(dev_bf16(x))
    wq, wsf, wg = nv.quantize(dev_bf16(w))
    og = dev_f32(0.01)
    a = [host(t) for t in nv.gemm_swiglu_quant(xq, xsf, xg, wq, wsf, wg, og)[1:]]
    b = [host(t) for t in nv.gemm_swiglu_quant(xq, xsf, xg, wq, wsf, wg, og)[1:]]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def test_l1_stage_rejects_bad_shapes(nv):
    z = torch.zeros((4, 40), dtype=torch.uint8, device="cuda:0")
    s = torch.zeros((4, 5), dtype=torch.uint8, device="cuda:0")
    g = dev_f32(1.0)
    with pytest.raises(nv.Nvfp4Error):
        nv.gemm_swiglu_quant(z, s, g, z, s, g, g)
