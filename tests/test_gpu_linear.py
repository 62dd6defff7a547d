"""GPU parity of the dense NVFP4 linear (nvfp4_linear) against the CPU
oracle: y = f32(g_x * g_w) * NVFP4(x) @ W^T.  Gate in fp32-output mode:
relative Frobenius error <= 1e-3 and cosine >= 0.9999; the activation global
scale is bit-exact.  bf16 output is compared with the oracle's y rounded to
bf16 (reported; bf16 rounding alone costs ~1.7e-3)."""
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


def _problem(nv, orc, M, K, N, seed):
    x, w = synth.dense_problem(M, K, N, seed=seed, device="cuda:0")
    wq, wsf, wg = nv.quantize(w)  # GPU operands, quantized by the GPU
    wb = synth.torch_bits(w)
    gw = orc.global_scale(wb)  # oracle operands, quantized by the oracle
    oq, osf = orc.quantize(wb, gw)
    torch.cuda.synchronize()
    return x, (wq, wsf, wg), (oq, osf, gw)


# 32-row tiles (M <= 64, K a multiple of 256 or 128; N 768: an odd number of
# column tiles), 256-row tiles with ragged rows, and K values with and
# without whole 256-K super-steps
SHAPES = [(1, 256, 256), (3, 128, 256), (64, 1280, 512), (65, 256, 256), (300, 512, 768),
          (257, 7168, 256), (40, 64, 256), (17, 1024, 768)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_linear_vs_oracle(nv, orc, M, K, N):
    x, (wq, wsf, wg), (oq, osf, gw) = _problem(nv, orc, M, K, N, seed=M + K + N)
    gx_out = torch.empty(1, dtype=torch.float32, device="cuda:0")
    y = nv.linear(dev_bf16(x), wq, wsf, wg, out_dtype=torch.float32, x_gs_out=gx_out)
    yb = nv.linear(dev_bf16(x), wq, wsf, wg, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, gx = orc.linear(x, oq, osf, gw)
    assert host(gx_out)[0] == gx
    assert host(wg)[0] == gw
    err, cos = rel_fro(host(y), ref), cosine(host(y), ref)
    yb_v = synth.bf16_values(host_bits(yb))
    errb = rel_fro(yb_v, synth.bf16_values(synth.bf16_bits(ref)))
    print(f"linear M{M} K{K} N{N}: rel_fro {err:.3e} cos {cos:.8f} | bf16 out vs bf16(oracle) {errb:.3e}")
    assert err <= 1e-3 and cos >= 0.9999
    assert errb <= 5e-3


def test_linear_supplied_scale(nv, orc):
    M, K, N = 48, 512, 256
    x, (wq, wsf, wg), (oq, osf, gw) = _problem(nv, orc, M, K, N, seed=3)
    g = np.float32(0.5 / 2688.0)  # clamps the largest blocks at the E4M3 maximum
    y = nv.linear(dev_bf16(x), wq, wsf, wg, out_dtype=torch.float32, x_gs=dev_f32(g))
    torch.cuda.synchronize()
    ref, _ = orc.linear(x, oq, osf, gw, x_gs=g)
    err, cos = rel_fro(host(y), ref), cosine(host(y), ref)
    assert err <= 1e-3 and cos >= 0.9999, (err, cos)


def test_linear_bench_shape_sampled(nv, orc):
    """M4096 K4096 N16384 (the bench's dense workload), oracle on sampled
    rows and columns of y: the rows on both sides of every 256-row tile
    edge, and 64 columns (the 256-column tile edges at both ends and in the
    middle, plus seeded ones)."""
    s = synth.DENSE_SHAPE
    x, w = synth.dense_problem(device="cuda:0")
    wq, wsf, wg = nv.quantize(w)
    y = nv.linear(dev_bf16(x), wq, wsf, wg, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.array(sorted({r for t in range(17) for r in (256 * t - 1, 256 * t) if 0 <= r < s["M"]}))
    fixed = [0, 255, 256, 257, 8191, 8192, 16383]
    rng = np.random.Generator(np.random.PCG64(17))
    cols = np.sort(np.concatenate([fixed, rng.choice(np.setdiff1d(np.arange(s["N"]), fixed), 64 - len(fixed),
                                                     replace=False)]))
    wb = synth.torch_bits(w[torch.from_numpy(cols).cuda()])
    gw = orc.global_scale(synth.torch_bits(w))
    oq, osf = orc.quantize(wb, gw)
    ref, _ = orc.linear(x, oq, osf, gw, rows=rows)
    got = host(y)[rows][:, cols]
    err, cos = rel_fro(got, ref), cosine(got, ref)
    print(f"dense {s}: sampled rel_fro {err:.3e} cos {cos:.8f}")
    assert err <= 1e-3 and cos >= 0.9999


def test_linear_empty_and_rejects(nv):
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda:0")
    wq = torch.zeros((256, 128), dtype=torch.uint8, device="cuda:0")
    wsf = torch.zeros((256, 16), dtype=torch.uint8, device="cuda:0")
    wg = torch.ones(1, dtype=torch.float32, device="cuda:0")
    y = nv.linear(x, wq, wsf, wg)
    assert y.shape == (0, 256)
    with pytest.raises(nv.Nvfp4Error):
        nv.linear(torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda:0"), wq[:200], wsf[:200], wg)
