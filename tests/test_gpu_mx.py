"""GPU parity of the MXFP4 variant (the OCP MX v1.0 format: E8M0 scale per 32
elements, E2M1 elements; a separately labelled format next to the pages'
NVFP4) against the CPU oracle: quantize and dequantize bit-exact; the GEMM
(mxfp4_linear) in fp32 output within relative Frobenius 1e-3 and cosine
0.9999 of the oracle's float64 product of the same (oracle-quantized, and
byte-identical) operands."""
import os

import numpy as np
import pytest
import torch

import synth
from gpu_util import cosine, dev_bf16, host, host_bits, rel_fro

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def nv():
    import quantization_nvfp4_quantize_amd as nv
    return nv


def _quantize_both(nv, orc, bits):
    q, sc = nv.mx_quantize(dev_bf16(bits))
    torch.cuda.synchronize()
    oq, osc = orc.mx_quantize(bits)
    return host(q), host(sc), oq, osc


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (64, 1024), (300, 7168)])
def test_mx_quantize_vs_oracle(nv, orc, M, K):
    bits = synth.quant_tensor(M, K, seed=M + K)
    q, sc, oq, osc = _quantize_both(nv, orc, bits)
    assert np.array_equal(sc, osc), f"{(sc != osc).sum()} scale codes differ"
    assert np.array_equal(q, oq), f"{(q != oq).sum()} nibble bytes differ"
    print(f"mx quantize {M}x{K}: bit-exact; codes {osc.min()}..{osc.max()}")


def test_mx_quantize_crafted_blocks(nv, orc):
    rows = []
    with open(os.path.join(GOLDEN, "mx_crafted_blocks.txt")) as f:
        for ln in f:
            ln = ln.split("#", 1)[0].strip()
            if ln:
                rows.append(ln)
    x = np.zeros((len(rows), 32), np.float32)
    want_q, want_c = [], []
    for i, ln in enumerate(rows):
        _, elems, code, hexbytes = [p.strip() for p in ln.split("|")]
        ev = [float(t) for t in elems.split()]
        x[i, :len(ev)] = ev
        want_c.append(int(code))
        want_q.append(np.frombuffer(bytes.fromhex(hexbytes.replace(" ", "")), np.uint8))
    q, sc, _, _ = _quantize_both(nv, orc, synth.bf16_bits(x))
    assert np.array_equal(sc[:, 0], np.array(want_c, np.uint8)), (sc[:, 0], want_c)
    assert np.array_equal(q, np.stack(want_q)), q


@pytest.mark.parametrize("anchor", [1.0, 2.0 ** -130, 3.0e38])
def test_mx_quantize_every_bf16(nv, orc, anchor):
    """Every finite bf16 value v, in a block [anchor, v, 0, ...]: covers every
    element rounding and every scale code the maximum can give (subnormal
    maxima, the clamp at code 0, the largest codes)."""
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((v >> 7) & 0xFF) != 0xFF
    v = v[finite]
    blocks = np.zeros((v.size, 32), np.uint16)
    blocks[:, 0] = synth.bf16_bits(np.array([anchor], np.float32))[0]
    blocks[:, 1] = v
    q, sc, oq, osc = _quantize_both(nv, orc, blocks)
    assert np.array_equal(sc, osc), f"{(sc != osc).sum()} scale codes differ"
    assert np.array_equal(q, oq), f"{(q != oq).sum()} bytes differ"


def test_mx_dequantize_vs_oracle(nv, orc):
    bits = synth.quant_tensor(128, 2048, seed=5)
    oq, osc = orc.mx_quantize(bits)
    ref = orc.mx_dequantize(oq, osc)
    qd = torch.from_numpy(oq).to("cuda:0")
    sd = torch.from_numpy(osc).to("cuda:0")
    y32 = host(nv.mx_dequantize(qd, sd, out_dtype=torch.float32))
    y16 = host_bits(nv.mx_dequantize(qd, sd, out_dtype=torch.bfloat16))
    assert np.array_equal(y32.astype(np.float64), ref), "fp32 dequantize differs"
    assert np.array_equal(y16, synth.bf16_bits(ref.astype(np.float32))), "bf16 dequantize differs"


def _mx_problem(nv, orc, M, K, N, seed):
    x, w = synth.dense_problem(M, K, N, seed=seed, device="cuda:0")
    wq, wsc = nv.mx_quantize(w)  # GPU operands, quantized by the GPU
    torch.cuda.synchronize()
    oq, osc = orc.mx_quantize(synth.torch_bits(w))  # oracle operands, quantized by the oracle
    assert np.array_equal(host(wq), oq) and np.array_equal(host(wsc), osc)
    return x, (wq, wsc), (oq, osc)


# ragged rows (partial 256-row tiles), several column tiles, K of 1 .. many steps
SHAPES = [(1, 128, 256), (37, 256, 512), (256, 512, 256), (300, 1024, 768), (513, 7168, 256)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_mx_linear_vs_oracle(nv, orc, M, K, N):
    x, (wq, wsc), (oq, osc) = _mx_problem(nv, orc, M, K, N, seed=M + K + N)
    y = nv.mx_linear(dev_bf16(x), wq, wsc, out_dtype=torch.float32)
    yb = nv.mx_linear(dev_bf16(x), wq, wsc, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    aq, asc = orc.mx_quantize(x)
    ref = orc.mx_linear(aq, asc, oq, osc)
    err, cos = rel_fro(host(y), ref), cosine(host(y), ref)
    errb = rel_fro(synth.bf16_values(host_bits(yb)), synth.bf16_values(synth.bf16_bits(ref.astype(np.float32))))
    print(f"mx linear M{M} K{K} N{N}: rel_fro {err:.3e} cos {cos:.8f} | bf16 out vs bf16(oracle) {errb:.3e}")
    assert err <= 1e-3 and cos >= 0.9999
    assert errb <= 5e-3


def test_mx_linear_both_gemm_kernels_agree(nv, orc):
    """K % 512 == 0 with 16-byte aligned scale codes takes the GEMM that loads
    the scale codes 4 steps at a time; weight scale codes 4 bytes past a
    16-byte boundary (the alignment the entry point asks for) take the
    general GEMM.  Both sum the same MFMA products in the same order,
    so their outputs agree bit for bit (ragged rows, two column tiles)."""
    M, K, N = 300, 1024, 512
    x, (wq, wsc), _ = _mx_problem(nv, orc, M, K, N, seed=11)
    buf = torch.empty(wsc.numel() + 16, dtype=torch.uint8, device="cuda:0")
    wsc_odd = buf[4:4 + wsc.numel()].view(wsc.shape)
    wsc_odd.copy_(wsc)
    assert wsc.data_ptr() % 16 == 0 and wsc_odd.data_ptr() % 16 == 4
    xd = dev_bf16(x)
    y0 = nv.mx_linear(xd, wq, wsc, out_dtype=torch.float32)
    y1 = nv.mx_linear(xd, wq, wsc_odd, out_dtype=torch.float32)
    b0 = nv.mx_linear(xd, wq, wsc, out_dtype=torch.bfloat16)
    b1 = nv.mx_linear(xd, wq, wsc_odd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    assert torch.equal(b0.view(torch.int16), b1.view(torch.int16))
    print(f"mx linear M{M} K{K} N{N}: both GEMM kernels bit-identical (fp32 and bf16 out)")


def test_mx_linear_full_size_sampled(nv, orc):
    """The benchmark's shape and launch (M4096 K4096 N16384, bf16 out): sampled
    rows and columns against the oracle (MXFP4 quantization is per row, so the
    oracle quantizes just the sampled rows)."""
    M, K, N = synth.DENSE_SHAPE["M"], synth.DENSE_SHAPE["K"], synth.DENSE_SHAPE["N"]
    x, w = synth.dense_problem(M, K, N, seed=5, device="cuda:0")
    wq, wsc = nv.mx_quantize(w)
    ws = nv.mx_linear_workspace(M, K, N, "cuda:0")
    y = nv.mx_linear(dev_bf16(x), wq, wsc, out_dtype=torch.bfloat16, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(M, 24, replace=False))
    cols = np.sort(rng.choice(N, 96, replace=False))
    aq, asc = orc.mx_quantize(x[rows])
    wb = synth.torch_bits(w[torch.from_numpy(cols).to("cuda:0")])
    oq, osc = orc.mx_quantize(wb)
    assert np.array_equal(host(wq)[cols], oq) and np.array_equal(host(wsc)[cols], osc)
    ref = orc.mx_linear(aq, asc, oq, osc)
    got = synth.bf16_values(host_bits(y)[np.ix_(rows, cols)])
    err = rel_fro(got, synth.bf16_values(synth.bf16_bits(ref.astype(np.float32))))
    print(f"mx linear {M}x{K}x{N} sampled 24 x 96: bf16 out vs bf16(oracle) {err:.3e}")
    assert err <= 5e-3 and cosine(got, ref) >= 0.9999


def test_mx_rejects_bad_args(nv):
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(nv.Nvfp4Error):
        nv.mx_quantize(torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda:0"))  # K % 32
    wq = torch.zeros((256, 48), dtype=torch.uint8, device="cuda:0")
    wsc = torch.zeros((256, 3), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(nv.Nvfp4Error):
        nv.mx_linear(x, wq, wsc)  # K % 128
    x0 = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda:0")
    wq = torch.zeros((256, 64), dtype=torch.uint8, device="cuda:0")
    wsc = torch.zeros((256, 4), dtype=torch.uint8, device="cuda:0")
    assert nv.mx_linear(x0, wq, wsc).shape == (0, 256)  # empty input: nothing launched
