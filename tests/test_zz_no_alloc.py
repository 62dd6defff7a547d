"""The allocation-free MoE entry point (moe_expert_ffn_nvfp4_noalloc, its
workspace a static per-GPU buffer) against the workspace entry point
(moe_expert_ffn_nvfp4) on the same inputs: every output bit-identical, on two
calls in a row with the second smaller, in both output dtypes, and an
oversized call rejected without touching the outputs."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_bf16, dev_f32, host, host_bits
from moe_util import gpu_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import quantization_nvfp4_quantize_amd as nv
    return nv


def _outputs(nv, cfg, T, out_dtype, dev):
    P, I, H = T * cfg.topk, cfg.I, cfg.H
    return dict(out=torch.full((T, H), 7.0, dtype=out_dtype, device=dev),
                xq=torch.zeros((T, H // 2), dtype=torch.uint8, device=dev),
                xsf=torch.zeros((T, H // 16), dtype=torch.uint8, device=dev),
                x_gs_out=torch.zeros(1, dtype=torch.float32, device=dev),
                l1_c=torch.zeros((P, I), dtype=torch.bfloat16, device=dev),
                l1_q=torch.zeros((P, I // 2), dtype=torch.uint8, device=dev),
                l1_sf=torch.zeros((P, I // 16), dtype=torch.uint8, device=dev),
                err_count=torch.full((1,), -5, dtype=torch.int32, device=dev))


def _run(nv, cfg, w, x, ids, wts, T, out_dtype, noalloc):
    dev = torch.device("cuda:0")
    o = _outputs(nv, cfg, T, out_dtype, dev)
    out = o.pop("out")
    a2 = dev_f32(cfg.a2_gs)
    args = nv.moe_args(x[:T], ids[:T], wts[:T], w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"],
                       a2, out, **o)
    if noalloc:
        nv.moe_expert_ffn_noalloc(args, dev)
    else:
        nv.moe_expert_ffn_raw(args, dev)
    torch.cuda.synchronize()
    got = {k: host_bits(v) if v.dtype == torch.bfloat16 else host(v) for k, v in o.items()}
    got["out"] = host_bits(out) if out_dtype == torch.bfloat16 else host(out).view(np.uint32)
    return got


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_moe_noalloc_matches_workspace_entry(nv, out_dtype):
    cfg = synth.DEC
    w = gpu_weights(nv, cfg)
    x = dev_bf16(synth.activations(cfg))
    ids, wts = synth.routing(cfg)
    ids = ids.copy()
    ids[9, 3] = -1  # a skipped pair
    ti, tw = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    # two calls in a row, the second with fewer tokens (and its own routing)
    for T in (cfg.T, 37):
        a = _run(nv, cfg, w, x, ti, tw, T, out_dtype, noalloc=True)
        b = _run(nv, cfg, w, x, ti, tw, T, out_dtype, noalloc=False)
        for k in b:
            assert np.array_equal(a[k], b[k]), (T, k)
        assert a["err_count"][0] == (1 if T > 9 else 0)
        print(f"T{T} {out_dtype}: allocation-free call equals the workspace call on every output")


def test_moe_noalloc_tiny_then_rejects_oversize(nv):
    """A small layer, then a call too large for the static buffer: rejected
    with NVFP4_ERR_WORKSPACE and nothing written; then the small layer again."""
    cfg = synth.TINY
    w = gpu_weights(nv, cfg)
    x = dev_bf16(synth.activations(cfg))
    ids, wts = synth.routing(cfg)
    ti, tw = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    a = _run(nv, cfg, w, x, ti, tw, cfg.T, torch.float32, noalloc=True)
    b = _run(nv, cfg, w, x, ti, tw, cfg.T, torch.float32, noalloc=False)
    assert all(np.array_equal(a[k], b[k]) for k in b)
    big = dataclasses.replace(cfg, T=1 << 16, name="tiny_big")
    xb = torch.zeros((big.T, cfg.H), dtype=torch.bfloat16, device="cuda:0")
    ib = torch.zeros((big.T, cfg.topk), dtype=torch.int32, device="cuda:0")
    wb = torch.ones((big.T, cfg.topk), dtype=torch.float32, device="cuda:0")
    yb = torch.full((big.T, cfg.H), 3.0, dtype=torch.float32, device="cuda:0")
    a2 = dev_f32(cfg.a2_gs)
    args = nv.moe_args(xb, ib, wb, w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"], a2, yb)
    assert nv.moe_workspace_size(args) > 64 << 20
    with pytest.raises(nv.Nvfp4Error) as ei:
        nv.moe_expert_ffn_noalloc(args, xb.device)
    assert ei.value.status == -3
    torch.cuda.synchronize()
    assert bool((yb == 3.0).all())
    c = _run(nv, cfg, w, x, ti, tw, cfg.T, torch.float32, noalloc=True)
    assert all(np.array_equal(c[k], b[k]) for k in b)
