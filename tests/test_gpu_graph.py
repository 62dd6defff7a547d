"""The C-ABI entry points under HIP graph capture: every replay must equal the
eager result (no hidden allocation, memset or host synchronization in the
launch sequence).  Replays are separated by eager work and synchronizations."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev_bf16, dev_f32, host
from moe_util import gpu_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import quantization_nvfp4_quantize_amd as nv
    return nv


def test_quantize_graph_replays(nv):
    x = dev_bf16(synth.quant_tensor(512, 7168, seed=8))
    ref = [host(t) for t in nv.quantize(x)]
    q = torch.empty_like(torch.from_numpy(ref[0])).cuda()
    sf = torch.empty_like(torch.from_numpy(ref[1])).cuda()
    g = torch.empty(1, dtype=torch.float32, device="cuda:0")
    nv.quantize(x, out=(q, sf, g))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.quantize(x, out=(q, sf, g))
    for _ in range(4):
        q.zero_()
        sf.zero_()
        g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(q), ref[0]) and np.array_equal(host(sf), ref[1])
        assert host(g)[0] == ref[2][0]
        _ = nv.quantize(x)  # eager work between replays


def test_moe_graph_replays(nv):
    cfg = synth.TINY
    w = gpu_weights(nv, cfg)
    x = dev_bf16(synth.activations(cfg))
    ids, wts = synth.routing(cfg)
    ti = torch.from_numpy(ids).cuda()
    tw = torch.from_numpy(wts).cuda()
    a2 = dev_f32(cfg.a2_gs)
    wl = (w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"])
    ref = host(nv.moe_expert_ffn(x, ti, tw, *wl, a2, out_dtype=torch.float32))
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda:0")
    args = nv.moe_args(x, ti, tw, *wl, a2, out)
    ws = torch.empty(nv.moe_workspace_size(args), dtype=torch.uint8, device="cuda:0")
    nv.moe_expert_ffn_raw(args, x.device, ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.moe_expert_ffn_raw(args, x.device, ws)
    for _ in range(4):
        out.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))
        _ = nv.moe_expert_ffn(x, ti, tw, *wl, a2)


def test_moe_graph_replays_aux_stream(nv):
    """A captured MoE layer whose mixed tiling forks its short tiles onto a
    second stream and joins them back: every replay equals the eager run."""
    import dataclasses
    counts = [266, 40, 289, 20]
    cfg = dataclasses.replace(synth.TINY, T=sum(counts), E=len(counts), topk=1, name="mixed")
    w = gpu_weights(nv, cfg)
    x = dev_bf16(synth.activations(cfg))
    rng = np.random.default_rng(5)
    ids = rng.permutation(np.repeat(np.arange(cfg.E), counts)).astype(np.int32)[:, None]
    ti = torch.from_numpy(ids).cuda()
    tw = torch.from_numpy(rng.uniform(0.5, 1.5, size=(cfg.T, 1)).astype(np.float32)).cuda()
    a2 = dev_f32(cfg.a2_gs)
    wl = (w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"])
    ref = host(nv.moe_expert_ffn(x, ti, tw, *wl, a2, out_dtype=torch.float32, tile_rows=288))
    stream = torch.cuda.Stream()
    evs = (torch.cuda.Event(), torch.cuda.Event())
    for e in evs:
        e.record()
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda:0")
    args = nv.moe_args(x, ti, tw, *wl, a2, out, tile_rows=288, aux=(stream, evs))
    ws = torch.empty(nv.moe_workspace_size(args), dtype=torch.uint8, device="cuda:0")
    nv.moe_expert_ffn_raw(args, x.device, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.moe_expert_ffn_raw(args, x.device, ws)
    for _ in range(4):
        out.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))
        _ = nv.moe_expert_ffn(x, ti, tw, *wl, a2, tile_rows=288)


def test_graph_keeps_its_workspace(nv):
    """A graph captured around calls that take their workspace from the
    binding (the dynamic-scale quantize and the MoE layer) keeps that
    workspace for itself: eager calls that need larger workspaces, and other
    tensors allocated and filled between the replays, do not disturb it."""
    x = dev_bf16(synth.quant_tensor(256, 7168, seed=12))
    ref = [host(t) for t in nv.quantize(x)]
    q = torch.empty(ref[0].shape, dtype=torch.uint8, device="cuda:0")
    sf = torch.empty(ref[1].shape, dtype=torch.uint8, device="cuda:0")
    g = torch.empty(1, dtype=torch.float32, device="cuda:0")
    cfg = synth.TINY
    w = gpu_weights(nv, cfg)
    xm = dev_bf16(synth.activations(cfg))
    ids, wts = synth.routing(cfg)
    ti, tw = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    wl = (w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"])
    a2 = dev_f32(cfg.a2_gs)
    yref = host(nv.moe_expert_ffn(xm, ti, tw, *wl, a2, out_dtype=torch.float32))
    y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda:0")
    nv.quantize(x, out=(q, sf, g))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.quantize(x, out=(q, sf, g))
        args = nv.moe_args(xm, ti, tw, *wl, a2, y)
        nv.moe_expert_ffn_raw(args, xm.device)
    import dataclasses
    for i in range(3):
        big = dev_bf16(synth.quant_tensor(1024 * (i + 2), 7168, seed=20 + i))
        nv.quantize(big)
        cbig = dataclasses.replace(cfg, T=512 * (i + 2), name="tiny_big")
        xb = dev_bf16(synth.activations(cbig))
        ib, wb = synth.routing(cbig)
        nv.moe_expert_ffn(xb, torch.from_numpy(ib).cuda(), torch.from_numpy(wb).cuda(), *wl, a2)
        junk = torch.full((1 << 24,), float(i + 7), dtype=torch.float32, device="cuda:0")
        q.zero_()
        sf.zero_()
        g.zero_()
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(q), ref[0]) and np.array_equal(host(sf), ref[1]), i
        assert host(g)[0] == ref[2][0], i
        assert np.array_equal(host(y).view(np.uint32), yref.view(np.uint32)), i
        del junk, big, xb


def test_moe_args_keep_their_tensors(nv):
    """A struct built from temporaries keeps them alive: the scale passed as
    a temporary is still the one the launch reads after other allocations
    have run."""
    import gc
    cfg = synth.TINY
    w = gpu_weights(nv, cfg)
    x = dev_bf16(synth.activations(cfg))
    ids, wts = synth.routing(cfg)
    ti, tw = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    wl = (w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"])
    y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda:0")
    used = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    args = nv.moe_args(x, ti, tw, *wl, dev_f32(cfg.a2_gs), y, a2_gs_out=used)
    gc.collect()
    junk = [torch.full((64,), 4.0, dtype=torch.float32, device="cuda:0") for _ in range(64)]
    nv.moe_expert_ffn_raw(args, x.device)
    torch.cuda.synchronize()
    assert host(used)[0] == np.float32(cfg.a2_gs)
    del junk
