"""Shared set-up for the MoE GPU tests: expert weights drawn by synth, then
quantized separately by each side (the GPU by nvfp4_quantize, the oracle by
its own quantizer) so no oracle input comes from the GPU path.  The weights
are drawn with torch's generator on cuda:0 for both sides (its CPU and GPU
streams differ) and copied to the host for the oracle."""
import numpy as np
import torch

import synth


def gpu_weights(nv, cfg, experts=None):
    """NVFP4 weights of all experts on cuda:0, quantized by the GPU path."""
    E, I, H = cfg.E, cfg.I, cfg.H
    dev = torch.device("cuda:0")
    w = dict(w1q=torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev),
             w1sf=torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=dev),
             w1gs=torch.empty(E, dtype=torch.float32, device=dev),
             w2q=torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev),
             w2sf=torch.empty((E, H, I // 16), dtype=torch.uint8, device=dev),
             w2gs=torch.empty(E, dtype=torch.float32, device=dev))
    for e in range(E) if experts is None else experts:
        w1, w2 = synth.expert_weights(cfg, e, device=dev)
        nv.quantize(w1, out=(w["w1q"][e], w["w1sf"][e], w["w1gs"][e:e + 1]))
        nv.quantize(w2, out=(w["w2q"][e], w["w2sf"][e], w["w2gs"][e:e + 1]))
    torch.cuda.synchronize()
    return w


def oracle_weights(orc, cfg, experts, device="cuda:0"):
    """Oracle-quantized weights for the listed experts (stacked in list
    order); the bf16 draws are regenerated from synth on `device`."""
    n = len(experts)
    E, I, H = cfg.E, cfg.I, cfg.H
    w = dict(w1q=np.zeros((n, 2 * I, H // 2), np.uint8), w1sf=np.zeros((n, 2 * I, H // 16), np.uint8),
             w1gs=np.zeros(n, np.float32), w2q=np.zeros((n, H, I // 2), np.uint8),
             w2sf=np.zeros((n, H, I // 16), np.uint8), w2gs=np.zeros(n, np.float32))
    for i, e in enumerate(experts):
        a, b = synth.expert_weights(cfg, int(e), device=device)
        a, b = synth.torch_bits(a), synth.torch_bits(b)
        w["w1gs"][i] = orc.global_scale(a)
        w["w1q"][i], w["w1sf"][i] = orc.quantize(a, w["w1gs"][i])
        w["w2gs"][i] = orc.global_scale(b)
        w["w2q"][i], w["w2sf"][i] = orc.quantize(b, w["w2gs"][i])
    return w


def oracle_tokens(orc, cfg, x_bits, ids, wts, tokens, device="cuda:0", want_pairs=True):
    """Oracle MoE for a subset of tokens, with only the experts they use."""
    tokens = np.asarray(tokens, np.int64)
    used = sorted(set(int(e) for e in ids[tokens].reshape(-1) if 0 <= e < cfg.E))
    remap = {e: i for i, e in enumerate(used)}
    ids_r = np.full_like(ids, -1)
    for t in tokens:
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            ids_r[t, j] = remap.get(e, -1)
    w = oracle_weights(orc, cfg, used, device=device)
    return orc.moe_tokens(x_bits, ids_r, wts, w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"],
                          w["w2gs"], cfg.a2_gs, tokens=tokens, want_pairs=want_pairs)
