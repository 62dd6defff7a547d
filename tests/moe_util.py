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


def expert_rows(ids, E):
    """The stable grouping of (token, expert) pairs by expert: for expert e,
    the pair ids p = t * k + j routed to it, in increasing order (its rows
    0, 1, ... in the grouped GEMMs).  Pairs with an id outside [0, E) are
    skipped.  Host-side test selection only."""
    flat = np.asarray(ids).reshape(-1)
    order = np.argsort(flat, kind="stable")
    fs = flat[order]
    return {e: order[np.searchsorted(fs, e, "left"):np.searchsorted(fs, e, "right")] for e in range(E)}


def boundary_tokens(ids, E, k, tile=256, short=64, short_tile=32, n_edge_experts=8, seed=0, extra=()):
    """Tokens chosen so that the oracle comparison reaches every kind of row
    of the mixed tiling at full size: for each expert whose last block of at
    most `short` rows goes on `short_tile`-row tiles, the token of a seeded
    row of each of those tiles (of its last row for every eighth such
    expert); for `n_edge_experts` experts with more than
    `tile` + 1 rows, the tokens of rows tile - 1, tile and tile + 1; the
    tokens of each expert's first row for experts with at most `short` rows
    in all; plus `extra`.  Returns (sorted token ids, dict of what each
    group holds)."""
    rows = expert_rows(ids, E)
    short_tok, edge_tok, small_tok, short_e = [], [], [], []
    edge_experts = [e for e in range(E) if rows[e].size > tile + 1]
    rng = np.random.Generator(np.random.PCG64(seed))
    if len(edge_experts) > n_edge_experts:
        edge_experts = sorted(rng.choice(edge_experts, n_edge_experts, replace=False).tolist())
    for e in range(E):
        n = rows[e].size
        rem = n % tile
        if n > tile and 0 < rem <= short:
            # a seeded row of each short tile; its last row for every 8th expert
            last = len(short_e) % 8 == 0
            for t0 in range(0, rem, short_tile):
                t1 = min(rem, t0 + short_tile)
                r = n - rem + (t1 - 1 if last else t0 + int(rng.integers(t1 - t0)))
                short_tok.append(rows[e][r] // k)
            short_e.append(e)
        if 0 < n <= short:
            small_tok.append(rows[e][0] // k)
    for e in edge_experts:
        edge_tok += [rows[e][tile - 1] // k, rows[e][tile] // k, rows[e][tile + 1] // k]
    toks = np.unique(np.array(list(short_tok) + list(edge_tok) + list(small_tok) + list(extra), np.int64))
    info = dict(short=np.unique(short_tok), edge=np.unique(edge_tok), small=np.unique(small_tok),
                edge_experts=edge_experts, short_experts=short_e)
    return toks, info
