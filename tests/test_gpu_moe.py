"""GPU parity of the full NVFP4 MoE expert FFN (moe_expert_ffn_nvfp4) against
the CPU oracle.

Gates (fp32-output mode): relative Frobenius error <= 1e-3 and cosine >=
0.9999 against the oracle's fp32 y.  The activation quantization (bytes and
global scale) is bit-exact; the L1 SwiGLU output meets the same tolerance;
the NVFP4 bytes of the L1 output (fused epilogue or separate pass, in every
flow) equal, bit for bit, the oracle's quantization of the GPU's own bf16
output under the same L1-output global scale.  bf16-output mode is compared with the oracle's
y rounded to bf16 (bounded loosely: bf16 rounding alone costs ~1.7e-3) and
with the fp32-output run of the same layer (its per-pair L2 rows go through
f16 with a power-of-two per row and 32 columns)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import cosine, dev_bf16, dev_f32, host, host_bits, rel_fro
from moe_util import gpu_weights, oracle_tokens, oracle_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import quantization_nvfp4_quantize_amd as nv
    return nv


# GEMM tilings: 32 (weights streamed), 256 (MFMA-bound), 288 (256-row tiles,
# each expert's last <= 64 rows on one or two 32-row tiles)
TILES = [32, 256, 288]


def _gpu_moe(nv, cfg, w, x_bits, ids, wts, out_dtype=torch.float32, tile_rows=0, dynamic=False,
             l1_unfused=False, paired=False):
    x = dev_bf16(x_bits)
    ti = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    tw = torch.from_numpy(np.ascontiguousarray(wts, np.float32)).cuda()
    a2 = None if dynamic else dev_f32(cfg.a2_gs)
    # paired: the 32-row tiles read row-paired copies of the weight scales
    ps = {}
    if paired and cfg.H % 1024 == 0:
        ps["w1_sf_paired"] = nv.pair_scales(w["w1sf"])
    if paired and cfg.I % 1024 == 0:
        ps["w2_sf_paired"] = nv.pair_scales(w["w2sf"])
    y, dbg = nv.moe_expert_ffn(x, ti, tw, w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"],
                               w["w2gs"], a2, out_dtype=out_dtype, debug=True,
                               tile_rows=tile_rows, l1_unfused=l1_unfused, **ps)
    torch.cuda.synchronize()
    return y, dbg


def _check_l1_bytes(orc, dbg, rows, g2):
    """The GPU's L1-output NVFP4 bytes on the listed pair rows == the
    oracle's quantization of the GPU's own bf16 rows under the scale g2."""
    c = host_bits(dbg["l1_c"])[rows]
    oq, osf = orc.quantize(c, np.float32(g2))
    gq, gsf = host(dbg["l1_q"])[rows], host(dbg["l1_sf"])[rows]
    bad = np.nonzero(gsf != osf)
    assert bad[0].size == 0, ("L1 scale bytes", bad[0].size, gsf[bad][:8], osf[bad][:8])
    bad = np.nonzero(gq != oq)
    assert bad[0].size == 0, ("L1 nibbles", bad[0].size, gq[bad][:8], oq[bad][:8])


def _check_tokens(nv, orc, cfg, w, x_bits, ids, wts, tokens, y, dbg, device="cuda:0", ref=None):
    if ref is None:
        ref = oracle_tokens(orc, cfg, x_bits, ids, wts, tokens, device=device)
    yg = host(y)[tokens]
    err, cos = rel_fro(yg, ref["y"]), cosine(yg, ref["y"])
    # activation quantization: bit-exact
    gx = orc.global_scale(x_bits)
    assert host(dbg["x_gs_out"])[0] == gx
    xq, xsf = orc.quantize(x_bits[tokens], gx)
    assert np.array_equal(host(dbg["xq"])[tokens], xq) and np.array_equal(host(dbg["xsf"])[tokens], xsf)
    # L1 compact output (pairs of the sampled tokens)
    k = cfg.topk
    pairs = (tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    valid = (ids[tokens] >= 0).reshape(-1) & (ids[tokens] < cfg.E).reshape(-1)
    cg = synth.bf16_values(host_bits(dbg["l1_c"])[pairs][valid])
    co = synth.bf16_values(ref["c"].reshape(-1, cfg.I)[valid])
    c_err, c_cos = rel_fro(cg, co), cosine(cg, co)
    # the L1 output's NVFP4 bytes == the oracle's quantization of the GPU's c
    assert host(dbg["a2_gs_out"])[0] == np.float32(cfg.a2_gs)
    _check_l1_bytes(orc, dbg, pairs[valid], cfg.a2_gs)
    # scale bytes that differ from the oracle's quantization of its own c
    flips = float((host(dbg["l1_sf"])[pairs][valid] != ref["a2_sf"].reshape(-1, cfg.I // 16)[valid]).mean())
    return err, cos, c_err, c_cos, flips


def _gate(err, cos, c_err, c_cos):
    assert err <= 1e-3 and cos >= 0.9999, (err, cos)
    assert c_err <= 1e-3 and c_cos >= 0.9999, (c_err, c_cos)


@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_tiny_full(nv, orc, tile_rows):
    cfg = synth.TINY
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), y, dbg)
    print("tiny: y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | sf flips %.2e" % res)
    _gate(*res[:4])
    assert host(dbg["err_count"])[0] == 0


def _check_bf16_vs_fp32(yb_dev, y32_dev):
    """A bf16-output run against the fp32-output run of the same layer: the
    bf16 path stores the per-pair L2 rows in f16 (relative error <= 2^-11
    each) before the combine, then rounds y to bf16 (<= 2^-9)."""
    yb = synth.bf16_values(host_bits(yb_dev))
    y32 = host(y32_dev)
    err = rel_fro(yb, y32)
    assert err <= 2e-3, err
    assert np.abs(yb - y32).max() <= 2.0 ** -8 * np.abs(y32).max()
    return err


@pytest.mark.parametrize("tile_rows", TILES)
@pytest.mark.parametrize("T", [64, 257])
def test_moe_bf16_output(nv, orc, tile_rows, T):
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, T=T, name=f"tiny{T}")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, _ = _gpu_moe(nv, cfg, w, x, ids, wts, out_dtype=torch.bfloat16, tile_rows=tile_rows)
    y32, _ = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    ref = oracle_tokens(orc, cfg, x, ids, wts, np.arange(cfg.T), device="cuda:0")
    yb = synth.bf16_values(host_bits(y))
    yo = synth.bf16_values(synth.bf16_bits(ref["y"]))
    err, cos = rel_fro(yb, yo), cosine(yb, yo)
    e32 = _check_bf16_vs_fp32(y, y32)
    print(f"T{T} tiles {tile_rows}: bf16 output vs bf16(oracle) rel_fro {err:.3e} cos {cos:.7f}; "
          f"vs the fp32-output run {e32:.3e}")
    assert err <= 5e-3 and cos >= 0.9999


@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_bf16_rows_extreme_weights(nv, tile_rows):
    """Routing weights from 2^-100 to 2^100 (and one token with all-zero
    weights), so that rows of one tile differ by up to 2^200: every row keeps
    its own f16 exponent, so every token of the bf16-output run matches the
    fp32-output run to bf16 precision."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, T=257, name="tiny257")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    exps = np.array([-100, -60, -20, 0, 20, 60, 100])
    wts = (wts * np.exp2(exps[np.arange(cfg.T) % len(exps)])[:, None]).astype(np.float32)
    wts[5] = 0.0
    yb, _ = _gpu_moe(nv, cfg, w, x, ids, wts, out_dtype=torch.bfloat16, tile_rows=tile_rows)
    y32, _ = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    yb = synth.bf16_values(host_bits(yb)).astype(np.float64)
    y32 = host(y32).astype(np.float64)
    assert np.all(yb[5] == 0.0) and np.all(y32[5] == 0.0)
    num = np.linalg.norm(yb - y32, axis=1)
    den = np.linalg.norm(y32, axis=1)
    rel = num[den > 0] / den[den > 0]
    print(f"tiles {tile_rows}: worst per-token rel error {rel.max():.3e}")
    assert rel.max() <= 4e-3


@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_invalid_ids_and_duplicates(nv, orc, tile_rows):
    cfg = synth.TINY
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    ids = ids.copy()
    ids[3, 0] = -1
    ids[7, 1] = cfg.E
    ids[11, 1] = 99
    ids[20, 1] = ids[20, 0]  # the same expert twice for one token
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    assert host(dbg["err_count"])[0] == 3
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), y, dbg)
    _gate(*res[:4])


@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_single_expert_topk1(nv, orc, tile_rows):
    """E = 1, k = 1, w = 1: the MoE reduces to one dense expert FFN."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, E=1, topk=1, name="dense")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids = np.zeros((cfg.T, 1), np.int32)
    wts = np.ones((cfg.T, 1), np.float32)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), y, dbg)
    _gate(*res[:4])


@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_ragged_token_counts(nv, orc, tile_rows):
    """Token counts that leave ragged row tiles (and an empty expert)."""
    import dataclasses
    for T in (1, 3, 130, 257):
        cfg = dataclasses.replace(synth.TINY, T=T, name=f"tiny{T}")
        w = gpu_weights(nv, cfg)
        x = synth.activations(cfg)
        ids, wts = synth.routing(cfg)
        y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
        res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(T), y, dbg)
        _gate(*res[:4])


@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_largest_expert_count_and_topk(nv, orc, tile_rows):
    """The largest supported routing: E = 512 experts and top-32, every token
    against the oracle."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, T=40, E=512, topk=32, name="e512k32")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    assert host(dbg["err_count"])[0] == 0
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), y, dbg)
    print("E512 top-32: y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | sf flips %.2e" % res)
    _gate(*res[:4])


@pytest.mark.parametrize("topk", [2, 32])
def test_moe_bf16_combine_skipped_pairs(nv, orc, topk):
    """The bf16-output combine (f16 per-pair rows) with skipped pairs (invalid
    expert ids) at top-2 (all k rows loaded before the sum) and at top-32
    (the loop for k above 8): against the fp32-output run of the same
    routing, and against the oracle."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, T=40, E=512 if topk == 32 else 8, topk=topk, name=f"bf16k{topk}")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    ids = ids.copy()
    ids[3, 0] = -1
    ids[7, topk - 1] = cfg.E
    ids[11, :] = -1  # a token without any valid pair: y = 0
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, out_dtype=torch.bfloat16)
    y32, _ = _gpu_moe(nv, cfg, w, x, ids, wts)
    assert host(dbg["err_count"])[0] == 2 + topk
    assert np.all(host_bits(y)[11] == 0)
    _check_bf16_vs_fp32(y, y32)
    ref = oracle_tokens(orc, cfg, x, ids, wts, np.arange(cfg.T), device="cuda:0")
    yb = synth.bf16_values(host_bits(y))
    yo = synth.bf16_values(synth.bf16_bits(ref["y"]))
    assert rel_fro(yb, yo) <= 5e-3 and cosine(yb, yo) >= 0.9999


@pytest.mark.parametrize("H,I", [(1280, 768), (1024, 512), (256, 1280), (1280, 1024)])
def test_moe_skinny_k_schedules(nv, orc, H, I):
    """32-row tiles with reduction lengths whose 256-K super-steps leave a
    partial group of four (H 1280: five, I 768: three), exactly one group
    (H 1024) and two groups and a half (I 1280), all against the oracle;
    H 1280 I 1024 gives the L2 an odd number of column tiles."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, T=40, H=H, I=I, E=4, name=f"mid{H}x{I}", a2_gs=4.0 / 2688.0)
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=32)
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), y, dbg)
    print(f"H{H} I{I}: y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | sf flips %.2e" % res)
    _gate(*res[:4])


@pytest.mark.parametrize("H,I", [(6400, 256), (256, 3072), (3328, 3328)])
def test_moe_skinny_tail_split(nv, orc, H, I):
    """32-row tiles where the launch's last items are split along K into
    pieces whose partial sums the last piece adds: with a handful of items per
    XCD every item is such a tail item.  H 6400 splits each L1 item into four
    pieces of 6, 6, 6 and 7 super-steps; I 3072 splits each L2 item in two;
    3328 splits both GEMMs' items into 6 + 7.  Against the oracle, and the
    same bytes on a second call (the arrival counters start from zero again)."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, T=40, H=H, I=I, E=4, name=f"split{H}x{I}", a2_gs=4.0 / 2688.0)
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=32)
    y2, _ = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=32)
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), y, dbg)
    print(f"H{H} I{I}: y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | sf flips %.2e" % res)
    _gate(*res[:4])


@pytest.mark.parametrize("tile_rows", TILES)
@pytest.mark.parametrize("flow", [1, "interleaved"])
def test_moe_unfused_static_matches_fused(nv, orc, tile_rows, flow):
    """The unfused flows with the supplied scale -- compact bf16 L1 output
    then a separate quantization pass, or the interleaved [SiLU(gate),
    SwiGLU] output then a deinterleave + quantize pass (the pages' earlier
    flow) -- against the oracle: y in fp32 mode within the GEMM gate, the L1
    output within the same gate, and its NVFP4 bytes equal to the oracle's
    quantization of the GPU's own bf16 rows.  They also reproduce the fused
    epilogue's bytes and y exactly."""
    cfg = synth.TINY
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    ya, da = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    yb, db = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows, l1_unfused=flow)
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), yb, db)
    print(f"flow {flow} tiles {tile_rows}: y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | "
          "sf flips %.2e" % res)
    _gate(*res[:4])
    assert host(db["a2_gs_out"])[0] == np.float32(cfg.a2_gs)
    assert host(da["a2_gs_out"])[0] == np.float32(cfg.a2_gs)
    assert np.array_equal(host_bits(da["l1_c"]), host_bits(db["l1_c"]))
    for key in ("l1_q", "l1_sf"):
        assert np.array_equal(host(da[key]), host(db[key])), key
    assert np.array_equal(host(ya).view(np.uint32), host(yb).view(np.uint32))


@pytest.mark.parametrize("tile_rows", TILES)
@pytest.mark.parametrize("shape", ["tiny", "mid"])
def test_moe_dynamic_l1_scale(nv, orc, tile_rows, shape):
    """Dynamic L1-output global scale (a2_gs NULL: amax of the valid pairs'
    bf16 SwiGLU rows / 2688, then a separate quantization pass) against the
    oracle's dynamic flow, with two skipped pairs whose rows must not count."""
    import dataclasses
    cfg = synth.TINY if shape == "tiny" else dataclasses.replace(synth.TINY, T=40, H=1280, I=768, E=4,
                                                                 name="mid1280x768")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    ids = ids.copy()
    ids[3, 0], ids[5, 1] = -1, cfg.E
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows, dynamic=True)
    used = sorted(set(int(e) for e in ids.reshape(-1) if 0 <= e < cfg.E))
    ow = oracle_weights(orc, cfg, used)
    remap = {e: i for i, e in enumerate(used)}
    ids_r = np.vectorize(lambda e: remap.get(int(e), -1))(ids).astype(np.int32)
    ref = orc.moe_tokens_dynamic(x, ids_r, wts, ow["w1q"], ow["w1sf"], ow["w1gs"], ow["w2q"], ow["w2sf"],
                                 ow["w2gs"])
    g_gpu = host(dbg["a2_gs_out"])[0]
    rel = abs(float(g_gpu) / float(ref["a2_gs"]) - 1.0)
    print(f"{shape}: dynamic a2_gs gpu {g_gpu!r} oracle {ref['a2_gs']!r} (rel {rel:.2e})")
    assert rel <= 2.0 ** -8
    # the GPU's scale is the oracle's global scale of the GPU's own valid
    # bf16 rows (skipped pairs excluded), bit for bit, and its bytes are the
    # oracle's quantization of those rows under that scale
    valid = ((ids >= 0) & (ids < cfg.E)).reshape(-1)
    rows = np.nonzero(valid)[0]
    assert g_gpu == orc.global_scale(host_bits(dbg["l1_c"])[rows])
    _check_l1_bytes(orc, dbg, rows, g_gpu)
    yg = host(y)
    err, cos = rel_fro(yg, ref["y"]), cosine(yg, ref["y"])
    print(f"{shape}: y rel_fro {err:.3e} cos {cos:.7f}")
    assert err <= 1e-3 and cos >= 0.9999


@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_many_route_groups(nv, orc, tile_rows):
    """Enough pairs (P = 9000) for the grouping to run over several
    workgroups (3 x 4096 pairs), with skipped ids spread over them, against
    the oracle on every token."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, T=4500, name="tiny4500")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    ids = ids.copy()
    ids[[5, 2100, 4400], [0, 1, 0]] = [-1, cfg.E, 77]
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    assert host(dbg["err_count"])[0] == 3
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), y, dbg)
    _gate(*res[:4])


@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_deterministic(nv, tile_rows):
    cfg = synth.TINY
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    a, _ = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    b, _ = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))


def test_moe_tile_modes_agree(nv):
    """The 32-row, the 256-row and the mixed GEMM tiles group K differently inside their
    MFMAs, but on this workload the fp32 sums of the exact NVFP4 products do
    not round (the products share a fine grid and the sums stay within 24
    significant bits), so their results are bit-identical (decode shape: every
    intermediate and the output)."""
    cfg = synth.DEC
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    ya, da = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=32)
    for tr in (256, 288):
        yb, db = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tr)
        assert np.array_equal(host_bits(da["l1_c"]), host_bits(db["l1_c"])), tr
        for key in ("l1_q", "l1_sf"):
            assert np.array_equal(host(da[key]), host(db[key])), (tr, key)
        assert np.array_equal(host(ya).view(np.uint32), host(yb).view(np.uint32)), tr


def _aux():
    stream = torch.cuda.Stream()
    evs = (torch.cuda.Event(), torch.cuda.Event())
    for e in evs:
        e.record()  # creates the underlying event
    return stream, evs


@pytest.mark.parametrize("flow", ["fused", "unfused", "interleaved", "dynamic"])
def test_moe_mixed_aux_stream(nv, flow):
    """The mixed tiling with the short tiles on a second stream gives the
    same bytes as on one stream, in every flow."""
    import dataclasses
    counts = [266, 544, 289, 255, 32, 0]
    cfg = dataclasses.replace(synth.TINY, T=sum(counts), E=len(counts), topk=1, name="mixed")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    rng = np.random.default_rng(11)
    ids = rng.permutation(np.repeat(np.arange(cfg.E), counts)).astype(np.int32)[:, None]
    wts = rng.uniform(0.5, 1.5, size=(cfg.T, 1)).astype(np.float32)
    xd = dev_bf16(x)
    ti = torch.from_numpy(ids).cuda()
    tw = torch.from_numpy(wts).cuda()
    a2 = None if flow == "dynamic" else dev_f32(cfg.a2_gs)
    unf = {"fused": False, "unfused": 1, "interleaved": 2, "dynamic": False}[flow]
    wl = (w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"])
    for out_dtype in (torch.float32, torch.bfloat16):
        ya, da = nv.moe_expert_ffn(xd, ti, tw, *wl, a2, out_dtype=out_dtype, debug=True, tile_rows=288,
                                   l1_unfused=unf)
        yb, db = nv.moe_expert_ffn(xd, ti, tw, *wl, a2, out_dtype=out_dtype, debug=True, tile_rows=288,
                                   l1_unfused=unf, aux=_aux())
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(da["l1_c"]), host_bits(db["l1_c"])), (flow, out_dtype)
        for key in ("l1_q", "l1_sf", "a2_gs_out"):
            assert np.array_equal(host(da[key]), host(db[key])), (flow, out_dtype, key)
        assert np.array_equal(host_bits(ya) if out_dtype == torch.bfloat16 else host(ya).view(np.uint32),
                              host_bits(yb) if out_dtype == torch.bfloat16 else host(yb).view(np.uint32))


def test_moe_mixed_tiles_remainders(nv, orc):
    """The mixed tiling on expert row counts chosen around its boundaries:
    256 + 10 (one 256-row tile and a 10-row short tile), 512 + 32 (two and a
    32-row short tile), 256 + 33 and 256 + 64 (a 256-row tile and two short
    tiles), 256 + 65 (a 65-row block stays on a 256-row tile), 255 and 32
    (one tile each), 0 (no tile): every token against the oracle, and
    bit-identical to the 256-row tiling."""
    import dataclasses
    counts = [266, 544, 289, 320, 321, 255, 32, 0]
    cfg = dataclasses.replace(synth.TINY, T=sum(counts), E=len(counts), topk=1, name="mixed")
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    rng = np.random.default_rng(7)
    ids = rng.permutation(np.repeat(np.arange(cfg.E), counts)).astype(np.int32)[:, None]
    wts = rng.uniform(0.5, 1.5, size=(cfg.T, 1)).astype(np.float32)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=288)
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), y, dbg)
    print("mixed: y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | sf flips %.2e" % res)
    _gate(*res[:4])
    yb, db = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=256)
    assert np.array_equal(host_bits(dbg["l1_c"]), host_bits(db["l1_c"]))
    assert np.array_equal(host(y).view(np.uint32), host(yb).view(np.uint32))


_ORACLE_CACHE = {}


def _oracle_cached(orc, cfg, x, ids, wts, tokens):
    """The oracle's result for a full-size workload's token sample, computed
    once per module (it does not depend on the GPU's tiling)."""
    key = (cfg.name, tuple(int(t) for t in tokens))
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = oracle_tokens(orc, cfg, x, ids, wts, tokens, device="cuda:0")
    return _ORACLE_CACHE[key]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tile_rows", TILES)
def test_moe_decode_config_sampled(nv, orc, tile_rows):
    """Decode-shaped layer (T128 H7168 I2048 E256 top-8, Zipf routing), full
    GPU run, every token against the oracle (all 186 touched experts, from
    the hottest with 111 rows to the many with a single row)."""
    cfg = synth.DEC
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows)
    tokens = np.arange(cfg.T)
    ref = _oracle_cached(orc, cfg, x, ids, wts, tokens)
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, tokens, y, dbg, ref=ref)
    print("decode: y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | sf flips %.2e" % res)
    _gate(*res[:4])
    # the same layer with the row-paired weight scales on its 32-row tiles
    # (H and I multiples of 1024; the L1's split pieces start 7, 14 and 21
    # super-steps in, inside a scale line): the same bytes
    yp, dbgp = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=tile_rows, paired=True)
    _assert_same(y, dbg, yp, dbgp)


@pytest.mark.timeout(900)
def test_moe_prefill_config_sampled(nv, orc):
    """Prefill-shaped layer (T16384, uniform top-8) in the mixed tiling, full
    GPU run; against the oracle on tokens chosen from the stable grouping:
    a row on each 32-row short tile of every expert that has them (125
    experts, 142 tiles), rows 255, 256 and 257 of eight experts' 256-row
    tiles, and the first, middle and last token."""
    from moe_util import boundary_tokens
    cfg = synth.PRE
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=288)
    tokens, info = boundary_tokens(ids, cfg.E, cfg.topk, extra=(0, cfg.T // 2, cfg.T - 1))
    # every short tile (142, of 125 experts) has a sampled row on it
    assert len(info["short_experts"]) == 125 and info["edge"].size >= 20, {k: len(v) for k, v in info.items()}
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, tokens, y, dbg, device="cuda:0")
    print(f"prefill ({tokens.size} tokens: {info['short'].size} on short tiles, {info['edge'].size} at "
          "256-row edges): y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | sf flips %.2e" % res)
    _gate(*res[:4])
    # row-paired weight scales on the short tiles: the same bytes
    yp, dbgp = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=288, paired=True)
    _assert_same(y, dbg, yp, dbgp)
    del dbg, dbgp
    # the bench's configuration (automatic tiling, bf16 output through f16
    # pair rows) matches this fp32-output run on every token
    yb, _ = _gpu_moe(nv, cfg, w, x, ids, wts, out_dtype=torch.bfloat16)
    print("prefill bf16 output vs the fp32-output run: rel_fro %.3e" % _check_bf16_vs_fp32(yb, y))


def _assert_same(y, dbg, yb, dbgb):
    """Bit-identical outputs and L1 intermediates of two runs."""
    assert np.array_equal(host(y).view(np.uint32), host(yb).view(np.uint32))
    assert np.array_equal(host_bits(dbg["l1_c"]), host_bits(dbgb["l1_c"]))
    for key in ("l1_q", "l1_sf", "xq", "xsf"):
        assert np.array_equal(host(dbg[key]), host(dbgb[key])), key


@pytest.mark.parametrize("H,I", [(1024, 3072), (3072, 1024)])
def test_moe_paired_scales_split(nv, orc, H, I):
    """Row-paired weight scales (nvfp4_pair_scales) on the 32-row tiles,
    where the launch's last items are split along K into two pieces of 6
    super-steps, the second starting inside a 128-byte scale line (I 3072:
    the L2's items; H 3072: the L1's): the same bytes as with the plain
    scales, and against the oracle."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, T=40, H=H, I=I, E=4, name=f"pair{H}x{I}", a2_gs=4.0 / 2688.0)
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=32)
    yp, dbgp = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=32, paired=True)
    _assert_same(y, dbg, yp, dbgp)
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, np.arange(cfg.T), yp, dbgp)
    print(f"paired H{H} I{I}: y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | sf flips %.2e" % res)
    _gate(*res[:4])


def test_moe_paired_scales_mixed(nv, orc):
    """The mixed tiling with row-paired scales: its short tiles read them,
    its 256-row tiles the plain ones; the same bytes as with the plain scales
    alone, and against the oracle on tokens of every short tile."""
    import dataclasses
    from moe_util import boundary_tokens
    cfg = dataclasses.replace(synth.TINY, T=1100, H=1024, I=1024, E=8, name="pairmixed", a2_gs=4.0 / 2688.0)
    w = gpu_weights(nv, cfg)
    x = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    y, dbg = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=288)
    yp, dbgp = _gpu_moe(nv, cfg, w, x, ids, wts, tile_rows=288, paired=True)
    _assert_same(y, dbg, yp, dbgp)
    tokens, info = boundary_tokens(ids, cfg.E, cfg.topk, n_edge_experts=2, extra=(0, cfg.T - 1))
    assert info["short"].size > 0
    res = _check_tokens(nv, orc, cfg, w, x, ids, wts, tokens, yp, dbgp)
    print(f"paired mixed ({tokens.size} tokens): y rel_fro %.3e cos %.7f | c rel_fro %.3e cos %.7f | "
          "sf flips %.2e" % res)
    _gate(*res[:4])


def test_moe_empty(nv):
    cfg = synth.TINY
    w = gpu_weights(nv, cfg, experts=[])
    x = torch.zeros((0, cfg.H), dtype=torch.bfloat16, device="cuda:0")
    ti = torch.zeros((0, cfg.topk), dtype=torch.int32, device="cuda:0")
    tw = torch.zeros((0, cfg.topk), dtype=torch.float32, device="cuda:0")
    y = nv.moe_expert_ffn(x, ti, tw, w["w1q"], w["w1sf"], w["w1gs"], w["w2q"], w["w2sf"], w["w2gs"],
                          dev_f32(cfg.a2_gs))
    torch.cuda.synchronize()
    assert y.shape == (0, cfg.H)
