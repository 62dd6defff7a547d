"""Benchmark of the NVFP4 MoE expert-FFN hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs quant,expert,dense,mx,dec,pre,tiny] [--no-cpu] [--no-modes]

Prints one JSON line.  `value` is the prefill-shaped MoE layer (T16384 H7168
I2048 E256 top-8: activation global scale + quantize, grouping, L1 GEMM with
fused SwiGLU -> bf16 -> NVFP4, L2 GEMM, weighted combine) in algorithmic
TFLOP/s (6 * P * H * I per step).  Other legs, reported alongside:
  quantize  8192 x 7168 bf16 -> NVFP4, supplied global scale (HBM-bound,
            2.5625 algorithmic bytes per element), inputs rotated over five
            copies (> 256 MiB Infinity Cache); also dynamic scale, dequantize
  expert    single-expert L1 stage M4096 K7168 N 2x2048
  dense     dense NVFP4 linear M4096 K4096 N16384 (quantize x + GEMM, bf16 out)
  mx        the separately labelled MXFP4 variant (OCP MX v1.0 format, E8M0
            scale per 32 elements) on the scaled FP4 MFMA: quantize
            8192 x 7168 and the dense linear M4096 K4096 N16384, against the
            FP4 MFMA peak
  dec       decode-shaped layer T128 (Zipf routing; weight-streaming bound)
  prefill_unfused / prefill_interleaved / prefill_dynamic  the same prefill
            layer with the L1 output written as bf16 and quantized in a
            separate pass: compact with the supplied scale (the fusion's
            saving), interleaved [SiLU(gate), SwiGLU] groups with a
            deinterleave + quantize pass (the pages' earlier flow), or
            compact with the dynamic amax / 2688 scale (and y's distance from
            the fused run)
  prefill_aux  the fused prefill layer with the mixed tiling's 32-row short
            tiles on a second stream, alongside the 256-row tiles
  tiny      the small MoE layer T64 H256 I128 E8 top-2 (launch-latency bound)
Timing: W untimed warmups, then K timed steps.  quantize, expert, dense and mx
replay a HIP graph of K launches between two events (no host gaps), then 50
more replays each between its own events for a median.  The MoE legs warm up
for W layers, and a short layer for more, up to ~100 ms of work while the
clock settles; then they run K layers eagerly between two events, then at
least 10 (prefill) or 50 (decode, tiny) layers with an event between
consecutive layers for a median, then K layers with the library's stage
events (HIP events between its stages on the same stream), which give every
stage's duration (the L1 GEMM's feeds `roofline.achieved`).
cpu_baseline: the CPU oracle, timed in the same run on this host's cores
(the CPUs this process may use, at most 16), on bounded samples: the prefill
layer (top level, the unit of `value`), and per leg the decode layer, the
quantize rows, the single-expert stage rows and the whole tiny layer.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 MFMA
FP4_PEAK_TFLOPS = 10100.0  # dense FP4 (scaled f8f6f4) MFMA
# intervals between the library's 9 stage events; l1_main / l2_main are the
# GEMM launches over the main tile list (256-row tiles in the prefill), and
# l1_rest / l2_rest the 32-row short tiles of the mixed tiling (and, in the
# unfused flows, the separate quantization pass)
STAGE_EVENTS = 9
STAGES = ["global_scale", "quantize_x", "route", "l1_main", "l1_rest", "l2_main", "l2_rest", "combine"]


def _ev():
    e = torch.cuda.Event(enable_timing=True)
    e.record()  # materialize the underlying hipEvent_t
    return e


def graph_time(fn, steps, warmup, replays=50, stats=None, warm_replays=3):
    """ms per call of fn(i): one replay of a graph of `steps` calls between
    two events (the mean), then `replays` more replays each between its own
    two events, whose median per-call time goes to stats["ms_median"].
    Before the timed replay, `warm_replays` untimed replays run back to back:
    a kernel trace showed the per-call time of an MFMA-bound stage still
    falling through the first two replays after the warm-up calls (211, then
    205 -> 189, then 181 us per call) while the clock settles."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    torch.cuda.synchronize()
    for _ in range(warm_replays):
        g.replay()
    torch.cuda.synchronize()
    a, b = _ev(), _ev()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    if stats is not None:
        evs = [(_ev(), _ev()) for _ in range(replays)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        per = [e0.elapsed_time(e1) / steps for e0, e1 in evs]
        stats.update(ms_median=float(np.median(per)), median_of=f"{replays} graph replays of {steps} calls")
    return ms


# ------------------------------------------------------------------ quantize
def bench_quantize(nv, steps, warmup):
    import synth
    M, K = synth.QUANT_SHAPE
    n = M * K
    dev = torch.device("cuda:0")
    bits = synth.quant_tensor()
    x0 = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    ncopy = 5
    xs = [x0] + [x0.clone() for _ in range(ncopy - 1)]
    outs = [(torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
             torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
             torch.empty(1, dtype=torch.float32, device=dev)) for _ in range(ncopy)]
    _, _, g = nv.quantize(x0)
    g = g.clone()
    deq = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(ncopy)]
    qst = {}
    q_ms = graph_time(lambda i: nv.quantize(xs[i % ncopy], g, out=outs[i % ncopy]), steps, warmup, stats=qst)
    d_ms = graph_time(lambda i: nv.quantize(xs[i % ncopy], None, out=outs[i % ncopy]), steps, warmup)
    dq_ms = graph_time(lambda i: nv.dequantize(outs[i % ncopy][0], outs[i % ncopy][1], g,
                                               out=deq[i % ncopy]), steps, warmup)
    qbytes = 2 * n + n // 2 + n // 16
    return dict(shape=[M, K], algorithmic_bytes=qbytes, quantize_ms=q_ms,
                quantize_GBps=qbytes / q_ms / 1e6, quantize_frac=qbytes / q_ms / 1e6 / HBM_PEAK_GBS,
                quantize_ms_median=qst["ms_median"], median_of=qst["median_of"],
                quantize_dynamic_ms=d_ms,
                quantize_dynamic_GBps=(qbytes + 2 * n) / d_ms / 1e6,
                dequantize_ms=dq_ms, dequantize_GBps=(n // 2 + n // 16 + 2 * n) / dq_ms / 1e6)


def bench_copy(steps):
    """A plain 512 MiB device-to-device copy (torch copy_, the runtime's copy
    kernel), launched eagerly `steps` times: the reference whose FETCH_SIZE
    and WRITE_SIZE counters calibrate the HBM traffic of the other kernels.
    Profile it in a run of its own (--legs copy), since the other legs also
    copy tensors with the same kernel."""
    dev = torch.device("cuda:0")
    n = 512 << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0, t1 = _ev(), _ev()
    t0.record()
    for _ in range(steps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    return dict(bytes_each_way=n, ms=ms, GBps=2 * n / ms / 1e6)


# ------------------------------------------------------------------ HBM traffic
# Kernel -> the sources it is compiled from.  Traffic taken by rocprofv3 is
# reported only while these files are byte-identical to the profiled ones.
KERNEL_SOURCES = {
    "l1_gemm_swiglu_quant_kernel": ["gemm.hip", "gemm_common.hpp", "nvfp4_device.hpp", "launch.hpp"],
    "l2_gemm_kernel": ["gemm.hip", "gemm_common.hpp", "nvfp4_device.hpp", "launch.hpp"],
    "quantize_kernel": ["quantize.hip", "nvfp4_device.hpp", "launch.hpp"],
    "dequantize_kernel": ["quantize.hip", "nvfp4_device.hpp", "launch.hpp"],
    "combine_kernel": ["moe.hip", "launch.hpp"],
    "combine_f16_kernel": ["moe.hip", "launch.hpp"],
    "amax_partial_kernel": ["quantize.hip", "nvfp4_device.hpp", "launch.hpp"],
    "l1_skinny_kernel": ["gemm_skinny.hip", "gemm_common.hpp", "nvfp4_device.hpp", "launch.hpp"],
    "l2_skinny_kernel": ["gemm_skinny.hip", "gemm_common.hpp", "nvfp4_device.hpp", "launch.hpp"],
    "mx_gemm_kernel": ["mxfp4.hip", "gemm_common.hpp", "nvfp4_device.hpp", "launch.hpp"],
    "mx_quantize_kernel": ["mxfp4.hip", "gemm_common.hpp", "nvfp4_device.hpp", "launch.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
# the dominant kernel of the headline workload: the prefill L1 GEMM (f16 activations)
ROOFLINE_KERNEL = "l1_gemm_swiglu_quant_kernel<false>"


def _code_only(text):
    """C++ source without comments and with whitespace collapsed, so that a
    comment-only edit does not mark a profile stale."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[_base(kernel)]:
        with open(os.path.join(ROOT, "quantization_nvfp4_quantize_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` in the bench leg `workload` from the
    committed counter summary, or None when absent or when the kernel's
    sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("traffic-json: "):
            d = json.loads(line[len("traffic-json: "):])
            if d.get("kernel") == kernel and d.get("workload") == workload and d.get("src") == source_hash(kernel):
                return d["bytes_per_launch"]
    return None


def _demangle_last(name):
    """Innermost identifier of an Itanium-mangled function name (_Z...), with
    its template arguments when they are bools or integers ("<true, 8>")."""
    i = 3 if name.startswith("_ZN") else 2
    last = name
    while i < len(name) and name[i].isdigit():
        j = i
        while name[j].isdigit():
            j += 1
        n = int(name[i:j])
        last = name[j:j + n]
        i = j + n
    if i < len(name) and name[i] == "I":
        import re
        m = re.match(r"I((?:L[bi]\d+E)+)E", name[i:])
        if m:
            args = re.findall(r"L([bi])(\d+)E", m.group(1))
            last += "<" + ", ".join(("true" if v == "1" else "false") if t == "b" else v for t, v in args) + ">"
    return last


def _short_name(name):
    """Kernel name without namespace and parameters, keeping template
    arguments: l1_gemm_swiglu_quant_kernel<false>."""
    if name.startswith("_Z"):
        return _demangle_last(name)
    base = name.replace("(anonymous namespace)::", "").replace("void ", "")
    base = base.split("(")[0]
    targs = ""
    if "<" in base:
        base, targs = base.split("<", 1)
        targs = "<" + targs
    return base.split("::")[-1].strip() + targs


def _base(kernel):
    """A kernel's name without its template arguments."""
    return kernel.split("<")[0]


def _read_counters(path, counter):
    import csv
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                rows.append((_short_name(r["Kernel_Name"]), int(r["Grid_Size"]), float(r["Counter_Value"])))
    return rows


def _split_legs(items):
    """'leg=path' arguments -> [(leg, path)]."""
    out = []
    for it in items:
        leg, _, path = it.partition("=")
        out.append((leg, path))
    return out


def traffic_summary(copy_fetch, copy_write, legs, cmds):
    """Markdown summary of counter runs (FETCH_SIZE and WRITE_SIZE in KiB per
    dispatch, one pair of runs per bench leg: legs = [(leg, fetch_csv,
    write_csv)]), each scaled by what the same counter reads for the 512 MiB
    copy of known size; one traffic-json line per (leg, kernel, grid)."""
    import collections
    n_copy = 512 << 20
    cf = [v for k, g, v in _read_counters(copy_fetch, "FETCH_SIZE") if _base(k) == "__amd_rocclr_copyBuffer"]
    cw = [v for k, g, v in _read_counters(copy_write, "WRITE_SIZE") if _base(k) == "__amd_rocclr_copyBuffer"]
    f_fac = n_copy / (np.median(cf) * 1024.0)
    w_fac = n_copy / (np.median(cw) * 1024.0)
    agg = collections.defaultdict(lambda: [[], []])
    for leg, fetch, write in legs:
        for i, (path, ctr) in enumerate(((fetch, "FETCH_SIZE"), (write, "WRITE_SIZE"))):
            for k, g, v in _read_counters(path, ctr):
                if _base(k) in KERNEL_SOURCES:
                    agg[(leg, k, g)][i].append(v)
    out = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated)", "",
           "Commands (from the repository root, on one MI355X; R = repository root; LEG is each of the",
           "bench legs listed in the table, one pair of counter runs per leg):", ""]
    out += ["    " + c for c in cmds]
    out += ["",
            f"Calibration: a 512 MiB device copy reads FETCH_SIZE {np.median(cf):.0f} KiB and "
            f"WRITE_SIZE {np.median(cw):.0f} KiB per dispatch (median of {len(cf)}, {len(cw)}), "
            f"so the scale factors are {f_fac:.4f} (fetch) and {w_fac:.4f} (write).", "",
            "| leg | kernel | grid | dispatches | FETCH KiB | WRITE KiB | HBM bytes per launch (scaled) |",
            "|---|---|---|---|---|---|---|"]
    js = []
    for (leg, k, g), (fv, wv) in sorted(agg.items()):
        if not fv or not wv:
            continue
        fk, wk = float(np.mean(fv)), float(np.mean(wv))
        b = fk * 1024 * f_fac + wk * 1024 * w_fac
        out.append(f"| {leg} | {k} | {g} | {len(fv)} | {fk:.0f} | {wk:.0f} | {b / 1e6:.2f} MB |")
        js.append("traffic-json: " + json.dumps({"kernel": k, "workload": leg, "grid": g, "src": source_hash(k),
                                                 "bytes_per_launch": b, "fetch_bytes": fk * 1024 * f_fac,
                                                 "write_bytes": wk * 1024 * w_fac}))
    out += ["", "Machine-readable lines (bench.py reads these; src = hash of the kernel's sources):", ""]
    out += js
    return "\n".join(out) + "\n"


def trace_summary(legs, cmd):
    """Markdown table of rocprofv3 kernel traces, one per bench leg (legs =
    [(leg, kernel_trace_csv)]): dispatches and average duration per (leg,
    kernel, grid)."""
    import collections
    import csv
    agg = collections.defaultdict(list)
    for leg, path in legs:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                agg[(leg, _short_name(r["Kernel_Name"]), grid)].append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    out = ["# Kernel trace (rocprofv3 --kernel-trace --stats), per bench leg", "",
           "Command (from the repository root, on one MI355X; R = repository root; LEG is each bench leg",
           "in the table):", "", "    " + cmd, "",
           "Kernels of the library (and the runtime's copy) only; torch's own kernels (weight generation)",
           "are left out.", "",
           "| leg | kernel | grid (work-items) | dispatches | avg us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    mine = set(KERNEL_SOURCES) | {"amax_rows_partial_kernel", "amax_finalize_kernel", "copy_scalar_kernel",
                                  "dequantize_f16_kernel", "route_kernel", "route_count_kernel",
                                  "route_scan_kernel", "route_place_kernel", "amax_route_kernel",
                                  "l1_skinny_kernel", "l2_skinny_kernel", "mx_dequantize_kernel",
                                  "__amd_rocclr_copyBuffer"}
    for (leg, k, g), v in sorted(agg.items(), key=lambda kv: (kv[0][0], -sum(kv[1]))):
        if _base(k) in mine:
            out.append(f"| {leg} | {k} | {g} | {len(v)} | {np.mean(v):.2f} | {np.min(v):.2f} | {np.max(v):.2f} |")
    return "\n".join(out) + "\n"


# ------------------------------------------------------------------ MFMA utilisation
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_util.md")
XCDS, SIMDS = 8, 1024  # MI355X: GRBM_GUI_ACTIVE is summed over the 8 XCDs; 256 CUs x 4 SIMDs
# MFMA operation counters (512 flops per MOP): f16 for the NVFP4 GEMMs, f6f4
# for the MXFP4 GEMM's scaled FP4 MFMA
MFMA_MOPS = ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F6F4")


def mfma_summary(legs, cmd):
    """Markdown table of rocprofv3 counter runs (SQ_VALU_MFMA_BUSY_CYCLES,
    GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_F16 / _F6F4) for the GEMM kernels, one
    run per bench leg (legs = [(leg, counter_csv)]).  Per dispatch: MFMA
    busy fraction = busy cycles summed over the SIMDs / (active cycles of one
    XCD x 1024 SIMDs), effective clock = active cycles of one XCD / duration,
    and the MFMA flops the counters report (512 per MOP)."""
    import collections
    import csv
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for leg, path in legs:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                k = _short_name(r["Kernel_Name"])
                if "gemm" not in k and "skinny" not in k and not k.startswith("Cijk"):
                    continue
                key = (leg, k if not k.startswith("Cijk") else "hipBLASLt f16 GEMM (torch.matmul)",
                       int(r["Grid_Size"]))
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
                agg[key][r["Counter_Name"]].append((float(r["Counter_Value"]), dur))
    out = ["# MFMA utilisation of the GEMM kernels (rocprofv3 counters), per bench leg", "",
           "Command (from the repository root, on one MI355X; R = repository root; LEG is each bench leg",
           "in the table):", "", "    " + cmd, "",
           f"Per dispatch: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs)",
           f"(rocprofv3 reports GRBM_GUI_ACTIVE summed over the {XCDS} XCDs); clock = GRBM_GUI_ACTIVE / {XCDS} /",
           "duration; MFMA TFLOP/s = 512 x (SQ_INSTS_VALU_MFMA_MOPS_F16 + SQ_INSTS_VALU_MFMA_MOPS_F6F4) /",
           "duration.  Durations are those of the counter runs.", "",
           "| leg | kernel | grid | dispatches | avg us | clock GHz | MFMA busy | MFMA TFLOP/s |",
           "|---|---|---|---|---|---|---|---|"]
    js = []
    for (leg, k, g), c in sorted(agg.items()):
        need = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
        mops = [m for m in MFMA_MOPS if m in c]
        if not all(n in c for n in need) or not mops:
            continue
        n = len(c["GRBM_GUI_ACTIVE"])
        busy = np.mean([x for x, _ in c["SQ_VALU_MFMA_BUSY_CYCLES"]])
        gui = np.mean([x for x, _ in c["GRBM_GUI_ACTIVE"]]) / XCDS
        dur = np.mean([d for _, d in c["GRBM_GUI_ACTIVE"]])
        flops = 512.0 * sum(np.mean([x for x, _ in c[m]]) for m in mops)
        util, clk = busy / (gui * SIMDS), gui / dur / 1e9
        out.append(f"| {leg} | {k} | {g} | {n} | {dur * 1e6:.1f} | {clk:.2f} | {100 * util:.1f} % | "
                   f"{flops / dur / 1e12:.0f} |")
        if _base(k) in KERNEL_SOURCES:
            js.append(json.dumps({"kernel": k, "workload": leg, "grid": g, "src": source_hash(k),
                                  "mfma_busy": util, "clock_ghz": clk, "mfma_flops": flops}))
    out += ["", "Machine-readable lines (bench.py reads these; src = hash of the kernel's sources):", ""]
    out += ["mfma-json: " + j for j in js]
    return "\n".join(out) + "\n"


def load_mfma(kernel, workload):
    """MFMA busy fraction and clock of `kernel` in bench leg `workload` from
    the committed counter summary, or None when absent or stale."""
    try:
        with open(MFMA_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("mfma-json: "):
            d = json.loads(line[len("mfma-json: "):])
            if d.get("kernel") == kernel and d.get("workload") == workload and d.get("src") == source_hash(kernel):
                return {"mfma_busy": d["mfma_busy"], "clock_ghz": d["clock_ghz"]}
    return None


# ------------------------------------------------------------------ MoE
def moe_weights(nv, cfg):
    """All experts' NVFP4 weights on the GPU (model preparation, untimed):
    (w1q, w1sf, w1gs, w2q, w2sf, w2gs, w1sf_paired, w2sf_paired), the last two
    the row-paired copies of the scales that the 32-row tiles read (None
    where H, resp. I, is not a multiple of 1024)."""
    import synth
    E, I, H = cfg.E, cfg.I, cfg.H
    dev = torch.device("cuda:0")
    w1q = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w1sf = torch.empty((E, 2 * I, H // 16), dtype=torch.uint8, device=dev)
    w1gs = torch.empty(E, dtype=torch.float32, device=dev)
    w2q = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    w2sf = torch.empty((E, H, I // 16), dtype=torch.uint8, device=dev)
    w2gs = torch.empty(E, dtype=torch.float32, device=dev)
    for e in range(E):
        a, b = synth.expert_weights(cfg, e, device=dev)
        nv.quantize(a, out=(w1q[e], w1sf[e], w1gs[e:e + 1]))
        nv.quantize(b, out=(w2q[e], w2sf[e], w2gs[e:e + 1]))
    w1p = nv.pair_scales(w1sf) if H % 1024 == 0 else None
    w2p = nv.pair_scales(w2sf) if I % 1024 == 0 else None
    torch.cuda.synchronize()
    return w1q, w1sf, w1gs, w2q, w2sf, w2gs, w1p, w2p


def bench_moe(nv, cfg, steps, warmup, w=None, mode="fused", median_iters=10):
    """One MoE layer config; mode "fused" (L1 output quantized in the GEMM
    epilogue with the supplied scale), "unfused" (compact bf16 L1 output,
    separate quantization pass, supplied scale), "interleaved" (interleaved
    [SiLU(gate), SwiGLU] bf16 output, deinterleave + quantize pass),
    "dynamic" (unfused, with the dynamic amax / 2688 scale) or "aux" (fused,
    with the mixed tiling's short tiles on a second stream alongside the
    256-row tiles)."""
    import synth
    dev = torch.device("cuda:0")
    if w is None:
        w = moe_weights(nv, cfg)
    xb = synth.activations(cfg)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    ids, wts = synth.routing(cfg)
    ti = torch.from_numpy(ids).to(dev)
    tw = torch.from_numpy(wts).to(dev)
    a2 = None if mode == "dynamic" else torch.tensor([cfg.a2_gs], dtype=torch.float32, device=dev)
    a2_out = torch.empty(1, dtype=torch.float32, device=dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    flow = {"fused": 0, "unfused": 1, "interleaved": 2, "dynamic": 0, "aux": 0}[mode]
    aux = None
    if mode == "aux":
        # the library forks the short tiles onto this stream and joins it back
        aux = (torch.cuda.Stream(), (torch.cuda.Event(), torch.cuda.Event()))
        for e in aux[1]:
            e.record()
    # the scale used is read back only in the dynamic flow (elsewhere it is the
    # supplied one, and asking for it would add a copy launch to every layer)
    args = nv.moe_args(x, ti, tw, *w[:6], a2, out, a2_gs_out=a2_out if mode == "dynamic" else None, l1_unfused=flow,
                       w1_sf_paired=w[6], w2_sf_paired=w[7],
                       aux=aux)
    ws = torch.empty(nv.moe_workspace_size(args), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        nv.moe_expert_ffn_raw(args, dev, ws)
    # The clock settles over about 0.1 s of sustained work: a short layer
    # (decode) gets more untimed layers, up to ~100 ms in all.  (With 3
    # warm-up layers the decode layer's mean came out 8 % above its median;
    # after 100 the two agreed within 1 %.)
    w0, w1 = _ev(), _ev()
    torch.cuda.synchronize()
    w0.record()
    nv.moe_expert_ffn_raw(args, dev, ws)
    w1.record()
    torch.cuda.synchronize()
    est = max(w0.elapsed_time(w1), 1e-3)
    for _ in range(int(min(2000, max(0.0, (100.0 - (warmup + 1) * est) / est)))):
        nv.moe_expert_ffn_raw(args, dev, ws)
    torch.cuda.synchronize()
    # the layer time: `steps` back-to-back layers between two events, with no
    # stage events inside (each event record costs the stream a few us)
    e0, e1 = _ev(), _ev()
    e0.record()
    for _ in range(steps):
        nv.moe_expert_ffn_raw(args, dev, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # per-layer times for a median: events between consecutive layers
    iters = max(steps, median_iters)
    bounds = [_ev() for _ in range(iters + 1)]
    torch.cuda.synchronize()
    bounds[0].record()
    for i in range(iters):
        nv.moe_expert_ffn_raw(args, dev, ws)
        bounds[i + 1].record()
    torch.cuda.synchronize()
    per_layer = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(iters)]
    # the stage breakdown: a second run with the library's stage events
    evs = [[_ev() for _ in range(STAGE_EVENTS)] for _ in range(steps)]
    handles = [(ctypes.c_void_p * STAGE_EVENTS)(*[e.cuda_event for e in row]) for row in evs]
    torch.cuda.synchronize()
    for i in range(steps):
        args.stage_events = ctypes.cast(handles[i], ctypes.POINTER(ctypes.c_void_p))
        nv.moe_expert_ffn_raw(args, dev, ws)
    torch.cuda.synchronize()
    args.stage_events = None
    evented_ms = evs[0][0].elapsed_time(evs[-1][STAGE_EVENTS - 1]) / steps
    stage_ms = {name: float(np.mean([evs[i][s].elapsed_time(evs[i][s + 1]) for i in range(steps)]))
                for s, name in enumerate(STAGES)}
    stage_ms_median = {name: float(np.median([evs[i][s].elapsed_time(evs[i][s + 1]) for i in range(steps)]))
                       for s, name in enumerate(STAGES)}
    stage_ms["l1_gemm_swiglu_quant"] = stage_ms["l1_main"] + stage_ms["l1_rest"]
    stage_ms["l2_gemm"] = stage_ms["l2_main"] + stage_ms["l2_rest"]
    flops = cfg.flops()
    used = np.unique(ids[(ids >= 0) & (ids < cfg.E)])
    wbytes_per_expert = (2 * cfg.I * cfg.H + cfg.H * cfg.I) * (0.5 + 1 / 16)
    l1_flops = 2.0 * cfg.P * cfg.H * 2 * cfg.I
    l2_flops = 2.0 * cfg.P * cfg.I * cfg.H
    # rows on the main (256-row) tiles: with more than 16 pairs per expert
    # (and H, I multiples of 256) the library picks the mixed tiling, whose
    # main list holds all but each expert's last block of at most 64 rows
    n = np.bincount(ids[(ids >= 0) & (ids < cfg.E)].reshape(-1), minlength=cfg.E)
    r = n % 256
    mixed = cfg.P > 16 * cfg.E
    main_rows = int(n.sum() - (r[(r > 0) & (r <= 64)].sum() if mixed else 0))
    l1_main_flops = 2.0 * main_rows * cfg.H * 2 * cfg.I
    return dict(
        workload=f"T{cfg.T} H{cfg.H} I{cfg.I} E{cfg.E} top{cfg.topk} ({cfg.routing} routing)",
        ms_per_step=ms, ms_median=float(np.median(per_layer)), median_of=f"{iters} layers",
        ms_per_step_with_stage_events=evented_ms, TFLOPs=flops / ms / 1e9, algorithmic_flops=flops,
        experts_touched=int(used.size),
        weight_GBps=used.size * wbytes_per_expert / ms / 1e6,
        stage_ms=stage_ms, stage_ms_median=stage_ms_median,
        l1_TFLOPs=l1_flops / stage_ms["l1_gemm_swiglu_quant"] / 1e9,
        l2_TFLOPs=l2_flops / stage_ms["l2_gemm"] / 1e9,
        l1_main_rows=main_rows, l1_main_flops=l1_main_flops,
        l1_main_TFLOPs=l1_main_flops / stage_ms["l1_main"] / 1e9,
        l1_flops=l1_flops, l2_flops=l2_flops, mode=mode,
        a2_gs=float(a2_out.item()) if mode == "dynamic" else float(a2.item()),
    ), (w, x, ids, wts, out.float())


def bench_expert(nv, steps, warmup):
    import synth
    dev = torch.device("cuda:0")
    M, K, I = synth.EXPERT_SHAPE["M"], synth.EXPERT_SHAPE["K"], synth.EXPERT_SHAPE["I"]
    xb, w1 = synth.expert_problem()
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    xq, xsf, xg = nv.quantize(x)
    wq, wsf, wg = nv.quantize(w1.to(dev))
    og = torch.tensor([synth.EXPERT_A2_GS], dtype=torch.float32, device=dev)
    outs = (torch.empty((M, I), dtype=torch.bfloat16, device=dev),
            torch.empty((M, I // 2), dtype=torch.uint8, device=dev),
            torch.empty((M, I // 16), dtype=torch.uint8, device=dev))
    st = {}
    ms = graph_time(lambda i: nv.gemm_swiglu_quant(xq, xsf, xg, wq, wsf, wg, og, out=outs), steps, warmup, stats=st)
    flops = 2.0 * M * K * 2 * I
    res = dict(workload=f"M{M} K{K} N2x{I}", ms=ms, TFLOPs=flops / ms / 1e9, algorithmic_flops=flops,
               frac=flops / ms / 1e9 / F16_PEAK_TFLOPS, ms_median=st["ms_median"], median_of=st["median_of"],
               frac_median=flops / st["ms_median"] / 1e9 / F16_PEAK_TFLOPS)
    # The same stage without a workspace: the GEMM reads the NVFP4
    # activations and dequantizes each K step into LDS itself (no separate
    # f16 expansion pass; the expansion then runs inside the MFMA loop).
    st2 = {}
    ms_lds = graph_time(lambda i: nv.gemm_swiglu_quant(xq, xsf, xg, wq, wsf, wg, og, out=outs, expand_a=False),
                        steps, warmup, stats=st2)
    res["nvfp4_activations_in_gemm"] = dict(ms=ms_lds, ms_median=st2["ms_median"], TFLOPs=flops / ms_lds / 1e9)
    # Context, not the product path: the vendor library's plain f16 GEMM
    # (torch -> hipBLASLt) on the same operand values, A [M][K] @ B^T with B
    # [2I][K] already dequantized (e2m1 * block scale, global scales left
    # out, so every value is exact in f16).  It reads 4x the weight bytes and
    # has no dequantization, SwiGLU or output quantization to do.
    one = torch.ones(1, dtype=torch.float32, device=dev)
    a16 = nv.dequantize(xq, xsf, one).to(torch.float16)
    b16 = nv.dequantize(wq, wsf, one).to(torch.float16).t().contiguous()  # [K][2I]
    c16 = torch.empty((M, 2 * I), dtype=torch.float16, device=dev)
    ms_v = graph_time(lambda i: torch.matmul(a16, b16, out=c16), steps, warmup)
    res["vendor_f16_gemm"] = dict(ms=ms_v, TFLOPs=flops / ms_v / 1e9,
                                  library="torch.matmul (hipBLASLt), f16 in/out, B pre-dequantized")
    return res


def bench_dense(nv, steps, warmup):
    """Dense NVFP4 linear M4096 K4096 N16384 (activation global scale +
    quantization + GEMM per call), bf16 output, graph-timed."""
    import synth
    dev = torch.device("cuda:0")
    M, K, N = synth.DENSE_SHAPE["M"], synth.DENSE_SHAPE["K"], synth.DENSE_SHAPE["N"]
    xb, w = synth.dense_problem(device=dev)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    wq, wsf, wg = nv.quantize(w)
    del w
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = nv.linear_workspace(M, K, N, dev)
    st = {}
    ms = graph_time(lambda i: nv.linear(x, wq, wsf, wg, out=out, ws=ws), steps, warmup, stats=st)
    flops = 2.0 * M * N * K
    # Context, not the product path: the vendor library's plain f16 GEMM
    # (torch -> hipBLASLt) on the same operand values, both already
    # dequantized (e2m1 * block scale, global scales left out: exact in f16),
    # f16 out; no quantization pass and 4x the weight bytes.
    one = torch.ones(1, dtype=torch.float32, device=dev)
    xq, xsf, _ = nv.quantize(x)
    a16 = nv.dequantize(xq, xsf, one).to(torch.float16)
    b16 = nv.dequantize(wq, wsf, one).to(torch.float16).t().contiguous()  # [K][N]
    c16 = torch.empty((M, N), dtype=torch.float16, device=dev)
    del xq, xsf
    ms_v = graph_time(lambda i: torch.matmul(a16, b16, out=c16), steps, warmup)
    return dict(workload=f"M{M} K{K} N{N}", ms=ms, TFLOPs=flops / ms / 1e9, algorithmic_flops=flops,
                frac=flops / ms / 1e9 / F16_PEAK_TFLOPS, ms_median=st["ms_median"], median_of=st["median_of"],
                vendor_f16_gemm=dict(ms=ms_v, TFLOPs=flops / ms_v / 1e9,
                                     library="torch.matmul (hipBLASLt), f16 in/out, operands pre-dequantized"))


def _vendor_mx_gemm(nv, x, wq, wsc, steps, warmup):
    """Context, not the product path: the vendor library's MXFP4 GEMM
    (torch._scaled_mm -> hipBLASLt) on the same operand bytes (E2M1 nibbles,
    one E8M0 code per 32 elements, the activations quantized once outside the
    timed calls), bf16 out, timed eagerly over back-to-back calls.  Its
    output is not checked (the library may expect another scale layout); None
    when this torch build has no MXFP4 GEMM."""
    f4, e8 = getattr(torch, "float4_e2m1fn_x2", None), getattr(torch, "float8_e8m0fnu", None)
    if f4 is None or e8 is None:
        return None
    try:
        xq, xsc = nv.mx_quantize(x)
        a, sa = xq.view(f4), xsc.view(e8)
        b, sb = wq.view(f4).t(), wsc.view(e8)
        fn = lambda: torch._scaled_mm(a, b, scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        for _ in range(max(warmup, 3)):
            fn()
        e0, e1 = _ev(), _ev()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        M, N, K = xq.shape[0], wq.shape[0], 2 * xq.shape[1]
        return dict(ms=ms, TFLOPs=2.0 * M * N * K / ms / 1e9,
                    library="torch._scaled_mm (hipBLASLt), MXFP4 operands, bf16 out; GEMM only, eager")
    except Exception as ex:  # not in this torch / hipBLASLt build
        return dict(unavailable=f"{type(ex).__name__}: {str(ex)[:120]}")


def bench_mx(nv, steps, warmup):
    """The separately labelled MXFP4 variant (OCP MX v1.0: E8M0 scale per 32
    elements) on the scaled FP4 MFMA: quantize 8192 x 7168 (inputs rotated
    like the NVFP4 quantize leg) and the dense linear M4096 K4096 N16384
    (activation quantization + GEMM, bf16 out), against the FP4 MFMA peak."""
    import synth
    dev = torch.device("cuda:0")
    M, K = synth.QUANT_SHAPE
    n = M * K
    x0 = torch.from_numpy(synth.quant_tensor().view(np.int16)).view(torch.bfloat16).to(dev)
    ncopy = 5
    xs = [x0] + [x0.clone() for _ in range(ncopy - 1)]
    outs = [(torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
             torch.empty((M, K // 32), dtype=torch.uint8, device=dev)) for _ in range(ncopy)]
    q_ms = graph_time(lambda i: nv.mx_quantize(xs[i % ncopy], out=outs[i % ncopy]), steps, warmup)
    qbytes = 2 * n + n // 2 + n // 32
    del xs, outs
    Md, Kd, Nd = synth.DENSE_SHAPE["M"], synth.DENSE_SHAPE["K"], synth.DENSE_SHAPE["N"]
    xb, w = synth.dense_problem(Md, Kd, Nd, device=dev)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    wq, wsc = nv.mx_quantize(w)
    del w
    out = torch.empty((Md, Nd), dtype=torch.bfloat16, device=dev)
    ws = nv.mx_linear_workspace(Md, Kd, Nd, dev)
    st = {}
    l_ms = graph_time(lambda i: nv.mx_linear(x, wq, wsc, out=out, ws=ws), steps, warmup, stats=st)
    flops = 2.0 * Md * Nd * Kd
    vendor = _vendor_mx_gemm(nv, x, wq, wsc, steps, warmup)
    return dict(format="MXFP4 (OCP MX v1.0, E8M0 scale per 32 elements; not NVFP4)", vendor_mxfp4_gemm=vendor,
                quantize_shape=[M, K], quantize_algorithmic_bytes=qbytes, quantize_ms=q_ms,
                quantize_GBps=qbytes / q_ms / 1e6, quantize_frac=qbytes / q_ms / 1e6 / HBM_PEAK_GBS,
                linear_workload=f"M{Md} K{Kd} N{Nd}", linear_ms=l_ms, linear_TFLOPs=flops / l_ms / 1e9,
                linear_algorithmic_flops=flops, linear_frac_fp4_peak=flops / l_ms / 1e9 / FP4_PEAK_TFLOPS,
                linear_ms_median=st["ms_median"], median_of=st["median_of"])


# ------------------------------------------------------------------ CPU oracle
# The oracle (plain C, fp64 GEMMs, never tuned) timed on this host's cores in
# the same run, on bounded samples of each workload.  Threads: the CPUs this
# process may run on, capped at 16 (one GPU's share of a shared host).
def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return dict(cpu_model=model, host_logical_cpus=os.cpu_count(), cpus_available=avail,
                threads=max(1, min(avail, 16)))


def _median_runs(fn, runs):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), ts


def _oracle_experts(orc, cfg, experts):
    """Oracle-quantized weights of the listed experts (model preparation,
    untimed like the GPU's), drawn on the GPU like the GPU path's."""
    import synth
    n = len(experts)
    W = dict(w1q=np.zeros((n, 2 * cfg.I, cfg.H // 2), np.uint8), w1sf=np.zeros((n, 2 * cfg.I, cfg.H // 16), np.uint8),
             w1gs=np.zeros(n, np.float32), w2q=np.zeros((n, cfg.H, cfg.I // 2), np.uint8),
             w2sf=np.zeros((n, cfg.H, cfg.I // 16), np.uint8), w2gs=np.zeros(n, np.float32))
    for i, e in enumerate(experts):
        a, b = synth.expert_weights(cfg, int(e), device="cuda:0")
        a, b = synth.torch_bits(a), synth.torch_bits(b)
        W["w1gs"][i] = orc.global_scale(a)
        W["w1q"][i], W["w1sf"][i] = orc.quantize(a, W["w1gs"][i])
        W["w2gs"][i] = orc.global_scale(b)
        W["w2q"][i], W["w2sf"][i] = orc.quantize(b, W["w2gs"][i])
    return W


def _few_expert_tokens(ids, E, ntok, pool):
    """ntok tokens from the first `pool` tokens, chosen greedily so that they
    share experts (each next token adds the fewest experts not yet used):
    the oracle's cost per pair does not depend on which experts, and fewer
    distinct experts keep its untimed weight preparation short."""
    used, chosen = set(), []
    cand = list(range(min(pool, ids.shape[0])))
    for _ in range(ntok):
        best = min(cand, key=lambda t: len(set(int(e) for e in ids[t] if 0 <= e < E) - used))
        cand.remove(best)
        chosen.append(best)
        used |= set(int(e) for e in ids[best] if 0 <= e < E)
    return np.array(sorted(chosen), np.int64), sorted(used)


def cpu_baseline_moe(cfg, ntok, runs, threads, pool=512):
    """The oracle's MoE layer (activation quantization, L1 + SwiGLU, L1-output
    quantization, L2, combine) on ntok tokens of the workload (all their
    top-k pairs), median of `runs`; algorithmic TFLOP/s as for the GPU."""
    import oracle
    import synth
    orc = oracle.default()
    x_bits = synth.activations(cfg)
    ids, wts = synth.routing(cfg)
    if ntok >= cfg.T:
        tokens, used = np.arange(cfg.T, dtype=np.int64), sorted(set(int(e) for e in ids.reshape(-1)))
    else:
        tokens, used = _few_expert_tokens(ids, cfg.E, ntok, pool)
    remap = {e: i for i, e in enumerate(used)}
    ids_r = np.vectorize(lambda e: remap.get(int(e), -1))(ids).astype(np.int32)
    W = _oracle_experts(orc, cfg, used)
    def run():  # the activation global scale spans all T tokens, as in the GPU layer
        g = orc.global_scale(x_bits)
        orc.moe_tokens(x_bits, ids_r, wts, W["w1q"], W["w1sf"], W["w1gs"], W["w2q"], W["w2sf"], W["w2gs"],
                       cfg.a2_gs, tokens=tokens, x_gs=g, threads=threads)
    med, ts = _median_runs(run, runs)
    pairs = int(((ids[tokens] >= 0) & (ids[tokens] < cfg.E)).sum())
    flops = 6.0 * pairs * cfg.H * cfg.I
    return {"value": flops / med / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": med, "runs": [round(t, 3) for t in ts],
            "sample": f"{tokens.size} of the {cfg.T} tokens of T{cfg.T} H{cfg.H} I{cfg.I} E{cfg.E} top-{cfg.topk} "
                      f"({pairs} pairs on {len(used)} experts; activation global scale over all T tokens, "
                      f"quantization, L1 + SwiGLU, L1-output quantization, L2, combine), median of {runs}; "
                      f"oracle weight quantization excluded"}


def cpu_baseline_expert(rows, runs, threads):
    """The oracle's single-expert stage (M4096 K7168 N 2x2048) on `rows` of
    its 4096 rows: activation quantization of those rows, L1 + SwiGLU, and
    quantization of the compact output; median of `runs`."""
    import oracle
    import synth
    orc = oracle.default()
    xb, w1 = synth.expert_problem(device="cuda:0")
    wb = synth.torch_bits(w1)
    gw = orc.global_scale(wb)
    wq, wsf = orc.quantize(wb, gw)
    K = xb.shape[1]
    sel = np.linspace(0, xb.shape[0] - 1, rows).astype(np.int64)
    xs = np.ascontiguousarray(xb[sel])
    gx = orc.global_scale(xb)
    def run():
        aq, asf = orc.quantize(xs, gx, threads=threads)
        c, _ = orc.l1_swiglu_rows(aq, asf, gx, wq, wsf, gw, np.arange(rows), threads=threads)
        orc.quantize(c, np.float32(synth.EXPERT_A2_GS), threads=threads)
    med, ts = _median_runs(run, runs)
    flops = 2.0 * rows * K * wq.shape[0]
    return {"value": flops / med / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": med, "runs": [round(t, 3) for t in ts],
            "sample": f"{rows} of the 4096 rows (quantize, L1 + SwiGLU, quantize), median of {runs}"}


def cpu_baseline_quantize(rows, runs, threads):
    import oracle
    import synth
    orc = oracle.default()
    bits = synth.quant_tensor(rows, synth.QUANT_SHAPE[1], seed=1)
    g = orc.global_scale(bits)
    med, ts = _median_runs(lambda: orc.quantize(bits, g, threads=threads), runs)
    n = rows * synth.QUANT_SHAPE[1]
    return {"value": (2 * n + n // 2 + n // 16) / med / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": med, "runs": [round(t, 3) for t in ts],
            "sample": f"{rows} x {synth.QUANT_SHAPE[1]} (of the 8192 x 7168 workload; supplied g), median of {runs}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="quant,expert,dense,mx,dec,pre,tiny")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the unfused and dynamic-scale runs of the prefill layer")
    ap.add_argument("--traffic-summary", nargs="+", metavar="CSV",
                    help="print the markdown HBM-traffic summary of rocprofv3 counter CSVs: COPY_FETCH "
                         "COPY_WRITE, then LEG=FETCH_CSV LEG=WRITE_CSV pairs")
    ap.add_argument("--trace-summary", nargs="+", metavar="LEG=KERNEL_TRACE_CSV",
                    help="print the markdown summary of rocprofv3 kernel traces, one per bench leg")
    ap.add_argument("--mfma-summary", nargs="+", metavar="LEG=COUNTER_CSV",
                    help="print the markdown MFMA-utilisation summary of rocprofv3 counter runs, one per bench leg")
    ap.add_argument("--cmd", action="append", default=[], help="command lines quoted in a summary")
    args = ap.parse_args()
    if args.traffic_summary:
        cf, cw, *rest = args.traffic_summary
        pairs = _split_legs(rest)
        legs = [(pairs[i][0], pairs[i][1], pairs[i + 1][1]) for i in range(0, len(pairs), 2)]
        sys.stdout.write(traffic_summary(cf, cw, legs, args.cmd))
        return
    if args.trace_summary:
        sys.stdout.write(trace_summary(_split_legs(args.trace_summary), " ".join(args.cmd)))
        return
    if args.mfma_summary:
        sys.stdout.write(mfma_summary(_split_legs(args.mfma_summary), " ".join(args.cmd)))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import quantization_nvfp4_quantize_amd as nv
    import synth
    legs = set(args.legs.split(","))
    res = {}
    if "copy" in legs:
        res["copy"] = bench_copy(args.steps)
    if "quant" in legs:
        res["quantize"] = bench_quantize(nv, args.steps, args.warmup)
        print("# quantize done", flush=True, file=sys.stderr)
    if "expert" in legs:
        res["expert_l1"] = bench_expert(nv, args.steps, args.warmup)
        print("# expert done", flush=True, file=sys.stderr)
    if "dense" in legs:
        res["dense_linear"] = bench_dense(nv, args.steps, args.warmup)
        print("# dense done", flush=True, file=sys.stderr)
    if "mx" in legs:
        res["mxfp4"] = bench_mx(nv, args.steps, args.warmup)
        print("# mxfp4 done", flush=True, file=sys.stderr)
        torch.cuda.empty_cache()
    if "dec" in legs:
        res["decode"], _ = bench_moe(nv, synth.DEC, args.steps, args.warmup, median_iters=50)
        print("# decode done", flush=True, file=sys.stderr)
        torch.cuda.empty_cache()
    pre = None
    if "pre" in legs:
        res["prefill"], pre = bench_moe(nv, synth.PRE, args.steps, args.warmup)
        print("# prefill done", flush=True, file=sys.stderr)
        if not args.no_modes:
            # the pages' unfused flows on the same layer: the fusion's saving,
            # and the dynamic L1-output scale against the supplied one
            y_static = pre[4]
            for mode in ("unfused", "interleaved", "dynamic", "aux"):
                r, extra = bench_moe(nv, synth.PRE, max(3, args.steps // 3), args.warmup, w=pre[0], mode=mode)
                r = {k: r[k] for k in ("ms_per_step", "ms_median", "median_of", "TFLOPs", "stage_ms", "a2_gs")}
                yd = extra[4]
                r["y_rel_fro_vs_fused"] = float(torch.linalg.norm(yd - y_static) / torch.linalg.norm(y_static))
                res["prefill_" + mode] = r
            for mode in ("unfused", "interleaved"):
                res["prefill_" + mode]["fusion_saving_ms"] = (res["prefill_" + mode]["ms_per_step"]
                                                             - res["prefill"]["ms_per_step"])
            print("# prefill modes done", flush=True, file=sys.stderr)
    if "tiny" in legs:
        # the small workload end to end (launch-latency bound)
        res["tiny"], _ = bench_moe(nv, synth.TINY, args.steps, args.warmup, median_iters=50)
        print("# tiny done", flush=True, file=sys.stderr)
    cpu = None
    if not args.no_cpu:
        # the oracle on this host's cores, same run, bounded samples of each leg
        info = cpu_info()
        th = info["threads"]
        del pre
        torch.cuda.empty_cache()
        if "prefill" in res:
            cpu = dict(cpu_baseline_moe(synth.PRE, ntok=16, runs=1, threads=th), **info)
        if "decode" in res:
            res["decode"]["cpu_baseline"] = cpu_baseline_moe(synth.DEC, ntok=8, runs=3, threads=th, pool=128)
        if "quantize" in res:
            res["quantize"]["cpu_baseline"] = cpu_baseline_quantize(rows=synth.QUANT_SHAPE[0], runs=3, threads=th)
        if "expert_l1" in res:
            res["expert_l1"]["cpu_baseline"] = cpu_baseline_expert(rows=32, runs=3, threads=th)
        if "tiny" in res:
            res["tiny"]["cpu_baseline"] = cpu_baseline_moe(synth.TINY, ntok=synth.TINY.T, runs=3, threads=th)
        print("# cpu baseline done", flush=True, file=sys.stderr)
    p = res.get("prefill")
    traffic = mfma = None
    if p:
        traffic = load_traffic(ROOFLINE_KERNEL, "pre")
        mfma = load_mfma(ROOFLINE_KERNEL, "pre")
    src = {"file": "profiles/hbm_traffic.md", "kernel_source_hash": source_hash(ROOFLINE_KERNEL)}
    line = {
        "metric": "MoE expert-FFN TFLOP/s + quantize GB/s, % of MI355X roofline (1 GPU)",
        "value": p["TFLOPs"] if p else None,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": p["ms_per_step"] if p else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "prefill-shaped NVFP4 MoE layer T16384 H7168 I2048 E256 top-8 "
                               "(uniform routing), bf16 in/out; plus standalone quantize 8192x7168",
                   "parallelism": "none (1 GPU)"},
        "roofline": ({"bound": "mfma", "kernel": ROOFLINE_KERNEL + " (256-row tiles)",
                      "achieved": p["l1_main_TFLOPs"], "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": p["l1_main_TFLOPs"] / F16_PEAK_TFLOPS, "traffic": traffic,
                      "traffic_unit": "bytes per launch (HBM, rocprofv3)",
                      "algorithmic_flops_per_launch": p["l1_main_flops"],
                      # rocprofv3 counters of the same kernel: MFMA-busy fraction of the SIMD
                      # cycles and the clock it ran at (the 2.5 PFLOP/s peak assumes 2.4 GHz)
                      "counters": mfma,
                      # traffic and counters are read from the committed rocprofv3 summaries (a
                      # profiler run of their own), and only while the kernel's sources hash to
                      # the value recorded with them; achieved comes from this run's HIP events
                      "traffic_source": dict(src, file="profiles/hbm_traffic.md") if traffic else None,
                      "counters_source": dict(src, file="profiles/mfma_util.md") if mfma else None,
                      "achieved_median": p["l1_main_flops"] / p["stage_ms_median"]["l1_main"] / 1e9}
                     if p else None),
        "cpu_baseline": cpu,
    }
    line.update(res)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
