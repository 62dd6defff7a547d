"""Benchmark of the NVFP4 MoE expert-FFN hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints one JSON line.  Legs:
  quantize   8192 x 7168 bf16 -> NVFP4 with a supplied global scale (HBM-bound,
             2.5625 algorithmic bytes per element), inputs rotated over enough
             copies that the 256 MiB Infinity Cache cannot serve repeats;
             also the dynamic-scale variant and dequantize.
  moe        the prefill-shaped MoE layer (T16384 H7168 I2048 E256 top-8) when
             the grouped GEMMs are available.
Timing: HIP events on the stream the library launches on (torch's current
stream), W untimed warmups then K timed steps between synchronizations.
cpu_baseline: the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def bench_quantize(nv, steps, warmup):
    import synth
    M, K = synth.QUANT_SHAPE
    n = M * K
    dev = torch.device("cuda:0")
    bits = synth.quant_tensor()
    x0 = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    ncopy = 5  # 5 x 117 MB inputs (> 256 MiB Infinity Cache)
    xs = [x0] + [x0.clone() for _ in range(ncopy - 1)]
    outs = [(torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
             torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
             torch.empty(1, dtype=torch.float32, device=dev)) for _ in range(ncopy)]
    _, _, g = nv.quantize(x0)
    torch.cuda.synchronize()

    def run(fn, nsteps, nwarm):
        for i in range(nwarm):
            fn(i % ncopy)
        torch.cuda.synchronize()
        ev = _events(nsteps + 1)
        ev[0].record()
        for i in range(nsteps):
            fn(i % ncopy)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(nsteps)]
        return float(np.mean(per)), float(np.median(per))

    q_ms, q_med = run(lambda i: nv.quantize(xs[i], g, out=outs[i]), steps, warmup)
    d_ms, _ = run(lambda i: nv.quantize(xs[i], None, out=outs[i]), steps, warmup)
    deq = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(ncopy)]
    dq_ms, _ = run(lambda i: nv.dequantize(outs[i][0], outs[i][1], g, out=deq[i]), steps, warmup)
    qbytes = 2 * n + n // 2 + n // 16
    return dict(
        shape=[M, K], algorithmic_bytes=qbytes,
        quantize_ms=q_ms, quantize_ms_median=q_med, quantize_GBps=qbytes / q_ms / 1e6,
        quantize_dynamic_ms=d_ms, quantize_dynamic_GBps=(qbytes + 2 * n) / d_ms / 1e6,
        dequantize_ms=dq_ms, dequantize_GBps=(n // 2 + n // 16 + 2 * n) / dq_ms / 1e6,
    )


def cpu_baseline_quantize(target_s=10.0):
    """Oracle quantize on a bounded sample of the 8192 x 7168 tensor's rows."""
    import oracle
    import synth
    orc = oracle.default()
    threads = oracle.default_threads()
    rows = 256
    bits = synth.quant_tensor(rows, synth.QUANT_SHAPE[1], seed=1)
    g = orc.global_scale(bits)
    t0 = time.time()
    reps = 0
    while time.time() - t0 < target_s:
        orc.quantize(bits, g, threads=threads)
        reps += 1
    dt = time.time() - t0
    n = rows * synth.QUANT_SHAPE[1] * reps
    gbs = (2 * n + n // 2 + n // 16) / dt / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"quantize of {rows} x {synth.QUANT_SHAPE[1]} rows of the workload, "
                      f"{reps} repetitions in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import quantization_nvfp4_quantize_amd as nv

    qres = bench_quantize(nv, args.steps, args.warmup)
    cpu = None if args.no_cpu else cpu_baseline_quantize()
    achieved = qres["quantize_GBps"]
    line = {
        "metric": "MoE expert-FFN TFLOP/s + quantize GB/s, % of MI355X roofline (1 GPU)",
        "value": achieved,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": qres["quantize_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "standalone NVFP4 quantize 8192x7168 bf16 (supplied global scale)",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "cpu_baseline": cpu,
        "quantize": qres,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
