"""Seeded synthetic inputs for the NVFP4 MoE expert FFN workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantization, no GEMM, no SwiGLU).  Both the CPU
oracle and the GPU path take their inputs from here.

Workloads (shapes and value distributions of the DeepSeek-style NVFP4 MoE on
the "nvfp4-megamoe-kernel" pages; no public dataset is involved):
  tiny  T64 H256 I128 E8 top-2, N(0,1) routing logits
  quant 8192 x 7168 bf16 N(0,1), 1% of elements x100, 1% of 16-blocks x1e-3
  expert single expert M4096 K7168 N 2x2048 (gate/up interleaved by 8)
  dec   T128 H7168 I2048 E256 top-8, Zipf(1.1)-skewed routing
  pre   T16384 H7168 I2048 E256 top-8, uniform routing
  dense NVFP4 linear M4096 K4096 N16384
Activations are bf16 N(0,1); weights bf16 N(0, 0.02).

Generators: numpy PCG64 with a fixed draw order for host tensors; expert
weights come from torch's generator (seeded per expert) on the requested
device, so the large configs can be drawn directly in GPU memory.  bf16
values are the round-to-nearest-even of the fp32 draws.
"""
from dataclasses import dataclass

import numpy as np
import torch


# ------------------------------------------------------------------ helpers
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp32 values (exact)."""
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def interleave_gate_up(w_gate_up, group: int = 8):
    """Rows [gate (I); up (I)] -> [gate_0..7, up_0..7, gate_8..15, up_8..15, ...].

    Works on numpy arrays and torch tensors of shape [2I, K] (a row
    permutation only)."""
    n2 = w_gate_up.shape[0]
    I = n2 // 2
    assert I % group == 0
    idx = np.empty(n2, np.int64)
    for j in range(I // group):
        idx[2 * group * j: 2 * group * j + group] = np.arange(group * j, group * j + group)
        idx[2 * group * j + group: 2 * group * (j + 1)] = I + np.arange(group * j, group * j + group)
    if isinstance(w_gate_up, torch.Tensor):
        return w_gate_up[torch.from_numpy(idx).to(w_gate_up.device)]
    return w_gate_up[idx]


# ------------------------------------------------------------------ configs
@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    topk: int
    routing: str        # "normal" (i.i.d. N(0,1) logits) or "zipf"
    seed: int
    a2_gs: float        # supplied global scale of the L1 output (kernel input)

    @property
    def P(self):
        return self.T * self.topk

    def flops(self):
        """Algorithmic GEMM flops of one forward: L1 2*P*H*2I + L2 2*P*I*H."""
        return 6.0 * self.P * self.H * self.I


# a2_gs: chosen so that the largest L1-output block scales stay below the
# E4M3 maximum for these distributions (|silu(g)*u| well under 2688*a2_gs).
TINY = MoeConfig("tiny", 64, 256, 128, 8, 2, "normal", 0, 0.75 / 2688.0)
DEC = MoeConfig("dec", 128, 7168, 2048, 256, 8, "zipf", 3, 64.0 / 2688.0)
PRE = MoeConfig("pre", 16384, 7168, 2048, 256, 8, "normal", 4, 64.0 / 2688.0)
MOE_CONFIGS = {c.name: c for c in (TINY, DEC, PRE)}

QUANT_SHAPE = (8192, 7168)
# dense NVFP4 linear: 4096 tokens through a projection with the (16384, 4096)
# weight shape the pages list for o_a_proj (out features x in features)
DENSE_SHAPE = dict(M=4096, K=4096, N=16384)
EXPERT_SHAPE = dict(M=4096, K=7168, I=2048)
EXPERT_A2_GS = 64.0 / 2688.0


# ------------------------------------------------------------------ tensors
def normal_bf16(shape, seed, std=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_bits(a)


def quant_tensor(M=QUANT_SHAPE[0], K=QUANT_SHAPE[1], seed=1):
    """Standalone quantize input: N(0,1); then 1% of elements (uniform
    positions) scaled by 100; then 1% of 16-element blocks replaced by
    N(0,1) * 1e-3.  Returns bf16 bits [M][K]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    flat = x.reshape(-1)
    n = flat.size
    out_idx = rng.choice(n, size=max(1, n // 100), replace=False)
    flat[out_idx] *= np.float32(100.0)
    nb = n // 16
    tiny_blocks = rng.choice(nb, size=max(1, nb // 100), replace=False)
    blocks = flat.reshape(nb, 16)
    blocks[tiny_blocks] = rng.standard_normal((tiny_blocks.size, 16), dtype=np.float32) * np.float32(1e-3)
    return bf16_bits(x)


def routing(cfg: MoeConfig):
    """Top-k expert ids (int32 [T][k], ties to the lower index) and weights
    (softmax over the selected logits, fp32 [T][k])."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed * 1000 + 7))
    T, E, k = cfg.T, cfg.E, cfg.topk
    if cfg.routing == "zipf":
        perm = rng.permutation(E)
        ranks = np.empty(E, np.float64)
        ranks[perm] = np.arange(1, E + 1, dtype=np.float64)
        logp = -1.1 * np.log(ranks)
        logp -= np.log(np.exp(logp).sum())
        gumbel = -np.log(-np.log(rng.uniform(size=(T, E))))
        logits = logp[None, :] + gumbel
    else:
        logits = rng.standard_normal((T, E))
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def activations(cfg: MoeConfig):
    return normal_bf16((cfg.T, cfg.H), cfg.seed * 1000 + 1)


def expert_weights(cfg: MoeConfig, e: int, device="cpu"):
    """bf16 torch tensors (w1 [2I][H] interleaved by 8, w2 [H][I]) of expert e,
    N(0, 0.02), drawn from torch's generator seeded by (config, expert)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed * 1_000_003 + e)
    w1 = torch.randn(2 * cfg.I, cfg.H, generator=gen, device=dev, dtype=torch.float32) * 0.02
    w2 = torch.randn(cfg.H, cfg.I, generator=gen, device=dev, dtype=torch.float32) * 0.02
    w1 = interleave_gate_up(w1.to(torch.bfloat16))
    return w1.contiguous(), w2.to(torch.bfloat16).contiguous()


def expert_problem(M=EXPERT_SHAPE["M"], K=EXPERT_SHAPE["K"], I=EXPERT_SHAPE["I"], seed=2,
                   device="cpu"):
    """Single-expert stage: activations bf16 bits [M][K] (numpy) and the
    interleaved weight w1 [2I][K] (bf16 torch tensor on `device`)."""
    x = normal_bf16((M, K), seed * 1000 + 1)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 1_000_003)
    w1 = torch.randn(2 * I, K, generator=gen, device=dev, dtype=torch.float32) * 0.02
    return x, interleave_gate_up(w1.to(torch.bfloat16)).contiguous()


def dense_problem(M=DENSE_SHAPE["M"], K=DENSE_SHAPE["K"], N=DENSE_SHAPE["N"], seed=5, device="cpu"):
    """Dense linear: activations bf16 bits [M][K] (numpy, N(0,1)) and the
    weight [N][K] (bf16 torch tensor on `device`, N(0, 0.02))."""
    x = normal_bf16((M, K), seed * 1000 + 1)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 1_000_003)
    w = torch.randn(N, K, generator=gen, device=dev, dtype=torch.float32) * 0.02
    return x, w.to(torch.bfloat16).contiguous()


def torch_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor (any device) -> uint16 numpy bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
