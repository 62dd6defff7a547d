"""Helpers shared by the GPU tests (device transfer of bf16 bit patterns)."""
import numpy as np
import torch


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> bf16 tensor on cuda:0."""
    b = np.ascontiguousarray(bits, np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda:0")


def host_bits(t):
    """bf16 tensor -> uint16 numpy bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return t.detach().to("cpu").numpy()


def dev_f32(v):
    return torch.tensor(np.atleast_1d(np.float32(v)), dtype=torch.float32, device="cuda:0")


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / max(np.linalg.norm(a) * np.linalg.norm(b), 1e-300))
