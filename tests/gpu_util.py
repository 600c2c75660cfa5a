"""Helpers of the GPU parity tests: device tensors from numpy, and the
relative-L2 metric  rel(a, b) = ||a - b|| / ||b||  with b the oracle."""

import numpy as np

from gpt_transformer_lm_amd import synthetic as S

FP32, BF16 = 0, 1


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch


def as_input(a, dtype):
    """The value the kernel sees for input a: float32, or float32 rounded to bf16."""
    a = np.asarray(a, dtype=np.float32)
    return S.bf16_round(a) if dtype == BF16 else a


def dev(a, dtype):
    """Device tensor holding as_input(a, dtype) in the storage type."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(as_input(a, dtype))).to("cuda")
    return t.to(torch.bfloat16) if dtype == BF16 else t


def dev_i32(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def empty(shape, dtype):
    torch = torch_mod()
    return torch.full(shape, float("nan"), dtype=torch.bfloat16 if dtype == BF16 else torch.float32,
                      device="cuda")


def empty32(shape, fill=float("nan")):
    torch = torch_mod()
    return torch.full(shape, fill, dtype=torch.float32, device="cuda")


def host(t):
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def say(*args):
    print(*args, flush=True)
