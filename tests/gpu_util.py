"""Helpers shared by the GPU tests: device placement and the oracle's true /
naive inputs.  No attention arithmetic lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(msg):
    """Name the GPU step about to run (flushed, so a fault still shows it)."""
    print(f"[gpu-step] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def true64(x: torch.Tensor) -> np.ndarray:
    """fp32 draws promoted to fp64: the 'true' inputs."""
    return x.detach().to("cpu", torch.float64).numpy()


def naive64(x: torch.Tensor) -> np.ndarray:
    """bf16-rounded draws (nearest even) in fp64: the kernel's real inputs."""
    return x.detach().to(torch.bfloat16).to("cpu", torch.float64).numpy()


def naive16(x: torch.Tensor) -> np.ndarray:
    """fp16-rounded draws (nearest even) in fp64: the kernel's inputs on the
    fp16 path."""
    return x.detach().to(torch.float16).to("cpu", torch.float64).numpy()


def to_gpu(x: torch.Tensor, dtype) -> torch.Tensor:
    return x.to(dtype).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()
