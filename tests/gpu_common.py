"""Device helpers for the GPU tests: bf16 bit patterns <-> torch tensors."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import workloads as WL


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to("cuda")


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def say(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def candidate(name: str):
    return WL.candidate_inputs(name)
