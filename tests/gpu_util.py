"""Helpers for the GPU tests: host arrays <-> device tensors, and the case
banner printed (and flushed) before each GPU step."""

import sys

import numpy as np
import torch


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()
