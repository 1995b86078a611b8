"""Host <-> device helpers for the GPU parity tests (no method arithmetic)."""

import numpy as np
import torch

DEV = "cuda:0"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def sync():
    torch.cuda.synchronize()


def show(msg: str):
    print(msg, flush=True)
