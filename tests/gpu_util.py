"""Helpers for the GPU parity tests: move channel-major numpy arrays to and from
device tensors in either layout.  Data movement only."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x_ct: np.ndarray, B: int, D: int, T: int, layout: str) -> torch.Tensor:
    """[C, T] channel-major -> device tensor [B, D, T] ('bdt') or [T, B, D] ('tbd')."""
    if layout == "bdt":
        arr = np.ascontiguousarray(x_ct).reshape(B, D, T)
    else:
        arr = np.ascontiguousarray(np.asarray(x_ct).T).reshape(T, B, D)
    return torch.from_numpy(arr).to(DEV)


def from_dev(t: torch.Tensor, B: int, D: int, T: int, layout: str) -> np.ndarray:
    x = t.detach().cpu().numpy()
    if layout == "bdt":
        return x.reshape(B * D, T)
    return np.ascontiguousarray(x.reshape(T, B * D).T)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)
