"""Small conversions shared by the tests (torch tensors <-> oracle numpy arrays)."""
import sys

import numpy as np
import torch


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy; bf16 is carried as uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_np(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def say(*args):
    """Name the case before a GPU step, so a failure can be traced to it."""
    print(*args, flush=True)
    sys.stdout.flush()


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    return a.shape == b.shape and a.tobytes() == b.tobytes()
