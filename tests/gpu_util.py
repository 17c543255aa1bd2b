"""Helpers for the GPU parity tests: host numpy bytes <-> device torch buffers."""
import sys

import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    """Copy a numpy array's bytes into a new device tensor of the same shape (raw bits)."""
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.uint8).reshape(-1).copy())
    out = t.to("cuda")
    return out


def dev_like(nbytes: int, fill_byte: int = 0, align: int = 1024):
    """A device byte buffer of `nbytes` whose start is `align`-aligned (a view into a
    slightly larger allocation)."""
    raw = torch.full((nbytes + align,), fill_byte, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % align
    return raw[off:off + nbytes]


def host(t: torch.Tensor, dtype, shape=None) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.cpu().numpy().view(dtype)
    return a.reshape(shape) if shape is not None else a


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def say(*args):
    """Name the case on stdout before a GPU step (flushed), so a fault is attributable."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()
