"""Moves synth host arrays to and from torch device tensors (storage formats kept bit for bit)."""
import numpy as np
import torch

from . import BF16, F32, FP8, Tensor


def to_device(t: Tensor, device="cuda") -> torch.Tensor:
    if t.kind == F32:
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)
    if t.kind == BF16:
        return torch.from_numpy(np.ascontiguousarray(t.data).view(np.int16)).to(device).view(torch.bfloat16)
    if t.kind == FP8:
        return torch.from_numpy(np.ascontiguousarray(t.data)).to(device)
    raise ValueError(t.kind)


def scale_to_device(t: Tensor, device="cuda"):
    return None if t.scale is None else torch.from_numpy(np.ascontiguousarray(t.scale)).to(device)


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (fp32 or bf16)."""
    return x.detach().to("cpu").to(torch.float64).numpy()


def empty_act(kind: str, shape, device="cuda") -> torch.Tensor:
    return torch.empty(shape, dtype=torch.float32 if kind == F32 else torch.bfloat16, device=device)


def bits(x: torch.Tensor) -> np.ndarray:
    """Raw storage bits of an fp32 / bf16 device tensor (for exact placement checks)."""
    if x.dtype == torch.float32:
        return x.detach().cpu().view(torch.int32).numpy()
    return x.detach().cpu().view(torch.int16).numpy()
