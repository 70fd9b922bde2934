"""Host <-> device helpers for the GPU tests (plumbing only)."""
import numpy as np
import torch

DEV = "cuda:0"


def up(a: np.ndarray) -> torch.Tensor:
    """Copy a host array to a new device tensor with the same bytes."""
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint64): np.int64,
            np.dtype(np.uint8): np.uint8, np.dtype(np.uint32): np.int32}[a.dtype]
    return torch.from_numpy(a.view(view)).to(DEV)


def down(t: torch.Tensor, dtype) -> np.ndarray:
    """Copy a device tensor back as a host array of `dtype` (same bytes)."""
    torch.cuda.synchronize()
    return t.cpu().numpy().view(dtype)


def filled(n: int, value: int, torch_dtype=torch.int16) -> torch.Tensor:
    v = value if value < 0x8000 or torch_dtype != torch.int16 else value - 0x10000
    return torch.full((n,), v, dtype=torch_dtype, device=DEV)
