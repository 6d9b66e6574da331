"""Helpers shared by the GPU parity tests: device transfer and bit views."""
import hashlib

import numpy as np
import torch

DEV = torch.device("cuda:0")
SENT = 0xFFFFFFFF


def dev_rows(x: np.ndarray, ld: int | None = None) -> torch.Tensor:
    """float32 rows or bfloat16 bit rows (uint16) -> device tensor [rows, ld] (pad NaN)."""
    x = np.ascontiguousarray(x)
    rows, V = x.shape
    ld = V if ld is None else ld
    if x.dtype == np.float32:
        buf = np.full((rows, ld), np.nan, np.float32)
        buf[:, :V] = x
        return torch.from_numpy(buf).to(DEV)
    assert x.dtype == np.uint16
    buf = np.full((rows, ld), 0x7FC0, np.uint16)
    buf[:, :V] = x
    return torch.from_numpy(buf.view(np.int16)).to(DEV).view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(DEV)


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def digest(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()
