"""Helpers for the GPU parity tests: host <-> device copies and strided buffers."""
import numpy as np
import torch

import workloads as wl


def require_gpu():
    assert torch.cuda.is_available(), "this test needs an MI355X; run it with -m gpu on a GPU host"
    return torch.device("cuda:0")


def to_device(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def strided_on_device(a: np.ndarray, ld: int, dev, extra_rows: int = 1, offset: int = 0):
    """Copy `a` into a device buffer with row stride ld, NaN in every gap, `extra_rows`
    NaN rows after the matrix and `offset` NaN floats before it.

    Returns (buffer, view); view has a's shape and row stride ld and starts `offset`
    floats into the buffer (offset 1 or 2 makes the start only 4-byte aligned).
    """
    buf, _ = wl.embed(a, ld, extra_rows=extra_rows)
    flat = np.concatenate([np.full(offset, np.nan, np.float32), buf.ravel()])
    dbuf = to_device(flat, dev)
    rows, cols = a.shape
    view = dbuf[offset:offset + buf.size].view(buf.shape)[:rows, :cols]
    return dbuf, view


def nan_output(rows: int, cols: int, ld: int, dev, extra_rows: int = 1):
    """A NaN-filled device buffer (rows + extra_rows) x ld and its rows x cols view."""
    buf = torch.full((rows + extra_rows, ld), float("nan"), dtype=torch.float32, device=dev)
    return buf, buf[:rows, :cols]


def outside_untouched(buf: torch.Tensor, rows: int, cols: int) -> bool:
    """True if every element of buf outside [:rows, :cols] is still NaN."""
    host = buf.cpu().numpy()
    mask = np.ones(host.shape, bool)
    mask[:rows, :cols] = False
    return bool(np.isnan(host[mask]).all())
