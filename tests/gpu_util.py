"""Shared helpers for the GPU parity tests (device transfer, guards, gates)."""

from __future__ import annotations

import numpy as np

GEMV_TOL = 2e-3   # floored elementwise relative error vs the fp64 oracle


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev):
    import torch
    a = np.array(a, copy=True, order="C")
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def guarded(shape, dtype, dev, pad=64, fill=float("nan")):
    """A tensor view with `pad` guard elements on each side, all set to `fill`.

    Returns (view, buffer); check_guards(buffer, view, pad) verifies them afterwards.
    """
    import torch
    count = int(np.prod(shape))
    buf = torch.full((count + 2 * pad,), fill, dtype=dtype, device=dev)
    return buf[pad:pad + count].view(*shape), buf


def guards_intact(buf, pad=64) -> bool:
    import torch
    head, tail = buf[:pad], buf[-pad:]
    if buf.dtype.is_floating_point:
        return bool(torch.isnan(head).all() and torch.isnan(tail).all())
    return bool((head == head[0]).all() and (tail == tail[0]).all())


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()
