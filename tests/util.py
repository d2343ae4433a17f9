"""Shared test helpers: device transfer of the seeded inputs and the parity metric."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_device(a: np.ndarray, dtype: str = "f32", device="cuda"):
    """float32 arrays -> float32 tensors; uint16 bf16 bit patterns -> bfloat16 tensors."""
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_f64(t) -> np.ndarray:
    return t.detach().to("cpu").to(dtype=__import__("torch").float64).numpy()


def device_inputs(inp, device="cuda"):
    return dict(x=to_device(inp.x, device=device), dt=to_device(inp.dt, device=device),
                A=to_device(inp.A, device=device), B=to_device(inp.B, device=device),
                C=to_device(inp.C, device=device), D=to_device(inp.D, device=device),
                init=to_device(inp.init, device=device))


def slice_rel_err(got: np.ndarray, ref: np.ndarray, head_axis: int, batch_axis: int = 0) -> float:
    """max over (batch, head) slices of max|got - ref| / max|ref| within the slice.

    The parity metric for y and for states: a normwise relative error per
    (b, h) slice, since the elementwise relative error is undefined where an
    output is near zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = np.moveaxis(got, (batch_axis, head_axis), (0, 1))
    r = np.moveaxis(ref, (batch_axis, head_axis), (0, 1))
    g = g.reshape(g.shape[0], g.shape[1], -1)
    r = r.reshape(r.shape[0], r.shape[1], -1)
    if g.shape[2] == 0:
        return 0.0
    err = np.max(np.abs(g - r), axis=2)
    den = np.maximum(np.max(np.abs(r), axis=2), 1e-30)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(err / den))


def _f64_of(inp, name, sl):
    from mamba_ssd_sequence_chunked_amd.inputs import bf16_to_f64
    a = getattr(inp, name)[sl]
    if a.dtype == np.uint16:
        return bf16_to_f64(np.ascontiguousarray(a))
    return np.ascontiguousarray(a, dtype=np.float64)


def head_slice(inp, b: int, h: int):
    """The inputs of one (batch, head) as a 1-batch, 1-head, 1-group fp64 problem
    (only that slice is converted, so it is cheap at full size)."""
    H = inp.x.shape[2]
    G = inp.B.shape[2]
    g = h // (H // G)
    return (_f64_of(inp, "x", np.s_[b:b + 1, :, h:h + 1, :]),
            _f64_of(inp, "dt", np.s_[b:b + 1, :, h:h + 1]),
            _f64_of(inp, "A", np.s_[h:h + 1]),
            _f64_of(inp, "B", np.s_[b:b + 1, :, g:g + 1, :]),
            _f64_of(inp, "C", np.s_[b:b + 1, :, g:g + 1, :]),
            _f64_of(inp, "D", np.s_[h:h + 1]),
            None if inp.init is None else _f64_of(inp, "init", np.s_[b:b + 1, h:h + 1]))
