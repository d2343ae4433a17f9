"""Parity of ssd_step (the recurrent mode) against the oracle's step, and of
step-by-step decoding against the chunked forward."""
import numpy as np
import pytest

import oracle
from mamba_ssd_sequence_chunked_amd.inputs import make_random
from util import TOL, slice_rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu

# (batch, nheads, headdim, dstate, ngroups, dtype)
CASES = [
    (3, 4, 16, 16, 1, "f32"),
    (2, 6, 32, 48, 3, "f32"),
    (4, 8, 64, 128, 1, "bf16"),
    (2, 4, 128, 256, 2, "bf16"),
    (5, 3, 64, 64, 3, "bf16"),
    (1, 2, 16, 240, 1, "f32"),
]


@pytest.mark.parametrize("c", CASES, ids=["b{}_H{}_P{}_N{}_G{}_{}".format(*c) for c in CASES])
def test_steps_match_oracle(c):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    b, H, P, N, G, dt = c
    T = 12
    inp = make_random(b, T, H, P, N, G, 16, dt, "shifted", True, seed=400 + CASES.index(c))
    st = to_device(inp.init)
    st_ref = inp.init.astype(np.float64)
    for t in range(T):
        x = to_device(np.ascontiguousarray(inp.x[:, t]))
        B = to_device(np.ascontiguousarray(inp.B[:, t]))
        C = to_device(np.ascontiguousarray(inp.C[:, t]))
        y = ssd.step(st, x, to_device(np.ascontiguousarray(inp.dt[:, t])), to_device(inp.A), B, C, to_device(inp.D))
        torch.cuda.synchronize()
        y_ref, st_ref = oracle.step(st_ref, inp.f64("x")[:, t], inp.dt[:, t], inp.A, inp.f64("B")[:, t],
                                    inp.f64("C")[:, t], inp.D)
        assert slice_rel_err(to_f64(y), y_ref, 1) <= TOL[dt], t
    assert slice_rel_err(to_f64(st), st_ref, 1) <= 1e-5


def test_step_sequence_equals_forward():
    """Decoding token by token reproduces the chunked forward (both on the GPU)."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_random(2, 70, 4, 64, 128, 2, 32, "f32", "shifted", True, seed=450)
    d = {k: to_device(getattr(inp, k)) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    y_fwd, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 32, d["init"])
    st = d["init"].clone()
    ys = []
    for t in range(70):
        ys.append(ssd.step(st, d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                           d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d["D"]))
    torch.cuda.synchronize()
    assert slice_rel_err(to_f64(torch.stack(ys, 1)), to_f64(y_fwd), 2) <= 1e-4
    assert slice_rel_err(to_f64(st), to_f64(fin), 1) <= 1e-4
