"""Parity at the full workload sizes, in the launch configuration the benchmark
times (one ssd_forward over the whole batch; ssd_step over the whole decode
batch): the forward checked on every (batch, head) slice against the fp64
oracle run on the whole problem, decode on sampled rows."""
import numpy as np
import pytest

import oracle
from mamba_ssd_sequence_chunked_amd.inputs import (CONFIGS, make_inputs, make_step_inputs,
                                                   make_step_params)
from util import TOL, slice_rel_err, to_device, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("name", ["l130m", "l2p7b", "long64k"])
def test_forward_full_size(name):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_inputs(name)
    b, L, H, P, N, G = inp.dims
    d = {k: to_device(getattr(inp, k)) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], inp.chunk_size, d["init"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y.float()).all()) and bool(torch.isfinite(fin).all())
    yg, fg = to_f64(y), to_f64(fin)
    del y, fin, d
    print(f"{name}: forward done, running the oracle", flush=True)
    y_ref, f_ref = oracle.forward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, inp.f64("init"))
    worst_y = slice_rel_err(yg, y_ref, 2)
    worst_f = slice_rel_err(fg, f_ref, 1)
    print(f"{name}: worst y err over all {b * H} (batch, head) slices {worst_y:.3e}, final err {worst_f:.3e}")
    assert worst_y <= TOL[inp.dtype], worst_y
    assert worst_f <= TOL[inp.dtype], worst_f


def test_decode_full_size():
    """1024 consecutive steps on the full (256, 80, 64, 128) fp32 state."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    c = CONFIGS["decode"]
    A, D, st0 = make_step_params("decode")
    rows = [0, 97, 255]
    st = to_device(st0)
    st_ref = st0[rows].astype(np.float64)
    dA, dD = to_device(A), to_device(D)
    worst = 0.0
    for t in range(c.seqlen):
        s = make_step_inputs("decode", t)
        y = ssd.step(st, to_device(s.x), to_device(s.dt), dA, to_device(s.B), to_device(s.C), dD)
        y_ref, st_ref = oracle.step(st_ref, s.f64("x")[rows], s.dt[rows], A, s.f64("B")[rows], s.f64("C")[rows], D)
        worst = max(worst, slice_rel_err(to_f64(y[rows]), y_ref, 1))
        if t % 256 == 255:
            print(f"step {t}: worst y err so far {worst:.3e}", flush=True)
    torch.cuda.synchronize()
    assert worst <= TOL["bf16"], worst
    assert slice_rel_err(to_f64(st[rows]), st_ref, 1) <= 1e-4
