"""Parity at the full workload sizes, in the launch configuration the benchmark
times (one ssd_forward over the whole batch; ssd_step over the whole decode
batch), checked on sampled (batch, head) slices that the fp64 oracle
computes one by one."""
import numpy as np
import pytest

import oracle
from mamba_ssd_sequence_chunked_amd.inputs import (CONFIGS, make_inputs, make_step_inputs,
                                                   make_step_params)
from util import TOL, head_slice, slice_rel_err, to_device, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _samples(b, H):
    return sorted({(0, 0), (b - 1, H - 1), (b // 2, H // 2 + 1), (0, H // 3), (b - 1, 1)})


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
    worst_y = worst_f = 0.0
    for (bi, h) in _samples(b, H):
        xs, dts, As, Bs, Cs, Ds, h0 = head_slice(inp, bi, h)
        y_ref, f_ref = oracle.forward(xs, dts, As, Bs, Cs, Ds, h0)
        ey = slice_rel_err(to_f64(y[bi:bi + 1, :, h:h + 1]), y_ref, 2)
        ef = slice_rel_err(to_f64(fin[bi:bi + 1, h:h + 1]), f_ref, 1)
        worst_y, worst_f = max(worst_y, ey), max(worst_f, ef)
    print(f"{name}: worst sampled y err {worst_y:.3e}, final err {worst_f:.3e}")
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
