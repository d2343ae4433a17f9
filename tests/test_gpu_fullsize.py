"""Parity at the full workload sizes, in the launch configuration the benchmark
times (one ssd_forward over the whole batch; ssd_step over the whole decode
batch): the forward checked on every (batch, head) slice against the fp64
oracle run on the whole problem, decode on every batch row, step and head."""
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
    """1024 consecutive steps on the full (256, 80, 64, 128) fp32 state, every batch row: y of every
    (batch row, step, head) and the final state of every (batch row, head) against the oracle.  The
    oracle runs the 1024 tokens of each row as one sequence from the same initial state (a step is one
    iteration of the recurrence; that L steps equal one forward over L tokens is pinned on the CPU),
    in slices of 32 batch rows."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    from mamba_ssd_sequence_chunked_amd.inputs import bf16_to_f64
    c = CONFIGS["decode"]
    b, T, H, P, N, G = c.batch, c.seqlen, c.nheads, c.headdim, c.dstate, c.ngroups
    A, D, st0 = make_step_params("decode")
    st = to_device(st0)
    dA, dD = to_device(A), to_device(D)
    # every step's inputs as stored (bf16 bit patterns, fp32 dt), token-major per batch row for the oracle
    xs = np.empty((b, T, H, P), dtype=np.uint16)
    dts = np.empty((b, T, H), dtype=np.float32)
    Bs = np.empty((b, T, G, N), dtype=np.uint16)
    Cs = np.empty((b, T, G, N), dtype=np.uint16)
    ys = torch.empty((T, b, H, P), dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        s = make_step_inputs("decode", t)
        xs[:, t], dts[:, t], Bs[:, t], Cs[:, t] = s.x, s.dt, s.B, s.C
        ys[t] = ssd.step(st, to_device(s.x), to_device(s.dt), dA, to_device(s.B), to_device(s.C), dD)
        if t % 256 == 255:
            print(f"decode: step {t} issued", flush=True)
    torch.cuda.synchronize()
    yg = ys.view(torch.int16).cpu().numpy().view(np.uint16)          # (T, b, H, P) bf16 bits
    sg = st.cpu().numpy()
    del ys, st
    worst_y = worst_f = 0.0
    for b0 in range(0, b, 32):
        rows = slice(b0, min(b, b0 + 32))
        y_ref, f_ref = oracle.forward(bf16_to_f64(xs[rows]), dts[rows], A, bf16_to_f64(Bs[rows]),
                                      bf16_to_f64(Cs[rows]), D, st0[rows])
        got = bf16_to_f64(np.ascontiguousarray(yg[:, rows].transpose(1, 0, 2, 3)))   # (rows, T, H, P)
        # per (batch row, step, head): max |error| over the head's P outputs / max |reference| there
        err = np.max(np.abs(got - y_ref), axis=3) / np.maximum(np.max(np.abs(y_ref), axis=3), 1e-30)
        assert np.all(np.isfinite(got))
        worst_y = max(worst_y, float(np.max(err)))
        worst_f = max(worst_f, slice_rel_err(sg[rows], f_ref, 1))
        print(f"decode rows {b0}..{rows.stop - 1}: worst y err {worst_y:.3e}, final {worst_f:.3e}", flush=True)
    assert worst_y <= TOL["bf16"], worst_y
    assert worst_f <= 1e-4, worst_f
