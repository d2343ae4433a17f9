"""Parity of the packed variable-length forward (state reset at every sequence start) against
the fp64 oracle, run on every sequence alone."""
import numpy as np
import pytest

import oracle
from mamba_ssd_sequence_chunked_amd.inputs import make_random, make_varlen, make_varlen_inputs
from util import TOL, slice_rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu

# (lengths, nheads, headdim, dstate, ngroups, chunk, dtype): sequences inside one chunk, across
# chunk borders, starting exactly at a chunk start, single tokens, empty sequences, ragged ends
CASES = [
    ([100, 1, 37, 256, 5], 4, 16, 16, 1, 64, "f32"),
    ([64, 64, 64], 2, 32, 32, 1, 64, "f32"),
    ([0, 10, 0, 200, 3, 0], 4, 32, 32, 2, 32, "f32"),
    ([257, 511, 1], 8, 64, 128, 2, 256, "bf16"),
    ([300], 4, 64, 64, 1, 128, "bf16"),
    (list(np.random.default_rng(7).integers(1, 13, 40)), 8, 64, 128, 1, 64, "bf16"),
    ([5, 700, 33, 129], 6, 128, 256, 3, 256, "bf16"),
    ([17, 48, 95], 3, 16, 48, 3, 16, "f32"),
    # chunks that are not whole 32-token stages, sequences starting inside the half-empty last stage
    ([300, 7, 150, 81, 1], 4, 64, 128, 1, 80, "bf16"),
    ([90, 250, 33], 2, 32, 64, 1, 208, "f32"),
]


def _run(inp):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    d = {k: to_device(getattr(inp, k)) for k in ("x", "dt", "A", "B", "C", "D")}
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    y, fin = ssd.forward_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], cu, inp.chunk_size)
    torch.cuda.synchronize()
    return to_f64(y), to_f64(fin)


def _check(y, fin, y_ref, fin_ref, cu, tol):
    for k in range(len(cu) - 1):
        a, e = int(cu[k]), int(cu[k + 1])
        if e > a:
            assert slice_rel_err(y[None, a:e], y_ref[None, a:e], 2) <= tol, f"y of sequence {k}"
        else:
            assert np.all(fin[k] == 0.0), f"final state of empty sequence {k}"
    nonempty = [k for k in range(len(cu) - 1) if cu[k + 1] > cu[k]]
    assert slice_rel_err(fin[nonempty], fin_ref[nonempty], 1) <= tol


@pytest.mark.parametrize("c", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_varlen_matches_oracle(c):
    lens, H, P, N, G, Q, dt = c
    inp = make_varlen(lens, H, P, N, G, Q, dt, "shifted", seed=700 + CASES.index(c))
    y, fin = _run(inp)
    y_ref, fin_ref = oracle.forward_varlen(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D,
                                           inp.cu_seqlens)
    _check(y, fin, y_ref, fin_ref, inp.cu_seqlens, TOL[dt])


def test_varlen_equal_lengths_match_batched_forward():
    """Equal-length sequences packed end to end give what the batched forward gives (GPU vs GPU)."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_random(3, 320, 4, 32, 64, 2, 64, "f32", "shifted", False, seed=760)
    d = {k: to_device(getattr(inp, k)) for k in ("x", "dt", "A", "B", "C", "D")}
    yb, fb = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64)
    cu = torch.tensor([0, 320, 640, 960], dtype=torch.int32, device="cuda")
    yv, fv = ssd.forward_varlen(d["x"].reshape(960, 4, 32), d["dt"].reshape(960, 4), d["A"],
                                d["B"].reshape(960, 2, 64), d["C"].reshape(960, 2, 64), d["D"], cu, 64)
    torch.cuda.synchronize()
    assert slice_rel_err(to_f64(yv).reshape(3, 320, 4, 32), to_f64(yb), 2) <= 1e-5
    assert slice_rel_err(to_f64(fv), to_f64(fb), 1) <= 1e-5


def test_varlen_no_tokens():
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    z = torch.empty((0, 2, 16), device="cuda")
    zb = torch.empty((0, 1, 16), device="cuda")
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    A = torch.full((2,), -1.0, device="cuda")
    y, fin = ssd.forward_varlen(z, torch.empty((0, 2), device="cuda"), A, zb, zb, torch.ones(2, device="cuda"), cu, 64)
    torch.cuda.synchronize()
    assert y.shape == (0, 2, 16) and fin.shape == (2, 2, 16, 16) and torch.all(fin == 0)


def test_varlen_full_size():
    """The 2.7B-layer shape over 16384 packed tokens of mixed lengths (the benchmark's launch
    configuration), every head of every sequence checked against the oracle run on each sequence."""
    inp = make_varlen_inputs("varlen2p7b")
    y, fin = _run(inp)
    print(f"varlen2p7b: {len(inp.cu_seqlens) - 1} sequences, GPU done, running the oracle", flush=True)
    y_ref, fin_ref = oracle.forward_varlen(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D,
                                           inp.cu_seqlens)
    _check(y, fin, y_ref, fin_ref, inp.cu_seqlens, TOL["bf16"])
