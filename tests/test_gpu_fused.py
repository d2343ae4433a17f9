"""Parity of ssd_forward_fused (one pass over the sequence per (batch, head), the state on chip)
against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from mamba_ssd_sequence_chunked_amd.inputs import make_inputs, make_random
from util import TOL, slice_rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu

# (batch, seqlen, nheads, headdim, dstate, ngroups, dtype, init): ragged last blocks, groups, every
# head size, state widths that fill and that pad the rounded-up width (16 -> 32, 48 -> 64), up to
# the widest supported (64 x 256)
CASES = [
    (1, 100, 4, 16, 16, 1, "f32", False),
    (2, 300, 4, 32, 64, 2, "f32", True),
    (1, 33, 2, 128, 128, 1, "f32", False),
    (1, 256, 4, 64, 128, 1, "bf16", False),
    (2, 77, 6, 128, 32, 3, "bf16", True),
    (1, 1000, 4, 64, 256, 2, "bf16", True),
    (1, 200, 8, 64, 48, 4, "bf16", False),
    (1, 1, 2, 32, 16, 1, "bf16", True),
]


def _run(inp):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    d = {k: to_device(getattr(inp, k)) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    y, fin = ssd.forward_fused(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init"])
    torch.cuda.synchronize()
    return to_f64(y), to_f64(fin)


@pytest.mark.parametrize("c", CASES, ids=["b{}_L{}_H{}_P{}_N{}_G{}_{}_i{}".format(*c) for c in CASES])
def test_fused_matches_oracle(c):
    b, L, H, P, N, G, dt, init = c
    inp = make_random(b, L, H, P, N, G, 64, dt, "shifted", init, seed=900 + CASES.index(c))
    y, fin = _run(inp)
    y_ref, f_ref = oracle.forward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, inp.f64("init"))
    assert slice_rel_err(y, y_ref, 2) <= TOL[dt]
    assert slice_rel_err(fin, f_ref, 1) <= TOL[dt]


def test_fused_empty_sequence():
    """No tokens: the final state is the initial state."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    z = torch.empty((1, 0, 2, 16), device="cuda")
    zb = torch.empty((1, 0, 1, 32), device="cuda")
    init = torch.randn((1, 2, 16, 32), device="cuda")
    _, fin = ssd.forward_fused(z, torch.empty((1, 0, 2), device="cuda"), torch.full((2,), -1.0, device="cuda"), zb,
                               zb, torch.ones(2, device="cuda"), init)
    torch.cuda.synchronize()
    assert torch.equal(fin, init)


def test_fused_full_size():
    """The 2.7B-layer workload (4 x 4096 tokens, 80 heads x 64, N = 128, bf16): every (batch, head)
    slice against the oracle run on the whole problem."""
    inp = make_inputs("l2p7b")
    b, L, H, P, N, G = inp.dims
    y, fin = _run(inp)
    print("l2p7b fused: forward done, running the oracle", flush=True)
    y_ref, f_ref = oracle.forward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, inp.f64("init"))
    ey, ef = slice_rel_err(y, y_ref, 2), slice_rel_err(fin, f_ref, 1)
    print(f"l2p7b fused: worst y err over all {b * H} slices {ey:.3e}, final err {ef:.3e}")
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]
