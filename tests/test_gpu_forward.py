"""Parity of ssd_forward (all four stages through the C ABI) against the fp64
oracle, plus the invariants of the chunked mode on the GPU."""
import numpy as np
import pytest

import oracle
from mamba_ssd_sequence_chunked_amd.inputs import make_inputs, make_random
from util import TOL, device_inputs, slice_rel_err, to_f64

pytestmark = pytest.mark.gpu

# (batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, dt_kind, init)
CASES = [
    (1, 512, 4, 16, 16, 1, 64, "f32", "shifted", False),     # the tiny configuration's shape
    (2, 700, 4, 32, 32, 2, 64, "f32", "shifted", True),      # ragged tail + groups + init, fp32
    (1, 1000, 3, 128, 64, 1, 128, "f32", "ranged", True),    # fp32, large headdim
    (2, 777, 8, 64, 128, 2, 256, "bf16", "shifted", True),   # several chunks + ragged tail
    (1, 1024, 4, 64, 256, 4, 256, "bf16", "ranged", False),  # dstate 256, G = H
    (3, 160, 5, 16, 48, 5, 32, "bf16", "shifted", True),
    (1, 48, 2, 64, 128, 1, 256, "bf16", "ranged", True),     # one partial chunk
    (1, 1, 2, 32, 32, 1, 16, "bf16", "shifted", True),       # a single token
    (1, 1, 2, 32, 32, 1, 16, "f32", "shifted", False),
    # chunks that are not whole 32-token stages: the last stage of every chunk is half empty
    (2, 500, 8, 64, 128, 1, 48, "bf16", "shifted", True),
    (1, 700, 4, 64, 128, 1, 176, "bf16", "ranged", False),
    # the largest head dimension with the largest state
    (1, 300, 3, 128, 256, 1, 256, "bf16", "shifted", True),
    (2, 200, 2, 128, 256, 2, 128, "f32", "shifted", True),
]


def _ids(c):
    return "b{}_L{}_H{}_P{}_N{}_G{}_Q{}_{}_{}{}".format(*c[:9], "_init" if c[9] else "")


def run_forward(inp):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    d = device_inputs(inp)
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], inp.chunk_size, d["init"])
    torch.cuda.synchronize()
    return y, fin


@pytest.mark.parametrize("c", CASES, ids=[_ids(c) for c in CASES])
def test_forward_matches_oracle(c):
    inp = make_random(*c, seed=200 + CASES.index(c))
    y, fin = run_forward(inp)
    y_ref, fin_ref = oracle.forward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, inp.f64("init"))
    ey = slice_rel_err(to_f64(y), y_ref, head_axis=2)
    ef = slice_rel_err(to_f64(fin), fin_ref, head_axis=1)
    print(f"{_ids(c)}: y err {ey:.3e}  final err {ef:.3e}")
    assert ey <= TOL[inp.dtype], ey
    assert ef <= TOL[inp.dtype], ef


def test_tiny_configuration():
    inp = make_inputs("tiny")
    y, fin = run_forward(inp)
    y_ref, fin_ref = oracle.forward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, None)
    assert slice_rel_err(to_f64(y), y_ref, 2) <= 1e-4
    assert slice_rel_err(to_f64(fin), fin_ref, 1) <= 1e-4


@pytest.mark.parametrize("Q", [16, 32, 48, 64, 80, 112, 128, 208, 240, 256])
def test_chunk_size_invariance(Q):
    """The chunk size changes how the work is blocked, not the result."""
    inp = make_random(2, 600, 4, 64, 64, 2, Q, "f32", "shifted", True, seed=300)
    y, fin = run_forward(inp)
    y_ref, fin_ref = oracle.forward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, inp.f64("init"))
    assert slice_rel_err(to_f64(y), y_ref, 2) <= 1e-4
    assert slice_rel_err(to_f64(fin), fin_ref, 1) <= 1e-4


def test_split_and_resume():
    """forward(x[:L1]) then forward(x[L1:], init=final) equals one pass."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_random(2, 900, 4, 64, 128, 1, 256, "bf16", "shifted", True, seed=301)
    d = device_inputs(inp)
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 256, d["init"])
    L1 = 333
    ya, fa = ssd.forward(d["x"][:, :L1].contiguous(), d["dt"][:, :L1].contiguous(), d["A"], d["B"][:, :L1].contiguous(),
                         d["C"][:, :L1].contiguous(), d["D"], 256, d["init"])
    yb, fb = ssd.forward(d["x"][:, L1:].contiguous(), d["dt"][:, L1:].contiguous(), d["A"], d["B"][:, L1:].contiguous(),
                         d["C"][:, L1:].contiguous(), d["D"], 256, fa)
    torch.cuda.synchronize()
    y2 = torch.cat([ya, yb], dim=1)
    assert slice_rel_err(to_f64(y2), to_f64(y), 2) <= 2e-2
    assert slice_rel_err(to_f64(fb), to_f64(fin), 1) <= 2e-2


def test_deterministic():
    """No atomics on the path: two runs are bitwise identical."""
    import torch
    inp = make_random(2, 1000, 8, 64, 128, 1, 256, "bf16", "ranged", True, seed=302)
    y1, f1 = run_forward(inp)
    y2, f2 = run_forward(inp)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_empty_sequence_returns_initial_state():
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_random(2, 0, 4, 32, 32, 1, 64, "bf16", "shifted", True, seed=303)
    d = device_inputs(inp)
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64, d["init"])
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(fin, d["init"])
    _, fin0 = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin0).item() == 0


def test_zero_batch_is_a_no_op():
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_random(0, 64, 2, 16, 16, 1, 16, "f32", "shifted", False, seed=304)
    d = device_inputs(inp)
    y, fin = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 16, None)
    torch.cuda.synchronize()
    assert y.shape == (0, 64, 2, 16) and fin.shape == (0, 2, 16, 16)


def test_causality_on_gpu():
    """Changing x at t0 leaves y[:t0] bit-identical (the kernels read no future token)."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_random(1, 600, 4, 64, 128, 1, 256, "bf16", "shifted", False, seed=305)
    d = device_inputs(inp)
    y1, _ = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 256, None)
    x2 = d["x"].clone()
    t0 = 300
    x2[:, t0:] = 0
    y2, _ = ssd.forward(x2, d["dt"], d["A"], d["B"], d["C"], d["D"], 256, None)
    torch.cuda.synchronize()
    assert torch.equal(y1[:, :t0], y2[:, :t0])
    assert not torch.equal(y1[:, t0:], y2[:, t0:])


def test_linear_attention_case_on_gpu():
    """A = 0 (unit decay) is causal linear attention; compare with that closed form."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_random(1, 300, 2, 32, 32, 1, 64, "f32", "shifted", False, seed=306)
    inp.A[:] = 0.0
    d = device_inputs(inp)
    y, _ = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64, None)
    torch.cuda.synchronize()
    X, Bm, Cm = inp.f64("x"), inp.f64("B"), inp.f64("C")
    dt = inp.dt.astype(np.float64)
    ref = np.empty_like(X)
    for h in range(2):
        V = dt[0, :, h, None] * X[0, :, h, :]
        ref[0, :, h, :] = np.tril(Cm[0, :, 0, :] @ Bm[0, :, 0, :].T) @ V + inp.D[h] * X[0, :, h, :]
    assert slice_rel_err(to_f64(y), ref, 2) <= 1e-4


def test_nan_in_x_reach():
    """A NaN in x at token t0, head h, column p of the head reaches y[:, h, p] from the first token
    of t0's 32-token block within its chunk on, not only from t0 on as in the recurrence: the block's
    masked scores are zero and zero times NaN is NaN on the matrix cores.  Nothing else changes: y
    before that block, the other columns and the other heads stay bit-identical, y[t0:, h, p] is NaN,
    and of the final state only row p of head h."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = make_random(1, 700, 4, 64, 128, 1, 256, "bf16", "shifted", True, seed=307)
    d = device_inputs(inp)
    y1, f1 = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 256, d["init"])
    t0, h, p = 256 + 77, 2, 5                 # token 77 of the second chunk: its block is tokens 64..95
    x2 = d["x"].clone()
    x2[0, t0, h, p] = float("nan")
    y2, f2 = ssd.forward(x2, d["dt"], d["A"], d["B"], d["C"], d["D"], 256, d["init"])
    torch.cuda.synchronize()
    first = 256 + 64
    keep = torch.ones_like(y1, dtype=torch.bool)
    keep[0, first:, h, p] = False
    assert torch.equal(y1[keep], y2[keep])
    assert bool(torch.isnan(y2[0, t0:, h, p]).all())
    fkeep = torch.ones_like(f1, dtype=torch.bool)
    fkeep[0, h, p] = False
    assert torch.equal(f1[fkeep], f2[fkeep])
    assert bool(torch.isnan(f2[0, h, p]).all())
