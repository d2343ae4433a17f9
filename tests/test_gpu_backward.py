"""Parity of the backward pass (ssd_backward) against the fp64 oracle's gradients."""
import numpy as np
import pytest

import oracle
from mamba_ssd_sequence_chunked_amd.inputs import make_inputs, make_random
from util import TOL, slice_rel_err, to_device, to_f64

pytestmark = pytest.mark.gpu

# (batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, init, dfinal): ragged last chunks,
# groups, every head size, dstate up to 256 (computed in two halves), with and without the
# initial state and the final-state gradient
CASES = [
    (1, 64, 2, 16, 16, 1, 16, "f32", False, False),
    (2, 100, 4, 16, 32, 2, 32, "f32", True, True),
    (2, 300, 4, 32, 64, 1, 64, "f32", True, True),
    (1, 256, 4, 64, 128, 1, 256, "bf16", False, True),
    (1, 200, 4, 64, 256, 2, 128, "bf16", True, False),
    (2, 77, 6, 128, 16, 3, 64, "f32", False, True),
    (1, 1000, 4, 64, 128, 1, 256, "bf16", True, True),
    # bf16 shapes for the in-kernel group sums of dB / dC: every head size, state width and chunk
    # multiple of 64, groups, and 32 heads per group (partial sums over two slices of the heads)
    (1, 300, 32, 32, 64, 1, 64, "bf16", True, True),
    (2, 200, 6, 128, 32, 3, 192, "bf16", False, True),
    (1, 130, 4, 32, 16, 2, 64, "bf16", True, False),
    # and one the per-head passes take (chunk not a multiple of 64, head size 16)
    (1, 100, 4, 16, 32, 1, 32, "bf16", False, True),
    # longer than one 4096-token pass of the suffix-sum kernel, with a chunk (192 tokens) that
    # straddles the pass boundary: the per-chunk restart carried across passes
    (1, 4500, 2, 16, 32, 1, 192, "f32", True, True),
    (1, 4500, 2, 32, 32, 1, 192, "bf16", False, True),
    # one chunk with both boundary values from the states (initial state and final-state gradient);
    # chunk 16 over 5000 tokens (256 chunks per pass of the scan); chunk 48 (passes of 4080 tokens)
    (1, 200, 4, 32, 64, 1, 256, "f32", True, True),
    (1, 5000, 2, 16, 16, 1, 16, "f32", True, True),
    (1, 4200, 2, 16, 32, 1, 48, "bf16", True, True),
    # one head per group (the one-head launch shape; group sums of a single head)
    (1, 300, 4, 64, 64, 4, 64, "bf16", True, True),
    (2, 150, 3, 32, 32, 3, 32, "f32", False, True),
    # the largest head dimension with the largest state
    (1, 150, 2, 128, 256, 1, 64, "bf16", True, True),
    (1, 100, 2, 128, 256, 1, 32, "f32", True, True),
]


def _grads(inp, dy, dfin):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    d = {k: to_device(getattr(inp, k)) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    g = ssd.backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], to_device(dy), inp.chunk_size, d["init"],
                     None if dfin is None else to_device(dfin))
    torch.cuda.synchronize()
    return {k: to_f64(v) for k, v in g.items()}


def _rel_all(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


@pytest.mark.parametrize("c", CASES, ids=["b{}_L{}_H{}_P{}_N{}_G{}_Q{}_{}_i{}_f{}".format(*c) for c in CASES])
def test_backward_matches_oracle(c):
    b, L, H, P, N, G, Q, dt, init, dfin = c
    inp = make_random(b, L, H, P, N, G, Q, dt, "shifted", init, seed=800 + CASES.index(c))
    rng = np.random.default_rng(850 + CASES.index(c))
    dy64 = rng.standard_normal((b, L, H, P))
    from mamba_ssd_sequence_chunked_amd.inputs import bf16_bits, bf16_to_f64
    dy = bf16_bits(dy64) if dt == "bf16" else dy64.astype(np.float32)
    dyf = bf16_to_f64(dy) if dt == "bf16" else dy.astype(np.float64)
    dfinal = (0.3 * rng.standard_normal((b, H, P, N))).astype(np.float32) if dfin else None
    g = _grads(inp, dy, dfinal)
    r = oracle.backward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, inp.f64("init"), dyf, dfinal)
    tol = TOL[dt]
    print("errors: " + ", ".join(f"{k} {slice_rel_err(g[k] if k != 'ddt' else g[k][..., None], r[k] if k != 'ddt' else r[k][..., None], 1 if k == 'dinit' else 2):.2e}"
                                 for k in ("dx", "ddt", "dB", "dC", "dinit")))
    assert slice_rel_err(g["dx"], r["dx"], 2) <= tol, "dx"
    assert slice_rel_err(g["ddt"][..., None], r["ddt"][..., None], 2) <= tol, "ddt"
    assert slice_rel_err(g["dB"], r["dB"], 2) <= tol, "dB"
    assert slice_rel_err(g["dC"], r["dC"], 2) <= tol, "dC"
    assert slice_rel_err(g["dinit"], r["dinit"], 1) <= tol, "dinit"
    # dA (one value per head) at the stated bar, normwise over the heads; its error relative to the
    # size of the per-token products it is summed from is printed beside it
    print(f"dA: normwise {_rel_all(g['dA'], r['dA']):.3e}, "
          f"of its terms' size {np.max(np.abs(g['dA'] - r['dA']) / r['dA_scale']):.3e}")
    assert _rel_all(g["dA"], r["dA"]) <= tol, "dA"
    assert _rel_all(g["dD"], r["dD"]) <= tol, "dD"


def test_backward_tiny_workload():
    """The small workload (1 x 512 tokens, 4 heads, P = N = 16, chunk 64, fp32): its dA is ~25 000 times
    smaller than the per-token products it is formed from, the hardest case here for dA's bar."""
    inp = make_inputs("tiny")
    dy = np.random.default_rng(11).standard_normal(inp.x.shape).astype(np.float32)
    g = _grads(inp, dy, None)
    r = oracle.backward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, None, dy.astype(np.float64))
    tol = TOL["f32"]
    assert slice_rel_err(g["dx"], r["dx"], 2) <= tol, "dx"
    assert slice_rel_err(g["ddt"][..., None], r["ddt"][..., None], 2) <= tol, "ddt"
    assert slice_rel_err(g["dB"], r["dB"], 2) <= tol, "dB"
    assert slice_rel_err(g["dC"], r["dC"], 2) <= tol, "dC"
    print(f"dA: normwise {_rel_all(g['dA'], r['dA']):.3e}, "
          f"of its terms' size {np.max(np.abs(g['dA'] - r['dA']) / r['dA_scale']):.3e}")
    assert _rel_all(g["dA"], r["dA"]) <= tol, "dA"
    assert _rel_all(g["dD"], r["dD"]) <= tol, "dD"


def test_backward_empty_sequence():
    """No tokens: the initial state's gradient is the final state's, the rest is zero-sized or zero."""
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    z = torch.empty((1, 0, 2, 16), device="cuda")
    zb = torch.empty((1, 0, 1, 16), device="cuda")
    dfin = torch.randn((1, 2, 16, 16), device="cuda")
    g = ssd.backward(z, torch.empty((1, 0, 2), device="cuda"), torch.full((2,), -1.0, device="cuda"), zb, zb,
                     torch.ones(2, device="cuda"), z, 64, None, dfin)
    torch.cuda.synchronize()
    assert torch.equal(g["dinit"], dfin)
    assert torch.all(g["dA"] == 0) and torch.all(g["dD"] == 0)


def test_backward_full_size():
    """The 2.7B-layer shape (4 x 4096 tokens, 80 heads, N = 128, bf16) in the benchmark's launch
    configuration (dB and dC summed over the 80 heads in the kernels, four head slices): every
    gradient against the oracle run on the whole problem, at the small cases' bars."""
    inp = make_inputs("l2p7b")
    b, L, H, P, N, G = inp.dims
    rng = np.random.default_rng(870)
    from mamba_ssd_sequence_chunked_amd.inputs import bf16_bits, bf16_to_f64
    dy = bf16_bits(rng.standard_normal((b, L, H, P)))
    g = _grads(inp, dy, None)
    print("l2p7b backward: gradients computed, running the oracle", flush=True)
    r = oracle.backward(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, inp.f64("init"),
                        bf16_to_f64(dy), None)
    tol = TOL["bf16"]
    assert slice_rel_err(g["dx"], r["dx"], 2) <= tol, "dx"
    assert slice_rel_err(g["ddt"][..., None], r["ddt"][..., None], 2) <= tol, "ddt"
    assert slice_rel_err(g["dB"], r["dB"], 2) <= tol, "dB"
    assert slice_rel_err(g["dC"], r["dC"], 2) <= tol, "dC"
    assert slice_rel_err(g["dinit"], r["dinit"], 1) <= tol, "dinit"
    print(f"dA: normwise {_rel_all(g['dA'], r['dA']):.3e}, "
          f"of its terms' size {np.max(np.abs(g['dA'] - r['dA']) / r['dA_scale']):.3e}")
    assert _rel_all(g["dA"], r["dA"]) <= tol, "dA"
    assert _rel_all(g["dD"], r["dD"]) <= tol, "dD"
