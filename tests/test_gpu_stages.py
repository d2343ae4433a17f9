"""Per-stage parity of the four chunked-mode kernels against the fp64 oracle.

Each stage is fed what the oracle says its inputs are wherever that is
possible (so a failure names the stage), and its output is compared element
by element with the oracle's value of the same quantity."""
import numpy as np
import pytest

import oracle
from mamba_ssd_sequence_chunked_amd.inputs import make_random
from util import TOL, device_inputs, slice_rel_err, to_f64

pytestmark = pytest.mark.gpu

# (batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, init)
CASES = [
    (1, 200, 4, 16, 16, 1, 64, "f32", False),        # ragged tail, tiny dims
    (2, 333, 6, 32, 48, 3, 32, "f32", True),          # groups, odd dstate, ragged
    (2, 300, 4, 64, 128, 2, 128, "bf16", True),       # 2.7B-like per-head dims
    (1, 520, 2, 128, 256, 1, 256, "bf16", False),     # largest tile shapes, ragged
    (1, 96, 3, 64, 64, 1, 16, "bf16", True),          # smallest chunk
]


def _ids(c):
    return "b{}_L{}_H{}_P{}_N{}_G{}_Q{}_{}{}".format(*c[:8], "_init" if c[8] else "")


@pytest.fixture(params=CASES, ids=[_ids(c) for c in CASES])
def case(request):
    b, L, H, P, N, G, Q, dt, init = request.param
    inp = make_random(b, L, H, P, N, G, Q, dt, "shifted", init, seed=100 + CASES.index(request.param))
    return inp


def test_dA_cumsum(case):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = case
    d = device_inputs(inp)
    cs, dtc = ssd.dA_cumsum(d["dt"], d["A"], inp.chunk_size)
    torch.cuda.synchronize()
    ref = oracle.chunk_log_decay(inp.dt, inp.A, inp.chunk_size)
    got = to_f64(cs)
    # fp32 prefix sums: absolute error grows with the magnitude of the running sum
    bound = 1e-5 * (1.0 + np.abs(ref))
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / (1 + np.abs(ref))))
    b, L, H = inp.dt.shape
    Q = inp.chunk_size
    nc = oracle.n_chunks(L, Q)
    dt_ref = np.zeros((b, H, nc * Q), dtype=np.float32)
    dt_ref[:, :, :L] = np.transpose(inp.dt, (0, 2, 1))
    assert np.array_equal(dtc.cpu().numpy().reshape(b, H, nc * Q), dt_ref)


def test_chunk_state(case):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = case
    d = device_inputs(inp)
    cs, dtc = ssd.dA_cumsum(d["dt"], d["A"], inp.chunk_size)
    st = ssd.chunk_state(d["x"], d["B"], dtc, cs, inp.chunk_size)
    torch.cuda.synchronize()
    ref = oracle.chunk_states(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, inp.chunk_size)
    err = slice_rel_err(to_f64(st), ref, head_axis=2)
    assert err <= TOL[inp.dtype], err


def test_state_passing(case):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = case
    d = device_inputs(inp)
    Q = inp.chunk_size
    cs, _ = ssd.dA_cumsum(d["dt"], d["A"], Q)
    # the oracle's chunk states as this stage's input
    chunk_ref = oracle.chunk_states(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"), inp.D, Q)
    st = torch.from_numpy(chunk_ref.astype(np.float32)).cuda()
    dtype = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    entry, final = ssd.state_passing(st, cs, d["init"], inp.x.shape[1], Q, dtype)
    torch.cuda.synchronize()
    entry_ref, fin_ref, _ = oracle.chunk_entry_states(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"),
                                                      inp.D, inp.f64("init"), Q)
    # entry states are rounded to T; the chain itself is fp32
    e1 = slice_rel_err(to_f64(entry), entry_ref, head_axis=2)
    e2 = slice_rel_err(to_f64(final), fin_ref, head_axis=1)
    tol_entry = TOL[inp.dtype] if inp.dtype == "bf16" else 2e-5
    assert e1 <= tol_entry, e1
    assert e2 <= 2e-5, e2


def test_chunk_scan(case):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    inp = case
    d = device_inputs(inp)
    Q = inp.chunk_size
    cs, dtc = ssd.dA_cumsum(d["dt"], d["A"], Q)
    entry_ref, _, y_ref = oracle.chunk_entry_states(inp.f64("x"), inp.dt, inp.A, inp.f64("B"), inp.f64("C"),
                                                    inp.D, inp.f64("init"), Q)
    dtype = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    entry = torch.from_numpy(entry_ref.astype(np.float32)).to("cuda", dtype=dtype)
    y = ssd.chunk_scan(d["x"], d["B"], d["C"], dtc, cs, entry, d["D"], Q)
    torch.cuda.synchronize()
    err = slice_rel_err(to_f64(y), y_ref, head_axis=2)
    assert err <= TOL[inp.dtype], err
