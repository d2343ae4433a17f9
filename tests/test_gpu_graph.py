"""The forward and the recurrent step captured in a HIP graph and replayed.

The no-allocation forward (static scratch, outputs passed in) and ssd_step (state updated in place,
y passed in) launch kernels only, so both can be recorded by stream capture.  Each graph is replayed
several times on new inputs copied into its input buffers, with eager work and synchronisations
between the replays, and every replay is compared bit for bit with the same calls made eagerly."""
import numpy as np
import pytest

from mamba_ssd_sequence_chunked_amd.inputs import make_random
from util import device_inputs

pytestmark = pytest.mark.gpu


def test_forward_noalloc_in_graph():
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    shape = (2, 700, 8, 64, 128, 1, 256, "bf16")
    inp = make_random(*shape, "shifted", True, seed=1200)
    d = device_inputs(inp)
    y = torch.empty_like(d["x"])
    fin = torch.empty_like(d["init"])
    args = lambda: (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], inp.chunk_size, d["init"])
    ssd.forward_noalloc(*args(), y=y, final_states=fin)      # eager first call: the scratch is looked up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ssd.forward_noalloc(*args(), y=y, final_states=fin)
    torch.cuda.synchronize()
    for k in range(3):
        new = make_random(*shape, "shifted", True, seed=1201 + k)
        nd = device_inputs(new)
        for key in ("x", "dt", "B", "C", "init"):
            d[key].copy_(nd[key])
        torch.cuda.synchronize()
        y_ref, fin_ref = ssd.forward(*args())                  # eager, plain allocations
        torch.cuda.synchronize()
        y.zero_()
        fin.zero_()
        print(f"forward graph replay {k}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), k
        assert torch.equal(fin, fin_ref), k


def test_decode_steps_in_graph():
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    b, H, P, N, G, T = 16, 8, 64, 128, 2, 8
    rng = np.random.default_rng(1300)
    dev = "cuda"
    A = torch.tensor(-np.exp(rng.uniform(0, np.log(16), H)), dtype=torch.float32, device=dev)
    D = torch.tensor(rng.standard_normal(H), dtype=torch.float32, device=dev)
    state = torch.empty((b, H, P, N), device=dev)
    xs = torch.empty((T, b, H, P), dtype=torch.bfloat16, device=dev)
    dts = torch.empty((T, b, H), device=dev)
    Bs = torch.empty((T, b, G, N), dtype=torch.bfloat16, device=dev)
    Cs = torch.empty((T, b, G, N), dtype=torch.bfloat16, device=dev)
    ys = torch.empty((T, b, H, P), dtype=torch.bfloat16, device=dev)

    def fill(seed):
        r = np.random.default_rng(seed)
        state.copy_(torch.tensor(0.1 * r.standard_normal((b, H, P, N)), dtype=torch.float32))
        xs.copy_(torch.tensor(r.standard_normal((T, b, H, P)), dtype=torch.float32).to(torch.bfloat16))
        dts.copy_(torch.tensor(np.log1p(np.exp(r.standard_normal((T, b, H)) - 2.0)), dtype=torch.float32))
        Bs.copy_(torch.tensor(r.standard_normal((T, b, G, N)) / np.sqrt(N), dtype=torch.float32).to(torch.bfloat16))
        Cs.copy_(torch.tensor(r.standard_normal((T, b, G, N)) / np.sqrt(N), dtype=torch.float32).to(torch.bfloat16))

    def steps():
        for t in range(T):
            ssd.step(state, xs[t], dts[t], A, Bs[t], Cs[t], D, y=ys[t])

    fill(1301)
    steps()                                                    # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    torch.cuda.synchronize()
    for k in range(3):
        fill(1310 + k)
        torch.cuda.synchronize()
        s0 = state.clone()
        steps()                                                # eager from the same start
        torch.cuda.synchronize()
        y_ref, st_ref = ys.clone(), state.clone()
        state.copy_(s0)
        ys.zero_()
        torch.cuda.synchronize()
        print(f"decode graph replay {k}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, y_ref), k
        assert torch.equal(state, st_ref), k
