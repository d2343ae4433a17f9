"""Guard bands around every output and workspace of the C ABI.

Each output (and the workspace) is a view into a larger allocation whose first and last GUARD
elements hold a canary bit pattern; after the call the canaries must be intact, the inputs
unchanged, and the outputs equal bit for bit to those of the same call on plain allocations.
Shapes are ragged (sequence lengths that are not multiples of the chunk or of 16, head counts
that are not multiples of a workgroup's heads, several groups), where a masked store that
slipped would land just outside a buffer."""
import ctypes

import numpy as np
import pytest

from mamba_ssd_sequence_chunked_amd.inputs import make_random
from util import to_device

pytestmark = pytest.mark.gpu

GUARD = 1 << 16          # elements on each side
CANARY = {4: 0x7FBADBAD, 2: 0x7FAB, 1: 0xA5}


def _lib():
    import mamba_ssd_sequence_chunked_amd as ssd
    return ssd.load_library()


class Guarded:
    """An output of `shape` and `dtype` inside a canary-filled allocation."""

    def __init__(self, shape, dtype):
        import torch
        self.n = int(np.prod(shape)) if len(shape) else 1
        self.es = torch.empty((), dtype=dtype).element_size()
        raw = {4: torch.int32, 2: torch.int16, 1: torch.uint8}[self.es]
        self.buf = torch.full((self.n + 2 * GUARD,), CANARY[self.es], dtype=raw, device="cuda")
        self.t = self.buf[GUARD:GUARD + self.n].view(dtype).view(shape)

    def intact(self):
        import torch
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.n:]
        return bool(torch.all(head == CANARY[self.es])) and bool(torch.all(tail == CANARY[self.es]))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _code(dt):
    return 1 if dt == "bf16" else 0


def _inputs(b, L, H, P, N, G, Q, dt, init, seed):
    inp = make_random(b, L, H, P, N, G, Q, dt, "shifted", init, seed=seed)
    d = {k: to_device(getattr(inp, k)) for k in ("x", "dt", "A", "B", "C", "D", "init")}
    return inp, d


def _snapshot(d):
    return {k: None if v is None else v.clone() for k, v in d.items()}


def _unchanged(d, snap):
    import torch
    return all((v is None and snap[k] is None) or torch.equal(v, snap[k]) for k, v in d.items())


FWD_CASES = [
    (2, 300, 6, 64, 128, 2, 256, "bf16", True),
    (1, 77, 5, 16, 48, 1, 64, "f32", False),
    (3, 129, 3, 32, 64, 3, 32, "bf16", False),
    (1, 1000, 4, 128, 128, 1, 128, "bf16", True),
]


@pytest.mark.parametrize("c", FWD_CASES, ids=["b{}_L{}_H{}_P{}_N{}_G{}_Q{}_{}_i{}".format(*c) for c in FWD_CASES])
def test_forward_guards(c):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    b, L, H, P, N, G, Q, dt, init = c
    lib = _lib()
    inp, d = _inputs(b, L, H, P, N, G, Q, dt, init, seed=900 + FWD_CASES.index(c))
    snap = _snapshot(d)
    code = _code(dt)
    y = Guarded((b, L, H, P), d["x"].dtype)
    fin = Guarded((b, H, P, N), torch.float32)
    wsb = lib.ssd_forward_workspace_bytes(b, L, H, P, N, Q, code)
    ws = Guarded((wsb,), torch.uint8)
    print(f"ssd_forward {c}", flush=True)
    rc = lib.ssd_forward(_p(d["x"]), _p(d["dt"]), _p(d["A"]), _p(d["B"]), _p(d["C"]), _p(d["D"]), _p(d["init"]),
                         _p(y.t), _p(fin.t), b, L, H, P, N, G, Q, code, _p(ws.t), wsb, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    assert y.intact() and fin.intact() and ws.intact()
    assert _unchanged(d, snap)
    y_ref, f_ref = ssd.forward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], Q, d["init"])
    torch.cuda.synchronize()
    assert torch.equal(y.t, y_ref) and torch.equal(fin.t, f_ref)

    # the one-pass forward and the entry point on the library's own scratch, same buffers
    for name in ("ssd_forward_fused", "ssd_forward_noalloc"):
        y2 = Guarded((b, L, H, P), d["x"].dtype)
        f2 = Guarded((b, H, P, N), torch.float32)
        print(f"{name} {c}", flush=True)
        if name == "ssd_forward_fused":
            rc = lib.ssd_forward_fused(_p(d["x"]), _p(d["dt"]), _p(d["A"]), _p(d["B"]), _p(d["C"]), _p(d["D"]),
                                       _p(d["init"]), _p(y2.t), _p(f2.t), b, L, H, P, N, G, code, _stream())
        else:
            rc = lib.ssd_forward_noalloc(_p(d["x"]), _p(d["dt"]), _p(d["A"]), _p(d["B"]), _p(d["C"]), _p(d["D"]),
                                         _p(d["init"]), _p(y2.t), _p(f2.t), b, L, H, P, N, G, Q, code, _stream())
        assert rc == 0, name
        torch.cuda.synchronize()
        assert y2.intact() and f2.intact(), name
        assert _unchanged(d, snap), name
        if name == "ssd_forward_noalloc":
            assert torch.equal(y2.t, y_ref) and torch.equal(f2.t, f_ref)
        else:
            yf, ff = ssd.forward_fused(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["init"])
            torch.cuda.synchronize()
            assert torch.equal(y2.t, yf) and torch.equal(f2.t, ff)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_step_guards(dt):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    b, H, P, N, G = 5, 6, 64, 48, 2
    lib = _lib()
    inp, d = _inputs(b, 1, H, P, N, G, 16, dt, True, seed=950)
    x, dtv, Bm, Cm = d["x"][:, 0].contiguous(), d["dt"][:, 0].contiguous(), d["B"][:, 0].contiguous(), \
        d["C"][:, 0].contiguous()
    ins = dict(x=x, dt=dtv, A=d["A"], B=Bm, C=Cm, D=d["D"])
    snap = _snapshot(ins)
    st = Guarded((b, H, P, N), torch.float32)
    st.t.copy_(d["init"])
    ref_state = d["init"].clone()
    y = Guarded((b, H, P), x.dtype)
    print(f"ssd_step {dt}", flush=True)
    rc = lib.ssd_step(_p(st.t), _p(x), _p(dtv), _p(d["A"]), _p(Bm), _p(Cm), _p(d["D"]), _p(y.t), b, H, P, N, G,
                      _code(dt), _stream())
    assert rc == 0
    torch.cuda.synchronize()
    assert st.intact() and y.intact()
    assert _unchanged(ins, snap)
    y_ref = ssd.step(ref_state, x, dtv, d["A"], Bm, Cm, d["D"])
    torch.cuda.synchronize()
    assert torch.equal(y.t, y_ref) and torch.equal(st.t, ref_state)


BWD_CASES = [
    (2, 300, 6, 64, 64, 2, 128, "bf16", True, True),      # bf16, dB / dC summed in the kernels
    (1, 100, 4, 16, 32, 1, 32, "bf16", False, True),      # bf16, per-head passes
    (2, 77, 5, 32, 64, 1, 64, "f32", True, False),       # fp32 (dstate one of 16 .. 256 for the backward)
]


@pytest.mark.parametrize("c", BWD_CASES, ids=["b{}_L{}_H{}_P{}_N{}_G{}_Q{}_{}_i{}_f{}".format(*c) for c in BWD_CASES])
def test_backward_guards(c):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    b, L, H, P, N, G, Q, dt, init, dfin = c
    lib = _lib()
    inp, d = _inputs(b, L, H, P, N, G, Q, dt, init, seed=960 + BWD_CASES.index(c))
    gen = torch.Generator(device="cuda").manual_seed(5)
    d["dy"] = torch.randn((b, L, H, P), generator=gen, device="cuda").to(d["x"].dtype)
    d["dfinal"] = torch.randn((b, H, P, N), generator=gen, device="cuda") if dfin else None
    snap = _snapshot(d)
    code = _code(dt)
    T = d["x"].dtype
    outs = dict(dx=Guarded((b, L, H, P), T), ddt=Guarded((b, L, H), torch.float32), dA=Guarded((H,), torch.float32),
                dB=Guarded((b, L, G, N), T), dC=Guarded((b, L, G, N), T), dD=Guarded((H,), torch.float32),
                dinit=Guarded((b, H, P, N), torch.float32))
    wsb = lib.ssd_backward_workspace_bytes(b, L, H, P, N, G, Q, code)
    ws = Guarded((wsb,), torch.uint8)
    print(f"ssd_backward {c}", flush=True)
    rc = lib.ssd_backward(_p(d["x"]), _p(d["dt"]), _p(d["A"]), _p(d["B"]), _p(d["C"]), _p(d["D"]), _p(d["init"]),
                          _p(d["dy"]), _p(d["dfinal"]), *[_p(outs[k].t) for k in ("dx", "ddt", "dA", "dB", "dC", "dD",
                                                                                     "dinit")],
                          b, L, H, P, N, G, Q, code, _p(ws.t), wsb, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    for k, o in outs.items():
        assert o.intact(), k
    assert ws.intact()
    assert _unchanged(d, snap)
    ref = ssd.backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dy"], Q, d["init"], d["dfinal"])
    torch.cuda.synchronize()
    for k, o in outs.items():
        assert torch.equal(o.t, ref[k]), k


def test_varlen_guards():
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    lens = [1, 200, 37, 300, 64, 5]
    T, H, P, N, G, Q = sum(lens), 6, 64, 128, 2, 64
    lib = _lib()
    inp, d = _inputs(1, T, H, P, N, G, Q, "bf16", False, seed=990)
    ins = dict(x=d["x"][0].contiguous(), dt=d["dt"][0].contiguous(), A=d["A"], B=d["B"][0].contiguous(),
               C=d["C"][0].contiguous(), D=d["D"])
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    ins["cu"] = cu
    snap = _snapshot(ins)
    nseq = len(lens)
    y = Guarded((T, H, P), ins["x"].dtype)
    fin = Guarded((nseq, H, P, N), torch.float32)
    wsb = lib.ssd_forward_varlen_workspace_bytes(T, H, P, N, Q, 1)
    ws = Guarded((wsb,), torch.uint8)
    print("ssd_forward_varlen", flush=True)
    rc = lib.ssd_forward_varlen(_p(ins["x"]), _p(ins["dt"]), _p(ins["A"]), _p(ins["B"]), _p(ins["C"]), _p(ins["D"]),
                                _p(cu), nseq, _p(y.t), _p(fin.t), T, H, P, N, G, Q, 1, _p(ws.t), wsb, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    assert y.intact() and fin.intact() and ws.intact()
    assert _unchanged(ins, snap)
    y_ref, f_ref = ssd.forward_varlen(ins["x"], ins["dt"], ins["A"], ins["B"], ins["C"], ins["D"], cu, Q)
    torch.cuda.synchronize()
    assert torch.equal(y.t, y_ref) and torch.equal(fin.t, f_ref)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_selective_scan_guards(dt):
    import torch
    import mamba_ssd_sequence_chunked_amd as ssd
    b, L, Dm, N = 2, 301, 200, 16
    lib = _lib()
    rng = np.random.default_rng(995)
    x = rng.standard_normal((b, L, Dm))
    delta = np.log1p(np.exp(rng.standard_normal((b, L, Dm)) - 3.0)).astype(np.float32)
    A = -np.exp(rng.standard_normal((Dm, N)) * 0.5).astype(np.float32)
    Bm, Cm = rng.standard_normal((b, L, N)), rng.standard_normal((b, L, N))
    Dv = rng.standard_normal(Dm).astype(np.float32)
    init = rng.standard_normal((b, Dm, N)).astype(np.float32)
    T = torch.bfloat16 if dt == "bf16" else torch.float32
    ins = dict(x=torch.tensor(x, device="cuda").to(T), delta=torch.tensor(delta, device="cuda"),
               A=torch.tensor(A, device="cuda"), B=torch.tensor(Bm, device="cuda").to(T),
               C=torch.tensor(Cm, device="cuda").to(T), D=torch.tensor(Dv, device="cuda"),
               init=torch.tensor(init, device="cuda"))
    snap = _snapshot(ins)
    y = Guarded((b, L, Dm), T)
    fin = Guarded((b, Dm, N), torch.float32)
    print(f"ssd_selective_scan {dt}", flush=True)
    rc = lib.ssd_selective_scan(_p(ins["x"]), _p(ins["delta"]), _p(ins["A"]), _p(ins["B"]), _p(ins["C"]),
                                _p(ins["D"]), _p(ins["init"]), _p(y.t), _p(fin.t), b, L, Dm, N, _code(dt), _stream())
    assert rc == 0
    torch.cuda.synchronize()
    assert y.intact() and fin.intact()
    assert _unchanged(ins, snap)
    y_ref, f_ref = ssd.selective_scan(ins["x"], ins["delta"], ins["A"], ins["B"], ins["C"], ins["D"], ins["init"])
    torch.cuda.synchronize()
    assert torch.equal(y.t, y_ref) and torch.equal(fin.t, f_ref)
