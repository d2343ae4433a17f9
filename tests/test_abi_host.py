"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/ssd.h declares, and rejects bad arguments with the
documented status before touching any memory.

The pointers passed here are never dereferenced: every call is one that the
host-side validation must reject, so nothing is enqueued."""
import ctypes
import os
import re

import pytest

import mamba_ssd_sequence_chunked_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WS, ERR_HIP, ERR_ALIAS = 0, -1, -2, -3, -4, -5, -6
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_A-Z0-9]+)\s*\(", text)))


def fake(i):
    """A distinct, 256-aligned, never-dereferenced address."""
    return P(0x10000000 + 0x1000000 * i)


def test_library_exports_every_declared_function():
    lib = ssd.load_library()
    names = declared_functions()
    assert {"ssd_forward", "ssd_step", "ssd_forward_workspace_bytes", "ssd_status_string", "ssd_dA_cumsum",
            "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan", "ssd_selective_scan", "ssd_forward_varlen",
            "ssd_forward_varlen_workspace_bytes", "ssd_backward", "ssd_backward_workspace_bytes", "ssd_forward_fused"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} is declared in include/ssd.h but not exported"


def test_status_strings():
    for code in (OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_WS, ERR_HIP, ERR_ALIAS, -7):
        assert ssd.status_string(code).startswith("SSD_")
    assert "unknown" in ssd.status_string(123)
    assert ssd.load_library().ssd_abi_version() == 104


def test_num_chunks_and_workspace():
    assert ssd.num_chunks(4096, 256) == 16
    assert ssd.num_chunks(4097, 256) == 17
    assert ssd.num_chunks(0, 64) == 0
    assert ssd.num_chunks(-1, 64) == -1
    ws = ssd.workspace_bytes(4, 4096, 80, 64, 128, 256, 1)
    nc = 16
    expect = 2 * 4 * 80 * nc * 256 * 4 + 4 * nc * 80 * 64 * 128 * 4 + 4 * nc * 80 * 64 * 128 * 2
    assert ws == expect
    assert ssd.workspace_bytes(1, 0, 4, 16, 16, 64, 0) >= 256
    assert ssd.workspace_bytes(1, 100, 4, 48, 16, 64, 0) == 0     # headdim 48 unsupported
    assert ssd.workspace_bytes(1, 100, 4, 16, 16, 64, 7) == 0     # bad dtype


def _forward(lib, **kw):
    args = dict(x=fake(1), dt=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6), init=None, y=fake(7),
                final=fake(8), batch=2, seqlen=100, nheads=4, headdim=16, dstate=16, ngroups=1, chunk=64,
                dtype=0, ws=fake(9), ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.ssd_forward(args["x"], args["dt"], args["A"], args["B"], args["C"], args["D"], args["init"],
                           args["y"], args["final"], args["batch"], args["seqlen"], args["nheads"],
                           args["headdim"], args["dstate"], args["ngroups"], args["chunk"], args["dtype"],
                           args["ws"], args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(headdim=48), ERR_SHAPE),
    (dict(headdim=256), ERR_SHAPE),
    (dict(dstate=8), ERR_SHAPE),
    (dict(dstate=264), ERR_SHAPE),
    (dict(dstate=40), ERR_SHAPE),
    (dict(ngroups=3), ERR_SHAPE),
    (dict(ngroups=0), ERR_SHAPE),
    (dict(chunk=24), ERR_SHAPE),
    (dict(chunk=512), ERR_SHAPE),
    (dict(chunk=0), ERR_SHAPE),
    (dict(seqlen=-1), ERR_SHAPE),
    (dict(batch=-1), ERR_SHAPE),
    (dict(nheads=0), ERR_SHAPE),
    (dict(nheads=65536), ERR_SHAPE),
    (dict(batch=65536), ERR_SHAPE),
    (dict(nheads=8200, headdim=128), ERR_SHAPE),     # nheads * headdim above 2^20
    (dict(nheads=8200, ngroups=8200, dstate=256), ERR_SHAPE),   # ngroups * dstate above 2^20
    (dict(dtype=2), ERR_DTYPE),
    (dict(x=None), ERR_NULL),
    (dict(final=None), ERR_NULL),
    (dict(ws=None), ERR_NULL),
    (dict(ws_bytes=100), ERR_WS),
    (dict(y=fake(1)), ERR_ALIAS),                    # y == x
    (dict(final=P(0x10000000 + 0x1000000 * 9 + 4096)), ERR_ALIAS),   # final inside the workspace
    (dict(x=P(0x10000008)), ERR_SHAPE),             # misaligned
])
def test_forward_rejects(kw, code):
    assert _forward(ssd.load_library(), **kw) == code


def test_step_rejects():
    lib = ssd.load_library()

    def call(**kw):
        a = dict(state=fake(1), x=fake(2), dt=fake(3), A=fake(4), B=fake(5), C=fake(6), D=fake(7), y=fake(8),
                 batch=2, nheads=4, headdim=16, dstate=16, ngroups=1, dtype=1)
        a.update(kw)
        return lib.ssd_step(a["state"], a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["y"], a["batch"],
                            a["nheads"], a["headdim"], a["dstate"], a["ngroups"], a["dtype"], None)

    assert call(headdim=20) == ERR_SHAPE
    assert call(dstate=0) == ERR_SHAPE
    assert call(ngroups=3) == ERR_SHAPE
    assert call(nheads=8200, headdim=128) == ERR_SHAPE
    assert call(dtype=-1) == ERR_DTYPE
    assert call(state=None) == ERR_NULL
    assert call(y=fake(2)) == ERR_ALIAS
    assert call(state=P(0x10000004)) == ERR_SHAPE
    assert call(batch=0) == OK                     # nothing to do, nothing enqueued


def test_forward_varlen_rejects():
    lib = ssd.load_library()

    def call(**kw):
        a = dict(x=fake(1), dt=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6), cu=fake(10), nseq=3, y=fake(7),
                 final=fake(8), T=300, H=4, P=16, N=16, G=1, Q=64, dtype=0, ws=fake(9), ws_bytes=1 << 30)
        a.update(kw)
        return lib.ssd_forward_varlen(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["cu"], a["nseq"], a["y"],
                                      a["final"], a["T"], a["H"], a["P"], a["N"], a["G"], a["Q"], a["dtype"], a["ws"],
                                      a["ws_bytes"], None)

    assert call(P=48) == ERR_SHAPE
    assert call(Q=24) == ERR_SHAPE
    assert call(nseq=-1) == ERR_SHAPE
    assert call(nseq=0) == ERR_SHAPE                 # tokens but no sequences
    assert call(nseq=0, T=0) == OK                   # nothing at all
    assert call(cu=None) == ERR_NULL
    assert call(final=None) == ERR_NULL
    assert call(dtype=5) == ERR_DTYPE
    assert call(ws_bytes=64) == ERR_WS
    assert call(y=fake(1)) == ERR_ALIAS
    assert call(final=P(0x10000000 + 0x1000000 * 10)) == ERR_ALIAS   # final over cu_seqlens
    ws = lib.ssd_forward_varlen_workspace_bytes(300, 4, 16, 16, 64, 0)
    nc = 5
    up = lambda v: (v + 255) // 256 * 256    # noqa: E731
    assert ws == 2 * up(4 * nc * 64 * 4) + up(nc * 4 * 16 * 16 * 4) * 2 + up(300 * 4) + up(nc * 16)
    assert lib.ssd_forward_varlen_workspace_bytes(300, 4, 48, 16, 64, 0) == 0


def test_noalloc_rejects():
    """ssd_forward_noalloc validates on the host, and refuses before any device work a problem whose single
    batch row needs more workspace than the static scratch (fake device pointers are never touched)."""
    lib = ssd.load_library()
    assert lib.ssd_forward_noalloc_scratch_bytes() == 64 << 20
    args = [fake(i) for i in range(1, 10)]

    def call(b=2, L=100, H=4, P=64, N=128, G=1, Q=64, dtype=1):
        return lib.ssd_forward_noalloc(*args, b, L, H, P, N, G, Q, dtype, None)

    assert call(L=65536, H=80, N=256, G=8, Q=256) == -7          # one row: 2.2 GB of workspace
    assert ssd.status_string(-7).startswith("SSD_ERR_SCRATCH")
    assert call(P=48) == ERR_SHAPE
    assert call(dtype=9) == ERR_DTYPE
    assert call(b=0) == OK                                       # nothing to do, nothing enqueued


def test_fused_rejects():
    """ssd_forward_fused validates on the host before any launch (fake device pointers are never touched)."""
    lib = ssd.load_library()
    args = [fake(i) for i in range(1, 10)]
    ok = dict(b=2, L=100, H=4, P=64, N=128, G=1)
    def call(dtype=1, **kw):
        d = {**ok, **kw}
        return lib.ssd_forward_fused(*args, d["b"], d["L"], d["H"], d["P"], d["N"], d["G"], dtype, None)
    assert call(P=128, N=256) == -2            # 128 x 256 state: beyond the on-chip limit
    assert call(P=48) == -2                     # not a head size
    assert call(G=3) == -2                      # heads not divisible by groups
    assert call(dtype=7) == -3                  # dtype
    assert call(b=0) == 0                       # nothing to do


def test_backward_rejects():
    lib = ssd.load_library()
    assert lib.ssd_backward_workspace_bytes(2, 100, 4, 16, 48, 1, 64, 0) == 0      # dstate 48: not a head size
    assert lib.ssd_backward_workspace_bytes(2, 100, 4, 16, 32, 1, 64, 0) > 0
    assert 0 < lib.ssd_backward_workspace_bytes(2, 100, 4, 16, 32, 1, 64, 1) < lib.ssd_backward_workspace_bytes(
        2, 100, 4, 16, 32, 1, 64, 0)                                                # bf16: operand copies in bf16

    def call(**kw):
        a = dict(x=fake(1), dt=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6), init=None, dy=fake(7),
                 dfinal=None, dx=fake(8), ddt=fake(9), dA=fake(10), dB=fake(11), dC=fake(12), dD=fake(13),
                 dinit=fake(14), b=2, L=100, H=4, P=16, N=32, G=1, Q=64, dtype=0, ws=fake(15), ws_bytes=1 << 30)
        a.update(kw)
        return lib.ssd_backward(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"], a["dy"], a["dfinal"],
                                a["dx"], a["ddt"], a["dA"], a["dB"], a["dC"], a["dD"], a["dinit"], a["b"], a["L"], a["H"],
                                a["P"], a["N"], a["G"], a["Q"], a["dtype"], a["ws"], a["ws_bytes"], None)

    assert call(N=48) == ERR_SHAPE
    assert call(dtype=4) == ERR_DTYPE
    assert call(dinit=None) == ERR_NULL
    assert call(dy=None) == ERR_NULL
    assert call(ws_bytes=1000) == ERR_WS
    assert call(dx=fake(1)) == ERR_ALIAS
    assert call(b=0) == OK                           # nothing to do, nothing enqueued


def test_selective_scan_rejects():
    lib = ssd.load_library()

    def call(**kw):
        a = dict(x=fake(1), delta=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6), init=None, y=fake(7),
                 final=fake(8), batch=2, seqlen=100, dim=64, dstate=16, dtype=1)
        a.update(kw)
        return lib.ssd_selective_scan(a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["init"], a["y"],
                                      a["final"], a["batch"], a["seqlen"], a["dim"], a["dstate"], a["dtype"], None)

    assert call(dim=60) == ERR_SHAPE                 # not a multiple of 8
    assert call(dim=0) == ERR_SHAPE
    assert call(dstate=12) == ERR_SHAPE
    assert call(dstate=128) == ERR_SHAPE
    assert call(batch=65536) == ERR_SHAPE
    assert call(seqlen=-1) == ERR_SHAPE
    assert call(dtype=3) == ERR_DTYPE
    assert call(final=None) == ERR_NULL
    assert call(delta=None) == ERR_NULL
    assert call(y=fake(1)) == ERR_ALIAS              # y == x
    assert call(final=P(0x10000000 + 0x1000000 * 7 + 64)) == ERR_ALIAS   # final inside y
    assert call(x=P(0x10000008)) == ERR_SHAPE        # misaligned
    assert call(batch=0) == OK                       # nothing to do, nothing enqueued


def test_stage_entry_points_reject():
    lib = ssd.load_library()
    assert lib.ssd_dA_cumsum(fake(1), fake(2), fake(3), fake(4), 1, 100, 4, 20, None) == ERR_SHAPE
    assert lib.ssd_dA_cumsum(None, fake(2), fake(3), fake(4), 1, 100, 4, 64, None) == ERR_NULL
    assert lib.ssd_dA_cumsum(fake(1), fake(2), fake(1), fake(4), 1, 100, 4, 64, None) == ERR_ALIAS
    assert lib.ssd_chunk_state(fake(1), fake(2), fake(3), fake(4), fake(5), 1, 100, 4, 16, 16, 1, 64, 5,
                               None) == ERR_DTYPE
    assert lib.ssd_state_passing(fake(1), fake(2), None, fake(3), None, 1, 100, 4, 16, 16, 64, 0,
                                 None) == ERR_NULL
    assert lib.ssd_chunk_scan(fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7), fake(1), 1, 100, 4,
                              16, 16, 1, 64, 0, None) == ERR_ALIAS


def test_no_device_reports_hip_error():
    """With no GPU, a valid call reaches the runtime and reports SSD_ERR_HIP (never crashes)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path")
    assert _forward(ssd.load_library()) == ERR_HIP


def test_python_binding_validates_before_calling():
    import torch
    x = torch.zeros(1, 8, 2, 16)
    with pytest.raises(ValueError):
        ssd.forward(x, torch.zeros(1, 8, 2), torch.zeros(2), torch.zeros(1, 8, 1, 16), torch.zeros(1, 8, 1, 16),
                    torch.zeros(2), 16)        # CPU tensors are refused
