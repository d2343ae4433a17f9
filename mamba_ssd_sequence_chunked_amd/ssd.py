"""Python binding of the C ABI in include/ssd.h (ctypes).

Argument marshalling only: shapes, dtypes, devices and contiguity are
checked, outputs and the workspace are allocated with torch on the
tensors' device, and the C entry point is called on torch's current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

from ._build import LIB_PATH

SSD_F32, SSD_BF16 = 0, 1
_STATUS_OK = 0

_lib = None


class SSDError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}")


def load_library():
    """Load libssd_mi355x.so (built by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"the SSD HIP library is not built ({LIB_PATH} missing); run __graft_entry__.build() "
            "or python -m mamba_ssd_sequence_chunked_amd._build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i64, i32, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [i32]
    lib.ssd_abi_version.restype = i32
    lib.ssd_abi_version.argtypes = []
    lib.ssd_num_chunks.restype = i64
    lib.ssd_num_chunks.argtypes = [i64, i64]
    lib.ssd_forward_workspace_bytes.restype = sz
    lib.ssd_forward_workspace_bytes.argtypes = [i64] * 6 + [i32]
    lib.ssd_forward.restype = i32
    lib.ssd_forward.argtypes = [vp] * 9 + [i64] * 7 + [i32, vp, sz, vp]
    lib.ssd_forward_noalloc.restype = i32
    lib.ssd_forward_noalloc.argtypes = [vp] * 9 + [i64] * 7 + [i32, vp]
    lib.ssd_forward_noalloc_scratch_bytes.restype = sz
    lib.ssd_forward_noalloc_scratch_bytes.argtypes = []
    lib.ssd_forward_fused.restype = i32
    lib.ssd_forward_fused.argtypes = [vp] * 9 + [i64] * 6 + [i32, vp]
    lib.ssd_dA_cumsum.restype = i32
    lib.ssd_dA_cumsum.argtypes = [fp] * 4 + [i64] * 4 + [vp]
    lib.ssd_chunk_state.restype = i32
    lib.ssd_chunk_state.argtypes = [vp] * 5 + [i64] * 7 + [i32, vp]
    lib.ssd_state_passing.restype = i32
    lib.ssd_state_passing.argtypes = [vp] * 5 + [i64] * 6 + [i32, vp]
    lib.ssd_chunk_scan.restype = i32
    lib.ssd_chunk_scan.argtypes = [vp] * 8 + [i64] * 7 + [i32, vp]
    lib.ssd_step.restype = i32
    lib.ssd_step.argtypes = [vp] * 8 + [i64] * 5 + [i32, vp]
    lib.ssd_forward_varlen_workspace_bytes.restype = sz
    lib.ssd_forward_varlen_workspace_bytes.argtypes = [i64] * 5 + [i32]
    lib.ssd_forward_varlen.restype = i32
    lib.ssd_forward_varlen.argtypes = [vp] * 7 + [i64] + [vp] * 2 + [i64] * 6 + [i32, vp, sz, vp]
    lib.ssd_backward_workspace_bytes.restype = sz
    lib.ssd_backward_workspace_bytes.argtypes = [i64] * 7 + [i32]
    lib.ssd_backward.restype = i32
    lib.ssd_backward.argtypes = [vp] * 16 + [i64] * 7 + [i32, vp, sz, vp]
    lib.ssd_selective_scan.restype = i32
    lib.ssd_selective_scan.argtypes = [vp] * 9 + [i64] * 4 + [i32, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssd_status_string(int(status)).decode()


def _check(fn: str, rc: int):
    if rc != _STATUS_OK:
        raise SSDError(fn, rc)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    raise ValueError(f"x/B/C must be float32 or bfloat16, got {t.dtype}")


def _need(t: Optional[torch.Tensor], name: str, shape, dtype, device) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def num_chunks(seqlen: int, chunk_size: int) -> int:
    return int(load_library().ssd_num_chunks(seqlen, chunk_size))


def workspace_bytes(batch, seqlen, nheads, headdim, dstate, chunk_size, dtype_code) -> int:
    return int(load_library().ssd_forward_workspace_bytes(batch, seqlen, nheads, headdim, dstate,
                                                          chunk_size, dtype_code))


def _forward_dims(x, B):
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be (batch, seqlen, nheads, headdim) and B, C (batch, seqlen, ngroups, dstate)")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return b, L, H, P, N, G


def forward(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
            D: torch.Tensor, chunk_size: int, init_states: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked (dual) mode: returns (y, final_states); see ssd_forward in include/ssd.h."""
    lib = load_library()
    b, L, H, P, N, G = _forward_dims(x, B)
    dev = x.device
    code = _dtype_code(x)
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    _need(D, "D", (H,), torch.float32, dev)
    if init_states is not None:
        _need(init_states, "init_states", (b, H, P, N), torch.float32, dev)
    y = torch.empty_like(x)
    final = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    ws_bytes = lib.ssd_forward_workspace_bytes(b, L, H, P, N, chunk_size, code)
    if ws_bytes == 0:
        _check("ssd_forward", -2)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rc = lib.ssd_forward(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_states), _ptr(y),
                         _ptr(final), b, L, H, P, N, G, chunk_size, code, _ptr(workspace),
                         workspace.numel(), _stream(dev))
    _check("ssd_forward", rc)
    return y, final


def forward_noalloc(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                    D: torch.Tensor, chunk_size: int, init_states: Optional[torch.Tensor] = None,
                    y: Optional[torch.Tensor] = None,
                    final_states: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """ssd_forward on the library's static scratch (no workspace; see ssd_forward_noalloc in
    include/ssd.h).  y and final_states may be passed in, so that the call allocates nothing."""
    lib = load_library()
    b, L, H, P, N, G = _forward_dims(x, B)
    dev = x.device
    code = _dtype_code(x)
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    _need(D, "D", (H,), torch.float32, dev)
    if init_states is not None:
        _need(init_states, "init_states", (b, H, P, N), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", (b, L, H, P), x.dtype, dev)
    if final_states is None:
        final_states = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    _need(final_states, "final_states", (b, H, P, N), torch.float32, dev)
    rc = lib.ssd_forward_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_states), _ptr(y),
                                 _ptr(final_states), b, L, H, P, N, G, chunk_size, code, _stream(dev))
    _check("ssd_forward_noalloc", rc)
    return y, final_states


def forward_fused(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                  D: torch.Tensor, init_states: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One pass over the sequence per (batch, head), the state on chip: returns (y, final_states);
    see ssd_forward_fused in include/ssd.h."""
    lib = load_library()
    b, L, H, P, N, G = _forward_dims(x, B)
    dev = x.device
    code = _dtype_code(x)
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    _need(D, "D", (H,), torch.float32, dev)
    if init_states is not None:
        _need(init_states, "init_states", (b, H, P, N), torch.float32, dev)
    y = torch.empty_like(x)
    final = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    rc = lib.ssd_forward_fused(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_states), _ptr(y),
                               _ptr(final), b, L, H, P, N, G, code, _stream(dev))
    _check("ssd_forward_fused", rc)
    return y, final


def step(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
         C: torch.Tensor, D: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Recurrent mode: advances ``state`` in place by one token and returns y; see ssd_step."""
    lib = load_library()
    if state.dim() != 4 or B.dim() != 3:
        raise ValueError("state must be (batch, nheads, headdim, dstate) and B, C (batch, ngroups, dstate)")
    b, H, P, N = state.shape
    G = B.shape[1]
    dev = state.device
    code = _dtype_code(x)
    _need(state, "state", (b, H, P, N), torch.float32, dev)
    _need(x, "x", (b, H, P), x.dtype, dev)
    _need(dt, "dt", (b, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, G, N), x.dtype, dev)
    _need(C, "C", (b, G, N), x.dtype, dev)
    _need(D, "D", (H,), torch.float32, dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", (b, H, P), x.dtype, dev)
    rc = lib.ssd_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y), b, H, P, N,
                      G, code, _stream(dev))
    _check("ssd_step", rc)
    return y


def backward(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
             D: torch.Tensor, dy: torch.Tensor, chunk_size: int, init_states: Optional[torch.Tensor] = None,
             dfinal: Optional[torch.Tensor] = None) -> dict:
    """Gradients of ``forward`` for dL/dy = dy and dL/d(final_states) = dfinal (None = 0); see
    ssd_backward.  Returns a dict with dx, ddt, dA, dB, dC, dD, dinit (dx, dB, dC in x's dtype)."""
    lib = load_library()
    b, L, H, P, N, G = _forward_dims(x, B)
    dev = x.device
    code = _dtype_code(x)
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    _need(D, "D", (H,), torch.float32, dev)
    _need(dy, "dy", (b, L, H, P), x.dtype, dev)
    if init_states is not None:
        _need(init_states, "init_states", (b, H, P, N), torch.float32, dev)
    if dfinal is not None:
        _need(dfinal, "dfinal", (b, H, P, N), torch.float32, dev)
    ws_bytes = lib.ssd_backward_workspace_bytes(b, L, H, P, N, G, chunk_size, code)
    if ws_bytes == 0:
        raise SSDError("ssd_backward_workspace_bytes", -2)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt), dA=torch.empty_like(A), dB=torch.empty_like(B),
               dC=torch.empty_like(C), dD=torch.empty_like(D),
               dinit=torch.empty((b, H, P, N), dtype=torch.float32, device=dev))
    rc = lib.ssd_backward(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_states), _ptr(dy),
                          _ptr(dfinal), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]),
                          _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]), b, L, H, P, N, G, chunk_size, code,
                          _ptr(ws), ws.numel(), _stream(dev))
    _check("ssd_backward", rc)
    return out


def forward_varlen(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                   D: torch.Tensor, cu_seqlens: torch.Tensor, chunk_size: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Packed variable-length batch; see ssd_forward_varlen.

    x (T, nheads, headdim); dt (T, nheads) fp32; A, D (nheads,) fp32; B, C (T, ngroups, dstate) in
    x's dtype; cu_seqlens int32 (nseq + 1,) on the same device.  Every sequence starts from a zero
    state.  Returns (y (T, nheads, headdim) in x's dtype, final_states (nseq, nheads, headdim, dstate))."""
    lib = load_library()
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be (T, nheads, headdim) and B, C (T, ngroups, dstate)")
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    dev = x.device
    code = _dtype_code(x)
    _need(x, "x", (T, H, P), x.dtype, dev)
    _need(dt, "dt", (T, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (T, G, N), x.dtype, dev)
    _need(C, "C", (T, G, N), x.dtype, dev)
    _need(D, "D", (H,), torch.float32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of nseq + 1 offsets")
    _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
    nseq = cu_seqlens.numel() - 1
    ws_bytes = lib.ssd_forward_varlen_workspace_bytes(T, H, P, N, chunk_size, code)
    if ws_bytes == 0:
        raise SSDError("ssd_forward_varlen_workspace_bytes", -2)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    final = torch.empty((nseq, H, P, N), dtype=torch.float32, device=dev)
    rc = lib.ssd_forward_varlen(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(cu_seqlens), nseq,
                                _ptr(y), _ptr(final), T, H, P, N, G, chunk_size, code, _ptr(workspace),
                                workspace.numel(), _stream(dev))
    _check("ssd_forward_varlen", rc)
    return y, final


def selective_scan(x: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                   D: torch.Tensor, init_states: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """The Mamba-1 selective scan (per-channel diagonal decays); see ssd_selective_scan.

    x (batch, seqlen, dim); delta (batch, seqlen, dim) fp32; A (dim, dstate) fp32;
    B, C (batch, seqlen, dstate) in x's dtype; D (dim,) fp32; init_states (batch, dim, dstate)
    fp32 or None.  Returns (y in x's dtype, final_states fp32)."""
    lib = load_library()
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, seqlen, dim) and A (dim, dstate)")
    b, L, Dm = x.shape
    N = A.shape[1]
    dev = x.device
    code = _dtype_code(x)
    _need(x, "x", (b, L, Dm), x.dtype, dev)
    _need(delta, "delta", (b, L, Dm), torch.float32, dev)
    _need(A, "A", (Dm, N), torch.float32, dev)
    _need(B, "B", (b, L, N), x.dtype, dev)
    _need(C, "C", (b, L, N), x.dtype, dev)
    _need(D, "D", (Dm,), torch.float32, dev)
    if init_states is not None:
        _need(init_states, "init_states", (b, Dm, N), torch.float32, dev)
    y = torch.empty_like(x)
    final = torch.empty((b, Dm, N), dtype=torch.float32, device=dev)
    rc = lib.ssd_selective_scan(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_states),
                                _ptr(y), _ptr(final), b, L, Dm, N, code, _stream(dev))
    _check("ssd_selective_scan", rc)
    return y, final


# --- the four stages of the chunked mode, one entry point each ---------------------------------

def dA_cumsum(dt: torch.Tensor, A: torch.Tensor, chunk_size: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stage 1: returns (dA_cs, dt_chunked), both (batch, nheads, nchunks, chunk_size) float32."""
    lib = load_library()
    if dt.dim() != 3:
        raise ValueError("dt must be (batch, seqlen, nheads)")
    b, L, H = dt.shape
    dev = dt.device
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    nc = num_chunks(L, chunk_size)
    if nc < 0:
        _check("ssd_dA_cumsum", -2)
    cs = torch.empty((b, H, nc, chunk_size), dtype=torch.float32, device=dev)
    dtc = torch.empty_like(cs)
    rc = lib.ssd_dA_cumsum(_ptr(dt), _ptr(A), _ptr(cs), _ptr(dtc), b, L, H, chunk_size, _stream(dev))
    _check("ssd_dA_cumsum", rc)
    return cs, dtc


def chunk_state(x: torch.Tensor, B: torch.Tensor, dt_chunked: torch.Tensor, dA_cs: torch.Tensor,
                chunk_size: int) -> torch.Tensor:
    """Stage 2: returns chunk_states (batch, nchunks, nheads, headdim, dstate) float32."""
    lib = load_library()
    b, L, H, P, N, G = _forward_dims(x, B)
    dev = x.device
    code = _dtype_code(x)
    nc = num_chunks(L, chunk_size)
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(dt_chunked, "dt_chunked", (b, H, nc, chunk_size), torch.float32, dev)
    _need(dA_cs, "dA_cs", (b, H, nc, chunk_size), torch.float32, dev)
    out = torch.empty((b, nc, H, P, N), dtype=torch.float32, device=dev)
    rc = lib.ssd_chunk_state(_ptr(x), _ptr(B), _ptr(dt_chunked), _ptr(dA_cs), _ptr(out), b, L, H, P, N, G,
                             chunk_size, code, _stream(dev))
    _check("ssd_chunk_state", rc)
    return out


def state_passing(chunk_states: torch.Tensor, dA_cs: torch.Tensor, init_states: Optional[torch.Tensor],
                  seqlen: int, chunk_size: int, dtype: torch.dtype) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stage 3: returns (entry_states (batch, nchunks, nheads, headdim, dstate) in ``dtype``,
    final_states (batch, nheads, headdim, dstate) float32)."""
    lib = load_library()
    b, nc, H, P, N = chunk_states.shape
    dev = chunk_states.device
    code = SSD_BF16 if dtype == torch.bfloat16 else SSD_F32
    _need(chunk_states, "chunk_states", (b, nc, H, P, N), torch.float32, dev)
    _need(dA_cs, "dA_cs", (b, H, nc, chunk_size), torch.float32, dev)
    if num_chunks(seqlen, chunk_size) != nc:
        raise ValueError("chunk_states does not match seqlen / chunk_size")
    if init_states is not None:
        _need(init_states, "init_states", (b, H, P, N), torch.float32, dev)
    entry = torch.empty((b, nc, H, P, N), dtype=dtype, device=dev)
    final = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    rc = lib.ssd_state_passing(_ptr(chunk_states), _ptr(dA_cs), _ptr(init_states), _ptr(entry), _ptr(final), b,
                               seqlen, H, P, N, chunk_size, code, _stream(dev))
    _check("ssd_state_passing", rc)
    return entry, final


def chunk_scan(x: torch.Tensor, B: torch.Tensor, C: torch.Tensor, dt_chunked: torch.Tensor,
               dA_cs: torch.Tensor, entry_states: torch.Tensor, D: torch.Tensor, chunk_size: int) -> torch.Tensor:
    """Stage 4: returns y (batch, seqlen, nheads, headdim) in x's dtype."""
    lib = load_library()
    b, L, H, P, N, G = _forward_dims(x, B)
    dev = x.device
    code = _dtype_code(x)
    nc = num_chunks(L, chunk_size)
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    _need(dt_chunked, "dt_chunked", (b, H, nc, chunk_size), torch.float32, dev)
    _need(dA_cs, "dA_cs", (b, H, nc, chunk_size), torch.float32, dev)
    _need(entry_states, "entry_states", (b, nc, H, P, N), x.dtype, dev)
    _need(D, "D", (H,), torch.float32, dev)
    y = torch.empty_like(x)
    rc = lib.ssd_chunk_scan(_ptr(x), _ptr(B), _ptr(C), _ptr(dt_chunked), _ptr(dA_cs), _ptr(entry_states), _ptr(D),
                            _ptr(y), b, L, H, P, N, G, chunk_size, code, _stream(dev))
    _check("ssd_chunk_scan", rc)
    return y
