"""fp64 CPU oracle of the Mamba-2 SSD layer core.

TEST INFRASTRUCTURE ONLY: the tests, the package's smoke entry and the
benchmark's CPU-baseline leg use it; the library never imports, links or
calls anything here, and nothing here imports the library.

``forward`` and ``step`` call the plain C recurrence in ``ssd_oracle.c``
(token by token, double precision, one independent (b, h, p) row per
OpenMP task); ``backward`` is the reverse-mode derivative of that
recurrence (the adjoint state run backwards over the stored states);
``forward_varlen`` runs ``forward`` on each sequence of a
packed batch; ``selective_scan`` calls the Mamba-1 recurrence there (one
(b, channel) row per task).  The helpers below it are written on top of those two calls
and plain numpy indexing only:

* ``chunk_log_decay`` - the exponent of the decay product of every prefix
  of a chunk, sum_{j<=l} dt_j A_h.  Its exponential is the product of the
  per-step decays a_j = exp(dt_j A_h) that appears in the matrix-mixer
  entries M_{t,i} = C_t (prod_{j=i+1..t} A_j) B_i ("Mamba-2" wiki note,
  section "Matrix Mixer View"), here restricted to one chunk.
* ``chunk_states`` - the state each chunk reaches from a zero state, i.e.
  the recurrence run over that chunk alone (the summary a chunk passes on;
  "Why Does Mamba-2 Resemble the Transformer?", section "The Core of SSD").
* ``chunk_entry_states`` - the state entering every chunk, i.e. the
  recurrence's state after the token before the chunk (the initial state
  for the first chunk).

Every function is pinned by the tests in ``tests/test_oracle_pins.py``
against closed forms, a brute-force dense quadratic form, textbook special
cases and invariants; none is pinned against the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP) into oracle/libssd_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib):
    lib.ssd_oracle_forward.restype = ctypes.c_int
    lib.ssd_oracle_forward.argtypes = [_dp] * 9 + [_i64] * 6 + [ctypes.POINTER(_i64), _i64, _dp,
                                                                ctypes.c_int]
    lib.ssd_oracle_step.restype = ctypes.c_int
    lib.ssd_oracle_step.argtypes = [_dp] * 8 + [_i64] * 5 + [ctypes.c_int]
    lib.ssd_oracle_backward.restype = ctypes.c_int
    lib.ssd_oracle_backward.argtypes = [_dp] * 17 + [_i64] * 6 + [ctypes.c_int]
    lib.ssd_oracle_selective_scan.restype = ctypes.c_int
    lib.ssd_oracle_selective_scan.argtypes = [_dp] * 9 + [_i64] * 4 + [ctypes.c_int]
    lib.ssd_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def load_variant(path: str):
    """Bind another build of ssd_oracle.c (used by the tests that plant a
    mistake in a copy of the oracle and check that a pin catches it)."""
    return _bind(ctypes.CDLL(os.path.abspath(path)))


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_dp)


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def forward(x, dt, A, B, C, D, init=None, record_t: Sequence[int] = (), nthreads: int = 0, lib=None):
    """Run the recurrence over a whole sequence.

    x (b,L,H,P); dt (b,L,H); A, D (H,); B, C (b,L,G,N); init (b,H,P,N) or None.
    Returns (y (b,L,H,P), final (b,H,P,N)) in fp64, plus the states after the
    tokens in ``record_t`` as (b, len(record_t), H, P, N) when it is not empty.
    """
    x, dt, A, B, C, D, init = (_f64(a) for a in (x, dt, A, B, C, D, init))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, L, H) and A.shape == (H,) and D.shape == (H,)
    assert B.shape == (b, L, G, N) and C.shape == (b, L, G, N)
    assert init is None or init.shape == (b, H, P, N)
    rec = np.ascontiguousarray(np.asarray(record_t, dtype=np.int64))
    if rec.size:
        assert np.all(np.diff(rec) >= 0) and rec[0] >= 0 and rec[-1] < L, "record_t must be ascending, in range"
    y = np.empty((b, L, H, P))
    final = np.empty((b, H, P, N))
    recorded = np.empty((b, rec.size, H, P, N)) if rec.size else None
    rc = (lib or _load()).ssd_oracle_forward(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init), _ptr(y), _ptr(final),
        b, L, H, P, N, G, rec.ctypes.data_as(ctypes.POINTER(_i64)) if rec.size else None, rec.size,
        _ptr(recorded), int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_forward rejected its arguments")
    if rec.size:
        return y, final, recorded
    return y, final


def step(state, x, dt, A, B, C, D, nthreads: int = 0, lib=None):
    """One recurrent step.  state (b,H,P,N) is NOT modified; returns (y (b,H,P), new_state)."""
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    x, dt, A, B, C, D = (_f64(a) for a in (x, dt, A, B, C, D))
    b, H, P, N = st.shape
    G = B.shape[1]
    assert x.shape == (b, H, P) and dt.shape == (b, H) and B.shape == (b, G, N) and C.shape == (b, G, N)
    y = np.empty((b, H, P))
    rc = (lib or _load()).ssd_oracle_step(_ptr(st), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                 _ptr(y), b, H, P, N, G, int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_step rejected its arguments")
    return y, st


def backward(x, dt, A, B, C, D, init, dy, dfinal=None, nthreads: int = 0, lib=None):
    """Gradients of the forward for dL/dy = dy and dL/dfinal = dfinal (None = 0).

    Shapes as in ``forward`` (dy like x, dfinal like init).  Returns a dict with dx, ddt, dA, dB,
    dC, dD and dinit (dinit is returned even when init is None: the gradient w.r.t. a zero
    initial state), and dA_scale: per head the size of the per-token products dA is formed from
    in a chunked pass, sum_t T_t (sum_p |dy yhat| + sum_p |u du|) with T_t the prefix sum of dt
    (dA's terms cancel strongly, so its errors are measured against this scale)."""
    x, dt, A, B, C, D, init, dy, dfinal = (_f64(a) for a in (x, dt, A, B, C, D, init, dy, dfinal))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dy.shape == x.shape and (dfinal is None or dfinal.shape == (b, H, P, N))
    out = dict(dx=np.empty((b, L, H, P)), ddt=np.empty((b, L, H)), dA=np.empty(H), dB=np.empty((b, L, G, N)),
               dC=np.empty((b, L, G, N)), dD=np.empty(H), dinit=np.empty((b, H, P, N)), dA_scale=np.empty(H))
    rc = (lib or _load()).ssd_oracle_backward(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init), _ptr(dy), _ptr(dfinal),
        _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
        _ptr(out["dinit"]), _ptr(out["dA_scale"]), b, L, H, P, N, G, int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_backward rejected its arguments")
    return out


def forward_varlen(x, dt, A, B, C, D, cu_seqlens, nthreads: int = 0, lib=None):
    """Packed variable-length sequences: sequence k is tokens cu_seqlens[k] .. cu_seqlens[k+1]-1
    of the packed arrays and starts from a zero state (the recurrence is reset at every sequence
    start); each sequence is run through ``forward`` on its own.

    x (T,H,P); dt (T,H); A, D (H,); B, C (T,G,N); cu_seqlens (nseq+1,) non-decreasing from 0 to T.
    Returns (y (T,H,P), final (nseq,H,P,N)) in fp64; an empty sequence's final state is zero."""
    x, dt, B, C = (_f64(a) for a in (x, dt, B, C))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, P = x.shape
    N = B.shape[2]
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0), "cu_seqlens must run from 0 to T"
    y = np.empty((T, H, P))
    final = np.zeros((len(cu) - 1, H, P, N))
    for k in range(len(cu) - 1):
        a, e = int(cu[k]), int(cu[k + 1])
        if e == a:
            continue
        yk, fk = forward(x[None, a:e], dt[None, a:e], A, B[None, a:e], C[None, a:e], D, None,
                         nthreads=nthreads, lib=lib)
        y[a:e] = yk[0]
        final[k] = fk[0]
    return y, final


def selective_scan(x, delta, A, B, C, D, init=None, nthreads: int = 0, lib=None):
    """The Mamba-1 selective scan (per-channel diagonal decays).

    x, delta (b,L,Dm); A (Dm,N); B, C (b,L,N); D (Dm,); init (b,Dm,N) or None.
    Returns (y (b,L,Dm), final (b,Dm,N)) in fp64."""
    x, delta, A, B, C, D, init = (_f64(a) for a in (x, delta, A, B, C, D, init))
    b, L, Dm = x.shape
    N = A.shape[1]
    assert delta.shape == (b, L, Dm) and A.shape == (Dm, N) and D.shape == (Dm,)
    assert B.shape == (b, L, N) and C.shape == (b, L, N)
    assert init is None or init.shape == (b, Dm, N)
    y = np.empty((b, L, Dm))
    final = np.empty((b, Dm, N))
    rc = (lib or _load()).ssd_oracle_selective_scan(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init), _ptr(y), _ptr(final),
        b, L, Dm, N, int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_selective_scan rejected its arguments")
    return y, final


def n_chunks(seqlen: int, chunk_size: int) -> int:
    return -(-seqlen // chunk_size)


def chunk_log_decay(dt, A, chunk_size: int) -> np.ndarray:
    """(b,H,nc,Q) fp64: sum of dt_j * A_h over j = chunk start .. l (inclusive).

    Positions past the end of a ragged last chunk repeat the chunk's last
    value (they carry no token)."""
    dt = _f64(dt)
    A = _f64(A)
    b, L, H = dt.shape
    nc = n_chunks(L, chunk_size)
    out = np.empty((b, H, nc, chunk_size))
    for c in range(nc):
        lo, hi = c * chunk_size, min(L, (c + 1) * chunk_size)
        run = np.cumsum(dt[:, lo:hi, :] * A[None, None, :], axis=1)  # (b, len, H)
        out[:, :, c, : hi - lo] = np.transpose(run, (0, 2, 1))
        out[:, :, c, hi - lo:] = out[:, :, c, hi - lo - 1: hi - lo]
    return out


def chunk_states(x, dt, A, B, C, D, chunk_size: int, nthreads: int = 0) -> np.ndarray:
    """(b,nc,H,P,N): the state each chunk reaches when run from a zero state."""
    b, L, H, P = np.shape(x)
    N = np.shape(B)[3]
    nc = n_chunks(L, chunk_size)
    out = np.empty((b, nc, H, P, N))
    for c in range(nc):
        lo, hi = c * chunk_size, min(L, (c + 1) * chunk_size)
        _, fin = forward(np.asarray(x)[:, lo:hi], np.asarray(dt)[:, lo:hi], A, np.asarray(B)[:, lo:hi],
                         np.asarray(C)[:, lo:hi], D, None, nthreads=nthreads)
        out[:, c] = fin
    return out


def chunk_entry_states(x, dt, A, B, C, D, init, chunk_size: int, nthreads: int = 0):
    """((b,nc,H,P,N) state entering each chunk, (b,H,P,N) final state, y)."""
    b, L, H, P = np.shape(x)
    N = np.shape(B)[3]
    nc = n_chunks(L, chunk_size)
    rec = [c * chunk_size - 1 for c in range(1, nc)]
    if rec:
        y, fin, recs = forward(x, dt, A, B, C, D, init, record_t=rec, nthreads=nthreads)
    else:
        y, fin = forward(x, dt, A, B, C, D, init, nthreads=nthreads)
        recs = np.empty((b, 0, H, P, N))
    entry = np.empty((b, nc, H, P, N))
    entry[:, 0] = 0.0 if init is None else _f64(init)
    entry[:, 1:] = recs
    return entry, fin, y
