"""Seeded synthetic inputs for the SSD layer core.

This module only draws random numbers and rounds them to the storage
types the kernels read (bf16 by round-to-nearest-even on the fp32 bit
pattern, fp32 by a plain cast).  It holds none of the method's
arithmetic: both the fp64 oracle and the HIP path receive the arrays it
returns, so input quantisation is never counted as error.

The workload shapes and distributions are the five configurations the
library is measured on:

  tiny     fp32, B=1 L=512 H=4 P=16 N=16 G=1 Q=64
  l130m    bf16, B=8 L=2048 H=24 P=64 N=128 G=1 Q=256, init state N(0, 0.1^2)
  l2p7b    bf16, B=4 L=4096 H=80 P=64 N=128 G=1 Q=256   (a 2.7B-class layer,
           d_inner 5120; the headline workload)
  long64k  bf16, B=1 L=65536 H=80 P=64 N=256 G=8 Q=256
  decode   bf16, batch 256 H=80 P=64 N=128 G=1, 1024 single-token steps on
           an fp32 state initialised N(0, 0.1^2)

packed variable-length batches,

  varlen2p7b the l2p7b layer shape over 16384 packed tokens split into
           sequences of seeded uniform lengths in [64, 4096] (the last one
           cut to fit), state reset at every sequence start; per-token draws
           as for a batch of one

and, for the Mamba-1 selective scan the SSD layer is compared with,

  scan2p7b bf16, B=4 L=4096 channels 5120 N=16 (the same 2.7B-class layer
           width, with Mamba-1's state size), delta drawn like "l2p7b"'s dt
           per (batch, token, channel), A[d, n] = -exp(U(0, log 16)) per
           (channel, state), draw order x, delta noise, delta uniform, A, B,
           C, D, initial state (if any)

Distributions: x ~ N(0,1); dt = softplus(z) with z ~ N(0,1) - 2
("tiny", "l130m", "decode") or z ~ N(0,1) + log(expm1(U(1e-3, 1e-1)))
("l2p7b", "long64k"); A_h = -exp(U(0, log 16)); B, C ~ N(0,1)/sqrt(N);
D ~ N(0,1).  Draw order per configuration: x, dt noise, dt uniform (if
any), A uniform, B, C, D, initial state (if any); all draws are fp64 from
``numpy.random.default_rng(seed)``.  The decode workload draws A, D and the
state from ``default_rng(seed)`` and step t's x, dt, B, C from
``default_rng([seed, t])`` so any step can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "CONFIGS", "SSDConfig", "SSDInputs", "StepInputs", "ScanInputs", "SCAN_CONFIGS", "bf16_bits",
    "bf16_to_f64", "make_inputs", "make_step_params", "make_step_inputs", "make_random",
    "make_scan_random", "make_scan_inputs", "VarlenInputs", "VARLEN_CONFIGS", "varlen_lengths",
    "make_varlen", "make_varlen_inputs",
]


@dataclasses.dataclass(frozen=True)
class SSDConfig:
    name: str
    batch: int
    seqlen: int            # for the decode workload: number of steps
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int        # 0 for the decode workload
    dtype: str             # "f32" or "bf16": storage type of x, B, C and y
    dt_kind: str           # "shifted" = softplus(N(0,1) - 2); "ranged" = softplus(N + log(expm1(U)))
    init: bool             # random N(0, 0.1^2) initial state
    seed: int

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


CONFIGS = {
    "tiny": SSDConfig("tiny", 1, 512, 4, 16, 16, 1, 64, "f32", "shifted", False, 0),
    "l130m": SSDConfig("l130m", 8, 2048, 24, 64, 128, 1, 256, "bf16", "shifted", True, 1),
    "l2p7b": SSDConfig("l2p7b", 4, 4096, 80, 64, 128, 1, 256, "bf16", "ranged", False, 2),
    "long64k": SSDConfig("long64k", 1, 65536, 80, 64, 256, 8, 256, "bf16", "ranged", False, 3),
    "decode": SSDConfig("decode", 256, 1024, 80, 64, 128, 1, 0, "bf16", "shifted", True, 4),
}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest-even on the fp32 bit pattern); returns uint16 bit patterns."""
    u = np.array(a, dtype=np.float32, copy=True, order="C").view(np.uint32)
    bias = np.right_shift(u, 16)
    np.bitwise_and(bias, 1, out=bias)
    bias += np.uint32(0x7FFF)
    u += bias
    del bias
    np.right_shift(u, 16, out=u)
    return u.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _softplus(z: np.ndarray) -> np.ndarray:
    # log(1 + e^z) without overflow for large z
    return np.logaddexp(0.0, z)


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(a64) if dtype == "bf16" else a64.astype(np.float32)


@dataclasses.dataclass
class SSDInputs:
    """One forward problem.  x, B, C hold float32 arrays (dtype "f32") or
    uint16 bf16 bit patterns (dtype "bf16"); dt, A, D, init are float32."""
    x: np.ndarray          # (batch, seqlen, nheads, headdim)
    dt: np.ndarray         # (batch, seqlen, nheads), positive
    A: np.ndarray          # (nheads,), negative
    B: np.ndarray          # (batch, seqlen, ngroups, dstate)
    C: np.ndarray          # (batch, seqlen, ngroups, dstate)
    D: np.ndarray          # (nheads,)
    init: Optional[np.ndarray]   # (batch, nheads, headdim, dstate) or None (zeros)
    chunk_size: int
    dtype: str

    @property
    def dims(self):
        b, l, h, p = self.x.shape
        return b, l, h, p, self.B.shape[3], self.B.shape[2]

    def f64(self, name: str) -> np.ndarray:
        """fp64 copy of one input (exact: every stored value is representable)."""
        a = getattr(self, name)
        if a is None:
            return None
        if name in ("x", "B", "C") and self.dtype == "bf16":
            return bf16_to_f64(a)
        return a.astype(np.float64)


def _draw_dt(rng: np.random.Generator, shape, kind: str) -> np.ndarray:
    z = rng.standard_normal(shape)
    if kind == "shifted":
        z = z - 2.0
    else:
        u = rng.uniform(1e-3, 1e-1, size=shape)
        z = z + np.log(np.expm1(u))
    return _softplus(z)


def make_random(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype="bf16",
                dt_kind="shifted", init=False, seed=0) -> SSDInputs:
    """Draw one forward problem of any shape with the workload distributions."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, nheads, headdim))
    dt = _draw_dt(rng, (batch, seqlen, nheads), dt_kind)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), size=nheads))
    Bm = rng.standard_normal((batch, seqlen, ngroups, dstate)) / np.sqrt(dstate)
    Cm = rng.standard_normal((batch, seqlen, ngroups, dstate)) / np.sqrt(dstate)
    D = rng.standard_normal(nheads)
    h0 = 0.1 * rng.standard_normal((batch, nheads, headdim, dstate)) if init else None
    return SSDInputs(
        x=_store(x, dtype), dt=dt.astype(np.float32), A=A.astype(np.float32),
        B=_store(Bm, dtype), C=_store(Cm, dtype), D=D.astype(np.float32),
        init=None if h0 is None else h0.astype(np.float32), chunk_size=chunk_size, dtype=dtype)


def make_inputs(name: str) -> SSDInputs:
    """The forward problem of a named configuration (not "decode")."""
    c = CONFIGS[name]
    if c.chunk_size == 0:
        raise ValueError(f"{name} is a decode workload; use make_step_params/make_step_inputs")
    return make_random(c.batch, c.seqlen, c.nheads, c.headdim, c.dstate, c.ngroups, c.chunk_size,
                       c.dtype, c.dt_kind, c.init, c.seed)


@dataclasses.dataclass
class StepInputs:
    x: np.ndarray    # (batch, nheads, headdim) storage dtype
    dt: np.ndarray   # (batch, nheads) float32
    B: np.ndarray    # (batch, ngroups, dstate) storage dtype
    C: np.ndarray    # (batch, ngroups, dstate) storage dtype
    dtype: str

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if name in ("x", "B", "C") and self.dtype == "bf16":
            return bf16_to_f64(a)
        return a.astype(np.float64)


def make_step_params(name: str = "decode", batch: Optional[int] = None):
    """Fixed decode parameters: (A, D, state0) as float32 arrays.

    ``batch`` below the configured batch returns the leading rows of the
    same draw, so a slice of the workload regenerates identically."""
    c = CONFIGS[name]
    rng = np.random.default_rng(c.seed)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), size=c.nheads))
    D = rng.standard_normal(c.nheads)
    state = 0.1 * rng.standard_normal((c.batch, c.nheads, c.headdim, c.dstate))
    b = c.batch if batch is None else batch
    return A.astype(np.float32), D.astype(np.float32), np.ascontiguousarray(state[:b].astype(np.float32))


def make_step_inputs(name: str, step: int, batch: Optional[int] = None) -> StepInputs:
    """Step ``step``'s fresh token inputs for the decode workload."""
    c = CONFIGS[name]
    rng = np.random.default_rng([c.seed, step])
    x = rng.standard_normal((c.batch, c.nheads, c.headdim))
    dt = _draw_dt(rng, (c.batch, c.nheads), c.dt_kind)
    Bm = rng.standard_normal((c.batch, c.ngroups, c.dstate)) / np.sqrt(c.dstate)
    Cm = rng.standard_normal((c.batch, c.ngroups, c.dstate)) / np.sqrt(c.dstate)
    b = c.batch if batch is None else batch
    return StepInputs(x=_store(x[:b], c.dtype), dt=dt[:b].astype(np.float32),
                      B=_store(Bm[:b], c.dtype), C=_store(Cm[:b], c.dtype), dtype=c.dtype)


@dataclasses.dataclass
class ScanInputs:
    """One selective-scan problem.  x, B, C in the storage dtype (float32 or
    uint16 bf16 bit patterns); delta, A, D, init float32."""
    x: np.ndarray          # (batch, seqlen, dim)
    delta: np.ndarray      # (batch, seqlen, dim), positive
    A: np.ndarray          # (dim, dstate), negative
    B: np.ndarray          # (batch, seqlen, dstate)
    C: np.ndarray          # (batch, seqlen, dstate)
    D: np.ndarray          # (dim,)
    init: Optional[np.ndarray]   # (batch, dim, dstate) or None (zeros)
    dtype: str

    @property
    def dims(self):
        b, l, d = self.x.shape
        return b, l, d, self.A.shape[1]

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if a is None:
            return None
        if name in ("x", "B", "C") and self.dtype == "bf16":
            return bf16_to_f64(a)
        return a.astype(np.float64)


SCAN_CONFIGS = {
    # name: (batch, seqlen, dim, dstate, dtype, dt_kind, init, seed)
    "scan2p7b": (4, 4096, 5120, 16, "bf16", "ranged", False, 5),
}


def make_scan_random(batch, seqlen, dim, dstate, dtype="bf16", dt_kind="ranged", init=False,
                     seed=0) -> ScanInputs:
    """Draw one selective-scan problem of any shape with the workload distributions."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, dim))
    delta = _draw_dt(rng, (batch, seqlen, dim), dt_kind)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), size=(dim, dstate)))
    Bm = rng.standard_normal((batch, seqlen, dstate)) / np.sqrt(dstate)
    Cm = rng.standard_normal((batch, seqlen, dstate)) / np.sqrt(dstate)
    D = rng.standard_normal(dim)
    h0 = 0.1 * rng.standard_normal((batch, dim, dstate)) if init else None
    return ScanInputs(
        x=_store(x, dtype), delta=delta.astype(np.float32), A=A.astype(np.float32),
        B=_store(Bm, dtype), C=_store(Cm, dtype), D=D.astype(np.float32),
        init=None if h0 is None else h0.astype(np.float32), dtype=dtype)


def make_scan_inputs(name: str) -> ScanInputs:
    b, l, d, n, dtype, kind, init, seed = SCAN_CONFIGS[name]
    return make_scan_random(b, l, d, n, dtype, kind, init, seed)


@dataclasses.dataclass
class VarlenInputs:
    """Packed sequences: sequence k is tokens cu_seqlens[k] .. cu_seqlens[k+1]-1."""
    x: np.ndarray          # (T, nheads, headdim) storage dtype
    dt: np.ndarray         # (T, nheads)
    A: np.ndarray          # (nheads,)
    B: np.ndarray          # (T, ngroups, dstate)
    C: np.ndarray          # (T, ngroups, dstate)
    D: np.ndarray          # (nheads,)
    cu_seqlens: np.ndarray  # (nseq + 1,) int32
    chunk_size: int
    dtype: str

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if name in ("x", "B", "C") and self.dtype == "bf16":
            return bf16_to_f64(a)
        return a.astype(np.float64)


def varlen_lengths(total: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Seeded sequence lengths, uniform integers in [lo, hi], the last cut so they sum to total."""
    rng = np.random.default_rng(seed)
    out = []
    left = total
    while left > 0:
        n = min(int(rng.integers(lo, hi + 1)), left)
        out.append(n)
        left -= n
    return np.array(out, dtype=np.int64)


def make_varlen(lengths, nheads, headdim, dstate, ngroups, chunk_size, dtype="bf16", dt_kind="ranged",
                seed=0) -> VarlenInputs:
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    p = make_random(1, T, nheads, headdim, dstate, ngroups, chunk_size, dtype, dt_kind, False, seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return VarlenInputs(x=p.x[0], dt=p.dt[0], A=p.A, B=p.B[0], C=p.C[0], D=p.D, cu_seqlens=cu,
                        chunk_size=chunk_size, dtype=dtype)


VARLEN_CONFIGS = {
    # name: (total tokens, length range, nheads, headdim, dstate, ngroups, chunk, dtype, dt_kind, seed)
    "varlen2p7b": (16384, (64, 4096), 80, 64, 128, 1, 256, "bf16", "ranged", 6),
}


def make_varlen_inputs(name: str) -> VarlenInputs:
    T, (lo, hi), H, P, N, G, Q, dtype, kind, seed = VARLEN_CONFIGS[name]
    return make_varlen(varlen_lengths(T, lo, hi, seed), H, P, N, G, Q, dtype, kind, seed)
