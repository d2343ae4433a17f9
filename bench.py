#!/usr/bin/env python3
"""Throughput of the SSD layer core on one MI355X.

A step is one ssd_forward call (the four chunked-mode kernels) over one batch
of the 2.7B-layer-shape workload (batch 4 x 4096 tokens, 80 heads of dim 64,
state 128, one group, chunk 256, bf16 x/B/C, fp32 dt/A/D), inputs resident in
HBM.  The JSON line reports tokens/s of the whole call, the roofline of its
dominant kernel measured with HIP events on the library's stream, the
recurrent-mode kernel on the decode workload (batch 256, fp32 state
256x80x64x128, single-token steps), and the fp64 CPU oracle timed on the
host beside it.

    python bench.py [--steps K] [--warmup W] [--workload l2p7b|l130m|long64k]

Order of the run: the secondary legs (decode, one-pass forward, packed
variable-length batch, backward, Mamba-1 scan, the 130M- and 64K-layer
workloads) run first, then the W untimed warmup steps and the K timed steps
of the headline, then per-call (warm and MALL-flushed) and per-kernel timings
of the same forward, then the CPU oracle.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores, published
KERNELS = ("dA_cumsum", "chunk_state", "state_passing", "chunk_scan")
KERNEL_SOURCES = {"dA_cumsum": "dA_cumsum.hip", "chunk_state": "chunk_state.hip",
                  "chunk_state_cumsum": "chunk_state.hip", "chunk_state_varlen": "chunk_state.hip",
                  "state_passing": "state_passing.hip", "state_passing_varlen": "state_passing.hip",
                  "chunk_scan": "chunk_scan.hip", "chunk_scan_varlen": "chunk_scan.hip", "ssd_step": "ssd_step.hip",
                  "selective_scan": "selective_scan.hip", "varlen_meta": "varlen_meta.hip",
                  "ssd_fused": "fused.hip",
                  # the backward's kernels: the pair-product (hi/lo) variants of the forward's and its own
                  "chunk_scan_split_dot": "chunk_scan.hip", "chunk_scan_split_grad": "chunk_scan.hip",
                  "chunk_scan_f32out": "chunk_scan.hip", "chunk_state_split": "chunk_state.hip",
                  "chunk_state_cumsum_split": "chunk_state.hip", "state_passing_split": "state_passing.hip",
                  **{k: "bwd.hip" for k in ("bwd_group_sum", "bwd_heads", "bwd_passing", "bwd_prep", "bwd_rows",
                                            "bwd_scan", "bwd_tables", "bwd_transpose", "bwd_zero")},
                  **{k: "bwd_dbc.hip" for k in ("bwd_dbc", "bwd_inter", "bwd_score")}}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # untimed; the GPU needs some tens of milliseconds of work to reach its full clocks
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="l2p7b", choices=["l130m", "l2p7b", "long64k"])
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true", help="skip the recurrent-mode leg")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--no-scan", action="store_true", help="skip the Mamba-1 selective-scan comparison leg")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed variable-length leg")
    ap.add_argument("--no-fused", action="store_true", help="skip the one-pass (fused) forward leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass leg")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip timing the forward on the 130M- and 64K-layer workloads")
    ap.add_argument("--no-cold", action="store_true", help="skip the MALL-flushed per-call timings")
    ap.add_argument("--backward-calls", type=int, default=20)
    ap.add_argument("--scan-calls", type=int, default=10)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (scale for HBM byte counters) and exit")
    return ap.parse_args()


# ------------------------------------------------------------------------------------------------
# Algorithmic work per launch (bytes that must cross HBM at least once; flops the method needs)

def kernel_work(b, L, H, P, N, G, Q, es, init):
    nc = -(-L // Q)
    x = b * L * H * P * es
    bc = b * L * G * N * es
    cs = b * H * nc * Q * 4
    st32 = b * nc * H * P * N * 4
    stT = b * nc * H * P * N * es
    fin = b * H * P * N * 4
    causal = Q * (Q + 1) // 2
    work = {
        "dA_cumsum": dict(bytes=b * L * H * 4 + 2 * cs, flops=2 * b * L * H),
        "chunk_state": dict(bytes=x + bc + 2 * cs + st32, flops=2 * b * L * H * P * N),
        "state_passing": dict(bytes=st32 + b * H * nc * 4 + (fin if init else 0) + stT + fin,
                              flops=2 * b * nc * H * P * N),
        # y = x + (causal C B^T once per group) masked @ X + C . S_in, plus D x
        "chunk_scan": dict(bytes=2 * x + 2 * bc + 2 * cs + stT + H * 4,
                           flops=2 * b * nc * G * causal * N + 2 * b * nc * H * causal * P
                           + 2 * b * L * H * N * P + 2 * b * L * H * P),
    }
    return work


def backward_work(b, L, H, P, N, G, Q, es):
    """Algorithmic bytes and flops of ssd_backward (bf16 inputs), whole pass and per dominant kernel.

    Whole pass: the minimum bytes are one read of x, dt, B, C, dy and one write of dx, ddt, dB, dC; the
    flops are the forward recomputed (y - D x), the adjoint readout du = g B (an SSD of the same shape),
    the scores dy . x^T inside chunks and their products with B and C, and the state terms of dB and dC
    (2 P N per token and head each).  Per kernel: the two pair-product readout passes, which read the
    hi and lo planes of the entry (resp. adjoint) states and each take every product twice."""
    nc = -(-L // Q)
    causal = Q * (Q + 1) // 2
    st = b * nc * H * P * N
    tab = b * H * nc * Q * 4
    fw = kernel_work(b, L, H, P, N, G, Q, es, False)
    fwd_flops = sum(v["flops"] for v in fw.values())
    total = dict(bytes=3 * b * L * H * P * es + 2 * b * L * H * 4 + 4 * b * L * G * N * es,
                 flops=2 * fwd_flops + 2 * b * nc * H * causal * P + 2 * 2 * b * nc * G * causal * N
                 + 2 * 2 * b * L * H * P * N)
    # the readout's matrix-core work taken twice (hi and lo operands): causal C.B^T once per group, G x,
    # and the state readout C . S
    split_flops = 2 * (2 * b * nc * G * causal * N + 2 * b * nc * H * causal * P + 2 * b * L * H * N * P)
    kernels = {
        # x, B, C, the decay tables, the entry states' hi and lo planes, dy; dy . yhat per (token, head) out
        "chunk_scan_split_dot": dict(bytes=2 * b * L * H * P * es + 2 * b * L * G * N * es + 2 * tab + 2 * st * es
                                     + b * H * L * 4, flops=split_flops),
        # dy (the input role, read again per token where it is then cached), reversed C and B, tables, the
        # adjoint states' planes; x and dt per token; dx, x . du and x . dy out
        "chunk_scan_split_grad": dict(bytes=3 * b * L * H * P * es + 2 * b * L * G * N * es + 2 * tab + 2 * st * es
                                      + b * L * H * 4 + 2 * b * H * L * 4, flops=split_flops),
    }
    return total, kernels


def trace_average_us(path_name, kernel_label):
    """Average duration of a kernel in a committed rocprofv3 trace summary (profiles/<path_name>), or
    None when the summary is missing, does not list the kernel, or its source digest no longer
    matches the backward's sources."""
    path = os.path.join(ROOT, "profiles", path_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    if not m_src or m_src.group(1) != backward_digest():
        return None
    m = re.search(rf"^\| {re.escape(kernel_label)} \(`[^`]*`\) \| \d+ \| ([0-9.]+) \|", text, re.M)
    return float(m.group(1)) if m else None


def backward_digest():
    h = hashlib.sha256()
    for f in ("bwd.hip", "bwd_dbc.hip", "chunk_scan.hip", "chunk_state.hip", "state_passing.hip", "common.hpp"):
        with open(os.path.join(ROOT, "mamba_ssd_sequence_chunked_amd", "csrc", f), "rb") as fh:
            h.update(_code_only(fh.read()))
    return h.hexdigest()[:16]


# Vector-ALU ceiling of the selective scan: each (token, channel, state) update needs four fp32
# VALU operations (delta*A, u*B, the state FMA, the readout FMA) and one exponential.  A SIMD
# retires 16 lanes of a plain VALU op per cycle and a transcendental at a quarter of that, so an
# update costs 8 lane-cycles: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz / 8 = 4.9e12 updates/s.
SCAN_UPDATE_PEAK = 256 * 4 * 16 * 2.4e9 / 8


def step_work(b, H, P, N, G, es):
    return dict(bytes=2 * b * H * P * N * 4 + 2 * b * H * P * es + 2 * b * G * N * es + b * H * 4 + 2 * H * 4,
                flops=5 * b * H * P * N)


def _code_only(text):
    """Source text with comments and blank lines removed, lines stripped: a change of
    comments alone leaves a kernel's counters valid."""
    text = re.sub(rb"/\*.*?\*/", b"", text, flags=re.S)
    text = re.sub(rb"//[^\n]*", b"", text)
    return b"\n".join(ln.strip() for ln in text.splitlines() if ln.strip())


def source_digest(name):
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[name], "common.hpp"):
        with open(os.path.join(ROOT, "mamba_ssd_sequence_chunked_amd", "csrc", f), "rb") as fh:
            h.update(_code_only(fh.read()))
    return h.hexdigest()[:16]


def measured_traffic(workload, name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    there is none for this kernel and workload or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{name}_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_src or not m_b or m_src.group(1) != source_digest(name):
        return None
    return float(m_b.group(1))


def counter_summary(workload, name):
    """Matrix-core counters per launch from the committed rocprofv3 summary
    (profiles/mfma_counters_<kernel>_<workload>.txt), or None when there is none for this kernel
    and workload or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"mfma_counters_{name}_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"^source_digest:\s*(\S+)", text, re.M)
    if not m_src or m_src.group(1) != source_digest(name):
        return None
    out = {}
    for key in ("mfma_instructions_per_launch", "mfma_flops_issued_per_launch", "mfma_busy_frac",
                "valu_instructions_per_launch", "lds_bank_conflict_cycles_per_launch"):
        m = re.search(rf"^{key}:\s*([0-9.eE+-]+)", text, re.M)
        if m:
            out[key] = float(m.group(1))
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stats_us(ms_list):
    v = sorted(1e3 * m for m in ms_list)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return dict(mean=round(sum(v) / n, 2), median=round(med, 2), min=round(v[0], 2), calls=n)


# ------------------------------------------------------------------------------------------------

def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the SSD layer core has no multi-GPU path in this library", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mamba_ssd_sequence_chunked_amd as ssd
    from mamba_ssd_sequence_chunked_amd.inputs import CONFIGS, make_inputs

    if args.copy_calibration:
        copy_calibration()
        return

    lib = ssd.load_library()
    dev = torch.device("cuda:0")
    inp = make_inputs(args.workload)
    b, L, H, P, N, G = inp.dims
    Q = inp.chunk_size
    es = 2 if inp.dtype == "bf16" else 4
    code = ssd.SSD_BF16 if inp.dtype == "bf16" else ssd.SSD_F32
    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32

    def t(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x, dt, A, B, C, D, init = (t(inp.x), t(inp.dt), t(inp.A), t(inp.B), t(inp.C), t(inp.D), t(inp.init))
    y = torch.empty_like(x)
    final = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    ws_bytes = ssd.workspace_bytes(b, L, H, P, N, Q, code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    nc = ssd.num_chunks(L, Q)
    cs = torch.empty((b, H, nc, Q), dtype=torch.float32, device=dev)
    dtc = torch.empty_like(cs)
    states = torch.empty((b, nc, H, P, N), dtype=torch.float32, device=dev)
    entry = torch.empty((b, nc, H, P, N), dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    p = lambda tt: None if tt is None else ctypes.c_void_p(tt.data_ptr())  # noqa: E731

    def forward():
        rc = lib.ssd_forward(p(x), p(dt), p(A), p(B), p(C), p(D), p(init), p(y), p(final), b, L, H, P, N, G, Q,
                             code, p(ws), ws_bytes, sp)
        if rc:
            raise ssd.SSDError("ssd_forward", rc)

    stage_calls = {
        "dA_cumsum": lambda: lib.ssd_dA_cumsum(p(dt), p(A), p(cs), p(dtc), b, L, H, Q, sp),
        "chunk_state": lambda: lib.ssd_chunk_state(p(x), p(B), p(dtc), p(cs), p(states), b, L, H, P, N, G, Q, code,
                                                   sp),
        "state_passing": lambda: lib.ssd_state_passing(p(states), p(cs), p(init), p(entry), p(final), b, L, H, P, N,
                                                       Q, code, sp),
        "chunk_scan": lambda: lib.ssd_chunk_scan(p(x), p(B), p(C), p(dtc), p(cs), p(entry), p(D), p(y), b, L, H, P,
                                                 N, G, Q, code, sp),
    }

    def time_region(fn, n):
        """ms per call of n back-to-back calls between two events on the library's stream"""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # ================================================================================================
    # secondary legs first (their results are reported beside the headline)

    # ---- recurrent mode on the decode workload
    decode = None
    if not args.no_decode:
        dc = CONFIGS["decode"]
        g = torch.Generator(device=dev)
        g.manual_seed(dc.seed)
        db, dH, dP, dN, dG = dc.batch, dc.nheads, dc.headdim, dc.dstate, dc.ngroups
        state = 0.1 * torch.randn((db, dH, dP, dN), generator=g, device=dev, dtype=torch.float32)
        dA = -torch.exp(torch.rand(dH, generator=g, device=dev) * float(np.log(16.0)))
        dD = torch.randn(dH, generator=g, device=dev)
        nset = 8
        sx = [torch.randn((db, dH, dP), generator=g, device=dev).to(torch.bfloat16) for _ in range(nset)]
        sdt = [torch.nn.functional.softplus(torch.randn((db, dH), generator=g, device=dev) - 2.0) for _ in range(nset)]
        sB = [(torch.randn((db, dG, dN), generator=g, device=dev) / dN ** 0.5).to(torch.bfloat16) for _ in range(nset)]
        sC = [(torch.randn((db, dG, dN), generator=g, device=dev) / dN ** 0.5).to(torch.bfloat16) for _ in range(nset)]
        yd = torch.empty((db, dH, dP), dtype=torch.bfloat16, device=dev)
        ctr = [0]

        def one():
            k = ctr[0] % nset
            ctr[0] += 1
            rc = lib.ssd_step(p(state), p(sx[k]), p(sdt[k]), p(dA), p(sB[k]), p(sC[k]), p(dD), p(yd), db, dH, dP, dN,
                              dG, ssd.SSD_BF16, sp)
            if rc:
                raise ssd.SSDError("ssd_step", rc)

        for _ in range(16):
            one()
        us = 1e3 * time_region(one, args.decode_steps)
        sw = step_work(db, dH, dP, dN, dG, 2)
        gbs = sw["bytes"] / us / 1e3
        decode = dict(workload="decode: batch 256, 80 heads x 64, state 128, bf16 tokens, fp32 state",
                      steps=args.decode_steps, us_per_step=round(us, 2), tokens_per_s=round(db / (us / 1e6), 1),
                      alg_bytes_per_step=sw["bytes"], gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                      traffic=measured_traffic("decode", "ssd_step"))
        print(f"[bench] ssd_step: {us:.1f} us/step, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
        del state, sx, sdt, sB, sC, yd

    # ---- the same forward as one pass over the sequence per (batch, head) (ssd_forward_fused)
    fused = None
    if not args.no_fused:
        fy = torch.empty_like(y)
        ffin = torch.empty_like(final)

        def fused_call():
            rc = lib.ssd_forward_fused(p(x), p(dt), p(A), p(B), p(C), p(D), p(init), p(fy), p(ffin), b, L, H, P, N, G,
                                       code, sp)
            if rc:
                raise ssd.SSDError("ssd_forward_fused", rc)

        for _ in range(5):
            fused_call()
        nf = max(1, min(args.steps, 20))
        us = 1e3 * time_region(fused_call, nf)
        # x read and y written once, B and C once per group, dt, the initial and final states
        fbytes = 2 * b * L * H * P * es + 2 * b * L * G * N * es + 4 * b * L * H + 2 * 4 * b * H * P * N
        fused = dict(workload=f"{args.workload}, one workgroup per (batch, head, 32-column slice of the head) "
                              "walking the sequence in 32-token blocks, the state on chip",
                     calls=nf, us_per_call=round(us, 1), tokens_per_s=round(b * L / (us / 1e6), 1),
                     algorithmic_bytes=fbytes, achieved_gbs=round(fbytes / (us * 1e3), 1),
                     traffic=measured_traffic(args.workload, "ssd_fused"))
        print(f"[bench] fused forward: {us:.1f} us/call", file=sys.stderr, flush=True)
        del fy, ffin

    # ---- packed variable-length batch: the same layer shape and token count, mixed sequence lengths
    varlen = None
    if not args.no_varlen and args.workload == "l2p7b":
        from mamba_ssd_sequence_chunked_amd.inputs import make_varlen_inputs
        vi = make_varlen_inputs("varlen2p7b")
        vT = vi.x.shape[0]
        vx, vdt, vB, vC = t(vi.x), t(vi.dt), t(vi.B), t(vi.C)
        vcu = torch.from_numpy(vi.cu_seqlens.astype(np.int32)).to(dev)
        nseq = len(vi.cu_seqlens) - 1
        vy = torch.empty_like(vx)
        vfin = torch.empty((nseq, H, P, N), dtype=torch.float32, device=dev)
        vws_bytes = lib.ssd_forward_varlen_workspace_bytes(vT, H, P, N, Q, code)
        vws = torch.empty(vws_bytes, dtype=torch.uint8, device=dev)

        def varlen_call():
            rc = lib.ssd_forward_varlen(p(vx), p(vdt), p(A), p(vB), p(vC), p(D), p(vcu), nseq, p(vy), p(vfin), vT, H,
                                        P, N, G, Q, code, p(vws), vws_bytes, sp)
            if rc:
                raise ssd.SSDError("ssd_forward_varlen", rc)

        for _ in range(5):
            varlen_call()
        us = 1e3 * time_region(varlen_call, max(1, min(args.steps, 20)))
        lens = np.diff(vi.cu_seqlens)
        varlen = dict(workload=f"varlen2p7b: {vT} packed tokens in {nseq} sequences (lengths {int(lens.min())}-"
                               f"{int(lens.max())}), 80 heads x 64, dstate 128, chunk 256, bf16",
                      us_per_call=round(us, 1), tokens_per_s=round(vT / (us / 1e6), 1))
        print(f"[bench] varlen forward: {us:.1f} us/call", file=sys.stderr, flush=True)
        del vx, vdt, vB, vC, vy, vws

    # ---- the backward pass on the same workload (gradients of every input; dL/dy drawn on the device)
    bwd = None
    if not args.no_backward:
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        dyb = torch.randn(x.shape, generator=g, device=dev).to(x.dtype)
        bws_bytes = lib.ssd_backward_workspace_bytes(b, L, H, P, N, G, Q, code)
        bws = torch.empty(bws_bytes, dtype=torch.uint8, device=dev)
        gx, gB, gC = torch.empty_like(x), torch.empty_like(B), torch.empty_like(C)
        gdt = torch.empty_like(dt)
        gA, gD = torch.empty_like(A), torch.empty_like(D)
        ginit = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)

        def bwd_call():
            rc = lib.ssd_backward(p(x), p(dt), p(A), p(B), p(C), p(D), p(init), p(dyb), None, p(gx), p(gdt), p(gA),
                                  p(gB), p(gC), p(gD), p(ginit), b, L, H, P, N, G, Q, code, p(bws), bws_bytes, sp)
            if rc:
                raise ssd.SSDError("ssd_backward", rc)

        for _ in range(3):
            bwd_call()
        us = 1e3 * time_region(bwd_call, args.backward_calls)
        bw_total, bw_kernels = backward_work(b, L, H, P, N, G, Q, es)
        bwd = dict(workload=f"{args.workload} backward: dx, ddt, dA, dB, dC, dD, dinit for a random dL/dy",
                   calls=args.backward_calls, us_per_call=round(us, 1), tokens_per_s=round(b * L / (us / 1e6), 1),
                   alg_bytes_min=bw_total["bytes"], alg_flops=bw_total["flops"],
                   hbm_frac_min_bytes=round(bw_total["bytes"] / us / 1e3 / HBM_PEAK_GBS, 4),
                   mfma_frac_alg=round(bw_total["flops"] / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                   note="the decay-gradient path takes fp32-accurate products: bf16 hi + lo pairs on the bf16 matrix "
                        "cores (see the library header)")
        if inp.dtype == "bf16":
            # the dominant kernels inside the pass, timed by the committed rocprofv3 trace of the same build
            dk = {}
            for kname, w in bw_kernels.items():
                kus = trace_average_us(f"kernel_trace_backward_{args.workload}.md", kname)
                dk[kname] = dict(alg_bytes=w["bytes"], issued_flops=w["flops"], us_trace=kus,
                                 hbm_frac=None if kus is None else round(w["bytes"] / kus / 1e3 / HBM_PEAK_GBS, 4),
                                 mfma_frac_issued=None if kus is None else
                                 round(w["flops"] / kus / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4))
            bwd["kernels"] = dk
        print(f"[bench] backward: {us:.1f} us/call", file=sys.stderr, flush=True)
        del dyb, bws, gx, gB, gC

    # ---- the Mamba-1 selective scan at the same layer width (for the SSD-vs-scan comparison)
    scan = None
    if not args.no_scan:
        from mamba_ssd_sequence_chunked_amd.inputs import SCAN_CONFIGS
        sb, sL, sD, sN, _, _, _, sseed = SCAN_CONFIGS["scan2p7b"]
        g = torch.Generator(device=dev)
        g.manual_seed(sseed)
        sx = torch.randn((sb, sL, sD), generator=g, device=dev).to(torch.bfloat16)
        sdl = torch.nn.functional.softplus(torch.randn((sb, sL, sD), generator=g, device=dev) + float(np.log(np.expm1(0.01))))
        sA = -torch.exp(torch.rand((sD, sN), generator=g, device=dev) * float(np.log(16.0)))
        sBm = (torch.randn((sb, sL, sN), generator=g, device=dev) / sN ** 0.5).to(torch.bfloat16)
        sCm = (torch.randn((sb, sL, sN), generator=g, device=dev) / sN ** 0.5).to(torch.bfloat16)
        sDv = torch.randn(sD, generator=g, device=dev)
        sy = torch.empty_like(sx)
        sfin = torch.empty((sb, sD, sN), dtype=torch.float32, device=dev)

        def scan_call():
            rc = lib.ssd_selective_scan(p(sx), p(sdl), p(sA), p(sBm), p(sCm), p(sDv), None, p(sy), p(sfin), sb, sL,
                                        sD, sN, ssd.SSD_BF16, sp)
            if rc:
                raise ssd.SSDError("ssd_selective_scan", rc)

        scan_call()
        us = 1e3 * time_region(scan_call, args.scan_calls)
        upd = sb * sL * sD * sN / (us / 1e6)
        scan = dict(workload=f"scan2p7b: Mamba-1 selective scan, batch {sb}, seqlen {sL}, {sD} channels, dstate {sN}, "
                             "bf16 x/B/C (inputs drawn on the device, timing only)",
                    calls=args.scan_calls, us_per_call=round(us, 1), tokens_per_s=round(sb * sL / (us / 1e6), 1),
                    bound="alu", updates_per_s=round(upd, 1), peak_updates_per_s=SCAN_UPDATE_PEAK,
                    frac=round(upd / SCAN_UPDATE_PEAK, 4))
        print(f"[bench] selective scan: {us:.1f} us/call", file=sys.stderr, flush=True)
        del sx, sdl, sBm, sCm, sy

    # ---- the forward on the other layer workloads (inputs drawn on the device: timing only; the
    # seeded host draws of the same shapes are what the parity tests check)
    others = None
    if not args.no_other_workloads:
        others = {}
        for wname in ("l130m", "l2p7b", "long64k"):
            if wname == args.workload:
                continue
            c = CONFIGS[wname]
            g = torch.Generator(device=dev)
            g.manual_seed(c.seed)
            ob, oL, oH, oP, oN, oG, oQ = c.batch, c.seqlen, c.nheads, c.headdim, c.dstate, c.ngroups, c.chunk_size
            ox = torch.randn((ob, oL, oH, oP), generator=g, device=dev).to(torch.bfloat16)
            z = torch.randn((ob, oL, oH), generator=g, device=dev)
            if c.dt_kind == "shifted":
                z = z - 2.0
            else:
                z = z + torch.log(torch.expm1(1e-3 + (1e-1 - 1e-3) * torch.rand((ob, oL, oH), generator=g, device=dev)))
            odt = torch.nn.functional.softplus(z)
            oA = -torch.exp(torch.rand(oH, generator=g, device=dev) * float(np.log(16.0)))
            oB = (torch.randn((ob, oL, oG, oN), generator=g, device=dev) / oN ** 0.5).to(torch.bfloat16)
            oC = (torch.randn((ob, oL, oG, oN), generator=g, device=dev) / oN ** 0.5).to(torch.bfloat16)
            oD = torch.randn(oH, generator=g, device=dev)
            oinit = 0.1 * torch.randn((ob, oH, oP, oN), generator=g, device=dev) if c.init else None
            oy = torch.empty_like(ox)
            ofin = torch.empty((ob, oH, oP, oN), dtype=torch.float32, device=dev)
            ows_bytes = ssd.workspace_bytes(ob, oL, oH, oP, oN, oQ, ssd.SSD_BF16)
            ows = torch.empty(ows_bytes, dtype=torch.uint8, device=dev)

            def other_call():
                rc = lib.ssd_forward(p(ox), p(odt), p(oA), p(oB), p(oC), p(oD), p(oinit), p(oy), p(ofin), ob, oL, oH,
                                     oP, oN, oG, oQ, ssd.SSD_BF16, p(ows), ows_bytes, sp)
                if rc:
                    raise ssd.SSDError("ssd_forward", rc)

            for _ in range(5):
                other_call()
            n_o = max(1, min(args.steps, 20))
            us = 1e3 * time_region(other_call, n_o)
            others[wname] = dict(workload=f"{wname}: batch {ob}, seqlen {oL}, {oH} heads x {oP}, dstate {oN}, "
                                          f"{oG} group(s), chunk {oQ}, bf16 x/B/C", calls=n_o, us_per_call=round(us, 1),
                                 tokens_per_s=round(ob * oL / (us / 1e6), 1))
            print(f"[bench] {wname} forward: {us:.1f} us/call", file=sys.stderr, flush=True)
            del ox, odt, oB, oC, oy, ofin, ows, oinit

    # ================================================================================================
    # the headline: W warmup steps, then exactly K timed steps (whole ssd_forward calls)
    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()
    print(f"[bench] {args.workload}: warmup {args.warmup} done", file=sys.stderr, flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        forward()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    tokens = b * L
    value = tokens / (ms_per_step / 1e3)
    print(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall * 1e6 / args.steps:.1f} us/step)",
          file=sys.stderr, flush=True)

    # ---- the same forward call by call: warm, and with L2 and the MALL evicted before every call
    def per_call(fn, n, flush=None):
        out = []
        for _ in range(n):
            if flush is not None:
                flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            out.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(c) for a, c in out]

    ncall = max(20, args.steps)
    fwd_warm = stats_us(per_call(forward, ncall))
    fwd_cold = None
    flush_buf = None
    if not args.no_cold:
        # a 512 MB read (a reduction into one value) between calls: it evicts the call's inputs from L2
        # and the 256 MB MALL without leaving dirty lines there for the timed call to write back
        flush_buf = torch.ones(128 << 20, dtype=torch.int32, device=dev)
        flush_out = torch.empty((), dtype=torch.int64, device=dev)

        def flush():
            torch.sum(flush_buf, dim=0, dtype=torch.int64, out=flush_out)

        fwd_cold = stats_us(per_call(forward, ncall, flush))
    print(f"[bench] forward per call: warm {fwd_warm}, cold {fwd_cold}", file=sys.stderr, flush=True)

    # ---- per-kernel durations: the same four launches with events between them, after one untimed set;
    # the queue is drained before each set and a one-element fill runs just before its first event, so
    # the first interval neither inherits the previous set's tail nor starts on an idle queue
    for name in KERNELS:
        stage_calls[name]()
    lead = torch.empty(1, dtype=torch.float32, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(KERNELS) + 1)] for _ in range(ncall)]
    for i in range(ncall):
        torch.cuda.synchronize()
        lead.fill_(float(i))
        evs[i][0].record(stream)
        for k, name in enumerate(KERNELS):
            rc = stage_calls[name]()
            if rc:
                raise ssd.SSDError(name, rc)
            evs[i][k + 1].record(stream)
    torch.cuda.synchronize()
    kern_ms = {name: [evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(ncall)] for k, name in enumerate(KERNELS)}
    kern_cold = {}
    if flush_buf is not None:
        # each stage alone after a flush (its inputs from HBM, as the first touch in a pipeline would be)
        for k, name in enumerate(KERNELS):
            kern_cold[name] = stats_us(per_call(stage_calls[name], ncall, flush))
    work = kernel_work(b, L, H, P, N, G, Q, es, init is not None)
    kernels = {}
    for name in KERNELS:
        st = stats_us(kern_ms[name])
        us = st["mean"]
        w = work[name]
        kernels[name] = dict(us=round(us, 2), us_median=st["median"], us_min=st["min"], alg_bytes=w["bytes"],
                             alg_flops=w["flops"], gbs=round(w["bytes"] / us / 1e3, 1),
                             hbm_frac=round(w["bytes"] / us / 1e3 / HBM_PEAK_GBS, 4),
                             tflops=round(w["flops"] / us / 1e6, 2),
                             mfma_frac=round(w["flops"] / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4))
        if name in kern_cold:
            kernels[name]["cold"] = kern_cold[name]
            kernels[name]["cold_hbm_frac"] = round(w["bytes"] / kern_cold[name]["median"] / 1e3 / HBM_PEAK_GBS, 4)
        cnt = counter_summary(args.workload, name)
        if cnt is not None and "mfma_flops_issued_per_launch" in cnt:
            issued = cnt["mfma_flops_issued_per_launch"]
            kernels[name]["mfma_issued"] = dict(
                flops_per_launch=issued, tflops=round(issued / us / 1e6, 2),
                frac=round(issued / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                busy_frac_counter=cnt.get("mfma_busy_frac"),
                source="rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per launch (committed counter summary) over the "
                       "live event-timed duration; busy_frac_counter = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE "
                       "per XCD x 1024 SIMDs) in the counter run")
    dominant = max(KERNELS, key=lambda n: kernels[n]["us"])
    dk = kernels[dominant]
    traffic = measured_traffic(args.workload, dominant)
    roofline = dict(kernel=dominant, bound="hbm", achieved=dk["gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(dk["gbs"] / HBM_PEAK_GBS, 4), traffic=traffic,
                    alg_bytes_per_launch=dk["alg_bytes"], us_per_launch=dk["us"], us_median=dk["us_median"],
                    us_min=dk["us_min"])
    if "mfma_issued" in dk:
        roofline["mfma"] = dict(alg_frac=dk["mfma_frac"], issued_frac=dk["mfma_issued"]["frac"],
                                busy_frac_counter=dk["mfma_issued"]["busy_frac_counter"])
    print(f"[bench] per-kernel us: {json.dumps({n: kernels[n]['us'] for n in KERNELS})}", file=sys.stderr, flush=True)

    if fused is not None:
        fused["time_over_chunked"] = round(fused["us_per_call"] / (1e3 * ms_per_step), 2)
    if bwd is not None:
        bwd["time_over_forward"] = round(bwd["us_per_call"] / (ms_per_step * 1e3), 2)
    if scan is not None and args.workload == "l2p7b":
        # same batch and tokens as the l2p7b forward (whose state is 8x larger)
        scan["time_over_ssd_forward"] = round(scan["us_per_call"] / (ms_per_step * 1e3), 3)

    # ---- the fp64 CPU oracle on the host, beside it
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        heads = H if args.workload != "long64k" else 8
        X64 = inp.f64("x")[:, :, :heads]
        B64, C64 = inp.f64("B"), inp.f64("C")
        hpg = H // G
        gsel = sorted({h // hpg for h in range(heads)})
        t0 = time.perf_counter()
        oracle.forward(X64, inp.dt[:, :, :heads], inp.A[:heads], B64[:, :, gsel], C64[:, :, gsel], inp.D[:heads],
                       None if inp.init is None else inp.init[:, :heads], nthreads=0)
        el = time.perf_counter() - t0
        # tokens/s of the whole workload = (token-heads per second) / heads
        cpu = dict(value=round(b * L * heads / el / H, 1), unit="tokens/s", cores=oracle.max_threads(),
                   kind="oracle", cpu_model=cpu_model(), threads=oracle.max_threads(), host_cpus=os.cpu_count(),
                   sample=f"{args.workload}: all {b}x{L} tokens, {heads} of {H} heads, fp64 token-by-token "
                          f"recurrence, {el:.2f} s wall")
        print(f"[bench] oracle: {el:.2f} s for {heads} heads", file=sys.stderr, flush=True)

    out = {
        "metric": "SSD fwd tokens/s at 2.7B-layer shape; % MFMA peak, % HBM BW for ssd_step",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if inp.dtype == "bf16" else "f32", "data": "synthetic (seeded numpy, inputs resident in HBM)",
        "config": {"workload": f"{args.workload}: batch {b}, seqlen {L}, {H} heads x {P}, dstate {N}, "
                               f"{G} group(s), chunk {Q}, {inp.dtype} x/B/C",
                   "global_batch": b, "seq_len": L, "parallelism": "single GPU"},
        "roofline": roofline,
        "forward_per_call_us": {"warm": fwd_warm, "cold_mall_flushed": fwd_cold},
        "kernels": kernels,
        "kernels_note": "the stage entry points timed one by one (mean, median, min over the calls); inside "
                        "ssd_forward stage 1 runs in the prologue of the stage-2 kernel, so the forward launches "
                        "three kernels; cold = each stage alone after a 512 MB read that evicts L2 and the MALL; "
                        "the events around each stage add a few us, which shows on the shortest one (dA_cumsum; "
                        "the committed kernel traces give the launches' own durations)",
        "other_workloads": others,
        "ssd_step": decode,
        "backward": bwd,
        "varlen": varlen,
        "fused_forward": fused,
        "selective_scan": scan,
        "order": "secondary legs, then warmup and the timed steps, then per-call and per-kernel timings",
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
