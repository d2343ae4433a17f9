"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle (the default
build, or a variant passed as ``lib``) disagrees with an independent
statement of the same result: a brute-force dense quadratic form, a closed
form, a textbook routine, a hand-worked example or an invariant.  None of
them re-types the recurrence loop itself.
"""
from __future__ import annotations

import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def _rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def rand_problem(seed, b=2, L=24, H=4, P=3, N=5, G=2, init=True, A_zero=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, L, H, P))
    dt = np.logaddexp(0.0, rng.standard_normal((b, L, H)) - 1.0)
    A = np.zeros(H) if A_zero else -np.exp(rng.uniform(0.0, np.log(16.0), H))
    Bm = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    h0 = 0.3 * rng.standard_normal((b, H, P, N)) if init else None
    return x, dt, A, Bm, Cm, D, h0


def dense_mixer(x, dt, A, Bm, Cm, D, h0):
    """y and final state from the explicit matrix-mixer expansion.

    M[t, i] = C_t . B_i * dt_i * prod_{j=i+1..t} a_j for i <= t, zero above
    the diagonal ("Mamba-2" wiki note, section "Matrix Mixer View";
    mohakchugh blog, section "The Duality"), y = M x + D x, plus the initial
    state carried by prod_{j<=t} a_j.  The decay products are formed as
    products of the per-step a_j = exp(dt_j A_h), not via a recurrence."""
    b, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((b, L, H, P))
    fin = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            a = np.exp(dt[bi, :, h] * A[h])
            dec = np.zeros((L, L))       # dec[t, i] = prod_{j=i+1..t} a_j
            for t in range(L):
                for i in range(t + 1):
                    dec[t, i] = np.prod(a[i + 1:t + 1])
            carry = np.array([np.prod(a[:t + 1]) for t in range(L)])
            CB = Cm[bi, :, g, :] @ Bm[bi, :, g, :].T          # (L, L): C_t . B_i
            M = np.tril(CB * dec * dt[bi, None, :, h])
            y[bi, :, h, :] = M @ x[bi, :, h, :] + D[h] * x[bi, :, h, :]
            if h0 is not None:
                y[bi, :, h, :] += carry[:, None] * (Cm[bi, :, g, :] @ h0[bi, h].T)
            w = dec[L - 1, :] * dt[bi, :, h]                  # weight of token i in the final state
            fin[bi, h] = (x[bi, :, h, :] * w[:, None]).T @ Bm[bi, :, g, :]
            if h0 is not None:
                fin[bi, h] += carry[L - 1] * h0[bi, h]
    return y, fin


# ----------------------------------------------------------------------------------------------
def pin_dense_quadratic_form(lib=None):
    """P1: recurrence == dense quadratic form (G in {1, 2}, with/without init)."""
    for seed, G, init in ((1, 1, False), (2, 2, True), (3, 4, True)):
        x, dt, A, Bm, Cm, D, h0 = rand_problem(seed, G=G, init=init)
        y, fin = oracle.forward(x, dt, A, Bm, Cm, D, h0, lib=lib)
        y_ref, fin_ref = dense_mixer(x, dt, A, Bm, Cm, D, h0)
        assert _rel(y, y_ref) < TOL, f"dense form y seed={seed}: {_rel(y, y_ref)}"
        assert _rel(fin, fin_ref) < TOL, f"dense form final seed={seed}: {_rel(fin, fin_ref)}"


def pin_linear_attention(lib=None):
    """P2: A = 0 (unit decay) is causal linear attention:
    y = tril(C B^T) (dt * x) + C h0^T + D x  ("Mamba-2" wiki note, mixer table;
    "Transformers are SSMs" paper card, "How It Works")."""
    x, dt, A, Bm, Cm, D, h0 = rand_problem(11, b=1, L=40, H=2, P=4, N=6, G=1, init=True, A_zero=True)
    y, fin = oracle.forward(x, dt, A, Bm, Cm, D, h0, lib=lib)
    for h in range(2):
        Q_ = Cm[0, :, 0, :]
        K_ = Bm[0, :, 0, :]
        V_ = dt[0, :, h, None] * x[0, :, h, :]
        ref = np.tril(Q_ @ K_.T) @ V_ + Q_ @ h0[0, h].T + D[h] * x[0, :, h, :]
        assert _rel(y[0, :, h, :], ref) < TOL, f"linear attention head {h}: {_rel(y[0, :, h, :], ref)}"
        fin_ref = h0[0, h] + V_.T @ K_
        assert _rel(fin[0, h], fin_ref) < TOL


def pin_scalar_closed_forms(lib=None):
    """P3: N = 1 (the scalar SSM of the mohakchugh blog, "The Duality").
    (i) constant dt, A; x = B = C = 1: geometric series y_t = dt (1 - a^{t+1}) / (1 - a) + D.
    (ii) constant coefficients, random x: a first-order IIR filter, scipy.signal.lfilter."""
    from scipy.signal import lfilter
    L = 50
    dtc, Ac, Dc = 0.3, -1.7, 0.25
    a = np.exp(dtc * Ac)
    ones = np.ones((1, L, 1, 1))
    y, fin = oracle.forward(ones, np.full((1, L, 1), dtc), np.array([Ac]), ones, ones, np.array([Dc]), None, lib=lib)
    t = np.arange(L)
    ref = dtc * (1 - a ** (t + 1)) / (1 - a) + Dc
    assert _rel(y[0, :, 0, 0], ref) < TOL, f"geometric series: {_rel(y[0, :, 0, 0], ref)}"
    assert _rel(fin[0, 0, 0, 0], ref[-1] - Dc) < TOL
    rng = np.random.default_rng(5)
    xs = rng.standard_normal(L)
    b0, c0 = 0.7, -1.3
    y, _ = oracle.forward(xs.reshape(1, L, 1, 1), np.full((1, L, 1), dtc), np.array([Ac]),
                          np.full((1, L, 1, 1), b0), np.full((1, L, 1, 1), c0), np.array([Dc]), None, lib=lib)
    ref = lfilter([c0 * dtc * b0], [1.0, -a], xs) + Dc * xs
    assert _rel(y[0, :, 0, 0], ref) < TOL, f"lfilter: {_rel(y[0, :, 0, 0], ref)}"


def _impulse_matrix(dt, A, Bm, Cm, L, lib=None):
    """Probe the mixing matrix column by column with unit impulses (P = 1, D = 0, zero state)."""
    M = np.zeros((L, L))
    for i in range(L):
        x = np.zeros((1, L, 1, 1))
        x[0, i, 0, 0] = 1.0
        y, _ = oracle.forward(x, dt, A, Bm, Cm, np.zeros(1), None, lib=lib)
        M[:, i] = y[0, :, 0, 0]
    return M


def pin_semiseparable_rank(lib=None):
    """P4: the mixing matrix is lower triangular and every block M[i:, :i+1] of
    its lower triangle has rank <= N ("Mamba-2" wiki note, "Structured
    Semiseparable Matrices"; mohakchugh blog, "The Duality")."""
    L = 24
    for N in (1, 2, 3):
        x, dt, A, Bm, Cm, D, _ = rand_problem(20 + N, b=1, L=L, H=1, P=1, N=N, G=1, init=False)
        A = 0.05 * A          # mild decay, so the far blocks keep a clean numerical rank
        M = _impulse_matrix(dt, A, Bm, Cm, L, lib=lib)
        assert np.all(np.triu(M, 1) == 0.0), "mixing matrix must be causal (lower triangular)"
        for i in range(L - 1):
            blk = M[i:, :i + 1]
            s = np.linalg.svd(blk, compute_uv=False)
            rank = int(np.sum(s > 1e-10 * max(s[0], 1e-300)))
            assert rank <= N, f"N={N} block at {i} has rank {rank}"
        # generic blocks reach rank N
        s = np.linalg.svd(M[L // 2:, :L // 2], compute_uv=False)
        assert int(np.sum(s > 1e-10 * s[0])) == min(N, L // 2)


def pin_skip_only(lib=None):
    """P5: with B = 0 (zero state) or C = 0, the output is exactly D x."""
    x, dt, A, Bm, Cm, D, h0 = rand_problem(31, init=True)
    y, fin = oracle.forward(x, dt, A, np.zeros_like(Bm), Cm, D, None, lib=lib)
    assert np.array_equal(y, D[None, None, :, None] * x), "B = 0 must give y = D x exactly"
    assert np.array_equal(fin, np.zeros_like(fin))
    y, _ = oracle.forward(x, dt, A, Bm, np.zeros_like(Cm), D, h0, lib=lib)
    assert np.array_equal(y, D[None, None, :, None] * x + 0.0), "C = 0 must give y = D x exactly"


def pin_zero_input(lib=None):
    """P6: x = 0 leaves only the decayed initial state:
    y_t = C_t . (prod_{j<=t} a_j) h0, final = prod_j a_j h0."""
    x, dt, A, Bm, Cm, D, h0 = rand_problem(41, init=True)
    x[:] = 0.0
    y, fin = oracle.forward(x, dt, A, Bm, Cm, D, h0, lib=lib)
    b, L, H, P = x.shape
    G = Bm.shape[2]
    for bi in range(b):
        for h in range(H):
            g = h // (H // G)
            carry = np.cumprod(np.exp(dt[bi, :, h] * A[h]))
            ref = carry[:, None] * (Cm[bi, :, g, :] @ h0[bi, h].T)
            assert _rel(y[bi, :, h, :], ref) < TOL
            assert _rel(fin[bi, h], carry[-1] * h0[bi, h]) < TOL


def pin_linearity_causality(lib=None):
    """P7: linear in x for a zero state; causal (a change at t0 leaves y[:t0]
    bit-identical); a NaN at t0 reaches only y[t0:] of its own (b, h, p) row."""
    x1, dt, A, Bm, Cm, D, _ = rand_problem(51, init=False)
    x2 = rand_problem(52, init=False)[0]
    al, be = 0.75, -2.5
    y1, _ = oracle.forward(x1, dt, A, Bm, Cm, D, None, lib=lib)
    y2, _ = oracle.forward(x2, dt, A, Bm, Cm, D, None, lib=lib)
    y12, _ = oracle.forward(al * x1 + be * x2, dt, A, Bm, Cm, D, None, lib=lib)
    assert _rel(y12, al * y1 + be * y2) < TOL
    t0 = 9
    xp = x1.copy()
    xp[:, t0] += 1.0
    yp, _ = oracle.forward(xp, dt, A, Bm, Cm, D, None, lib=lib)
    assert np.array_equal(yp[:, :t0], y1[:, :t0])
    assert not np.array_equal(yp[:, t0:], y1[:, t0:])
    xn = x1.copy()
    xn[1, t0, 2, 1] = np.nan
    yn, _ = oracle.forward(xn, dt, A, Bm, Cm, D, None, lib=lib)
    bad = np.isnan(yn)
    expect = np.zeros_like(bad)
    expect[1, t0:, 2, 1] = True
    assert np.array_equal(bad, expect), "NaN must poison exactly y[t0:] of its row"


def pin_split_resume(lib=None):
    """P8: running the first L1 tokens, then the rest from the returned state,
    equals one pass ("Why Does Mamba-2 Resemble the Transformer?",
    "Mamba-2 Changes More Than the Algorithm": the recurrent state is what
    crosses a split of the sequence)."""
    x, dt, A, Bm, Cm, D, h0 = rand_problem(61, L=30, init=True)
    y, fin = oracle.forward(x, dt, A, Bm, Cm, D, h0, lib=lib)
    for L1 in (1, 13, 29):
        ya, fa = oracle.forward(x[:, :L1], dt[:, :L1], A, Bm[:, :L1], Cm[:, :L1], D, h0, lib=lib)
        yb, fb = oracle.forward(x[:, L1:], dt[:, L1:], A, Bm[:, L1:], Cm[:, L1:], D, fa, lib=lib)
        assert _rel(np.concatenate([ya, yb], axis=1), y) < TOL
        assert _rel(fb, fin) < TOL


def pin_groups(lib=None):
    """P9: G groups == one group per head after repeating B, C to the heads
    that share them (heads are assigned to groups in contiguous blocks)."""
    x, dt, A, Bm, Cm, D, h0 = rand_problem(71, H=6, G=3, init=True)
    y, fin = oracle.forward(x, dt, A, Bm, Cm, D, h0, lib=lib)
    Br = np.repeat(Bm, 2, axis=2)
    Cr = np.repeat(Cm, 2, axis=2)
    y2, fin2 = oracle.forward(x, dt, A, Br, Cr, D, h0, lib=lib)
    assert np.array_equal(y, y2) and np.array_equal(fin, fin2)
    # and heads in different groups really see different B, C
    y3, _ = oracle.forward(x, dt, A, Bm[:, :, ::-1].copy(), Cm[:, :, ::-1].copy(), D, h0, lib=lib)
    assert not np.array_equal(y, y3)


def pin_step_matches_forward(lib=None):
    """P10: the recurrent mode, one token at a time, equals the whole-sequence
    call ("Transformers are SSMs" paper card, "Why It Matters": O(1) decode)."""
    x, dt, A, Bm, Cm, D, h0 = rand_problem(81, init=True)
    y, fin = oracle.forward(x, dt, A, Bm, Cm, D, h0, lib=lib)
    st = h0
    for t in range(x.shape[1]):
        yt, st = oracle.step(st, x[:, t], dt[:, t], A, Bm[:, t], Cm[:, t], D, lib=lib)
        assert _rel(yt, y[:, t]) < TOL
    assert _rel(st, fin) < TOL


def load_hand_example():
    vals = {}
    with open(os.path.join(GOLDEN, "hand_example_n2.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            vals[k] = np.array([float(t) for t in v])
    return vals


def pin_hand_example(lib=None):
    """P11: the hand-worked example in tests/golden/hand_example_n2.txt."""
    v = load_hand_example()
    L = 3
    x = v["x"].reshape(1, L, 1, 1)
    dt = v["dt"].reshape(1, L, 1)
    Bm = np.stack([v["B0"], v["B1"], v["B2"]]).reshape(1, L, 1, 2)
    Cm = np.stack([v["C0"], v["C1"], v["C2"]]).reshape(1, L, 1, 2)
    h0 = v["init"].reshape(1, 1, 1, 2)
    y, fin = oracle.forward(x, dt, v["A"], Bm, Cm, v["D"], h0, lib=lib)
    assert np.max(np.abs(y.ravel() - v["y"])) < 1e-13, f"hand example y {y.ravel()} vs {v['y']}"
    assert np.max(np.abs(fin.ravel() - v["final"])) < 1e-13
    # the same example through the recurrent step
    st = h0
    for t in range(L):
        yt, st = oracle.step(st, x[:, t], dt[:, t], v["A"], Bm[:, t], Cm[:, t], v["D"], lib=lib)
        assert abs(yt.ravel()[0] - v["y"][t]) < 1e-13


def pin_chunk_helpers(lib=None):
    """P12: the chunk-level helpers against closed forms.
    * exp(chunk_log_decay) is the decay product the recurrence applies to a
      unit state (B = 0, C = 1, h0 = 1, D = 0: y_t = prod_{j<=t} a_j within the chunk);
    * chunk_states and chunk_entry_states against the dense expansion
      sum_i (prod_{j=i+1..end} a_j) dt_i x_i B_i^T (+ carried init)."""
    Q = 8
    x, dt, A, Bm, Cm, D, h0 = rand_problem(91, b=2, L=29, H=4, P=3, N=5, G=2, init=True)
    cs = oracle.chunk_log_decay(dt, A, Q)
    b, L, H, P = x.shape
    nc = oracle.n_chunks(L, Q)
    for c in range(nc):
        lo, hi = c * Q, min(L, (c + 1) * Q)
        n = hi - lo
        ones = np.ones((b, n, 1, 1))
        for h in range(H):
            yy, _ = oracle.forward(np.zeros((b, n, 1, 1)), dt[:, lo:hi, h:h + 1], A[h:h + 1],
                                   np.zeros((b, n, 1, 1)), ones, np.zeros(1), np.ones((b, 1, 1, 1)), lib=lib)
            assert _rel(np.exp(cs[:, h, c, :n]), yy[:, :, 0, 0]) < TOL
    st = oracle.chunk_states(x, dt, A, Bm, Cm, D, Q)
    entry, fin, _ = oracle.chunk_entry_states(x, dt, A, Bm, Cm, D, h0, Q)
    G = Bm.shape[2]
    for bi in range(b):
        for h in range(H):
            g = h // (H // G)
            a = np.exp(dt[bi, :, h] * A[h])
            for c in range(nc):
                lo, hi = c * Q, min(L, (c + 1) * Q)
                w = np.array([np.prod(a[i + 1:hi]) * dt[bi, i, h] for i in range(lo, hi)])
                ref = (x[bi, lo:hi, h, :] * w[:, None]).T @ Bm[bi, lo:hi, g, :]
                assert _rel(st[bi, c, h], ref) < TOL
                w0 = np.array([np.prod(a[i + 1:lo]) * dt[bi, i, h] for i in range(0, lo)])
                ref_in = np.prod(a[:lo]) * h0[bi, h]
                if lo:
                    ref_in = ref_in + (x[bi, :lo, h, :] * w0[:, None]).T @ Bm[bi, :lo, g, :]
                assert _rel(entry[bi, c, h], ref_in) < TOL


ALL_PINS = [
    pin_dense_quadratic_form, pin_linear_attention, pin_scalar_closed_forms, pin_semiseparable_rank,
    pin_skip_only, pin_zero_input, pin_linearity_causality, pin_split_resume, pin_groups,
    pin_step_matches_forward, pin_hand_example, pin_chunk_helpers,
]


# ----------------------------------------------------------------------------------------------
# The Mamba-1 selective scan (per-channel diagonal decays; mohakchugh blog, "Mamba-1: Selective
# State Spaces").  Pins S1-S5.

def rand_scan_problem(seed, b=2, L=20, Dm=5, N=4, init=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, L, Dm))
    delta = np.logaddexp(0.0, rng.standard_normal((b, L, Dm)) - 1.0)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), (Dm, N)))
    Bm = rng.standard_normal((b, L, N)) / np.sqrt(N)
    Cm = rng.standard_normal((b, L, N)) / np.sqrt(N)
    D = rng.standard_normal(Dm)
    h0 = 0.3 * rng.standard_normal((b, Dm, N)) if init else None
    return x, delta, A, Bm, Cm, D, h0


def dense_scan(x, delta, A, Bm, Cm, D, h0):
    """y and final state of the selective scan from its explicit expansion: the
    contribution of token i to y_t is sum_n C_t[n] B_i[n] delta_i x_i prod_{j=i+1..t} a_j[n],
    a_j[n] = exp(delta_j A[d, n]), formed as explicit products (no recurrence)."""
    b, L, Dm = x.shape
    N = A.shape[1]
    y = np.zeros((b, L, Dm))
    fin = np.zeros((b, Dm, N))
    for bi in range(b):
        for d in range(Dm):
            a = np.exp(delta[bi, :, d, None] * A[d][None, :])          # (L, N)
            for t in range(L):
                acc = D[d] * x[bi, t, d]
                for i in range(t + 1):
                    dec = np.prod(a[i + 1:t + 1], axis=0)             # (N,)
                    acc += np.sum(Cm[bi, t] * Bm[bi, i] * dec) * delta[bi, i, d] * x[bi, i, d]
                if h0 is not None:
                    acc += np.sum(Cm[bi, t] * np.prod(a[:t + 1], axis=0) * h0[bi, d])
                y[bi, t, d] = acc
            for i in range(L):
                fin[bi, d] += np.prod(a[i + 1:], axis=0) * Bm[bi, i] * delta[bi, i, d] * x[bi, i, d]
            if h0 is not None:
                fin[bi, d] += np.prod(a, axis=0) * h0[bi, d]
    return y, fin


def pin_scan_dense_form(lib=None):
    """S1: selective scan == its explicit expansion (with and without an initial state)."""
    for seed, init in ((21, False), (22, True)):
        x, delta, A, Bm, Cm, D, h0 = rand_scan_problem(seed, init=init)
        y, fin = oracle.selective_scan(x, delta, A, Bm, Cm, D, h0, lib=lib)
        y_ref, fin_ref = dense_scan(x, delta, A, Bm, Cm, D, h0)
        assert _rel(y, y_ref) < TOL, f"scan dense form y seed={seed}: {_rel(y, y_ref)}"
        assert _rel(fin, fin_ref) < TOL, f"scan dense form final seed={seed}: {_rel(fin, fin_ref)}"


def pin_scan_scalar_identity(lib=None):
    """S2: with every state entry of a channel decaying at one rate (A[d, n] = A_d, the
    scalar-times-identity restriction of the "Transformers are SSMs" paper card, "How It
    Works"), the selective scan is the SSD layer with one head per channel, head dimension 1
    and B, C shared: its dense matrix-mixer form (pin P1's builder)."""
    x, delta, A, Bm, Cm, D, h0 = rand_scan_problem(23, b=2, L=16, Dm=3, N=4, init=True)
    A_h = A[:, 0].copy()
    A = np.repeat(A_h[:, None], A.shape[1], axis=1)
    y, fin = oracle.selective_scan(x, delta, A, Bm, Cm, D, h0, lib=lib)
    y_ref, fin_ref = dense_mixer(x[..., None], delta, A_h, Bm[:, :, None, :], Cm[:, :, None, :], D,
                                 h0[:, :, None, :])
    assert _rel(y, y_ref[..., 0]) < TOL, f"scalar identity y: {_rel(y, y_ref[..., 0])}"
    assert _rel(fin, fin_ref[:, :, 0, :]) < TOL, f"scalar identity final: {_rel(fin, fin_ref[:, :, 0, :])}"


def pin_scan_one_hot_filters(lib=None):
    """S3: with delta constant per channel, B constant and C picking one state entry n0, every
    channel is a first-order IIR filter with pole exp(delta_d A[d, n0]) (scipy.signal.lfilter);
    this fixes which entry of A each (channel, state) pair decays with."""
    from scipy.signal import lfilter
    rng = np.random.default_rng(24)
    L, Dm, N = 40, 3, 5
    x = rng.standard_normal((1, L, Dm))
    dl = np.array([0.2, 0.45, 0.7])
    delta = np.broadcast_to(dl, (1, L, Dm)).copy()
    A = -np.exp(rng.uniform(0.0, np.log(16.0), (Dm, N)))
    D = rng.standard_normal(Dm)
    b0, c0 = 0.8, -1.1
    Bm = np.full((1, L, N), b0)
    for n0 in range(N):
        Cm = np.zeros((1, L, N))
        Cm[0, :, n0] = c0
        y, _ = oracle.selective_scan(x, delta, A, Bm, Cm, D, None, lib=lib)
        for d in range(Dm):
            ref = lfilter([c0 * dl[d] * b0], [1.0, -np.exp(dl[d] * A[d, n0])], x[0, :, d]) + D[d] * x[0, :, d]
            assert _rel(y[0, :, d], ref) < TOL, f"one-hot filter n0={n0} d={d}: {_rel(y[0, :, d], ref)}"


def pin_scan_zero_input(lib=None):
    """S4: x = 0 leaves only the decayed initial state:
    y_t[d] = sum_n C_t[n] exp(A[d, n] sum_{j<=t} delta_j[d]) h0[d, n] (a closed form through
    the running sum of delta), and the final state is exp(A[d, n] sum_j delta_j[d]) h0[d, n]."""
    x, delta, A, Bm, Cm, D, h0 = rand_scan_problem(25, b=2, L=30, Dm=4, N=3, init=True)
    x = np.zeros_like(x)
    y, fin = oracle.selective_scan(x, delta, A, Bm, Cm, D, h0, lib=lib)
    cum = np.cumsum(delta, axis=1)                                     # (b, L, Dm)
    dec = np.exp(cum[..., None] * A[None, None])                       # (b, L, Dm, N)
    ref = np.einsum("btn,btdn,bdn->btd", Cm, dec, h0)
    assert _rel(y, ref) < TOL, f"scan zero input: {_rel(y, ref)}"
    assert _rel(fin, dec[:, -1] * h0) < TOL


def pin_scan_split_resume(lib=None):
    """S5: scanning a prefix, then the rest from the prefix's final state, equals one scan."""
    x, delta, A, Bm, Cm, D, h0 = rand_scan_problem(26, b=2, L=33, Dm=4, N=6, init=True)
    y, fin = oracle.selective_scan(x, delta, A, Bm, Cm, D, h0, lib=lib)
    L1 = 14
    y1, f1 = oracle.selective_scan(x[:, :L1], delta[:, :L1], A, Bm[:, :L1], Cm[:, :L1], D, h0, lib=lib)
    y2, f2 = oracle.selective_scan(x[:, L1:], delta[:, L1:], A, Bm[:, L1:], Cm[:, L1:], D, f1, lib=lib)
    assert _rel(np.concatenate([y1, y2], axis=1), y) < TOL
    assert _rel(f2, fin) < TOL


SCAN_PINS = [pin_scan_dense_form, pin_scan_scalar_identity, pin_scan_one_hot_filters, pin_scan_zero_input,
             pin_scan_split_resume]
ALL_PINS = ALL_PINS + SCAN_PINS


# ----------------------------------------------------------------------------------------------
# Packed variable-length batches (state reset at every sequence start).  Pins V1-V3.

def dense_mixer_packed(x, dt, A, Bm, Cm, D, seq_id):
    """y of a packed stream from the dense matrix-mixer form over ALL its tokens, with the
    entries that connect two different sequences set to zero (a block-diagonal mixer): the
    decays are explicit products of a_j over the whole stream, so a missing reset would leave
    cross-sequence entries nonzero."""
    T, H, P = x.shape
    G = Bm.shape[1]
    hpg = H // G
    y = np.zeros((T, H, P))
    same = seq_id[:, None] == seq_id[None, :]
    for h in range(H):
        g = h // hpg
        a = np.exp(dt[:, h] * A[h])
        dec = np.zeros((T, T))
        for t in range(T):
            for i in range(t + 1):
                dec[t, i] = np.prod(a[i + 1:t + 1])
        M = np.tril((Cm[:, g, :] @ Bm[:, g, :].T) * dec * dt[None, :, h]) * same
        y[:, h, :] = M @ x[:, h, :] + D[h] * x[:, h, :]
    return y


def _packed(seed, lens, H=3, P=2, N=4, G=1):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    x = rng.standard_normal((T, H, P))
    dt = np.logaddexp(0.0, rng.standard_normal((T, H)) - 1.0)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), H))
    Bm = rng.standard_normal((T, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((T, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return x, dt, A, Bm, Cm, D, cu


def pin_varlen_dense_form(lib=None):
    """V1: the packed forward == the block-diagonal dense mixer of the whole stream."""
    for seed, lens, G in ((31, [5, 1, 9, 7], 1), (32, [12, 3, 3, 6], 3)):
        x, dt, A, Bm, Cm, D, cu = _packed(seed, lens, G=G)
        seq_id = np.repeat(np.arange(len(lens)), lens)
        y, _ = oracle.forward_varlen(x, dt, A, Bm, Cm, D, cu, lib=lib)
        ref = dense_mixer_packed(x, dt, A, Bm, Cm, D, seq_id)
        assert _rel(y, ref) < TOL, f"varlen dense form seed={seed}: {_rel(y, ref)}"


def pin_varlen_equal_lengths_batch(lib=None):
    """V2: sequences of one length packed end to end == the same sequences as a batch."""
    x, dt, A, Bm, Cm, D, h0 = rand_problem(33, b=3, L=11, H=4, P=3, N=5, G=2, init=False)
    yb, fb = oracle.forward(x, dt, A, Bm, Cm, D, None, lib=lib)
    cu = np.arange(4) * 11
    y, f = oracle.forward_varlen(x.reshape(33, 4, 3), dt.reshape(33, 4), A, Bm.reshape(33, 2, 5),
                                 Cm.reshape(33, 2, 5), D, cu, lib=lib)
    assert _rel(y, yb.reshape(33, 4, 3)) < TOL
    assert _rel(f, fb) < TOL


def pin_varlen_final_states(lib=None):
    """V3: a sequence's final state is the dense form's: sum_i prod_{j>i} a_j dt_i x_i B_i^T over
    its own tokens only; an empty sequence's is zero."""
    lens = [4, 0, 6, 1]
    x, dt, A, Bm, Cm, D, cu = _packed(34, lens, H=2, P=2, N=3)
    _, f = oracle.forward_varlen(x, dt, A, Bm, Cm, D, cu, lib=lib)
    for k in range(len(lens)):
        a, e = cu[k], cu[k + 1]
        for h in range(2):
            ref = np.zeros((2, 3))
            for i in range(a, e):
                w = np.prod(np.exp(dt[i + 1:e, h] * A[h])) * dt[i, h]
                ref += w * np.outer(x[i, h], Bm[i, 0])
            assert np.max(np.abs(f[k, h] - ref)) < TOL * max(1.0, np.max(np.abs(ref))), (k, h)


VARLEN_PINS = [pin_varlen_dense_form, pin_varlen_equal_lengths_batch, pin_varlen_final_states]
ALL_PINS = ALL_PINS + VARLEN_PINS


# ----------------------------------------------------------------------------------------------
# Gradients (the backward pass).  Pins W1-W2.

def _loss(x, dt, A, Bm, Cm, D, h0, dy, dfin, lib=None):
    y, fin = oracle.forward(x, dt, A, Bm, Cm, D, h0, lib=None)
    return float(np.sum(y * dy) + np.sum(fin * dfin))


def pin_backward_finite_differences(lib=None):
    """W1: every gradient equals the central finite difference of L = <y, dy> + <final, dfinal>
    computed with the forward recurrence (step 1e-6 in fp64), on a problem with groups and an
    initial state; all coordinates of every input are probed."""
    rng = np.random.default_rng(41)
    x, dt, A, Bm, Cm, D, h0 = rand_problem(41, b=2, L=7, H=4, P=2, N=3, G=2, init=True)
    dy = rng.standard_normal(x.shape)
    dfin = rng.standard_normal(h0.shape)
    gr = oracle.backward(x, dt, A, Bm, Cm, D, h0, dy, dfin, lib=lib)
    args = dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, init=h0)
    names = dict(x="dx", dt="ddt", A="dA", B="dB", C="dC", D="dD", init="dinit")
    eps = 1e-6
    for k, a in args.items():
        fd = np.zeros_like(a)
        for i in np.ndindex(a.shape):
            old = a[i]
            a[i] = old + eps
            lp = _loss(args["x"], args["dt"], args["A"], args["B"], args["C"], args["D"], args["init"], dy, dfin)
            a[i] = old - eps
            lm = _loss(args["x"], args["dt"], args["A"], args["B"], args["C"], args["D"], args["init"], dy, dfin)
            a[i] = old
            fd[i] = (lp - lm) / (2 * eps)
        assert _rel(gr[names[k]], fd) < 1e-6, f"d{k}: {_rel(gr[names[k]], fd)}"


def pin_backward_structure(lib=None):
    """W2: closed forms: dD_h = sum of x . dy over tokens; with C = 0 and no final-state gradient
    only the skip path remains (dx = D dy, dB = dC's partner terms vanish: dB = 0, ddt = 0, dA = 0);
    the gradients are linear in (dy, dfinal)."""
    rng = np.random.default_rng(42)
    x, dt, A, Bm, Cm, D, h0 = rand_problem(42, b=1, L=9, H=2, P=3, N=4, G=1, init=True)
    dy = rng.standard_normal(x.shape)
    dfin = rng.standard_normal(h0.shape)
    gr = oracle.backward(x, dt, A, Bm, Cm, D, h0, dy, dfin, lib=lib)
    assert _rel(gr["dD"], np.einsum("blhp,blhp->h", x, dy)) < TOL
    z = oracle.backward(x, dt, A, Bm, np.zeros_like(Cm), D, h0, dy, None, lib=lib)
    assert _rel(z["dx"], D[None, None, :, None] * dy) < TOL
    assert np.max(np.abs(z["dB"])) == 0.0 and np.max(np.abs(z["ddt"])) == 0.0 and np.max(np.abs(z["dA"])) == 0.0
    g1 = oracle.backward(x, dt, A, Bm, Cm, D, h0, dy, None, lib=lib)
    g2 = oracle.backward(x, dt, A, Bm, Cm, D, h0, np.zeros_like(dy), dfin, lib=lib)
    for k in gr:
        if k in ("dD", "dA_scale"):          # dD does not depend on dfinal; the scale is not linear
            continue
        assert _rel(gr[k], g1[k] + g2[k]) < TOL, f"linearity {k}"


def pin_backward_dA_scale(lib=None):
    """W3: dA_scale, rebuilt from the dense quadratic form instead of the adjoint recurrence.

    The scale is sum over (b, t) of T_t (sum_p |dy_t[p] yhat_t[p]| + sum_p |u_t[p] du_t[p]|),
    with T_t = sum_{j <= t} dt_j, yhat = y - D x (the mixer part of y, from ``dense_mixer``),
    u_t = dt_t x_t and du_t = g_t B_t.  The adjoint state g_t = dL/dh_t is written out as the
    transpose of the matrix mixer: g_t[p, :] = sum_{t' >= t} (prod_{j=t+1..t'} a_j) dy_t'[p] C_t'
    + (prod_{j=t+1..L-1} a_j) dfinal[p, :], so du_t[p] = sum_t' dec[t', t] (C_t' . B_t) dy_t'[p]
    + dec[L-1, t] (dfinal[p, :] . B_t), the decay products again formed as explicit products."""
    rng = np.random.default_rng(43)
    for G, use_dfin in ((1, True), (2, False)):
        x, dt, A, Bm, Cm, D, h0 = rand_problem(43 + G, b=2, L=11, H=4, P=3, N=4, G=G, init=True)
        dy = rng.standard_normal(x.shape)
        dfin = rng.standard_normal(h0.shape) if use_dfin else None
        gr = oracle.backward(x, dt, A, Bm, Cm, D, h0, dy, dfin, lib=lib)
        y, _ = dense_mixer(x, dt, A, Bm, Cm, D, h0)
        b, L, H, P = x.shape
        hpg = H // G
        ref = np.zeros(H)
        for bi in range(b):
            for h in range(H):
                g = h // hpg
                a = np.exp(dt[bi, :, h] * A[h])
                dec = np.zeros((L, L))
                for t in range(L):
                    for i in range(t + 1):
                        dec[t, i] = np.prod(a[i + 1:t + 1])
                CB = Cm[bi, :, g, :] @ Bm[bi, :, g, :].T           # CB[t', t] = C_t' . B_t
                du = np.tril(CB * dec).T @ dy[bi, :, h, :]          # du[t, p]
                if dfin is not None:
                    du += dec[L - 1, :, None] * (Bm[bi, :, g, :] @ dfin[bi, h].T)
                yhat = y[bi, :, h, :] - D[h] * x[bi, :, h, :]
                u = dt[bi, :, h, None] * x[bi, :, h, :]
                T = np.cumsum(dt[bi, :, h])
                mag = np.sum(np.abs(dy[bi, :, h, :] * yhat), axis=1) + np.sum(np.abs(u * du), axis=1)
                ref[h] += np.sum(T * mag)
        assert _rel(gr["dA_scale"], ref) < 1e-12, f"dA_scale: {_rel(gr['dA_scale'], ref)}"


BACKWARD_PINS = [pin_backward_finite_differences, pin_backward_structure, pin_backward_dA_scale]
ALL_PINS = ALL_PINS + BACKWARD_PINS
