"""Plant plausible mistakes in copies of the oracle (CPU only) and check that
at least one pin catches each of them.  This guards the pins themselves: a
pin set that a dropped term, a wrong sign or index, or a swapped operand
slips through would not pin the oracle."""
import os
import subprocess

import pytest

import oracle
from oracle_pins import (BACKWARD_PINS, SCAN_PINS, pin_dense_quadratic_form, pin_groups, pin_hand_example, pin_skip_only,
                         pin_step_matches_forward, pin_zero_input, pin_scalar_closed_forms)

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

MUTANTS = {
    "dropped_skip_term": [("acc + D[h] * xv", "acc")],
    "decay_sign": [("exp(dtv * A[h])", "exp(-dtv * A[h])")],
    "input_not_scaled_by_dt": [("const double u = dtv * xv;", "const double u = xv;")],
    "B_C_swapped_in_update": [("S[n] = a * S[n] + u * Bt[n];", "S[n] = a * S[n] + u * Ct[n];")],
    "B_C_swapped_in_readout": [("acc += Ct[n] * S[n];", "acc += Bt[n] * S[n];")],
    "readout_before_update": [("S[n] = a * S[n] + u * Bt[n];\n                    acc += Ct[n] * S[n];",
                               "acc += Ct[n] * S[n];\n                    S[n] = a * S[n] + u * Bt[n];")],
    "decay_after_input": [("S[n] = a * S[n] + u * Bt[n];", "S[n] = a * (S[n] + u * Bt[n]);")],
    "group_map_interleaved": [("const int64_t g = h / heads_per_group;", "const int64_t g = h % ngroups;")],
    "init_ignored": [("init ? init[state_off + n] : 0.0", "0.0")],
    "dt_of_neighbour_head": [("dt[(b * seqlen + t) * nheads + h]", "dt[(b * seqlen + t) * nheads + (h + 1) % nheads]")],
    # forward only (the first occurrence): the step has no previous token
    "decay_uses_previous_dt": [("const double a = exp(dtv * A[h]);",
                                "const double a = exp((t ? dt[(b * seqlen + t - 1) * nheads + h] : dtv) * A[h]);", 1)],
}

# mistakes planted in the selective scan (the Mamba-1 recurrence), caught by its own pins
SCAN_MUTANTS = {
    "scan_dropped_skip_term": [("y[bt * dim + d] = acc + D[d] * xv;", "y[bt * dim + d] = acc;")],
    "scan_decay_sign": [("exp(dl * A[d * dstate + n])", "exp(-dl * A[d * dstate + n])")],
    "scan_A_transposed": [("A[d * dstate + n]", "A[n * dim + d]")],
    "scan_decay_shared_over_states": [("A[d * dstate + n]", "A[d * dstate]")],
    "scan_input_not_scaled_by_delta": [("const double u = dl * xv;", "const double u = xv;")],
    "scan_B_C_swapped_in_update": [("S[n] = a * S[n] + u * Bm[bt * dstate + n];",
                                    "S[n] = a * S[n] + u * Cm[bt * dstate + n];")],
    "scan_readout_before_update": [("S[n] = a * S[n] + u * Bm[bt * dstate + n];\n                    acc += Cm[bt * dstate + n] * S[n];",
                                    "acc += Cm[bt * dstate + n] * S[n];\n                    S[n] = a * S[n] + u * Bm[bt * dstate + n];")],
    "scan_decay_after_input": [("S[n] = a * S[n] + u * Bm[bt * dstate + n];", "S[n] = a * (S[n] + u * Bm[bt * dstate + n]);")],
    "scan_init_ignored": [("init ? init[r * dstate + n] : 0.0", "0.0")],
    "scan_delta_of_neighbour_channel": [("const double dl = delta[bt * dim + d];",
                                         "const double dl = delta[bt * dim + (d + 1) % dim];")],
}

# mistakes planted in the backward, caught by the gradient pins
BACKWARD_MUTANTS = {
    "bwd_decay_before_dy": [("for (int64_t n = 0; n < N; ++n) gs[p * N + n] += dyt[p] * Ct[n];",
                             "for (int64_t n = 0; n < N; ++n) gs[p * N + n] = a * gs[p * N + n] + dyt[p] * Ct[n];")],
    "bwd_ddt_missing_decay_term": [("ddt[bt * nheads + h] = xdu + A[h] * a * da;", "ddt[bt * nheads + h] = xdu;")],
    "bwd_dB_missing_dt": [("sb += gs[p * N + n] * dtv * xt[p];", "sb += gs[p * N + n] * xt[p];")],
    "bwd_dC_previous_state": [("sc += hs[(t + 1) * PN + p * N + n] * dyt[p];", "sc += hs[t * PN + p * N + n] * dyt[p];")],
    "bwd_dx_missing_skip": [("dx[(bt * nheads + h) * P + p] = dtv * acc + D[h] * dyt[p];",
                             "dx[(bt * nheads + h) * P + p] = dtv * acc;")],
    "bwd_dA_missing_dt": [("dA_acc += dtv * a * da;", "dA_acc += a * da;")],
    "bwd_dinit_not_decayed": [("for (int64_t i = 0; i < PN; ++i) gs[i] *= a;",
                               "if (t > 0) for (int64_t i = 0; i < PN; ++i) gs[i] *= a;")],
    # the scale dA's error is measured against
    "bwd_scale_prefix_exclusive": [("for (int64_t j = 0; j <= t; ++j) T += dt", "for (int64_t j = 0; j < t; ++j) T += dt")],
    "bwd_scale_previous_state": [("yh += hs[(t + 1) * PN + p * N + n] * Ct[n];", "yh += hs[t * PN + p * N + n] * Ct[n];")],
    "bwd_scale_missing_du_term": [("mag += fabs(dyt[p] * yh) + fabs(dtv * xt[p] * du[p]);", "mag += fabs(dyt[p] * yh);")],
    "bwd_scale_missing_dt": [("fabs(dtv * xt[p] * du[p])", "fabs(xt[p] * du[p])")],
}

PINS = [pin_hand_example, pin_skip_only, pin_zero_input, pin_scalar_closed_forms, pin_groups,
        pin_dense_quadratic_form, pin_step_matches_forward]


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(SCAN_MUTANTS) + sorted(BACKWARD_MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    if name in MUTANTS:
        edits, pins = MUTANTS[name], PINS
    elif name in SCAN_MUTANTS:
        edits, pins = SCAN_MUTANTS[name], SCAN_PINS
    else:
        edits, pins = BACKWARD_MUTANTS[name], BACKWARD_PINS
    for old, new, *count in edits:
        assert old in src, f"mutation site for {name} not found"
        src = src.replace(old, new, *count)
    path = tmp_path / "ssd_oracle_mutant.c"
    path.write_text(src)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(so), str(path), "-lm"])
    lib = oracle.load_variant(str(so))
    caught = []
    for pin in pins:
        try:
            pin(lib=lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


# mistakes planted in the packed variable-length driver (Python), each caught by the varlen pins
def _varlen_no_reset(x, dt, A, B, C, D, cu_seqlens, nthreads=0, lib=None):
    """the whole packed stream run as one sequence (state carried across sequence starts)"""
    import numpy as np
    y, f = oracle.forward(np.asarray(x)[None], np.asarray(dt)[None], A, np.asarray(B)[None], np.asarray(C)[None], D,
                          None, lib=lib)
    cu = np.asarray(cu_seqlens)
    fin = np.zeros((len(cu) - 1,) + f.shape[1:])
    return y[0], fin


def _varlen_shifted_boundary(x, dt, A, B, C, D, cu_seqlens, nthreads=0, lib=None):
    """every sequence start moved one token late"""
    import numpy as np
    cu = np.asarray(cu_seqlens).copy()
    cu[1:-1] = np.minimum(cu[1:-1] + 1, cu[-1])
    return _ORIG_VARLEN(x, dt, A, B, C, D, cu, nthreads=nthreads, lib=lib)


_ORIG_VARLEN = oracle.forward_varlen


@pytest.mark.parametrize("mutant", [_varlen_no_reset, _varlen_shifted_boundary], ids=["no_reset", "shifted_boundary"])
def test_varlen_mutant_is_caught(mutant, monkeypatch):
    from oracle_pins import VARLEN_PINS
    monkeypatch.setattr(oracle, "forward_varlen", mutant)
    caught = []
    for pin in VARLEN_PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutant.__name__}"
