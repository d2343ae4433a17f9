"""Seeded input generators (CPU only): determinism, shapes, bf16 rounding."""
import numpy as np
import torch

from mamba_ssd_sequence_chunked_amd.inputs import (CONFIGS, bf16_bits, bf16_to_f64, make_random,
                                                   make_step_inputs, make_step_params)


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -0.0, 3.0e38, 1e-40, 1.00390625, 1.01171875], dtype=np.float32)])
    ours = bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy())


def test_same_seed_same_bytes():
    a = make_random(2, 100, 4, 16, 32, 2, 32, "bf16", "ranged", True, seed=7)
    b = make_random(2, 100, 4, 16, 32, 2, 32, "bf16", "ranged", True, seed=7)
    for k in ("x", "dt", "A", "B", "C", "D", "init"):
        assert getattr(a, k).tobytes() == getattr(b, k).tobytes()
    c = make_random(2, 100, 4, 16, 32, 2, 32, "bf16", "ranged", True, seed=8)
    assert a.x.tobytes() != c.x.tobytes()


def test_shapes_and_ranges():
    inp = make_random(3, 70, 6, 16, 32, 3, 32, "f32", "shifted", False, seed=1)
    assert inp.x.shape == (3, 70, 6, 16) and inp.x.dtype == np.float32
    assert inp.B.shape == (3, 70, 3, 32) and inp.dt.shape == (3, 70, 6)
    assert np.all(inp.dt > 0) and np.all(inp.A < 0) and np.all(inp.A >= -16.0) and inp.init is None
    assert inp.dims == (3, 70, 6, 16, 32, 3)


def test_decode_slices_regenerate():
    A, D, st = make_step_params("decode", batch=3)
    assert A.shape == (80,) and st.shape == (3, 80, 64, 128)
    s5 = make_step_inputs("decode", 5, batch=3)
    s5b = make_step_inputs("decode", 5, batch=3)
    assert s5.x.tobytes() == s5b.x.tobytes()
    assert s5.x.shape == (3, 80, 64) and s5.B.shape == (3, 1, 128)


def test_config_table():
    assert CONFIGS["l2p7b"].tokens == 16384
    assert CONFIGS["long64k"].nheads % CONFIGS["long64k"].ngroups == 0
