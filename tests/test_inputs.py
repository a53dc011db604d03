"""The seeded input generator: determinism, storage rounding, shapes and ranges."""
import math

import numpy as np
import pytest

from non_linear_matrix_amd.inputs import CONFIGS, bf16_bits_to_fp32, fp32_to_bf16_bits, generate, scaled


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.5, 3.0e38, 1e-40, 0.0, -0.0], np.float32)
    b = fp32_to_bf16_bits(x)
    back = bf16_bits_to_fp32(b)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == np.float32(1.0 + 2.0 ** -6)
    assert back[3] == -1.5 and back[6] == 0.0 and np.signbit(back[7])
    # every bf16 value round-trips exactly
    allbits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_fp32(allbits)
    fin = np.isfinite(vals)
    assert np.array_equal(fp32_to_bf16_bits(vals[fin]), allbits[fin])


def test_generation_is_deterministic_and_seeded():
    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=8)
    a, b, c = generate(cfg, 0), generate(cfg, 0), generate(cfg, 1)
    for key in ("k", "v", "q", "f", "W", "H0"):
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])


@pytest.mark.parametrize("name", list(CONFIGS))
def test_shapes_dtypes_and_ranges(name):
    cfg = CONFIGS[name]
    small = scaled(cfg, T=min(cfg.T, 16), B=min(cfg.B, 2))
    x = generate(small, 0)
    B, H, K, V, T = small.B, small.H, small.K, small.V, small.T
    store = np.float32 if cfg.dtype == "f32" else np.uint16
    assert x["k"].shape == (B, H, T, K) and x["k"].dtype == store
    assert x["q"].shape == (B, H, T, K) and x["v"].shape == (B, H, T, V)
    assert x["f"].shape == (B, H, T) and x["W"].shape == (H, V, V)
    val = (lambda a: a) if cfg.dtype == "f32" else bf16_bits_to_fp32
    f = val(x["f"])
    assert np.all(f >= 0) and np.all(f <= 1)
    w = val(x["W"]).astype(np.float64)
    assert abs(w.std() * math.sqrt(V) - 1) < 0.1
    if cfg.h0 == "zero":
        assert x["H0"] is None
    else:
        assert x["H0"].dtype == np.float32 and np.max(np.abs(x["H0"])) <= 0.5


def test_qkv_scale_and_gate_means():
    x = generate(scaled(CONFIGS["C2"], T=64), 0)
    k = bf16_bits_to_fp32(x["k"]).astype(np.float64)
    assert abs(k.std() * 8 - 1) < 0.05               # N(0, 1) / sqrt(64)
    y = generate(scaled(CONFIGS["C3"], T=32, B=1), 0)
    k3 = bf16_bits_to_fp32(y["k"]).astype(np.float64)
    assert abs(k3.std() - 1) < 0.05                  # unscaled
    f = bf16_bits_to_fp32(generate(scaled(CONFIGS["C5"], T=256), 0)["f"]).astype(np.float64)
    f = np.clip(f, 1e-6, 1 - 1e-6)
    logit = np.log(f / (1 - f))
    assert abs(np.median(logit) - 3) < 0.1
