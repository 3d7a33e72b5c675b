"""Pins of the oracle's bf16 expansion of NVFP4 weights (CPU only)."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import expand as oexp
import workload


def _bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern, from the format's fields."""
    s = -1 if bits >> 15 else 1
    e, m = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:
        return s * Fraction(m, 128) * Fraction(2) ** -126
    return s * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def _nearest_even_bf16(v: Fraction, negative: bool = False) -> int:
    """Brute force: the finite bf16 nearest to v, ties to an even pattern
    (`negative` gives the sign of a zero)."""
    best = None
    sign = 0x8000 if v < 0 or (v == 0 and negative) else 0
    for b in range(0x7F80):                                  # every finite magnitude
        d = abs(abs(v) - _bf16_value(b))
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return best[1] | sign


def test_round_to_bf16_is_nearest_even_by_brute_force():
    g = workload.rng(3)
    vals = list(g.standard_normal(12) * 10.0 ** g.integers(-40, 38, 12))
    vals += [1.51171875, 1.5078125 + 2.0 ** -9, -(1 + 2.0 ** -8), 1 + 3 * 2.0 ** -8, 2.0 ** -130,
             3 * 2.0 ** -134, 2.0 ** -134, 2.0 ** -126 - 2.0 ** -134, 0.0]
    got = oracle.round_to_bf16(np.array(vals))
    for v, b in zip(vals, got):
        assert int(b) == _nearest_even_bf16(Fraction(v), np.signbit(v)), v


def test_round_to_bf16_matches_fp32_conversion_on_fp32_values():
    # For a value that is already fp32, torch's fp32 -> bf16 cast is one
    # round-to-nearest-even: the oracle must agree on every such value,
    # including subnormals, exact midpoints and values next to them.
    g = workload.rng(4)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-90, 88, 20000))).astype(np.float32)
    mids = (np.arange(0, 1 << 16, 7, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    x = x[np.isfinite(x) & (np.abs(x) < 3.3e38)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to_bf16(x.astype(np.float64)), want)


def test_dequant_bf16_without_scale_is_exact_and_with_scale_rounds_once():
    packed, scales = workload.random_codes(9, 64, 5)
    scales[0, :] = 0x01                                       # smallest subnormal scale
    t = float(np.float32(3.7e-5))
    exact = oracle.dequant(packed, scales, 1.0)
    got = oracle.dequant_bf16(packed, scales, t, apply_tensor_scale=False)
    assert np.array_equal(workload.bf16_bits_to_f32(got).astype(np.float64), exact)
    scaled = oracle.dequant_bf16(packed, scales, t, apply_tensor_scale=True)
    full = oracle.dequant(packed, scales, t)
    for b, v in zip(scaled.ravel()[::37], full.ravel()[::37]):
        assert int(b) == _nearest_even_bf16(Fraction(float(v)), np.signbit(v))


def test_round_to_bf16_nan_and_overflow():
    got = oracle.round_to_bf16(np.array([np.nan, 2.0 ** 128, -(2.0 ** 128), 3.4e38]))
    assert got[0] == 0x7FC0 and got[1] == 0x7F80 and got[2] == 0xFF80 and got[3] == 0x7F80
