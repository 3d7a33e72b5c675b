"""Pins of the oracle's fused forms: silu(gate) * up and the de-interleaved
output order (CPU only)."""
import numpy as np
import scipy.special

import oracle
import workload


def test_silu_against_the_logistic_function():
    # silu(g) = g * sigma(g) with sigma the logistic function (scipy's expit,
    # a library routine), and its limits: 0 at 0, g for large g, 0 for very
    # negative g.
    g = np.concatenate([workload.rng(1).standard_normal(1000) * 8, [0.0, 50.0, -50.0, 1e-30, -800.0]])
    ref = g * scipy.special.expit(g)
    assert np.allclose(oracle.silu(g), ref, rtol=4e-16, atol=0)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([60.0]))[0] == 60.0
    assert abs(oracle.silu(np.array([-800.0]))[0]) == 0.0


def test_silu_mul_bf16_rounds_the_float64_product_once():
    g = workload.activations_bf16(4, 256, 2)
    u = workload.activations_bf16(4, 256, 3, outliers=True)
    got = oracle.silu_mul_bf16(g, u)
    gf = workload.bf16_bits_to_f32(g).astype(np.float64)
    uf = workload.bf16_bits_to_f32(u).astype(np.float64)
    exact = gf * scipy.special.expit(gf) * uf
    val = workload.bf16_bits_to_f32(got).astype(np.float64)
    # nearest bf16: within half a bf16 step (2^-8 of the value's binade)
    half_step = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(exact), 1e-300))).astype(int) - 8)
    assert np.all(np.abs(val - exact) <= half_step * (1 + 1e-12))


def test_deinterleave_printed_layouts():
    # Q|gate per head, 2 heads of 3: [q0 q0 q0 g0 g0 g0 q1 q1 q1 g1 g1 g1]
    # is stored as [q0 q0 q0 q1 q1 q1 g0 g0 g0 g1 g1 g1].
    names = ["q0a", "q0b", "q0c", "g0a", "g0b", "g0c", "q1a", "q1b", "q1c", "g1a", "g1b", "g1c"]
    out = oracle.deinterleave(np.array([names]), [3, 3])[0].tolist()
    assert out == ["q0a", "q0b", "q0c", "q1a", "q1b", "q1c", "g0a", "g0b", "g0c", "g1a", "g1b", "g1c"]
    # Q, K, V, Z per group with unequal widths (2, 1, 1, 2), 2 groups
    rows = ["Q0", "Q0'", "K0", "V0", "Z0", "Z0'", "Q1", "Q1'", "K1", "V1", "Z1", "Z1'"]
    out = oracle.deinterleave(np.array([rows]), [2, 1, 1, 2])[0].tolist()
    assert out == ["Q0", "Q0'", "Q1", "Q1'", "K0", "K1", "V0", "V1", "Z0", "Z0'", "Z1", "Z1'"]


def test_deinterleave_columns_is_a_permutation():
    for n, widths in [(8192, [128, 128]), (12288, [256, 128, 128, 256]), (48, [48]), (30, [1, 2, 3, 4])]:
        cols = oracle.deinterleave_columns(n, widths)
        assert np.array_equal(np.sort(cols), np.arange(n))
    assert np.array_equal(oracle.deinterleave_columns(7, [7]), np.arange(7))   # one part: identity
