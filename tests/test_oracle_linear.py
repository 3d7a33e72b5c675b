"""Pins of the oracle's dequantisation and product (CPU only)."""
from fractions import Fraction
import os

import numpy as np
import pytest

import oracle
from oracle import linear as olin
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                vals[int(c)] = Fraction(float(v))
    return vals


def _exact_e4m3(byte):
    # Exact rational value from the OFP8 E4M3 definition (bias 7).
    s = -1 if byte >> 7 else 1
    e, m = (byte >> 3) & 15, byte & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _bf16_fraction(bits):
    return Fraction(float(workload.bf16_bits_to_f32(np.array([bits], np.uint16))[0]))


def _brute_force(x_bits, packed, scales, t):
    """Exact rationals, element by element, reading the nibbles one at a time."""
    e2m1 = _golden_e2m1()
    m, k = x_bits.shape
    n = packed.shape[0]
    tf = Fraction(float(np.float32(t)))
    y = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                byte = int(packed[j, kk // 2])
                code = (byte & 0xF) if kk % 2 == 0 else (byte >> 4)
                w = tf * _exact_e4m3(int(scales[j, kk // 16])) * e2m1[code]
                acc += _bf16_fraction(int(x_bits[i, kk])) * w
            y[i][j] = acc
    return y


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 16, 1), (2, 3, 32, 2), (3, 5, 48, 3),
                                        (2, 2, 256, 4), (3, 4, 64, 5)])
def test_linear_ref_matches_exact_rationals(m, n, k, seed):
    packed, scales = workload.random_codes(n, k, seed)
    x = workload.activations_bf16(m, k, seed + 100, outliers=True)
    t = 0.000123
    y = oracle.linear_ref(x, packed, scales, t)
    bnd = oracle.bound(x, packed, scales, t)
    exact = _brute_force(x, packed, scales, t)
    u = 2.0 ** -53
    gamma = k * u / (1 - k * u)
    for i in range(m):
        for j in range(n):
            err = abs(Fraction(float(y[i, j])) - exact[i][j])
            assert err <= Fraction(gamma) * Fraction(float(bnd[i, j])) * (1 + Fraction(1, 10**6))


def test_dequant_is_exact():
    n, k = 4, 64
    packed, scales = workload.random_codes(n, k, 7)
    t = float(np.float32(3.3e-5))
    wd = oracle.dequant(packed, scales, t)
    e2m1 = _golden_e2m1()
    for j in range(n):
        for kk in range(k):
            byte = int(packed[j, kk // 2])
            code = (byte & 0xF) if kk % 2 == 0 else (byte >> 4)
            exact = Fraction(t) * _exact_e4m3(int(scales[j, kk // 16])) * e2m1[code]
            assert Fraction(float(wd[j, kk])) == exact


def _one_hot_ok():
    """A single non-zero nibble at (n, k) with x = e_k gives y = that weight alone."""
    n, k = 3, 256
    ok = True
    for row in range(n):
        for col in (0, 1, 2, 15, 16, 17, 31, 32, 130, 255):
            packed = np.zeros((n, k // 2), np.uint8)
            scales = np.full((n, k // 16), 0x38, np.uint8)           # scale 1.0
            scales[row, col // 16] = 0x40                            # scale 2.0 on that group only
            code = 7                                                 # e2m1 6.0
            packed[row, col // 2] = code if col % 2 == 0 else code << 4
            x = np.zeros((1, k), np.uint16)
            x[0, col] = 0x3F80                                       # bf16 1.0
            y = oracle.linear_ref(x, packed, scales, 1.0)
            want = np.zeros((1, n))
            want[0, row] = 12.0
            ok &= np.array_equal(y, want)
            # the neighbouring element of the same byte contributes nothing
            x2 = np.zeros((1, k), np.uint16)
            x2[0, col ^ 1] = 0x3F80
            ok &= np.array_equal(oracle.linear_ref(x2, packed, scales, 1.0), np.zeros((1, n)))
    return ok


def test_layout_one_hot():
    assert _one_hot_ok()


def test_mutant_nibble_order_fails_one_hot(monkeypatch):
    monkeypatch.setattr(olin, "nibble_shift", lambda k: 4 * (1 - k % 2))
    assert not _one_hot_ok()


def test_mutant_scale_group_fails_one_hot(monkeypatch):
    monkeypatch.setattr(olin, "scale_index", lambda k: k // 32)
    assert not _one_hot_ok()


def test_unit_scales_reduce_to_plain_matmul():
    # All group scales e4m3 1.0 and t = 1: y is x times the e2m1 code values,
    # a small matrix of halves; numpy's float64 matmul is exact on it.
    n, k, m = 7, 128, 3
    g = workload.rng(5)
    codes = g.integers(0, 16, size=(n, k), dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((n, k // 16), 0x38, np.uint8)
    e2m1 = _golden_e2m1()
    dense = np.array([[float(e2m1[int(c)]) for c in row] for row in codes])
    xb = workload.activations_bf16(m, k, 6)
    x = workload.bf16_bits_to_f32(xb).astype(np.float64)
    # make x small integers / 2 so the matmul is exact in float64
    x = np.round(x * 4) / 4
    xb = workload.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(oracle.linear_ref(xb, packed, scales, 1.0), x @ dense.T)


def test_tensor_scale_multiplies_the_weight():
    packed, scales = workload.random_codes(5, 64, 9)
    x = workload.activations_bf16(2, 64, 10)
    y1 = oracle.linear_ref(x, packed, scales, 1.0)
    y2 = oracle.linear_ref(x, packed, scales, 0.25)
    assert np.array_equal(y2, y1 * 0.25)


def test_column_sampling_matches_full():
    packed, scales = workload.random_codes(300, 256, 12)
    x = workload.activations_bf16(3, 256, 13)
    full = oracle.linear_ref(x, packed, scales, 0.01)
    cols = np.array([0, 5, 299, 128])
    bfull = oracle.bound(x, packed, scales, 0.01)
    # BLAS may block the sum differently for another shape: agree to fp64 rounding.
    gamma = 2 * 256 * 2.0 ** -53
    got = oracle.linear_ref(x, packed, scales, 0.01, cols)
    assert np.all(np.abs(got - full[:, cols]) <= gamma * bfull[:, cols])
    assert np.allclose(oracle.bound(x, packed, scales, 0.01, cols), bfull[:, cols], rtol=gamma, atol=0)


def test_row_blocks_do_not_change_the_result(monkeypatch):
    packed, scales = workload.random_codes(50, 64, 14)
    x = workload.activations_bf16(2, 64, 15)
    a = oracle.linear_ref(x, packed, scales, 0.5)
    bnd = oracle.bound(x, packed, scales, 0.5)
    monkeypatch.setattr(olin, "ROW_BLOCK", 7)
    gamma = 2 * 64 * 2.0 ** -53
    assert np.all(np.abs(oracle.linear_ref(x, packed, scales, 0.5) - a) <= gamma * bnd)


def _exact_abs_sums(x_bits, packed, scales, t):
    """Sum over k of |x[m, k] * Wd[n, k]| in exact rationals, nibble by nibble."""
    e2m1 = _golden_e2m1()
    m, k = x_bits.shape
    n = packed.shape[0]
    tf = Fraction(float(np.float32(t)))
    out = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                byte = int(packed[j, kk // 2])
                code = (byte & 0xF) if kk % 2 == 0 else (byte >> 4)
                w = tf * _exact_e4m3(int(scales[j, kk // 16])) * e2m1[code]
                acc += abs(_bf16_fraction(int(x_bits[i, kk])) * w)
            out[i][j] = acc
    return out


# Bound cases: tensor scales away from 1 (so a bound that drops t is caught),
# shapes with several 16-k groups per row and rows in several row blocks.
_BOUND_CASES = [(2, 9, 64, 0.000123, 31), (3, 5, 48, 37.5, 32), (1, 12, 32, 2.0 ** -20, 33)]


def _bound_pinned(bound_fn, monkeypatch) -> bool:
    """bound_fn(x, packed, scales, t, cols) equals the exact sum of |x * Wd|
    to within the float64 rounding of a K-term sum, for full outputs (row-block
    path, with blocks smaller than N) and for sampled columns."""
    monkeypatch.setattr(olin, "ROW_BLOCK", 4)
    ok = True
    for m, n, k, t, seed in _BOUND_CASES:
        packed, scales = workload.random_codes(n, k, seed)
        scales[:, 0] = 0x7E                      # include the largest group scale
        x = workload.activations_bf16(m, k, seed + 50, outliers=True)
        exact = _exact_abs_sums(x, packed, scales, t)
        gamma = Fraction(k + 1) * Fraction(1, 2 ** 53) * 2
        cols = np.array([n - 1, 0, 3])
        full = bound_fn(x, packed, scales, t, None)
        some = bound_fn(x, packed, scales, t, cols)
        for i in range(m):
            for j in range(n):
                e = exact[i][j]
                ok &= abs(Fraction(float(full[i, j])) - e) <= gamma * e
            for c, j in enumerate(cols):
                e = exact[i][int(j)]
                ok &= abs(Fraction(float(some[i, c])) - e) <= gamma * e
    return bool(ok)


def test_bound_is_sum_of_absolute_products(monkeypatch):
    assert _bound_pinned(oracle.bound, monkeypatch)


def test_bound_mutants_fail_the_pin(monkeypatch):
    # Plausible mistakes in bound(): the tensor scale dropped, a constant
    # factor, a signed (not absolute) sum, the activations' sign kept.
    real = oracle.bound
    mutants = {
        "drops t": lambda x, p, s, t, c: real(x, p, s, 1.0, c),
        "x4": lambda x, p, s, t, c: 4.0 * real(x, p, s, t, c),
        "signed": lambda x, p, s, t, c: oracle.linear_ref(x, p, s, t, c),
        "abs of x only": lambda x, p, s, t, c: (np.abs(olin.bf16_bits_to_f64(x)) @
                                                (olin.dequant(p[c], s[c], t) if c is not None
                                                 else olin.dequant(p, s, t)).T),
    }
    for name, fn in mutants.items():
        assert not _bound_pinned(fn, monkeypatch), name


def test_accept_tolerance():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    bnd = np.array([[10.0, 10.0, 0.0]])
    assert oracle.accept(y_ref, y_ref, bnd)
    assert oracle.accept(y_ref + np.array([[0.0199, -0.0199, 0]]), y_ref, bnd)
    assert not oracle.accept(y_ref + np.array([[0.0201, 0, 0]]), y_ref, bnd)
    assert oracle.accept(y_ref + np.array([[0, 0, 9e-7]]), y_ref, bnd)
    assert not oracle.accept(y_ref + np.array([[0, 0, 2e-6]]), y_ref, bnd)
    nan = y_ref.copy(); nan[0, 1] = np.nan
    assert not oracle.accept(nan, y_ref, bnd)
    assert oracle.accept(nan, nan, bnd)


def test_bf16_output_allowance_covers_exact_rounding():
    # One dominating product: |y| equals the bound, and the nearest bf16 of the
    # exact result misses it by almost 2^-8 of |y| -- more than 2e-3 * bound.
    import torch
    y_ref = np.array([[4175.84]])
    bnd = y_ref.copy()
    y16 = torch.from_numpy(y_ref).to(torch.bfloat16).double().numpy()
    assert not oracle.accept(y16, y_ref, bnd, out="f32")
    assert oracle.accept(y16, y_ref, bnd, out="bf16")
    # random sums: the nearest bf16 of the exact result is always accepted
    packed, scales = workload.random_codes(50, 256, 20)
    x = workload.activations_bf16(8, 256, 21, outliers=True)
    y_ref = oracle.linear_ref(x, packed, scales, 0.03)
    bnd = oracle.bound(x, packed, scales, 0.03)
    y16 = torch.from_numpy(y_ref).to(torch.bfloat16).double().numpy()
    assert oracle.accept(y16, y_ref, bnd, out="bf16")
    # but not an output a further bf16 step away.  One product decides the
    # sum: x = 1 + 2^-7 (bf16), w = e2m1 1.5 at scale 1, so y_ref = bound =
    # 1.51171875, halfway between the bf16 neighbours 1.5078125 and 1.515625.
    # Both neighbours are accepted (they miss by 2^-8, which the 2e-3 term
    # alone would reject); 1.5234375, one more step up, is not.
    one_x = np.zeros((1, 32), np.uint16)
    one_x[0, 3] = 0x3F81                                      # bf16 1 + 2^-7
    one_p = np.zeros((1, 16), np.uint8)
    one_p[0, 1] = 0x30                                        # k = 3: code 3 = 1.5
    one_s = np.full((1, 2), 0x38, np.uint8)                   # scale 1.0
    y1 = oracle.linear_ref(one_x, one_p, one_s, 1.0)
    b1 = oracle.bound(one_x, one_p, one_s, 1.0)
    assert y1[0, 0] == 1.51171875 and b1[0, 0] == y1[0, 0]
    for near in (1.5078125, 1.515625):
        assert not oracle.accept(np.array([[near]]), y1, b1, out="f32")
        assert oracle.accept(np.array([[near]]), y1, b1, out="bf16")
    assert not oracle.accept(np.array([[1.5234375]]), y1, b1, out="bf16")
    assert not oracle.accept(np.array([[1.5]]), y1, b1, out="bf16")
    with pytest.raises(ValueError):
        oracle.tolerance(y_ref, bnd, out="f16")
