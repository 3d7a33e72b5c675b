"""Pins of the oracle's FP8 block-scaled product (W8A16) and its quantiser
(CPU only)."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import fp8 as of8
import workload


def _e4m3_exact(byte):
    s = -1 if byte >> 7 else 1
    e, m = (byte >> 3) & 15, byte & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _random_fp8(n, k, seed):
    g = workload.rng(seed)
    codes = g.integers(0, 256, size=(n, k), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                    # no NaN codes
    scales = (g.uniform(0.5, 2.0, size=(n // 128, k // 128)) * 2.0 ** -7).astype(np.float32)
    return codes, scales


def test_linear_fp8_matches_exact_rationals():
    n, k, m = 256, 256, 2
    codes, scales = _random_fp8(n, k, 1)
    x = workload.activations_bf16(m, k, 2, outliers=True)
    y = oracle.linear_fp8_ref(x, codes, scales)
    bnd = oracle.bound_fp8(x, codes, scales)
    for i in range(m):
        for j in (0, 1, 127, 128, 200, 255):
            acc, aabs = Fraction(0), Fraction(0)
            for kk in range(k):
                w = _e4m3_exact(int(codes[j, kk])) * Fraction(float(scales[j // 128, kk // 128]))
                p = Fraction(float(workload.bf16_bits_to_f32(x[i:i + 1, kk])[0])) * w
                acc += p
                aabs += abs(p)
            gamma = Fraction(2 * k, 2 ** 53)
            assert abs(Fraction(float(y[i, j])) - acc) <= gamma * aabs
            assert abs(Fraction(float(bnd[i, j])) - aabs) <= gamma * aabs


def test_block_scale_indexing_one_hot():
    # one weight at (n, k) with every scale distinct: y picks S[n // 128, k // 128]
    n, k = 384, 512
    scales = (np.arange(1, 3 * 4 + 1, dtype=np.float32).reshape(3, 4))
    for row, col in [(0, 0), (127, 129), (128, 127), (300, 511), (255, 256)]:
        codes = np.zeros((n, k), np.uint8)
        codes[row, col] = 0x38                               # 1.0
        x = np.zeros((1, k), np.uint16)
        x[0, col] = 0x3F80
        y = oracle.linear_fp8_ref(x, codes, scales)
        want = np.zeros((1, n))
        want[0, row] = scales[row // 128, col // 128]
        assert np.array_equal(y, want), (row, col)


def test_quantizer_matches_torch_fp8_cast_and_round_trips():
    w = workload.weights_f32(256, 384, 3)
    codes, s = oracle.quantize_fp8_ref(w)
    # each block's scale is its absmax / 448 in fp32, so |W / S| <= 448 (up to
    # the scale's rounding) and the codes are the e4m3 cast of W / S
    blocks = w.reshape(2, 128, 3, 128)
    assert np.array_equal(s, (np.abs(blocks).max(axis=(1, 3)).astype(np.float64) / 448.0).astype(np.float32))
    v = (w.astype(np.float64) / np.repeat(np.repeat(s, 128, 0), 128, 1).astype(np.float64)).astype(np.float32)
    v = np.clip(v, -448, 448)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # float32 rounding of W / S may move a value across a tie; compare where it did not
    exact = (w.astype(np.float64) / np.repeat(np.repeat(s, 128, 0), 128, 1)) == v.astype(np.float64)
    assert np.array_equal(codes[exact], want[exact])
    # weights built as e4m3 * S come back exactly
    sc = np.array([[2.0 ** -5, 3.0 * 2 ** -9], [0.75, 1.0]], np.float32)
    c0 = workload.rng(4).integers(0, 0x7F, size=(256, 256), dtype=np.uint8)
    c0[0, 0], c0[0, 128], c0[128, 0], c0[128, 128] = 0x7E, 0x7E, 0x7E, 0x7E   # each block's max is 448
    w2 = (oracle.E4M3[c0] * np.repeat(np.repeat(sc, 128, 0), 128, 1)).astype(np.float32)
    c2, s2 = oracle.quantize_fp8_ref(w2)
    assert np.array_equal(s2, sc) and np.array_equal(c2, c0)


def test_mutant_block_index_fails(monkeypatch):
    # scale blocks indexed by k // 64 instead of 128 would change one-hot results
    codes = np.zeros((128, 256), np.uint8)
    codes[5, 100] = 0x38
    scales = np.array([[1.0, 2.0]], np.float32)
    x = np.zeros((1, 256), np.uint16)
    x[0, 100] = 0x3F80
    assert oracle.linear_fp8_ref(x, codes, scales)[0, 5] == 1.0
    monkeypatch.setattr(of8, "BLOCK", 64)
    try:
        assert oracle.linear_fp8_ref(x, codes, np.array([[1.0, 2.0, 3.0, 4.0], [5.0] * 4], np.float32))[0, 5] != 1.0
    finally:
        monkeypatch.setattr(of8, "BLOCK", 128)
