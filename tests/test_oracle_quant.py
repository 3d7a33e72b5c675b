"""Pins of the oracle's reference quantiser (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quant as oq
import workload


def test_e4m3_round_matches_torch_cast_on_fp32_values():
    # torch's fp32 -> float8_e4m3fn cast rounds to nearest even; inside the
    # finite range it is the same rule as Q3.
    g = workload.rng(3)
    u = np.concatenate([
        g.uniform(0, 448, 20000),
        np.exp(g.uniform(np.log(2.0 ** -12), np.log(448), 20000)),
        oracle.E4M3[:0x7F],                                   # exact points
        (oracle.E4M3[:0x7E] + oracle.E4M3[1:0x7F]) / 2,       # every midpoint
    ]).astype(np.float32)
    lib = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.e4m3_round(u.astype(np.float64))
    assert np.array_equal(ours, lib)


def test_e4m3_round_saturates():
    assert oracle.e4m3_round(np.array([448.0, 448.0001, 464.0, 1e30])).tolist() == [0x7E] * 4
    assert oracle.e4m3_round(np.array([0.0, 2.0 ** -10, 2.0 ** -10 * 1.0001])).tolist() == [0, 0, 1]


@pytest.mark.parametrize("v,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
                                    (3.5, 6), (5.0, 6), (-0.25, 0), (-0.75, 10),
                                    (-1.25, 10), (-1.75, 12), (-2.5, 12), (-3.5, 14),
                                    (-5.0, 14), (7.0, 7), (-100.0, 15), (6.0, 7),
                                    (0.2499, 0), (0.2501, 1), (-0.0, 0)])
def test_e2m1_round_ties_and_saturation(v, code):
    # Ties go to the even code: 0.25 -> 0 (0.0), 0.75 -> 2 (1.0), 1.25 -> 2,
    # 1.75 -> 4 (2.0), 2.5 -> 4, 3.5 -> 6 (4.0), 5 -> 6; |v| > 6 -> 6.
    assert int(oracle.e2m1_round(np.array([v]))[0]) == code


def test_e2m1_round_is_nearest():
    g = workload.rng(4)
    v = g.uniform(-8, 8, 50000)
    c = oracle.e2m1_round(v)
    got = oracle.E2M1[c]
    grid = oracle.E2M1[:8]
    best = np.min(np.abs(np.abs(v)[:, None] - grid[None, :]), axis=1)
    assert np.all(np.abs(np.abs(v) - np.abs(got)) <= best)
    assert np.all((np.sign(got) == np.sign(v)) | (got == 0))


def _round_trip_case(seed):
    """W = t * E4M3[s] * E2M1[c] with every group's largest |code| 6 and one
    group at s = 0x7E, t an fp32 with 16 significant bits: every Q-step is
    exact, so the quantiser must return (c, s, t)."""
    g = workload.rng(seed)
    n, k = 6, 64
    mant = int(g.integers(2 ** 15, 2 ** 16))
    t = float(np.float32(mant * 2.0 ** -30))
    s = g.integers(1, 0x7E, size=(n, k // 16), dtype=np.uint8)
    s[2, 1] = 0x7E
    mag = g.integers(0, 8, size=(n, k))
    sign = g.integers(0, 2, size=(n, k))
    codes = (mag | (sign << 3)).astype(np.uint8)
    codes[mag == 0] = 0                                   # no -0 codes
    for r in range(n):
        for gi in range(k // 16):
            j = gi * 16 + int(g.integers(0, 16))
            codes[r, j] = 7 | (int(sign[r, j]) << 3)      # group max |code| = 6
    w = t * oracle.E4M3[s][:, np.arange(k) // 16] * oracle.E2M1[codes]
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return w32, packed, s, t


@pytest.mark.parametrize("seed", range(5))
def test_quantize_round_trip_closed_form(seed):
    w, packed, s, t = _round_trip_case(seed)
    p2, s2, t2 = oracle.quantize_ref(w)
    assert t2 == t
    assert np.array_equal(s2, s)
    assert np.array_equal(p2, packed)


def test_quantize_error_bound():
    w = workload.weights_f32(64, 256, 8)
    packed, s, t = oracle.quantize_ref(w)
    wd = oracle.dequant(packed, s, t)
    big_s = oracle.E4M3[s][:, np.arange(256) // 16] * np.float64(np.float32(t))
    v = np.abs(w.astype(np.float64)) / big_s
    # half the e2m1 grid spacing at |v|: 0.25 below 2, 0.5 below 4, 1 up to 6
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    sat = np.maximum(v - 6.0, 0.0)
    assert np.all(np.abs(w - wd) <= big_s * (half + sat) * (1 + 1e-12))
    # groups keep their largest weight within e4m3's relative step (2^-4)
    amax = np.max(np.abs(w.reshape(64, 16, 16)), axis=2)
    wmax = np.max(np.abs(wd.reshape(64, 16, 16)), axis=2)
    assert np.all(np.abs(wmax - amax) <= amax * 2.0 ** -3)


def test_quantize_special_cases():
    z = np.zeros((2, 32), np.float32)
    p, s, t = oracle.quantize_ref(z)
    assert t == 1.0 and not p.any() and not s.any()
    w = np.zeros((2, 32), np.float32)
    w[0, 3] = 1.0                             # one non-zero group; the rest are zero groups
    p, s, t = oracle.quantize_ref(w)
    assert s[0, 0] == 0x7E and s[0, 1] == 0 and not s[1].any()
    assert t == float(np.float32(1.0 / 2688.0))
    assert (p[0, 1] >> 4) == 7 and p[0, 0] == 0
    with pytest.raises(ValueError):
        oracle.quantize_ref(np.full((1, 16), np.nan, np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_ref(np.full((1, 16), np.inf, np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_ref(np.zeros((1, 8), np.float32))
    # negative weights carry the sign bit; tiny negatives that round to 0 do not
    w = np.zeros((1, 16), np.float32)
    w[0, 0] = -6.0
    w[0, 1] = -0.1
    p, s, t = oracle.quantize_ref(w)
    assert (p[0, 0] & 0xF) == 15 and (p[0, 0] >> 4) == 0


def test_mutant_tie_rule_fails_the_tie_pins(monkeypatch):
    # Planting "ties away from zero" in the oracle must break a tie pin.
    def away(values, grid):
        values = np.asarray(values, dtype=np.float64)
        d = np.abs(values[:, None] - grid[None, :])
        best = d.min(axis=1, keepdims=True)
        return np.where(d == best, np.arange(len(grid)), -1).max(axis=1)
    monkeypatch.setattr(oq, "_nearest_code", away)
    assert int(oq.e2m1_round(np.array([0.75]))[0]) != 2 or \
        int(oq.e2m1_round(np.array([2.5]))[0]) != 4
