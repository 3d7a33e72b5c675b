"""Pins of the oracle's e2m1 and e4m3 tables (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_e2m1_matches_published_values():
    rows = _read("e2m1_ocp_mx.txt")
    assert len(rows) == 16
    for code_s, value_s in rows:
        code, value = int(code_s), float(value_s)
        got = oracle.E2M1[code]
        assert got == value
        assert math.copysign(1.0, got) == math.copysign(1.0, value)


def test_e2m1_magnitudes_are_monotone_in_code():
    mags = oracle.E2M1[:8]
    assert np.all(np.diff(mags) > 0)
    assert np.array_equal(oracle.E2M1[8:], -mags)


def test_e4m3_spot_values_match_published_table():
    for byte_s, value_s, _ in _read("e4m3_ocp_fp8.txt"):
        byte = int(byte_s, 16)
        got = oracle.E4M3[byte]
        if value_s == "nan":
            assert math.isnan(got)
        else:
            assert got == float(value_s)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(value_s))


def test_e4m3_table_matches_torch_float8_e4m3fn():
    # A library decoder of the same OCP format, written independently.
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    lib = lib.to(torch.float64).numpy()
    ours = oracle.E4M3
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(lib[ok]))


def test_e4m3_structure():
    pos = oracle.E4M3[:0x7F]
    assert np.all(np.diff(pos) > 0)                    # 127 increasing values
    assert np.array_equal(oracle.E4M3[0x80:0xFF], -pos)
    assert np.isnan(oracle.E4M3[0x7F]) and np.isnan(oracle.E4M3[0xFF])
    assert np.isfinite(oracle.E4M3).sum() == 254
    assert not np.isinf(oracle.E4M3).any()


def test_every_e2m1_times_e4m3_product_is_exact_in_fp16_and_bf16():
    # "10 Kernels" section 10.2: an e2m1 value times an e4m3 scale needs six
    # significant bits, so fp16 (eleven) holds it exactly.  bf16 (eight) does too.
    scales = oracle.E4M3[np.isfinite(oracle.E4M3)]
    prods = (oracle.E2M1[:, None] * scales[None, :]).ravel()
    assert prods.size == 16 * 254
    as_f16 = prods.astype(np.float16).astype(np.float64)
    assert np.array_equal(as_f16, prods)
    as_bf16 = torch.from_numpy(prods).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, prods)
    # and the magnitude needs at most six significant bits
    nz = np.abs(prods[prods != 0])
    m, _ = np.frexp(nz)
    assert np.all((m * 64) == np.round(m * 64))


def test_mutant_e2m1_sign_bit_fails_the_pin(monkeypatch):
    # A planted mistake in the oracle (sign taken from bit 2) must be caught.
    from oracle import formats

    def wrong(code):
        sign = -1.0 if (code >> 2) & 1 else 1.0
        return sign * abs(formats.e2m1_value(code))

    table = np.array([wrong(c) for c in range(16)])
    rows = _read("e2m1_ocp_mx.txt")
    assert any(table[int(c)] != float(v) for c, v in rows)
