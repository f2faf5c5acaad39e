"""Pins of the oracle's FP8 E4M3 codec against the OCP FP8 table and the
definition of round-to-nearest-even (not against the oracle's own formulas)."""
import math
import struct

import numpy as np
import pytest

from oracle import fp8
from tests.golden_io import load


def test_ocp_table_points():
    g = load("ocp_fp8_e4m3.txt")
    for k, v in g.items():
        code = int(k, 16)
        got = fp8.E4M3_TABLE[code]
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v)


def test_table_shape():
    finite = fp8.E4M3_TABLE[~np.isnan(fp8.E4M3_TABLE)]
    assert finite.size == 254
    pos = np.unique(np.abs(finite))
    assert pos.size == 127 and pos.max() == 448.0
    # codes 0..0x7E are strictly increasing (the RNE search relies on it)
    assert np.all(np.diff(fp8.E4M3_TABLE[:0x7F]) > 0)


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.E4M3_TABLE[codes].astype(np.float32)
    assert np.array_equal(fp8.e4m3_encode_rne(vals), codes)


def _f32_next(x, direction):
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    if x == 0:
        return np.float32(direction * 1e-45)
    b += direction if x > 0 else -direction
    return np.float32(struct.unpack("<f", struct.pack("<I", b))[0])


def test_ties_go_to_even_and_neighbours_to_nearest():
    for c in range(0, 0x7E):
        lo, hi = fp8.E4M3_TABLE[c], fp8.E4M3_TABLE[c + 1]
        mid = np.float32((lo + hi) / 2)          # exact: both have <= 4 significant bits
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode_rne(np.array([mid]))[0] == even
        assert fp8.e4m3_encode_rne(np.array([_f32_next(float(mid), -1)]))[0] == c
        assert fp8.e4m3_encode_rne(np.array([_f32_next(float(mid), +1)]))[0] == c + 1
        # negative side mirrors with the sign bit
        assert fp8.e4m3_encode_rne(np.array([-mid]))[0] == (even | 0x80)


def test_saturation_and_signed_zero():
    y = np.array([448.0, 460.0, 463.99, 500.0, 1e30, -1e30], dtype=np.float32)
    assert fp8.e4m3_encode_rne(y).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    z = np.array([0.0, -0.0, -1e-30], dtype=np.float32)
    assert fp8.e4m3_encode_rne(z).tolist() == [0x00, 0x80, 0x80]


def test_vector_encode_rules():
    x = np.zeros((2, 16), dtype=np.float32)
    c, s = fp8.fp8_encode(x)
    assert (c == 0).all() and (s == 0).all()
    rng = np.random.default_rng(1)
    x = rng.standard_normal((500, 256)).astype(np.float32)
    c, s = fp8.fp8_encode(x)
    amax = np.abs(x).max(-1)
    # the largest magnitude lands on +-448 and the scale is amax/448 in fp32
    j = np.abs(x).argmax(-1)
    assert np.all((c[np.arange(500), j] & 0x7F) == 0x7E)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # relative error of normal-range values is at most half an ulp: 2^-4
    xh = fp8.fp8_decode(c, s)
    normal = np.abs(x) >= amax[:, None] * (2.0 ** -6) / 448 * 1.01
    rel = np.abs(xh - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4 * 1.0001
    # subnormal-range values are within half a subnormal step
    sub_err = np.abs(xh - x)[~normal] / s.repeat(256).reshape(500, 256)[~normal]
    assert sub_err.size == 0 or sub_err.max() <= 2.0 ** -10 * 1.01


def test_demote_rows_are_exact_products():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    c, s = fp8.fp8_encode(x)
    r = fp8.fp8_decode_f32(c, s)
    assert r.dtype == np.float32
    assert np.array_equal(r.astype(np.float64), np.float32(fp8.fp8_decode(c, s)).astype(np.float64))
