"""Pins of the oracle's fractional-level TQ codes (SemKV, section 4.1).

What fixes them from outside the codec: the page's printed packing densities
(three five-level codes in 7 bits = 2.333 bits a value, +0.49% over log2 5;
five six-level codes in 13 bits = 2.600, +0.58% over log2 6), Max's 1960
table for the 5- and 6-level Gaussian quantizers, exhaustive digit checks of
the mixed-radix groups, brute-force nearest-centroid search, and the
SemKV operating point's average width (25% of tokens at 2.585 bits, the rest
at 2.322: 2.39 bits)."""
import itertools
import math

import numpy as np
import pytest

from oracle import tq, tqf
from tests.golden_io import load


@pytest.mark.parametrize("levels,printed_bits,printed_overhead", [(5, 2.333, 0.49), (6, 2.600, 0.58)])
def test_packing_density_as_printed(levels, printed_bits, printed_overhead):
    b = tqf.bits_per_value(levels)
    assert round(b, 3) == printed_bits
    assert round(100 * (b / math.log2(levels) - 1), 2) == printed_overhead
    k, nbits = tqf.GROUPS[levels]
    assert levels ** k <= 2 ** nbits < levels ** (k + 1)      # k digits fit, k + 1 would not
    assert tqf.row_bytes(128, levels) == (-(-128 // k) * nbits + 7) // 8


def test_semkv_operating_point_width():
    assert round(0.25 * math.log2(6) + 0.75 * math.log2(5), 2) == 2.39


@pytest.mark.parametrize("levels", [5, 6])
def test_lloyd_max_matches_max_1960(levels):
    g = load("lloyd_max_gaussian.txt")
    c, dist = tq.lloyd_max_gaussian(levels)
    pos = np.atleast_1d(g[f"levels_{levels}"])
    if levels % 2:
        assert abs(c[levels // 2]) < 1e-12                      # the middle level is 0
    assert np.allclose(c[-len(pos):], pos, rtol=0, atol=6e-4)
    assert np.allclose(c, -c[::-1], atol=1e-12)
    assert abs(dist - g[f"mse_{levels}"]) <= 6e-4 * g[f"mse_{levels}"]
    c16, t32 = tqf.codebook_levels(levels)
    assert np.all(np.diff(c16.astype(np.float64)) > 0) and len(t32) == levels - 1


@pytest.mark.parametrize("levels", [5, 6])
def test_every_group_round_trips(levels):
    k, nbits = tqf.GROUPS[levels]
    if levels ** k > 10000:
        digits = list(itertools.islice(itertools.product(range(levels), repeat=k), 0, None, 7))
    else:
        digits = list(itertools.product(range(levels), repeat=k))
    for dg in digits:
        row = np.array(dg, np.uint8)
        packed = tqf.pack_row(row, levels)
        assert len(packed) == (nbits + 7) // 8
        v = int.from_bytes(bytes(packed), "little")
        assert v == sum(int(c) * levels ** i for i, c in enumerate(dg)) < 2 ** nbits
        assert np.array_equal(tqf.unpack_row(packed, k, levels), row)


@pytest.mark.parametrize("levels", [5, 6])
@pytest.mark.parametrize("d", [128, 256])
def test_rows_round_trip_and_codes_are_nearest(levels, d):
    rng = np.random.default_rng(levels * d)
    x = rng.standard_normal((8, d)).astype(np.float32)
    s = tq.signs_from_bits(rng.integers(0, 2 ** 32, d // 32, dtype=np.uint64).astype(np.uint32), d)
    codes, sigma = tqf.encode(x, s, levels)
    assert codes.max() < levels
    for r in range(8):
        packed = tqf.pack_row(codes[r], levels)
        assert len(packed) == tqf.row_bytes(d, levels)
        assert np.array_equal(tqf.unpack_row(packed, d, levels), codes[r])
    # brute force: every code is a nearest fp16 centroid of the normalized
    # rotated coordinate (ties aside)
    c16, _ = tqf.codebook_levels(levels)
    w = tq.fwht((x * s).astype(np.float32)).astype(np.float64)
    n = np.sqrt((x.astype(np.float64) ** 2).sum(-1))[:, None]
    dist = np.abs(w[..., None] / n[..., None] - c16.astype(np.float64))
    best = dist.min(-1)
    assert np.all(dist[np.arange(8)[:, None], np.arange(d)[None, :], codes] <= best + 1e-6)
    # decode restores the norm to within the fp16 rounding of sigma
    xh = tqf.decode(codes, sigma, s, levels)
    assert np.allclose(np.linalg.norm(xh, axis=-1), n[:, 0], rtol=1e-3)
