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


# ---------------------------------------------------------------- page layout
@pytest.mark.parametrize("levels,d,row", [(5, 128, 38), (6, 128, 43), (5, 256, 76), (6, 256, 85)])
def test_head_block_and_token_bytes(levels, d, row):
    """Row bytes from the printed densities by hand: ceil(d / k) groups of
    nbits bits, rounded up to bytes (d = 128, L = 5: 43 groups x 7 = 301 bits
    = 38 bytes). A head block is P key rows, P value rows, 2 x P fp16
    sigmas; a token-head costs 2 rows + 4 bytes."""
    from oracle import accounting as acc, layout as OL
    from oracle.attention import FMT_TQF5, FMT_TQF6, head_block_bytes
    assert tqf.row_bytes(d, levels) == row
    fmt = FMT_TQF5 if levels == 5 else FMT_TQF6
    for P in (16, 32):
        assert OL.tqf_head_bytes(P, d, levels) == head_block_bytes(fmt, P, d) == P * (2 * row + 4)
    assert acc.token_head_bytes(fmt, d) == 2 * row + 4


@pytest.mark.parametrize("levels", [5, 6])
def test_packed_head_puts_each_digit_where_the_rule_says(levels):
    """Hand-placed digits: code c at dim j of token t sits in group j // k as
    digit j % k (weight L^(j % k)), at bit (j // k) * nbits of row t."""
    from oracle import layout as OL
    k, nbits = tqf.GROUPS[levels]
    P, d = 16, 128
    R = tqf.row_bytes(d, levels)
    kc = np.zeros((P, d), np.uint8)
    vc = np.zeros((P, d), np.uint8)
    placed = [(0, 0, 1), (3, 5, levels - 1), (7, d - 1, 2), (15, 64, 3)]
    for t, j, c in placed:
        kc[t, j] = c
    vc[9, 100] = 4
    ks = np.arange(P, dtype=np.float16)
    vs = -np.arange(P, dtype=np.float16)
    blk = OL.tqf_pack_head(kc, vc, ks, vs, levels)
    assert len(blk) == OL.tqf_head_bytes(P, d, levels)
    for t, j, c in placed:
        row = int.from_bytes(bytes(blk[t * R:(t + 1) * R]), "little")
        g, i = divmod(j, k)
        assert (row >> (g * nbits)) & ((1 << nbits) - 1) == c * levels ** i
    vrow = int.from_bytes(bytes(blk[(P + 9) * R:(P + 10) * R]), "little")
    assert vrow == 4 * levels ** (100 % k) << ((100 // k) * nbits)
    got = OL.tqf_unpack_head(blk, P, d, levels)
    assert np.array_equal(got[0], kc) and np.array_equal(got[1], vc)
    assert np.array_equal(got[2], ks) and np.array_equal(got[3], vs)


@pytest.mark.parametrize("levels", [5, 6])
def test_cache_page_dequant_and_rebuild_follow_the_codec(levels):
    """A TQF page of the cache builder holds the codec's codes and sigmas;
    its dequantization is sigma * s * FWHT(c) / sqrt(d) computed directly, and
    the fp32 rebuild used by promotion agrees with it to fp32 rounding."""
    import math
    from oracle import attention as A, cache as OC, layout as OL, promote as PR
    from oracle.attention import FMT_TQF5, FMT_TQF6
    from scipy.linalg import hadamard
    fmt = FMT_TQF5 if levels == 5 else FMT_TQF6
    rng = np.random.default_rng(levels)
    P, Hkv, d = 16, 2, 128
    K = rng.standard_normal((P, Hkv, d)).astype(np.float32)
    V = rng.standard_normal((P, Hkv, d)).astype(np.float32)
    words = rng.integers(0, 2 ** 32, (Hkv, 2, d // 32), dtype=np.uint64).astype(np.uint32)
    page = OC.encode_page(fmt, K, V, 11, words)                 # slots 11.. empty
    hb = A.head_block_bytes(fmt, P, d)
    c16, _ = tqf.codebook_levels(levels)
    H = hadamard(d).astype(np.float64)
    for g in range(Hkv):
        sk = tq.signs_from_bits(words[g, 0], d)
        sv = tq.signs_from_bits(words[g, 1], d)
        blk = page[g * hb:(g + 1) * hb]
        kc, vc, ksig, vsig = OL.tqf_unpack_head(blk, P, d, levels)
        ck, sgk = tqf.encode(np.where(np.arange(P)[:, None] < 11, K[:, g], 0), sk, levels)
        assert np.array_equal(kc, ck) and np.array_equal(ksig.view(np.uint16), sgk.view(np.uint16))
        assert np.all(kc[11:] == 0) and np.all(ksig[11:] == 0)
        k_hat, v_hat = A.dequant_page_head(fmt, blk, P, d, sk, sv)
        want = ksig.astype(np.float64)[:, None] * sk * (c16.astype(np.float64)[kc] @ H) / math.sqrt(d)
        assert np.allclose(k_hat, want, rtol=0, atol=1e-12)
        k32, v32 = PR.reconstruct_head_f32(fmt, blk, P, d, sk, sv)
        assert np.allclose(k32, k_hat, rtol=2e-7, atol=1e-30)
        assert np.allclose(v32, v_hat, rtol=2e-7, atol=1e-30)
