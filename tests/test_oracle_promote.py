"""Pins of the oracle's promotion (compressed page -> FP8 page).

What fixes them from outside the promotion code: the fp64 TQ decode and the
FP8 codec (both pinned in their own tests), a 60-digit decimal square root
for the 1/sqrt(d) constant, the closed form of a constant code row (its
Hadamard transform is a single spike), the E4M3 rounding bound (3 mantissa
bits: half-ulp 2^-4 relative, 2^-10 of the scale below the normal range),
and codes taken straight from the encoder before any packing (so a wrong tile
index or role in the unpack shows up)."""
import decimal

import numpy as np
import pytest

import workloads as W
from oracle import fp8, layout as L, promote, tq, tqk
from oracle.attention import FMT_FP8, FMT_TQ2, FMT_TQ3, FMT_TQK, head_block_bytes
from oracle.cache import encode_page

F32 = np.float32


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
def test_inv_sqrt_constant_is_the_nearest_fp32(d):
    decimal.getcontext().prec = 60
    t = decimal.Decimal(1) / decimal.Decimal(d).sqrt()
    r = promote.inv_sqrt_f32(d)
    lo, hi = np.nextafter(r, F32(0)), np.nextafter(r, F32(1))
    err = abs(decimal.Decimal(float(r)) - t)
    assert err <= abs(decimal.Decimal(float(lo)) - t)
    assert err <= abs(decimal.Decimal(float(hi)) - t)
    if d in (16, 64, 256):
        assert float(r) == 1.0 / np.sqrt(d)          # powers of 4: exact


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [32, 128, 256])
def test_fwht_of_centroids_is_exact_in_fp32(bits, d):
    c16, _ = tq.codebook(bits)
    rng = np.random.default_rng(bits * 1000 + d)
    rows = [np.full(d, len(c16) - 1), np.zeros(d, np.int64), rng.integers(0, len(c16), d)]
    for codes in rows:
        c = c16.astype(F32)[codes]
        assert np.array_equal(tq.fwht(c).astype(np.float64), tq.fwht(c.astype(np.float64)))


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256])
def test_reconstruction_is_the_decode_within_two_roundings(bits, d):
    rng = np.random.default_rng(7 * bits + d)
    x = rng.standard_normal((64, d)).astype(F32)
    s = tq.signs_from_bits(rng.integers(0, 2 ** 32, d // 32, dtype=np.uint64).astype(np.uint32), d)
    codes, sigma = tq.tq_encode(x, s, bits)
    got = promote.tq_reconstruct_f32(codes, sigma, s, bits).astype(np.float64)
    ref = tq.tq_decode(codes, sigma, s, bits)
    assert np.all(np.abs(got - ref) <= 2.0 ** -22 * np.abs(ref) + 1e-30)
    assert np.array_equal(np.signbit(got[ref != 0]), np.signbit(ref[ref != 0]))


@pytest.mark.parametrize("bits", [2, 3])
def test_constant_code_row_is_one_spike(bits):
    d = 256
    c16, _ = tq.codebook(bits)
    code = len(c16) - 1
    sigma = np.array([1.5], np.float16)
    words = np.array([0x80000001, 0x7, 0, 0, 0, 0, 0, 0x80000000], np.uint32)
    s = tq.signs_from_bits(words, d)
    x = promote.tq_reconstruct_f32(np.full((1, d), code, np.uint8), sigma, s, bits)[0]
    # FWHT of a constant row c is (d c, 0, ..., 0): x_0 = sigma s_0 sqrt(d) c
    assert x[0] == F32(1.5 * s[0] * 16 * float(c16[code]))
    assert np.all(x[1:] == 0)
    assert np.array_equal(np.signbit(x[1:]), s[1:] < 0)          # zeros keep the sign flip
    codes, scale = fp8.fp8_encode(x[None, :])
    assert codes[0, 0] == (0xFE if x[0] < 0 else 0x7E)          # the spike saturates to 448
    assert np.array_equal(codes[0, 1:], np.where(s[1:] < 0, 0x80, 0x00).astype(np.uint8))
    assert scale[0] == F32(abs(x[0]) / F32(448))


def _fp8_bound(xhat, scale):
    """E4M3 rounding bound per element: 2^-4 relative for normal codes,
    2^-10 of the scale in the subnormal range; plus fp32 slack."""
    return np.maximum(np.abs(xhat) * 2.0 ** -4, 2.0 ** -10 * scale[..., None]) * (1 + 2.0 ** -20) + 1e-30


@pytest.mark.parametrize("fmt,d", [(FMT_TQ3, 256), (FMT_TQ3, 128), (FMT_TQ2, 128)])
def test_promoted_page_decodes_to_the_compressed_page(fmt, d):
    P, Hkv, n_valid = 16, 2, 13
    bits = 3 if fmt == FMT_TQ3 else 2
    rng = np.random.default_rng(fmt * 100 + d)
    Kp = rng.standard_normal((P, Hkv, d)).astype(F32)
    Vp = rng.standard_normal((P, Hkv, d)).astype(F32)
    signs = rng.integers(0, 2 ** 32, (Hkv, 2, d // 32), dtype=np.uint64).astype(np.uint32)
    page = encode_page(fmt, Kp, Vp, n_valid, signs)
    out = promote.promote_page(fmt, page, Hkv, P, d, signs)
    assert out.size == Hkv * head_block_bytes(FMT_FP8, P, d)
    hb = head_block_bytes(FMT_FP8, P, d)
    for g in range(Hkv):
        kc8, vc8, ks, vs = L.fp8_unpack_head(out[g * hb:(g + 1) * hb], P, d)
        for role, (c8, sc, X) in enumerate([(kc8, ks, Kp), (vc8, vs, Vp)]):
            s = tq.signs_from_bits(signs[g, role], d)
            x = X[:, g, :].copy()
            x[n_valid:] = 0
            codes, sigma = tq.tq_encode(x, s, bits)               # codes before any packing
            ref = tq.tq_decode(codes, sigma, s, bits)
            got = fp8.fp8_decode(c8, sc)
            assert np.all(np.abs(got - ref) <= _fp8_bound(ref, sc)), (g, role)
            assert np.all(c8[n_valid:] == 0) and np.all(sc[n_valid:] == 0)
            assert np.all(sc[:n_valid] > 0)


def test_promoted_grouped_key_page_decodes_to_the_compressed_page():
    w = W.WORKLOADS["l70b"]
    P, d, Hkv = 32, 128, 2
    rates = W.make_tqk_rates(w, 3, 0)[:Hkv]
    rng = np.random.default_rng(11)
    Kp = rng.standard_normal((P, Hkv, d)).astype(F32)
    Vp = rng.standard_normal((P, Hkv, d)).astype(F32)
    signs = rng.integers(0, 2 ** 32, (Hkv, 2, d // 32), dtype=np.uint64).astype(np.uint32)
    page = encode_page(FMT_TQK, Kp, Vp, P, signs, tqk=rates)
    out = promote.promote_page(FMT_TQK, page, Hkv, P, d, signs, tqk=rates)
    hb = head_block_bytes(FMT_FP8, P, d)
    for g in range(Hkv):
        kc8, vc8, ks, vs = L.fp8_unpack_head(out[g * hb:(g + 1) * hb], P, d)
        sk = tq.signs_from_bits(signs[g, 0], d)
        sv = tq.signs_from_bits(signs[g, 1], d)
        perm, segs = tqk.segments(rates[g])
        kref = tqk.decode_key(tqk.encode_key(Kp[:, g, :], perm, segs, sk), perm, segs, sk)
        vcodes, vsig = tq.tq_encode(Vp[:, g, :], sv, 3)
        vref = tq.tq_decode(vcodes, vsig, sv, 3)
        assert np.all(np.abs(fp8.fp8_decode(kc8, ks) - kref) <= _fp8_bound(kref, ks))
        assert np.all(np.abs(fp8.fp8_decode(vc8, vs) - vref) <= _fp8_bound(vref, vs))


def test_promoting_an_empty_page_gives_an_empty_fp8_page():
    P, d, Hkv = 16, 128, 1
    signs = np.zeros((Hkv, 2, d // 32), np.uint32)
    page = np.zeros(Hkv * head_block_bytes(FMT_TQ3, P, d), np.uint8)
    out = promote.promote_page(FMT_TQ3, page, Hkv, P, d, signs)
    assert not out.any()


def test_fp8_pages_cannot_be_promoted():
    with pytest.raises(ValueError):
        promote.reconstruct_head_f32(FMT_FP8, np.zeros(8, np.uint8), 16, 128, None, None)
