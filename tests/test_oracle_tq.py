"""Pins of the oracle's TQ codec: the Gaussian Lloyd-Max table (Max 1960),
dense Hadamard products, brute-force nearest-centroid search, closed-form
special cases and the codec-coordinate identities the kernels rely on."""
import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import tq
from tests.golden_io import load


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_max_1960(bits):
    g = load("lloyd_max_gaussian.txt")
    L = 1 << bits
    c, dist = tq.lloyd_max_gaussian(L)
    pos = np.atleast_1d(g[f"levels_{L}"])
    assert np.allclose(c[L // 2:], pos, rtol=0, atol=6e-4)
    assert np.allclose(c[:L // 2], -pos[::-1], rtol=0, atol=6e-4)
    assert abs(dist - g[f"mse_{L}"]) <= 6e-4 * g[f"mse_{L}"] + 1e-6
    # the distortion formula agrees with direct integration of (x - c)^2
    assert abs(tq.gaussian_distortion(c) - dist) < 1e-12


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fp16_codebook_and_thresholds(bits):
    c16, t32 = tq.codebook(bits)
    c64, dist = tq.lloyd_max_gaussian(1 << bits)
    # fp16 rounding is the nearest fp16 value
    assert np.all(np.abs(c16.astype(np.float64) - c64) <= np.abs(c64) * 2.0 ** -11)
    # symmetric, ascending, thresholds are exact midpoints between them
    assert np.array_equal(c16, -c16[::-1])
    assert np.all(np.diff(c16.astype(np.float64)) > 0)
    mid = (c16[:-1].astype(np.float64) + c16[1:].astype(np.float64)) / 2
    assert np.array_equal(t32.astype(np.float64), mid)
    # rounding the centroids to fp16 leaves the distortion unchanged to 6 decimals
    assert abs(tq.gaussian_distortion(c16.astype(np.float64)) - dist) < 1e-6


@pytest.mark.parametrize("d", [4, 8, 128, 256])
def test_fwht_is_sylvester_hadamard(d):
    rng = np.random.default_rng(d)
    u = rng.standard_normal((5, d))
    assert np.allclose(tq.fwht(u), u @ hadamard(d).T, rtol=0, atol=1e-10)


def test_rotation_is_orthogonal():
    d = 256
    rng = np.random.default_rng(3)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    R = np.stack([tq.rotate(e, s) for e in np.eye(d)], axis=1)   # columns R e_j
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-12)
    x = rng.standard_normal(d)
    assert abs(np.linalg.norm(tq.rotate(x, s)) - np.linalg.norm(x)) < 1e-12


def test_halving_tree_is_a_sum():
    rng = np.random.default_rng(4)
    t = rng.standard_normal((3, 64))
    assert np.allclose(tq.halving_tree_sum(t), t.sum(-1), atol=1e-12)
    # fp32 order: element 0 gets ((t0 + t32) + (t16 + t48)) + ...
    a = np.arange(8, dtype=np.float32)
    assert tq.halving_tree_sum(a) == np.float32(((0 + 4) + (2 + 6)) + ((1 + 5) + (3 + 7)))


def test_signs_from_bits():
    words = np.array([0b1011, 0x80000000], dtype=np.uint32)
    s = tq.signs_from_bits(words, 64)
    assert s[0] == -1 and s[1] == -1 and s[2] == 1 and s[3] == -1 and s[31] == 1 and s[63] == -1
    assert (s == -1).sum() == 4


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d", [4, 8])
def test_codes_are_nearest_centroid_bruteforce(bits, d):
    """For tiny d, compare with an fp64 search over every centroid: the
    threshold rule may only differ within 1e-6 (relative) of a boundary."""
    c16, t32 = tq.codebook(bits)
    c = c16.astype(np.float64)
    rng = np.random.default_rng(10 * bits + d)
    x = rng.standard_normal((4000, d)).astype(np.float32)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    codes, sigma = tq.tq_encode(x, s, bits)
    x64 = x.astype(np.float64)
    n = np.sqrt((x64 * x64).sum(-1))
    z = (x64 * s) @ hadamard(d).T / n[:, None]          # w / n, ~N(0,1)
    best = np.abs(z[..., None] - c).argmin(-1)
    near = np.min(np.abs(z[..., None] - (c[:-1] + c[1:]) / 2), axis=-1) < 1e-6
    assert np.array_equal(codes[~near], best[~near])
    # sigma restores the input norm: sigma * ||c_code|| = ||x|| (fp16 rounding)
    cn = np.sqrt((c[codes] ** 2).sum(-1))
    assert np.allclose(sigma.astype(np.float64) * cn, n, rtol=2.0 ** -11, atol=0)


def test_ties_go_to_the_lower_code():
    for bits in (2, 3, 4):
        c16, t32 = tq.codebook(bits)
        n = np.float32(3.0)
        for k, t in enumerate(t32):
            w = np.float32(n * t)           # exactly on threshold k
            assert tq.tq_quantize(np.array([w]), n, bits)[0] == k
            up = np.nextafter(w, np.float32(np.inf))
            assert tq.tq_quantize(np.array([up]), n, bits)[0] == k + 1


def test_zero_and_spike_vectors():
    d = 128
    s = np.ones(d)
    codes, sigma = tq.tq_encode(np.zeros((1, d), np.float32), s, 3)
    assert (codes == 0).all() and sigma[0] == 0
    # x = a e_0: every rotated coordinate is +-a = +-||x||, i.e. +-1 in units
    # of the norm, which falls between thresholds 0.5005 and 1.0498 -> codes
    # 5 (+0.7559) or 2 (-0.7559), sigma = a / (0.755859375 sqrt(d))
    a = np.float32(2.5)
    x = np.zeros((1, d), np.float32)
    x[0, 0] = a
    codes, sigma = tq.tq_encode(x, s, 3)
    assert set(np.unique(codes).tolist()) == {5}
    assert sigma[0] == np.float16(a / (0.755859375 * math.sqrt(d)))
    x[0, 0] = -a
    codes, _ = tq.tq_encode(x, s, 3)
    assert set(np.unique(codes).tolist()) == {2}
    # a coordinate that rotates to exactly 0 sits on the zero threshold -> lower code 3
    x = np.zeros((1, 4), np.float32)
    x[0, :2] = 1.0                      # FWHT(1,1,0,0) = (2,0,2,0)
    codes, _ = tq.tq_encode(x, np.ones(4), 3)
    assert codes[0].tolist()[1] == 3 and codes[0].tolist()[3] == 3


@pytest.mark.parametrize("bits,expect", [(2, 0.1175), (3, 0.0348), (4, 0.0095)])
def test_gaussian_relative_mse(bits, expect):
    """E||x - x_hat||^2 / ||x||^2 for x ~ N(0, I_256) tracks the Gaussian
    distortion D (with renormalization it is 2 - 2 sqrt(1 - D))."""
    rng = np.random.default_rng(bits)
    d = 256
    x = rng.standard_normal((2000, d)).astype(np.float32)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    codes, sigma = tq.tq_encode(x, s, bits)
    xh = tq.tq_decode(codes, sigma, s, bits)
    rel = ((xh - x) ** 2).sum(-1) / (x.astype(np.float64) ** 2).sum(-1)
    assert abs(rel.mean() - expect) < 0.12 * expect


def test_codec_coordinate_identities():
    """q . x_hat = sigma (R q) . c and sum_i p_i x_hat_i = R^T sum_i p_i sigma_i c_i."""
    rng = np.random.default_rng(7)
    d = 256
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x = rng.standard_normal((64, d)).astype(np.float32)
    codes, sigma = tq.tq_encode(x, s, 3)
    c = tq.codebook(3)[0].astype(np.float64)[codes]
    xh = tq.tq_decode(codes, sigma, s, 3)
    q = rng.standard_normal(d)
    lhs = xh @ q
    rhs = sigma.astype(np.float64) * (c @ tq.rotate(q, s))
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    p = rng.random(64)
    acc_rot = (p * sigma.astype(np.float64)) @ c
    back = s * tq.fwht(acc_rot) / math.sqrt(d)          # R^T y = D_s H y / sqrt(d)
    assert np.allclose(back, p @ xh, rtol=1e-12, atol=1e-12)


def test_encode_is_fp32_deterministic_under_batching():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((33, 128)).astype(np.float32)
    s = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    a = tq.tq_encode(x, s, 3)
    b = [tq.tq_encode(x[i:i + 1], s, 3) for i in range(33)]
    assert np.array_equal(a[0], np.concatenate([t[0] for t in b]))
    assert np.array_equal(a[1], np.concatenate([t[1] for t in b]))


@pytest.mark.parametrize("bits", [2, 3])
def test_sigma_overflows_to_inf_beyond_the_fp16_range(bits):
    """sigma is an fp16 number (IEEE 754 binary16: largest finite 65504, and
    round-to-nearest-even sends every value of 65520 or more to +inf). For a
    spike x = a e_0 every rotated coordinate has |w_j| = a, so every code is
    the level just above w / n = +-1 and ||c_code|| = |c| sqrt(d) in closed
    form; sigma = a / ||c_code|| is finite below 65520 and +inf above it,
    with no warning (it is the defined result, not an error)."""
    import warnings
    d = 128
    c16, t32 = tq.codebook(bits)
    mag = float(np.abs(c16.astype(np.float64)[np.searchsorted(t32, 1.0)]))
    norm_c = mag * np.sqrt(d)
    signs = np.ones(d)
    for target, finite in ((60000.0, True), (65500.0, True), (65540.0, False), (1e6, False)):
        x = np.zeros((1, d), np.float32)
        x[0, 0] = np.float32(target * norm_c)
        with warnings.catch_warnings():
            warnings.simplefilter("error")
            codes, sigma = tq.tq_encode(x, signs, bits)
        ratio = float(x[0, 0]) / norm_c
        if finite:
            assert np.isfinite(sigma[0]) and abs(float(sigma[0]) - ratio) <= 32.0
        else:
            assert np.isposinf(sigma[0])
            with np.errstate(invalid="ignore"):
                xh = tq.tq_decode(codes, sigma, signs, bits)
            assert not np.all(np.isfinite(xh))
