"""TurboQuant-MSE-style b-bit codec of Stale pages (TQ3, and TQ2/TQ4 segments).

Minima-KV, section 3.1 "Stale (S, TQ3)": a three-bit rotated scalar quantizer
with codes, scales and metadata stored next to the page; section 4.3: the
conversion is normalize-rotate-pack; section 4.1: per page and KV head, 3-bit
K codes with an fp16 norm correction and 3-bit V codes with fp16 metadata.
Block-GTQ, appendix B.1: one rotation per group generated once from a fixed
seed and reused for every token; Lloyd-Max centroids under the Gaussian
coordinate model; the decoded direction is renormalized and the stored input
norm restored. SemKV, section 4.9: TurboQuant-MSE = random rotation followed by
a Gaussian-optimal Lloyd-Max codebook with one stored scalar per row.

Readings this oracle fixes where the pages are silent:
  * rotation R = H D_s / sqrt(d): flip signs s (an input), then the Sylvester
    Hadamard transform H, for one (layer, KV head, role);
  * codebook: N(0,1) Lloyd-Max centroids for 2^b levels, rounded to fp16;
    decision thresholds are the fp32 midpoints of adjacent fp16 centroids;
  * the renormalize-then-restore step is folded into one stored fp16
    sigma = ||x|| / ||c_code||, so x_hat = sigma * R^T c_code;
  * values use the same codec with their own signs (one fp16 sigma).

Encode of one vector x (fp32, length d), every step fp32 RNE, no FMA:
  1. t_j = x_j * x_j; halving tree: for h = d/2, d/4, .., 1: t[:h] += t[h:2h];
     n = sqrt(t_0)
  2. u = s * x                       (sign flips, exact)
  3. w = FWHT(u), unnormalized, stages h = 1, 2, 4, .., d/2:
     (u_i, u_{i+h}) <- (u_i + u_{i+h}, u_i - u_{i+h})
  4. T_k = n * t_k; code_j = #{k : w_j > T_k}   (a tie goes to the lower code)
  5. cn2 = halving-tree sum of c[code_j]^2; sigma = fp16_RNE(n / sqrt(cn2))
  zero vector -> codes 0, sigma 0.
Decode (fp64): x_hat = sigma * s * FWHT(c[code]) / sqrt(d).
"""
from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# Gaussian Lloyd-Max scalar quantizer (Lloyd's method I)
# --------------------------------------------------------------------------
def _phi(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x: float) -> float:
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def lloyd_max_gaussian(levels: int, iters: int = 20000, tol: float = 1e-15):
    """Centroids (ascending, fp64) and MSE distortion of the N(0,1) Lloyd-Max
    quantizer with `levels` levels: alternate nearest-neighbour cells (midpoint
    thresholds) and conditional-mean centroids until nothing moves."""
    c = [(_inv_Phi((k + 0.5) / levels)) for k in range(levels)]
    for _ in range(iters):
        t = [-math.inf] + [(c[k] + c[k + 1]) / 2 for k in range(levels - 1)] + [math.inf]
        new = []
        for k in range(levels):
            a, b = t[k], t[k + 1]
            pa = 0.0 if a == -math.inf else _phi(a)
            pb = 0.0 if b == math.inf else _phi(b)
            mass = _Phi(b) - _Phi(a)
            new.append((pa - pb) / mass)
        delta = max(abs(x - y) for x, y in zip(new, c))
        c = new
        if delta < tol:
            break
    t = [-math.inf] + [(c[k] + c[k + 1]) / 2 for k in range(levels - 1)] + [math.inf]
    dist = 1.0
    for k in range(levels):
        mass = _Phi(t[k + 1]) - _Phi(t[k])
        dist -= c[k] * c[k] * mass
    return np.array(c, dtype=np.float64), dist


def _inv_Phi(p: float) -> float:
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _Phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def gaussian_distortion(centroids: np.ndarray) -> float:
    """MSE of N(0,1) quantized to the nearest of the given (ascending) centroids."""
    c = [float(v) for v in centroids]
    t = [-math.inf] + [(c[k] + c[k + 1]) / 2 for k in range(len(c) - 1)] + [math.inf]
    total = 0.0
    for k in range(len(c)):
        a, b = t[k], t[k + 1]
        # integral of (x - c)^2 phi(x) over (a, b)
        pa = 0.0 if a == -math.inf else _phi(a)
        pb = 0.0 if b == math.inf else _phi(b)
        aa = 0.0 if a == -math.inf else a * _phi(a)
        bb = 0.0 if b == math.inf else b * _phi(b)
        m0 = _Phi(b) - _Phi(a)
        m1 = pa - pb
        m2 = m0 + aa - bb
        total += m2 - 2 * c[k] * m1 + c[k] * c[k] * m0
    return total


_CODEBOOK_CACHE = {}


def codebook(bits: int):
    """(centroids fp16 [2^b] ascending, thresholds fp32 [2^b - 1] ascending)."""
    if bits not in _CODEBOOK_CACHE:
        c64, _ = lloyd_max_gaussian(1 << bits)
        c16 = c64.astype(np.float16)
        c32 = c16.astype(np.float32)
        t32 = ((c32[:-1] + c32[1:]) / np.float32(2)).astype(np.float32)
        _CODEBOOK_CACHE[bits] = (c16, t32)
    return _CODEBOOK_CACHE[bits]


# --------------------------------------------------------------------------
# rotation pieces
# --------------------------------------------------------------------------
def fwht(u: np.ndarray) -> np.ndarray:
    """Unnormalized Walsh-Hadamard transform along the last axis, in the dtype
    of `u`, with butterfly stages h = 1, 2, 4, ..."""
    w = np.array(u, copy=True)
    d = w.shape[-1]
    assert d & (d - 1) == 0
    h = 1
    while h < d:
        v = w.reshape(w.shape[:-1] + (d // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        w = v.reshape(w.shape)
        h *= 2
    return w


def halving_tree_sum(t: np.ndarray) -> np.ndarray:
    """Sum along the last axis by t[:h] += t[h:2h], h = d/2, d/4, .., 1."""
    t = np.array(t, copy=True)
    h = t.shape[-1] // 2
    while h >= 1:
        t[..., :h] = t[..., :h] + t[..., h:2 * h]
        h //= 2
    return t[..., 0]


def signs_from_bits(words: np.ndarray, d: int) -> np.ndarray:
    """Sign vector (+1/-1 float) from packed bits: bit j of word j//32 set = -1."""
    words = np.asarray(words, dtype=np.uint32)
    j = np.arange(d)
    bit = (words[..., j // 32] >> (j % 32).astype(np.uint32)) & 1
    return np.where(bit == 1, -1.0, 1.0)


# --------------------------------------------------------------------------
# encode / decode
# --------------------------------------------------------------------------
def tq_quantize(w: np.ndarray, n: np.ndarray, bits: int) -> np.ndarray:
    """code_j = #{k : w_j > fp32(n * t_k)} along the last axis of w (fp32)."""
    _, t32 = codebook(bits)
    w = np.asarray(w, dtype=np.float32)
    n = np.asarray(n, dtype=np.float32)
    T = (n[..., None] * t32).astype(np.float32)                    # [..., 2^b-1]
    return (w[..., :, None] > T[..., None, :]).sum(axis=-1).astype(np.uint8)


def tq_encode(x: np.ndarray, signs: np.ndarray, bits: int):
    """Encode vectors along the last axis. `signs` (+-1) broadcasts against x.
    Returns (codes uint8 [..., d], sigma float16 [...])."""
    x = np.asarray(x, dtype=np.float32)
    c16, _ = codebook(bits)
    c32 = c16.astype(np.float32)
    # 1. norm
    n2 = halving_tree_sum((x * x).astype(np.float32))
    n = np.sqrt(n2).astype(np.float32)
    # 2-3. rotate (sign flip, unnormalized FWHT)
    u = (x * np.asarray(signs, dtype=np.float32)).astype(np.float32)
    w = fwht(u)
    # 4. thresholds scaled by the norm; count the thresholds strictly below w
    codes = tq_quantize(w, n, bits)
    # 5. norm correction
    cn2 = halving_tree_sum((c32[codes] * c32[codes]).astype(np.float32))
    ratio = (n / np.sqrt(cn2).astype(np.float32)).astype(np.float32)
    # fp16 round-to-nearest-even; a ratio of 65520 or more rounds to +inf,
    # which is what an fp16 sigma is for such a vector (no clamping)
    with np.errstate(over="ignore"):
        sigma = ratio.astype(np.float16)
    zero = n2 == 0
    codes[zero] = 0
    sigma[zero] = 0
    return codes, sigma


def tq_decode(codes: np.ndarray, sigma: np.ndarray, signs: np.ndarray, bits: int) -> np.ndarray:
    """x_hat = sigma * s * FWHT(c[code]) / sqrt(d), in fp64."""
    c16, _ = codebook(bits)
    c = c16.astype(np.float64)[np.asarray(codes)]
    d = c.shape[-1]
    y = fwht(c) / math.sqrt(d)
    return np.asarray(sigma, dtype=np.float64)[..., None] * np.asarray(signs, dtype=np.float64) * y


def rotate(q: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R q = H (s * q) / sqrt(d) in fp64 (the codec-coordinate query)."""
    q = np.asarray(q, dtype=np.float64)
    return fwht(q * np.asarray(signs, dtype=np.float64)) / math.sqrt(q.shape[-1])
