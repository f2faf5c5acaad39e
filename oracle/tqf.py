"""Fractional-level TQ codes: non-power-of-two level counts, mixed-radix packed.

TEST INFRASTRUCTURE ONLY (see the package docstring).

SemKV, section 4.1 ("Quantization", "Memory accounting") and section 4.9:
fractional bit widths are non-power-of-two level counts (log2 5 = 2.322,
log2 6 = 2.585 bits); the TurboQuant-MSE reimplementation takes a random
rotation and a Gaussian-optimal Lloyd-Max codebook extended to those level
counts; non-power-of-two codes are stored by mixed-radix packing, three
five-level codes in 7 bits and five six-level codes in 13 bits.

Readings fixed here (the page gives no arithmetic beyond that):
  * the codec is the TQ codec of oracle.tq with an L-level codebook: the
    Gaussian Lloyd-Max centroids for L levels rounded to fp16, thresholds at
    the fp32 midpoints, code = number of thresholds strictly below the
    rotated coordinate (ties to the lower code), one fp16 norm correction;
  * a group of k codes (c_0 .. c_{k-1}) is the integer sum_i c_i L^i (the
    first code is the least significant digit), written in nbits bits; a row
    of d codes is ceil(d / k) groups (the last padded with code 0) in one
    little-endian bitstream, ceil(groups * nbits / 8) bytes.
"""
from __future__ import annotations

import math

import numpy as np

from . import tq as _tq

# level count -> (codes per group, bits per group)
GROUPS = {5: (3, 7), 6: (5, 13)}

_CACHE = {}


def codebook_levels(levels: int):
    """(centroids fp16 [L] ascending, thresholds fp32 [L - 1])."""
    if levels not in _CACHE:
        c64, _ = _tq.lloyd_max_gaussian(levels)
        c16 = c64.astype(np.float16)
        c32 = c16.astype(np.float32)
        t32 = ((c32[:-1] + c32[1:]) / np.float32(2)).astype(np.float32)
        _CACHE[levels] = (c16, t32)
    return _CACHE[levels]


def encode(x: np.ndarray, signs: np.ndarray, levels: int):
    """TQ encode along the last axis with an L-level codebook: (codes uint8
    [..., d] in [0, L), sigma float16 [...]). Same steps and fp32 arithmetic
    as oracle.tq.tq_encode."""
    x = np.asarray(x, dtype=np.float32)
    c16, t32 = codebook_levels(levels)
    c32 = c16.astype(np.float32)
    n2 = _tq.halving_tree_sum((x * x).astype(np.float32))
    n = np.sqrt(n2).astype(np.float32)
    w = _tq.fwht((x * np.asarray(signs, dtype=np.float32)).astype(np.float32))
    T = (n[..., None] * t32).astype(np.float32)
    codes = (w[..., :, None] > T[..., None, :]).sum(axis=-1).astype(np.uint8)
    cn2 = _tq.halving_tree_sum((c32[codes] * c32[codes]).astype(np.float32))
    with np.errstate(over="ignore"):        # a ratio >= 65520 rounds to +inf in fp16
        sigma = (n / np.sqrt(cn2).astype(np.float32)).astype(np.float32).astype(np.float16)
    zero = n2 == 0
    codes[zero] = 0
    sigma[zero] = 0
    return codes, sigma


def decode(codes: np.ndarray, sigma: np.ndarray, signs: np.ndarray, levels: int) -> np.ndarray:
    """x_hat = sigma * s * FWHT(c[code]) / sqrt(d), fp64."""
    c16, _ = codebook_levels(levels)
    c = c16.astype(np.float64)[np.asarray(codes)]
    return (np.asarray(sigma, dtype=np.float64)[..., None] * np.asarray(signs, dtype=np.float64)
            * _tq.fwht(c) / math.sqrt(c.shape[-1]))


def row_bytes(d: int, levels: int) -> int:
    k, nbits = GROUPS[levels]
    return (-(-d // k) * nbits + 7) // 8


def pack_row(codes: np.ndarray, levels: int) -> np.ndarray:
    """Mixed-radix bitstream of one row of codes (uint8 [d]) -> uint8 bytes."""
    k, nbits = GROUPS[levels]
    codes = [int(c) for c in np.asarray(codes).ravel()]
    if any(c < 0 or c >= levels for c in codes):
        raise ValueError("code out of range")
    n_groups = -(-len(codes) // k)
    codes += [0] * (n_groups * k - len(codes))
    acc = 0
    for g in range(n_groups):
        v = sum(codes[g * k + i] * levels ** i for i in range(k))
        acc |= v << (g * nbits)
    nbytes = (n_groups * nbits + 7) // 8
    return np.frombuffer(acc.to_bytes(nbytes, "little"), dtype=np.uint8).copy()


def unpack_row(data: np.ndarray, d: int, levels: int) -> np.ndarray:
    """Inverse of pack_row: uint8 bytes -> codes uint8 [d]."""
    k, nbits = GROUPS[levels]
    acc = int.from_bytes(bytes(np.asarray(data, dtype=np.uint8)), "little")
    out = []
    n_groups = -(-d // k)
    for g in range(n_groups):
        v = (acc >> (g * nbits)) & ((1 << nbits) - 1)
        for _ in range(k):
            out.append(v % levels)
            v //= levels
    return np.array(out[:d], dtype=np.uint8)


def bits_per_value(levels: int) -> float:
    k, nbits = GROUPS[levels]
    return nbits / k
