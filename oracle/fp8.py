"""FP8 E4M3 codec of Recent and Anchor pages.

Minima-KV (arxiv 2608.23834), section 3.1 "Recent (R, FP8)" and "Anchor (A,
FP8)", and section 4.1: new KV is appended in FP8; each page keeps its scales
next to the codes. The pages do not fix the FP8 variant or the scale rule;
this oracle reads them as the OCP 8-bit floating point E4M3 format (bias 7,
no infinities, 0x7F/0xFF = NaN, largest finite 448) with one fp32 scale per
(token, KV head, role) vector, scale = amax / 448.

Encode of one vector x (fp32, length d), every operation fp32 RNE:
    amax = max_j |x_j|
    amax == 0  ->  all codes 0x00, scale 0
    inv  = 448 / amax
    y_j  = x_j * inv
    e_j  = nearest finite E4M3 value to y_j, ties to the even code,
           magnitudes >= 448 saturate to 448, sign kept (also for a zero)
    scale = amax / 448
Decode: x_hat_j = value(e_j) * scale (exact in fp64).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code from its fields (OCP FP8 spec, E4M3 column)."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** (1 - 7)        # subnormal
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)  # normal
    return sign * mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite magnitudes, codes 0x00..0x7E in ascending order
_MAGS = E4M3_TABLE[:0x7F]


def e4m3_encode_rne(y: np.ndarray) -> np.ndarray:
    """Round fp32 values to E4M3 codes: nearest, ties to even, saturating."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    idx = np.searchsorted(_MAGS, a, side="left")
    idx = np.clip(idx, 1, 0x7E)
    lo = idx - 1
    hi = idx
    dlo = a - _MAGS[lo]
    dhi = _MAGS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def fp8_encode(x: np.ndarray):
    """Encode vectors along the last axis. Returns (codes uint8, scale float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)
    codes = np.where(zero[..., None], np.uint8(0), e4m3_encode_rne(y)).astype(np.uint8)
    scale = np.where(zero, np.float32(0), (amax / np.float32(E4M3_MAX)).astype(np.float32)).astype(np.float32)
    return codes, scale


def fp8_decode(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x_hat = value(code) * scale, in fp64 (exact)."""
    return E4M3_TABLE[np.asarray(codes)] * np.asarray(scale, dtype=np.float64)[..., None]


def fp8_decode_f32(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp32(value(code) * scale): the fp32 rows an FP8 page is demoted from."""
    v = E4M3_TABLE[np.asarray(codes)].astype(np.float32)
    return (v * np.asarray(scale, dtype=np.float32)[..., None]).astype(np.float32)
