"""Byte accounting of the formats (what a decode step must move).

Minima-KV Eq. 1: per live token the KV payload is m = 2 L_f H_kv d_h s bytes
(the 2 counts K and V); Eq. 2-3 evaluate it for 16 full-attention layers, 4
KV heads and d_h = 256. Eq. 10: b_eff = 8 (p_R + p_A) + b_S p_S + b_meta and
C_BF16 = 16 / b_eff. Eq. 14: C_mem(L) = floor((M - W) / (D + K(L))).
Block-GTQ appendix B.1 separates logical payload rate, total effective rate
and allocated physical footprint; appendix H.1 stores 1-4-bit codes in nibble
containers plus one fp16 norm per row, which gives its 132-byte figure.
"""
from __future__ import annotations

import math

import numpy as np

FMT_FP8, FMT_TQ3, FMT_TQ2, FMT_TQK, FMT_TQF5, FMT_TQF6 = 0, 1, 2, 3, 4, 5


def kv_bytes_per_token(L_f: int, H_kv: int, d_h: int, s: float) -> float:
    """Minima-KV Eq. 1."""
    return 2 * L_f * H_kv * d_h * s


def fp8_token_head_bytes(d: int) -> int:
    """K and V codes (d bytes each) plus one fp32 scale each."""
    return 2 * d + 8


def tq_token_head_bytes(d: int, bits: int) -> int:
    """K and V dense b-bit codes plus one fp16 sigma each."""
    return 2 * (bits * d // 8 + 2)


def tq_nibble_token_head_bytes(d: int) -> int:
    """Block-GTQ H.1 container accounting: codes of 1-4 bits in 4-bit nibbles."""
    return 2 * (d // 2 + 2)


def tqk_token_head_bytes(d: int, seg_dims=(32, 64, 32), seg_bits=(2, 3, 4), v_bits: int = 3) -> int:
    """Grouped mixed-rate keys: each segment's codes plus one fp16 sigma per
    segment; values uniform b-bit codes plus one fp16 sigma."""
    k = sum(n * b // 8 + 2 for n, b in zip(seg_dims, seg_bits))
    return k + v_bits * d // 8 + 2


def tqf_token_head_bytes(d: int, levels: int) -> int:
    """Fractional-level TQ (SemKV section 4.1 "Memory accounting"): K and V
    rows of ceil(d / k) mixed-radix groups of nbits bits (k codes per group),
    rounded up to whole bytes, plus one fp16 sigma each."""
    k, nbits = {5: (3, 7), 6: (5, 13)}[levels]
    return 2 * ((-(-d // k) * nbits + 7) // 8 + 2)


def token_head_bytes(fmt: int, d: int) -> int:
    if fmt == FMT_FP8:
        return fp8_token_head_bytes(d)
    if fmt == FMT_TQ3:
        return tq_token_head_bytes(d, 3)
    if fmt == FMT_TQ2:
        return tq_token_head_bytes(d, 2)
    if fmt == FMT_TQK:
        return tqk_token_head_bytes(d)
    if fmt == FMT_TQF5:
        return tqf_token_head_bytes(d, 5)
    if fmt == FMT_TQF6:
        return tqf_token_head_bytes(d, 6)
    raise ValueError(fmt)


def b_eff(p_R: float, p_A: float, p_S: float, b_S: float, b_meta: float = 0.0) -> float:
    """Minima-KV Eq. 10 (bits per scalar)."""
    return 8.0 * (p_R + p_A) + b_S * p_S + b_meta


def c_bf16(beff: float) -> float:
    return 16.0 / beff


def capacity(M: float, W: float, D: float, K: float) -> int:
    """Minima-KV Eq. 14."""
    return int(math.floor((M - W) / (D + K)))


def decode_kv_bytes(page_format: np.ndarray, seq_lens: np.ndarray, P: int, Hkv: int, d: int) -> int:
    """Bytes of every page a decode step scans (whole pages, all KV heads)."""
    total = 0
    for b in range(page_format.shape[0]):
        n_pages = (int(seq_lens[b]) + P - 1) // P
        for f in page_format[b, :n_pages]:
            total += P * Hkv * token_head_bytes(int(f), d)
    return total
