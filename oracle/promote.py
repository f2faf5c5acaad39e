"""Promotion of a compressed (TQ) page back into an FP8 page.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Minima-KV (arxiv 2608.23834), algorithm 1 step "Promote": a Stale page that
re-enters the protected budget is reconstructed into a newly allocated FP8
page, whose mapping is then published; section 3.1 "Anchor" and figure 2
("promotion reconstructs into FP8 before publication"). The pages give no
arithmetic for the reconstruction. Readings fixed here:

  * the reconstruction is the TQ decode x = sigma * s (.) FWHT(c[code]) /
    sqrt(d_s) (Block-GTQ appendix B.1: renormalized direction, stored norm
    restored), evaluated in IEEE fp32 in this order:
      1. c_j = centroid of code_j (fp16 values, exact in fp32);
      2. F = unnormalized FWHT(c). Every centroid is a multiple of 2^-13 below
         2^2 in magnitude, so every partial sum of at most 256 of them is a
         multiple of 2^-13 below 2^23: exact in fp32, in any order;
      3. u_j = fp32(F_j * r), r = the fp32 value nearest to 1/sqrt(d_s);
      4. x_j = fp32(sigma * u_j), then the sign flip s_j (exact);
  * grouped mixed-rate keys reconstruct segment by segment, each at its own
    width d_s with its own sigma and signs; the coordinate permutation is
    undone afterwards (exact);
  * the FP8 page is the FP8 codec (oracle.fp8: one amax scale per token,
    KV head and role) applied to those fp32 rows, so promoting a page is an
    Append of its reconstruction;
  * slots of the source page that hold no token have sigma 0; they rebuild
    to zero rows and become codes 0, scale 0 (the empty-slot rule of the
    encoders).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import fp8 as _fp8
from . import layout as _layout
from . import tq as _tq
from . import tqk as _tqk
from .attention import FMT_TQ2, FMT_TQ3, FMT_TQK, TQ_BITS

F32 = np.float32


def inv_sqrt_f32(d: int) -> np.float32:
    """fp32 value nearest to t = 1/sqrt(d), decided in exact rationals: find
    the fp32 pair lo <= t < hi (lo^2 <= 1/d < hi^2), then t lies below their
    midpoint m exactly when 1/d < m^2 (ties go to the even significand)."""
    target = Fraction(1, d)
    lo = F32(1.0 / np.sqrt(float(d)))
    while Fraction(float(lo)) ** 2 > target:
        lo = np.nextafter(lo, F32(0))
    while Fraction(float(np.nextafter(lo, F32(1)))) ** 2 <= target:
        lo = np.nextafter(lo, F32(1))
    hi = np.nextafter(lo, F32(1))
    if Fraction(float(lo)) ** 2 == target:
        return F32(lo)
    m2 = ((Fraction(float(lo)) + Fraction(float(hi))) / 2) ** 2
    if target < m2:
        return F32(lo)
    if target > m2:
        return F32(hi)
    return F32(lo) if (lo.view(np.uint32) & 1) == 0 else F32(hi)


def tq_reconstruct_f32(codes: np.ndarray, sigma: np.ndarray, signs: np.ndarray, bits: int) -> np.ndarray:
    """fp32 rows of TQ-coded vectors along the last axis (steps 1-4 above).
    codes uint8 [..., d_s], sigma float16 [...], signs +-1 [d_s]."""
    c16, _ = _tq.codebook(bits)
    c = c16.astype(F32)[np.asarray(codes)]
    F = _tq.fwht(c)                                   # fp32, exact
    r = inv_sqrt_f32(c.shape[-1])
    u = (F * r).astype(F32)
    x = (np.asarray(sigma).astype(F32)[..., None] * u).astype(F32)
    return (x * np.asarray(signs, dtype=F32)).astype(F32)


def tqf_reconstruct_f32(codes: np.ndarray, sigma: np.ndarray, signs: np.ndarray, levels: int) -> np.ndarray:
    """The same rebuild with an L-level codebook (fractional-level TQ): the
    FWHT of fp16 centroids is exact in fp32 here too (for L = 5, 6 every
    partial sum is a multiple of 2^-12 below 2^10)."""
    from . import tqf as _tqf
    c16, _ = _tqf.codebook_levels(levels)
    c = c16.astype(F32)[np.asarray(codes)]
    F = _tq.fwht(c)
    r = inv_sqrt_f32(c.shape[-1])
    u = (F * r).astype(F32)
    x = (np.asarray(sigma).astype(F32)[..., None] * u).astype(F32)
    return (x * np.asarray(signs, dtype=F32)).astype(F32)


def tqk_key_reconstruct_f32(seg_codes, perm: np.ndarray, segs, signs_perm: np.ndarray) -> np.ndarray:
    """fp32 key rows from grouped mixed-rate segments; permutation undone."""
    parts, j0 = [], 0
    for (bits, width), (codes, sigma) in zip(segs, seg_codes):
        parts.append(tq_reconstruct_f32(codes, sigma, signs_perm[j0:j0 + width], bits))
        j0 += width
    xp = np.concatenate(parts, axis=-1)
    x = np.zeros_like(xp)
    x[..., perm] = xp
    return x


def reconstruct_head_f32(fmt: int, blk: np.ndarray, P: int, d: int, sk: np.ndarray, sv: np.ndarray,
                         block_bits=None):
    """fp32 K, V [P, d] of one compressed (page, KV head) block."""
    if fmt in (FMT_TQ3, FMT_TQ2):
        b = TQ_BITS[fmt]
        kc, vc, ksig, vsig = _layout.tq_unpack_head(blk, P, d, b)
        return tq_reconstruct_f32(kc, ksig, sk, b), tq_reconstruct_f32(vc, vsig, sv, b)
    if fmt == FMT_TQK:
        perm, segs = _tqk.segments(block_bits)
        kc, ksig, vc, vsig = _layout.tqk_unpack_head(blk, P, d)
        seg_codes, j0 = [], 0
        for i, (_, width) in enumerate(segs):
            seg_codes.append((kc[:, j0:j0 + width], ksig[i]))
            j0 += width
        k = tqk_key_reconstruct_f32(seg_codes, perm, segs, sk)
        return k, tq_reconstruct_f32(vc, vsig, sv, _tqk.V_BITS)
    from .attention import TQF_LEVELS
    if fmt in TQF_LEVELS:
        L = TQF_LEVELS[fmt]
        kc, vc, ksig, vsig = _layout.tqf_unpack_head(blk, P, d, L)
        return tqf_reconstruct_f32(kc, ksig, sk, L), tqf_reconstruct_f32(vc, vsig, sv, L)
    raise ValueError(f"format {fmt} cannot be promoted")


def promote_page(fmt: int, page: np.ndarray, Hkv: int, P: int, d: int, signs_words, tqk=None) -> np.ndarray:
    """Bytes of the FP8 page (all KV heads) that promoting one compressed page
    of format `fmt` writes. signs_words uint32 [Hkv][2][d/32]; tqk = per-head
    block widths for grouped keys."""
    from .attention import head_block_bytes
    hb = head_block_bytes(fmt, P, d)
    out = []
    for g in range(Hkv):
        blk = np.asarray(page[g * hb:(g + 1) * hb], dtype=np.uint8)
        sk = _tq.signs_from_bits(signs_words[g, 0], d)
        sv = _tq.signs_from_bits(signs_words[g, 1], d)
        k, v = reconstruct_head_f32(fmt, blk, P, d, sk, sv, None if tqk is None else tqk[g])
        kc, ks = _fp8.fp8_encode(k)
        vc, vs = _fp8.fp8_encode(v)
        out.append(_layout.fp8_pack_head(kc, vc, ks, vs))
    return np.concatenate(out)
