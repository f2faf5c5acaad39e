"""Grouped mixed-rate keys (TQK): equal-rate groups of RoPE blocks.

Block-GTQ, appendix A.7 ("Equal-rate grouping"): a key's RoPE blocks
(x_{2i}, x_{2i+1}) that are assigned the same width b form one group, and every
nonempty group is encoded by one TQ-MSE encoder at b bits. Appendix B.1: each
group has its own rotation, drawn once from a fixed seed; Lloyd-Max centroids
under the Gaussian model; the decoded direction is renormalized and the stored
norm restored. Appendix H.1: blocks with the same rate are permuted into one
contiguous segment of the key's code row, with one fp16 norm per nonempty
segment, next to a uniform-rate value row with one fp16 value norm. Appendix
H.2: the query is permuted and rotated group by group into the codec
coordinates, so q . k_hat needs no inverse rotation of the key.

Readings this oracle fixes (the pages leave them open):
  * segments are ordered by ascending rate; inside a segment the blocks keep
    ascending block index, each block contributing coordinates 2i, 2i + 1;
  * a segment of width d_s is the TQ codec of oracle.tq at length d_s
    (norm, sign flips, unnormalized FWHT, threshold count, sigma) with the
    sign bits at the segment's positions of the key sign vector, i.e. the
    key signs are indexed in permuted order;
  * values are uniform TQ3 over the whole head (oracle.tq);
  * the workloads allocate d/8, d/4 and d/8 blocks at 2, 3 and 4 bits (mean
    3 bits per coordinate), so the segments are d/4, d/2 and d/4 wide.

Decode of a key: the segment's x_hat_s = sigma_s * s_s * FWHT(c[code_s]) /
sqrt(d_s), in fp64, then the permutation is undone.
"""
from __future__ import annotations

import numpy as np

from . import layout as _layout
from . import tq as _tq

KEY_RATES = (2, 3, 4)     # allowed block widths, in segment order
V_BITS = 3


def segments(block_bits) -> tuple:
    """(perm [d], [(bits, width)]) for one (layer, KV head).

    perm[j] is the original coordinate at permuted position j: blocks sorted
    by rate (ascending), ties kept in block order. Empty segments are dropped."""
    block_bits = [int(b) for b in np.asarray(block_bits).ravel()]
    perm, segs = [], []
    for b in KEY_RATES:
        blocks = [i for i, bb in enumerate(block_bits) if bb == b]
        if blocks:
            segs.append((b, 2 * len(blocks)))
            for i in blocks:
                perm += [2 * i, 2 * i + 1]
    if len(perm) != 2 * len(block_bits):
        raise ValueError("block widths must be 2, 3 or 4 bits")
    return np.array(perm, dtype=np.int64), segs


def encode_key(x: np.ndarray, perm: np.ndarray, segs, signs_perm: np.ndarray):
    """x float32 [..., d]; signs_perm (+-1) [d] in permuted order.
    Returns [(codes uint8 [..., d_s], sigma float16 [...])] per segment."""
    xp = np.asarray(x, dtype=np.float32)[..., perm]
    out, j0 = [], 0
    for bits, width in segs:
        out.append(_tq.tq_encode(xp[..., j0:j0 + width], signs_perm[j0:j0 + width], bits))
        j0 += width
    return out


def decode_key(seg_codes, perm: np.ndarray, segs, signs_perm: np.ndarray) -> np.ndarray:
    """Inverse of encode_key up to codec error: x_hat [..., d] in fp64."""
    parts, j0 = [], 0
    for (bits, width), (codes, sigma) in zip(segs, seg_codes):
        parts.append(_tq.tq_decode(codes, sigma, signs_perm[j0:j0 + width], bits))
        j0 += width
    xp = np.concatenate(parts, axis=-1)
    x = np.zeros_like(xp)
    x[..., perm] = xp
    return x


def codes_in_row(seg_codes) -> np.ndarray:
    """Segment codes concatenated in permuted order, uint8 [..., d]."""
    return np.concatenate([c for c, _ in seg_codes], axis=-1)


def head_bytes(P: int, d: int) -> int:
    return _layout.tqk_head_bytes(P, d)


def _check_layout_segments(segs, d):
    if [(b, w) for b, w in segs] != [(2, d // 4), (3, d // 2), (4, d // 4)]:
        raise ValueError(f"the page layout holds segments of d/4, d/2, d/4 at 2, 3, 4 bits, got {segs}")


def encode_page_head(k: np.ndarray, v: np.ndarray, sk: np.ndarray, sv: np.ndarray, block_bits) -> np.ndarray:
    """k, v float32 [P, d] of one KV head; sk (+-1, permuted order), sv (+-1)
    [d]; block_bits [d/2] -> the head block's bytes."""
    P, d = k.shape
    perm, segs = segments(block_bits)
    _check_layout_segments(segs, d)
    ks = encode_key(k, perm, segs, sk)
    vc, vsig = _tq.tq_encode(v, sv, V_BITS)
    return _layout.tqk_pack_head(codes_in_row(ks), np.stack([s for _, s in ks], axis=0), vc, vsig)


def dequant_page_head(blk: np.ndarray, P: int, d: int, sk: np.ndarray, sv: np.ndarray, block_bits):
    """Dequantized K, V [P, d] (fp64) of one TQK head block."""
    perm, segs = segments(block_bits)
    _check_layout_segments(segs, d)
    kc, ksig, vc, vsig = _layout.tqk_unpack_head(blk, P, d)
    seg_codes, j0 = [], 0
    for i, (bits, width) in enumerate(segs):
        seg_codes.append((kc[:, j0:j0 + width], ksig[i]))
        j0 += width
    return decode_key(seg_codes, perm, segs, sk), _tq.tq_decode(vc, vsig, sv, V_BITS)


def rotate_query(q: np.ndarray, perm: np.ndarray, segs, signs_perm: np.ndarray) -> np.ndarray:
    """Codec-coordinate query (Block-GTQ H.2): permute, then R_s per segment
    (R_s q_s = H (s_s * q_s) / sqrt(d_s)), fp64."""
    qp = np.asarray(q, dtype=np.float64)[..., perm]
    out, j0 = [], 0
    for _, width in segs:
        out.append(_tq.rotate(qp[..., j0:j0 + width], signs_perm[j0:j0 + width]))
        j0 += width
    return np.concatenate(out, axis=-1)
