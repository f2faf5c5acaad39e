"""Byte layout of one page of each physical format.

The pages fix what a page holds but not where each bit goes: Minima-KV
section 4.1 lists, per Stale page and KV head, 3-bit K codes, an fp16 K norm
correction, 3-bit V codes and fp16 V metadata, with FP8 pages holding codes
plus scales (section 3.1). This module is the oracle's own statement of the
one dense layout this build uses; it is written from the layout rules below,
not from the HIP sources.

A pool is [num_pages][page bytes]; a page is [Hkv][head block]. With P the
page size (a multiple of 16) and d the head dim, a head block is

  FP8:  K tiles | V tiles | K scales fp32[P] | V scales fp32[P]     2Pd + 8P B
  TQb:  K tiles | V tiles | K sigma fp16[P]  | V sigma fp16[P]   2Pdb/8 + 4P B
  TQK:  K tiles | V tiles | K sigma fp16[3][P] | V sigma fp16[P] P(3d/4 + 8) B
        (grouped mixed-rate keys; the rule is stated with the TQK section below)
  TQF:  K rows  | V rows  | K sigma fp16[P]  | V sigma fp16[P]   2P R + 4P B
        (fractional-level codes: row t is the token's mixed-radix bitstream of
        R = row_bytes(d, L) bytes, oracle.tqf.pack_row; rows in slot order)

Tiles cover 16 tokens (slots 16*tau .. 16*tau+15 of the page) and one role.
Inside a tile the 16*d elements are dealt to 64 "lanes", D_L = d/4 each:
  K: lane l, element i  <->  token  l % 16,                 dim (l // 16) * D_L + i
  V: lane l, element i  <->  token  4 * (l // 16) + i % 4,  dim  l % 16 + 16 * (i // 4)
FP8 element (l, i) is the byte at ((i // 16) * 64 + l) * 16 + i % 16.
TQb: lane l's D_L codes occupy W = D_L * b / 32 little-endian 32-bit words.
Word w of lane l sits in a 16-, 8- or 4-byte region (regions greedily take 4,
then 2, then 1 of the remaining words; region r of width k words starts after
the earlier regions, and lane l's slice of it is at l * 4k).
Codes are taken in groups of four: group g = elements 4g .. 4g+3, and slot
s = i % 4 always lives in byte s of a word.
  b = 2: group g -> word g // 4, bits 2*(g % 4) .. +1 of byte s
  b = 4: group g -> word g // 2, bits 4*(g % 2) .. +3 of byte s
  b = 3: words go in triples; triple m holds groups 8m .. 8m+7, q = g - 8m:
         q = 0, 1 -> word 3m,   bits 0-2 / 3-5 of byte s
         q = 2, 3 -> word 3m+1, bits 0-2 / 3-5
         q = 4, 5 -> word 3m+2, bits 0-2 / 3-5
         q = 6    -> code bits 0-1 in word 3m bits 6-7, code bit 2 in word 3m+2 bit 6
         q = 7    -> code bits 0-1 in word 3m+1 bits 6-7, code bit 2 in word 3m+2 bit 7
"""
from __future__ import annotations

import numpy as np

TILE = 16


def fp8_head_bytes(P: int, d: int) -> int:
    return 2 * P * d + 8 * P


def tq_head_bytes(P: int, d: int, bits: int) -> int:
    return 2 * P * d * bits // 8 + 4 * P


def lane_element_token_dim(role: int, d: int):
    """(token [64, D_L], dim [64, D_L]) of every (lane, element) of a tile."""
    DL = d // 4
    l = np.arange(64)[:, None]
    i = np.arange(DL)[None, :]
    if role == 0:
        tok = np.broadcast_to(l % 16, (64, DL))
        dim = (l // 16) * DL + i
    else:
        tok = 4 * (l // 16) + i % 4
        dim = l % 16 + 16 * (i // 4)
    return np.array(tok), np.array(dim)


def word_regions(W: int):
    """[(first word, width in words)] in storage order."""
    regs, w = [], 0
    for width in (4, 2, 1):
        while W - w >= width:
            regs.append((w, width))
            w += width
    return regs


def word_byte_offset(l: int, w: int, W: int) -> int:
    """Byte offset inside a TQ tile of word w of lane l."""
    base = 0
    for first, width in word_regions(W):
        if first <= w < first + width:
            return base + l * 4 * width + 4 * (w - first)
        base += 64 * 4 * width
    raise ValueError("word out of range")


def code_bit_positions(i: int, bits: int):
    """[(word, bit in word, code bit)] for element i of a lane."""
    g, s = i // 4, i % 4
    if bits == 2:
        return [(g // 4, 8 * s + 2 * (g % 4) + k, k) for k in range(2)]
    if bits == 4:
        return [(g // 2, 8 * s + 4 * (g % 2) + k, k) for k in range(4)]
    if bits == 3:
        m, q = g // 8, g % 8
        if q < 6:
            word = 3 * m + q // 2
            lo = 3 * (q % 2)
            return [(word, 8 * s + lo + k, k) for k in range(3)]
        word = 3 * m + (q - 6)
        hibit = 6 + (q - 6)
        return [(word, 8 * s + 6, 0), (word, 8 * s + 7, 1), (3 * m + 2, 8 * s + hibit, 2)]
    raise ValueError(bits)


# --------------------------------------------------------------------------
# index maps (vectorized packing uses these; the loop versions below state the
# same rules element by element and pin the maps in the tests)
# --------------------------------------------------------------------------
_MAPS = {}


def _fp8_map(role: int, d: int):
    """Flat (token*d + dim) source of every byte of an FP8 tile."""
    key = ("fp8", role, d)
    if key not in _MAPS:
        tok, dim = lane_element_token_dim(role, d)
        DL = d // 4
        src = np.zeros(16 * d, dtype=np.int64)
        l = np.arange(64)[:, None]
        i = np.arange(DL)[None, :]
        off = ((i // 16) * 64 + l) * 16 + i % 16
        src[off.ravel()] = (tok * d + dim).ravel()
        _MAPS[key] = src
    return _MAPS[key]


def _tq_map(role: int, d: int, bits: int):
    """For every (tile byte, bit in byte): (flat element source, code bit)."""
    key = ("tq", role, d, bits)
    if key not in _MAPS:
        tok, dim = lane_element_token_dim(role, d)
        DL = d // 4
        W = DL * bits // 32
        nbytes = 16 * d * bits // 8
        src = np.full((nbytes, 8), -1, dtype=np.int64)
        cbit = np.zeros((nbytes, 8), dtype=np.int64)
        for i in range(DL):
            for (w, pos, cb) in code_bit_positions(i, bits):
                for l in range(64):
                    byte = word_byte_offset(l, w, W) + pos // 8
                    src[byte, pos % 8] = tok[l, i] * d + dim[l, i]
                    cbit[byte, pos % 8] = cb
        assert (src >= 0).all()
        _MAPS[key] = (src, cbit)
    return _MAPS[key]


# --------------------------------------------------------------------------
# FP8
# --------------------------------------------------------------------------
def fp8_pack_tiles(codes: np.ndarray, role: int) -> np.ndarray:
    """codes uint8 [n, 16, d] -> tile bytes [n, 16*d]."""
    n, _, d = codes.shape
    return codes.reshape(n, 16 * d)[:, _fp8_map(role, d)]


def fp8_unpack_tiles(tiles: np.ndarray, role: int, d: int) -> np.ndarray:
    n = tiles.shape[0]
    out = np.zeros((n, 16 * d), dtype=np.uint8)
    out[:, _fp8_map(role, d)] = tiles
    return out.reshape(n, 16, d)


def fp8_pack_head(kc, vc, ks, vs) -> np.ndarray:
    """kc, vc uint8 [P, d]; ks, vs float32 [P] -> head block bytes."""
    P, d = kc.shape
    parts = [fp8_pack_tiles(kc.reshape(P // TILE, TILE, d), 0).ravel(),
             fp8_pack_tiles(vc.reshape(P // TILE, TILE, d), 1).ravel(),
             np.asarray(ks, dtype="<f4").view(np.uint8),
             np.asarray(vs, dtype="<f4").view(np.uint8)]
    out = np.concatenate(parts)
    assert out.size == fp8_head_bytes(P, d)
    return out


def fp8_unpack_head(blk: np.ndarray, P: int, d: int):
    blk = np.asarray(blk, dtype=np.uint8)
    nt = P // TILE
    kc = fp8_unpack_tiles(blk[:P * d].reshape(nt, 16 * d), 0, d).reshape(P, d)
    vc = fp8_unpack_tiles(blk[P * d:2 * P * d].reshape(nt, 16 * d), 1, d).reshape(P, d)
    off = 2 * P * d
    ks = blk[off:off + 4 * P].copy().view("<f4")
    vs = blk[off + 4 * P:off + 8 * P].copy().view("<f4")
    return kc, vc, ks, vs


def fp8_tile_pack_loop(codes16: np.ndarray, role: int, d: int) -> np.ndarray:
    """Element-by-element statement of the FP8 tile rule (small inputs only)."""
    tok, dim = lane_element_token_dim(role, d)
    out = np.zeros(16 * d, dtype=np.uint8)
    for l in range(64):
        for i in range(d // 4):
            out[((i // 16) * 64 + l) * 16 + i % 16] = codes16[tok[l, i], dim[l, i]]
    return out


# --------------------------------------------------------------------------
# TQb
# --------------------------------------------------------------------------
def tq_pack_tiles(codes: np.ndarray, role: int, bits: int) -> np.ndarray:
    """codes uint8 [n, 16, d] (values < 2^bits) -> tile bytes [n, 16*d*bits/8]."""
    n, _, d = codes.shape
    src, cbit = _tq_map(role, d, bits)
    flat = codes.reshape(n, 16 * d).astype(np.uint16)
    b = (flat[:, src] >> cbit.astype(np.uint16)) & 1            # [n, nbytes, 8]
    weights = (1 << np.arange(8)).astype(np.uint16)
    return (b * weights).sum(axis=-1).astype(np.uint8)


def tq_unpack_tiles(tiles: np.ndarray, role: int, d: int, bits: int) -> np.ndarray:
    n = tiles.shape[0]
    src, cbit = _tq_map(role, d, bits)
    bitv = (tiles[:, :, None].astype(np.uint16) >> np.arange(8, dtype=np.uint16)) & 1
    out = np.zeros((n, 16 * d), dtype=np.uint16)
    contrib = bitv << cbit.astype(np.uint16)
    np.add.at(out, (np.arange(n)[:, None], src.reshape(1, -1).repeat(n, 0)), contrib.reshape(n, -1))
    return out.astype(np.uint8).reshape(n, 16, d)


def tq_pack_head(kc, vc, ksig, vsig, bits: int) -> np.ndarray:
    """kc, vc uint8 codes [P, d]; ksig, vsig float16 [P] -> head block bytes."""
    P, d = kc.shape
    parts = [tq_pack_tiles(kc.reshape(P // TILE, TILE, d), 0, bits).ravel(),
             tq_pack_tiles(vc.reshape(P // TILE, TILE, d), 1, bits).ravel(),
             np.asarray(ksig, dtype="<f2").view(np.uint8),
             np.asarray(vsig, dtype="<f2").view(np.uint8)]
    out = np.concatenate(parts)
    assert out.size == tq_head_bytes(P, d, bits)
    return out


def tq_unpack_head(blk: np.ndarray, P: int, d: int, bits: int):
    blk = np.asarray(blk, dtype=np.uint8)
    nt = P // TILE
    T = 16 * d * bits // 8
    kc = tq_unpack_tiles(blk[:nt * T].reshape(nt, T), 0, d, bits).reshape(P, d)
    vc = tq_unpack_tiles(blk[nt * T:2 * nt * T].reshape(nt, T), 1, d, bits).reshape(P, d)
    off = 2 * nt * T
    ksig = blk[off:off + 2 * P].copy().view("<f2")
    vsig = blk[off + 2 * P:off + 4 * P].copy().view("<f2")
    return kc, vc, ksig, vsig


def tq_tile_pack_loop(codes16: np.ndarray, role: int, d: int, bits: int) -> np.ndarray:
    """Element-by-element statement of the TQ tile rule (small inputs only)."""
    tok, dim = lane_element_token_dim(role, d)
    DL = d // 4
    W = DL * bits // 32
    out = np.zeros(16 * d * bits // 8, dtype=np.uint8)
    for l in range(64):
        words = [0] * W
        for i in range(DL):
            c = int(codes16[tok[l, i], dim[l, i]])
            for (w, pos, cb) in code_bit_positions(i, bits):
                if (c >> cb) & 1:
                    words[w] |= 1 << pos
        for w in range(W):
            off = word_byte_offset(l, w, W)
            out[off:off + 4] = np.frombuffer(int(words[w]).to_bytes(4, "little"), dtype=np.uint8)
    return out


# --------------------------------------------------------------------------
# TQK: grouped mixed-rate keys, uniform TQ3 values
# --------------------------------------------------------------------------
# Head block: K tiles | V tiles | K sigma fp16[3][P] (segment-major) |
# V sigma fp16[P]; P (3d/4 + 8) bytes. The key row is in permuted order with
# segments [0, d/4) at 2 bits, [d/4, 3d/4) at 3 bits, [3d/4, d) at 4 bits.
# V tiles follow the TQ3 rule above. A K tile deals 16 tokens to 64 lanes in
# 32-coordinate chunks, so that one chunk never straddles two segments:
#   K: lane l, element i  <->  token l % 16,  dim 32 * (i // 8) + 8 * (l // 16) + i % 8
# Groups g = i // 4 of a lane: the first d/64 are 2-bit, the next d/32 3-bit,
# the last d/64 4-bit (n2 = d/64, n3 = d/32). The lane's W = 3d/128 words go in
# triples; triple m holds, at byte s = i % 4 of each word:
#   word 3m:     4-bit group n2 + n3 + 2m at bits 0-3, group n2 + n3 + 2m + 1 at bits 4-7
#   word 3m + 1: 3-bit group n2 + 4m at bits 0-2, group n2 + 4m + 1 at bits 3-5,
#                2-bit group 2m at bits 6-7
#   word 3m + 2: 3-bit group n2 + 4m + 2 at bits 0-2, group n2 + 4m + 3 at bits 3-5,
#                2-bit group 2m + 1 at bits 6-7
# Words sit in per-lane regions exactly as for TQ3 (word_byte_offset).
def tqk_head_bytes(P: int, d: int) -> int:
    return P * (2 * (3 * d // 8) + 8)


def tqk_key_lane_map(d: int):
    """(token [64, d/4], permuted dim [64, d/4]) of every (lane, element) of a K tile."""
    DL = d // 4
    l = np.arange(64)[:, None]
    i = np.arange(DL)[None, :]
    tok = np.broadcast_to(l % 16, (64, DL))
    dim = 32 * (i // 8) + 8 * (l // 16) + i % 8
    return np.array(tok), np.array(dim)


def tqk_element_bits(i: int, d: int) -> int:
    g = i // 4
    n2, n3 = d // 64, d // 32
    return 2 if g < n2 else (3 if g < n2 + n3 else 4)


def tqk_code_bit_positions(i: int, d: int):
    """[(word, bit in word, code bit)] for element i of a lane of a TQK K tile."""
    g, s = i // 4, i % 4
    n2, n3 = d // 64, d // 32
    if g < n2:
        m, k = g // 2, g % 2
        return [(3 * m + 1 + k, 8 * s + 6 + b, b) for b in range(2)]
    if g < n2 + n3:
        m, q = (g - n2) // 4, (g - n2) % 4
        return [(3 * m + 1 + q // 2, 8 * s + 3 * (q % 2) + b, b) for b in range(3)]
    m, k = (g - n2 - n3) // 2, (g - n2 - n3) % 2
    return [(3 * m, 8 * s + 4 * k + b, b) for b in range(4)]


def _tqk_key_map(d: int):
    key = ("tqk", d)
    if key not in _MAPS:
        tok, dim = tqk_key_lane_map(d)
        DL = d // 4
        W = 3 * d // 128
        nbytes = 16 * d * 3 // 8
        src = np.full((nbytes, 8), -1, dtype=np.int64)
        cbit = np.zeros((nbytes, 8), dtype=np.int64)
        for i in range(DL):
            for (w, pos, cb) in tqk_code_bit_positions(i, d):
                for l in range(64):
                    byte = word_byte_offset(l, w, W) + pos // 8
                    src[byte, pos % 8] = tok[l, i] * d + dim[l, i]
                    cbit[byte, pos % 8] = cb
        assert (src >= 0).all()
        _MAPS[key] = (src, cbit)
    return _MAPS[key]


def tqk_pack_key_tiles(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [n, 16, d] (permuted order, each below 2^(its bits)) -> bytes [n, 6d]."""
    n, _, d = codes.shape
    src, cbit = _tqk_key_map(d)
    flat = codes.reshape(n, 16 * d).astype(np.uint16)
    b = (flat[:, src] >> cbit.astype(np.uint16)) & 1
    weights = (1 << np.arange(8)).astype(np.uint16)
    return (b * weights).sum(axis=-1).astype(np.uint8)


def tqk_unpack_key_tiles(tiles: np.ndarray, d: int) -> np.ndarray:
    n = tiles.shape[0]
    src, cbit = _tqk_key_map(d)
    bitv = (tiles[:, :, None].astype(np.uint16) >> np.arange(8, dtype=np.uint16)) & 1
    out = np.zeros((n, 16 * d), dtype=np.uint16)
    contrib = bitv << cbit.astype(np.uint16)
    np.add.at(out, (np.arange(n)[:, None], src.reshape(1, -1).repeat(n, 0)), contrib.reshape(n, -1))
    return out.astype(np.uint8).reshape(n, 16, d)


def tqk_key_tile_pack_loop(codes16: np.ndarray, d: int) -> np.ndarray:
    """Element-by-element statement of the TQK K tile rule (small inputs only)."""
    tok, dim = tqk_key_lane_map(d)
    W = 3 * d // 128
    out = np.zeros(16 * d * 3 // 8, dtype=np.uint8)
    for l in range(64):
        words = [0] * W
        for i in range(d // 4):
            c = int(codes16[tok[l, i], dim[l, i]])
            for (w, pos, cb) in tqk_code_bit_positions(i, d):
                if (c >> cb) & 1:
                    words[w] |= 1 << pos
        for w in range(W):
            off = word_byte_offset(l, w, W)
            out[off:off + 4] = np.frombuffer(int(words[w]).to_bytes(4, "little"), dtype=np.uint8)
    return out


def tqk_pack_head(kc, ksig, vc, vsig) -> np.ndarray:
    """kc uint8 [P, d] key codes in permuted order; ksig float16 [3, P];
    vc uint8 [P, d] TQ3 value codes; vsig float16 [P] -> head block bytes."""
    P, d = kc.shape
    parts = [tqk_pack_key_tiles(kc.reshape(P // TILE, TILE, d)).ravel(),
             tq_pack_tiles(vc.reshape(P // TILE, TILE, d), 1, 3).ravel(),
             np.ascontiguousarray(ksig, dtype="<f2").view(np.uint8).ravel(),
             np.asarray(vsig, dtype="<f2").view(np.uint8)]
    out = np.concatenate(parts)
    assert out.size == tqk_head_bytes(P, d)
    return out


def tqk_unpack_head(blk: np.ndarray, P: int, d: int):
    blk = np.asarray(blk, dtype=np.uint8)
    nt = P // TILE
    T = 16 * d * 3 // 8
    kc = tqk_unpack_key_tiles(blk[:nt * T].reshape(nt, T), d).reshape(P, d)
    vc = tq_unpack_tiles(blk[nt * T:2 * nt * T].reshape(nt, T), 1, d, 3).reshape(P, d)
    off = 2 * nt * T
    ksig = blk[off:off + 6 * P].copy().view("<f2").reshape(3, P)
    vsig = blk[off + 6 * P:off + 8 * P].copy().view("<f2")
    return kc, ksig, vc, vsig


# --------------------------------------------------------------------------
# fractional-level TQ (TQF5 / TQF6): one mixed-radix bitstream per token row
# --------------------------------------------------------------------------
def tqf_head_bytes(P: int, d: int, levels: int) -> int:
    from . import tqf as _tqf
    return 2 * P * _tqf.row_bytes(d, levels) + 4 * P


def tqf_pack_head(kc, vc, ksig, vsig, levels: int) -> np.ndarray:
    """kc, vc uint8 codes [P, d] in [0, L); ksig, vsig float16 [P] -> head
    block bytes: the P key rows, the P value rows, then the two sigma arrays."""
    from . import tqf as _tqf
    rows = [_tqf.pack_row(r, levels) for r in np.asarray(kc)] + [_tqf.pack_row(r, levels) for r in np.asarray(vc)]
    return np.concatenate(rows + [np.asarray(ksig, np.float16).view(np.uint8),
                                  np.asarray(vsig, np.float16).view(np.uint8)])


def tqf_unpack_head(blk: np.ndarray, P: int, d: int, levels: int):
    """Inverse of tqf_pack_head: (kc, vc, ksig, vsig)."""
    from . import tqf as _tqf
    blk = np.asarray(blk, dtype=np.uint8)
    R = _tqf.row_bytes(d, levels)
    kc = np.stack([_tqf.unpack_row(blk[t * R:(t + 1) * R], d, levels) for t in range(P)])
    vc = np.stack([_tqf.unpack_row(blk[(P + t) * R:(P + t + 1) * R], d, levels) for t in range(P)])
    o = 2 * P * R
    ksig = blk[o:o + 2 * P].view(np.float16)
    vsig = blk[o + 2 * P:o + 4 * P].view(np.float16)
    return kc, vc, ksig, vsig
