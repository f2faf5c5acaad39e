"""Pins of the page byte layout: sizes against the per-token byte formulas,
bijectivity, the vectorized packers against the element-by-element rule, and
hand-derived bit placements."""
import numpy as np
import pytest

from oracle import accounting, layout as L


@pytest.mark.parametrize("P", [16, 32])
@pytest.mark.parametrize("d", [128, 256])
def test_head_block_sizes(P, d):
    assert L.fp8_head_bytes(P, d) == P * accounting.fp8_token_head_bytes(d)
    for b in (2, 3, 4):
        assert L.tq_head_bytes(P, d, b) == P * accounting.tq_token_head_bytes(d, b)
    # the per-token-head numbers the configs use
    assert accounting.fp8_token_head_bytes(256) == 520 and accounting.fp8_token_head_bytes(128) == 264
    assert accounting.tq_token_head_bytes(256, 3) == 196 and accounting.tq_token_head_bytes(128, 3) == 100
    assert accounting.tq_token_head_bytes(128, 2) == 68


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("role", [0, 1])
def test_lane_map_is_a_bijection(d, role):
    tok, dim = L.lane_element_token_dim(role, d)
    flat = (tok * d + dim).ravel()
    assert np.array_equal(np.sort(flat), np.arange(16 * d))


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_every_tile_bit_used_once(d, bits):
    DL = d // 4
    W = DL * bits // 32
    seen = set()
    for i in range(DL):
        for (w, pos, cb) in L.code_bit_positions(i, bits):
            assert 0 <= w < W and 0 <= pos < 32
            for l in range(64):
                key = L.word_byte_offset(l, w, W) * 8 + pos
                assert key not in seen
                seen.add(key)
    assert len(seen) == 16 * d * bits


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("role", [0, 1])
def test_vectorized_tq_pack_matches_rule(d, bits, role):
    rng = np.random.default_rng(d + bits + role)
    c = rng.integers(0, 1 << bits, size=(2, 16, d)).astype(np.uint8)
    t = L.tq_pack_tiles(c, role, bits)
    for k in range(2):
        assert np.array_equal(t[k], L.tq_tile_pack_loop(c[k], role, d, bits))
    assert np.array_equal(L.tq_unpack_tiles(t, role, d, bits), c)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("role", [0, 1])
def test_vectorized_fp8_pack_matches_rule(d, role):
    rng = np.random.default_rng(d + role)
    c = rng.integers(0, 256, size=(2, 16, d)).astype(np.uint8)
    t = L.fp8_pack_tiles(c, role)
    for k in range(2):
        assert np.array_equal(t[k], L.fp8_tile_pack_loop(c[k], role, d))
    assert np.array_equal(L.fp8_unpack_tiles(t, role, d), c)


def test_hand_placed_bits_tq3_d128():
    # K role, token 0, dim 24 -> lane 0, element 24 -> group 6, slot 0 (q = 6):
    # code bits 0-1 in word 0 bits 6-7, code bit 2 in word 2 bit 6.
    # d = 128 -> W = 3 words per lane: regions (words 0-1: 8 B/lane), (word 2: 4 B/lane)
    c = np.zeros((1, 16, 128), np.uint8)
    c[0, 0, 24] = 7
    t = L.tq_pack_tiles(c, 0, 3)[0]
    nz = {int(i): int(t[i]) for i in np.nonzero(t)[0]}
    assert nz == {0: 0xC0, 512: 0x40}
    # V role, token 5, dim 18: lane = 18 % 16 + 16 * (5 // 4) = 18, element
    # i = 4 * (18 // 16) + 5 % 4 = 5 -> group 1, slot 1: word 0 bits 3-5 of byte 1
    c = np.zeros((1, 16, 128), np.uint8)
    c[0, 5, 18] = 5
    t = L.tq_pack_tiles(c, 1, 3)[0]
    nz = {int(i): int(t[i]) for i in np.nonzero(t)[0]}
    assert nz == {18 * 8 + 1: 5 << 3}


def test_hand_placed_fp8_bytes():
    # K role d = 256: token 3, dim 70 -> lane 3 + 16 * (70 // 64) = 19, element 6
    # -> byte ((6 // 16) * 64 + 19) * 16 + 6 = 310
    c = np.zeros((1, 16, 256), np.uint8)
    c[0, 3, 70] = 0xAB
    t = L.fp8_pack_tiles(c, 0)[0]
    assert np.nonzero(t)[0].tolist() == [310]
    # V role d = 256: token 9, dim 37 -> lane 37 % 16 + 16 * (9 // 4) = 37,
    # element 4 * (37 // 16) + 9 % 4 = 9 -> byte (0 * 64 + 37) * 16 + 9 = 601
    c = np.zeros((1, 16, 256), np.uint8)
    c[0, 9, 37] = 0xCD
    t = L.fp8_pack_tiles(c, 1)[0]
    assert np.nonzero(t)[0].tolist() == [601]


def test_head_pack_roundtrip_and_order():
    rng = np.random.default_rng(5)
    P, d = 32, 128
    kc = rng.integers(0, 8, (P, d)).astype(np.uint8)
    vc = rng.integers(0, 8, (P, d)).astype(np.uint8)
    ks = rng.random(P).astype(np.float16)
    vs = rng.random(P).astype(np.float16)
    blk = L.tq_pack_head(kc, vc, ks, vs, 3)
    out = L.tq_unpack_head(blk, P, d, 3)
    for a, b in zip(out, (kc, vc, ks, vs)):
        assert np.array_equal(a, b)
    # sigma arrays sit at the end, K then V, in slot order
    assert np.array_equal(blk[-4 * P:-2 * P].view("<f2"), ks)
    kc8 = rng.integers(0, 256, (P, d)).astype(np.uint8)
    vc8 = rng.integers(0, 256, (P, d)).astype(np.uint8)
    ks8 = rng.random(P).astype(np.float32)
    vs8 = rng.random(P).astype(np.float32)
    blk = L.fp8_pack_head(kc8, vc8, ks8, vs8)
    out = L.fp8_unpack_head(blk, P, d)
    for a, b in zip(out, (kc8, vc8, ks8, vs8)):
        assert np.array_equal(a, b)
    assert np.array_equal(blk[-4 * P:].view("<f4"), vs8)
