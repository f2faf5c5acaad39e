"""Pins of the oracle's grouped mixed-rate key codec (TQK) and its page layout.

What fixes them from outside the oracle: the rate accounting of Block-GTQ
appendix A.7 (a key row carries d * mean-rate code bits), the reduction of a
one-segment key to the already pinned TQ codec, dense Hadamard and
permutation matrices for the codec-coordinate query (appendix H.2), the
per-segment norm restore (appendix B.1), brute-force placement checks of the
layout, and the Gaussian distortion per rate."""
import math

import numpy as np
import pytest
from scipy.linalg import hadamard

import workloads as W
from oracle import accounting, layout as L, tq, tqk


def _rates(d, seed):
    nb = d // 2
    r = np.zeros(nb, np.int64)
    p = np.random.default_rng(seed).permutation(nb)
    r[p[:nb // 4]] = 2
    r[p[nb // 4:3 * nb // 4]] = 3
    r[p[3 * nb // 4:]] = 4
    return r


@pytest.mark.parametrize("d", [128, 256])
def test_segments_group_blocks_by_rate(d):
    rates = _rates(d, d)
    perm, segs = tqk.segments(rates)
    assert segs == [(2, d // 4), (3, d // 2), (4, d // 4)]
    assert np.array_equal(np.sort(perm), np.arange(d))             # a permutation
    # brute force: walk positions, each pair is one whole block, widths never
    # decrease, and inside one width the block index increases
    prev = (0, -1)
    for j in range(0, d, 2):
        a, b = perm[j], perm[j + 1]
        assert a % 2 == 0 and b == a + 1
        blk = a // 2
        key = (rates[blk], blk)
        assert key > prev
        prev = key
    # mean rate 3: the key row holds d * 3 code bits (Block-GTQ A.7: 2 sum b_i = d b_bar)
    assert 2 * rates.sum() == 3 * d
    assert sum(b * w for b, w in segs) == 3 * d


def test_workload_permutation_matches_the_grouping_rule():
    w = W.WORKLOADS["l70b"]
    rates = W.make_tqk_rates(w, 4, 0)
    perm = W.make_tqk_perm(w, 4, 0)
    assert perm.shape == (w.num_kv_heads, w.head_dim)
    for h in range(w.num_kv_heads):
        p, segs = tqk.segments(rates[h])
        assert np.array_equal(perm[h].astype(np.int64), p)
        assert segs == [(2, 32), (3, 64), (4, 32)]


def test_single_segment_is_the_plain_tq_codec():
    """All blocks at one rate and no reordering: the grouped key codec is the
    uniform codec of oracle.tq, bit for bit."""
    rng = np.random.default_rng(1)
    d = 64
    x = rng.standard_normal((50, d)).astype(np.float32)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    for bits in (2, 3, 4):
        perm, segs = tqk.segments(np.full(d // 2, bits))
        assert np.array_equal(perm, np.arange(d)) and segs == [(bits, d)]
        (codes, sigma), = tqk.encode_key(x, perm, segs, s)
        c2, s2 = tq.tq_encode(x, s, bits)
        assert np.array_equal(codes, c2) and np.array_equal(sigma, s2)


def test_codec_coordinate_query_identity():
    """q . k_hat = sum_s sigma_s (R_s (P q)_s) . c_s with R_s = H_s D_s / sqrt(d_s),
    checked with dense Hadamard and permutation matrices (fp64)."""
    rng = np.random.default_rng(2)
    d = 128
    rates = _rates(d, 5)
    perm, segs = tqk.segments(rates)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x = rng.standard_normal((40, d)).astype(np.float32) * np.repeat(rng.uniform(0.1, 3, d // 2), 2)
    seg = tqk.encode_key(x, perm, segs, s)
    kh = tqk.decode_key(seg, perm, segs, s)
    q = rng.standard_normal(d)
    Pm = np.zeros((d, d))
    Pm[np.arange(d), perm] = 1.0                                   # (P q)_j = q[perm[j]]
    qp = Pm @ q
    rhs = np.zeros(40)
    j0 = 0
    for (bits, width), (codes, sigma) in zip(segs, seg):
        R = hadamard(width) @ np.diag(s[j0:j0 + width]) / math.sqrt(width)
        c = tq.codebook(bits)[0].astype(np.float64)[codes]
        rhs += sigma.astype(np.float64) * (c @ (R @ qp[j0:j0 + width]))
        j0 += width
    assert np.allclose(kh @ q, rhs, rtol=1e-12, atol=1e-12)
    qr = tqk.rotate_query(q, perm, segs, s)
    allc = tqk.codes_in_row(seg)
    sig = np.stack([sg for _, sg in seg]).astype(np.float64)        # [3, n]
    j0, rhs2 = 0, np.zeros(40)
    for i, (bits, width) in enumerate(segs):
        c = tq.codebook(bits)[0].astype(np.float64)[allc[:, j0:j0 + width]]
        rhs2 += sig[i] * (c @ qr[j0:j0 + width])
        j0 += width
    assert np.allclose(rhs2, rhs, rtol=1e-12, atol=1e-12)


def test_each_segment_restores_its_norm():
    rng = np.random.default_rng(3)
    d = 128
    rates = _rates(d, 9)
    perm, segs = tqk.segments(rates)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x = rng.standard_normal((30, d)).astype(np.float32)
    x[0] = 0
    seg = tqk.encode_key(x, perm, segs, s)
    kh = tqk.decode_key(seg, perm, segs, s)
    assert np.all(kh[0] == 0)
    j0 = 0
    for (bits, width), (codes, sigma) in zip(segs, seg):
        idx = perm[j0:j0 + width]
        n_in = np.linalg.norm(x[1:, idx].astype(np.float64), axis=-1)
        n_out = np.linalg.norm(kh[1:, idx], axis=-1)
        assert np.allclose(n_out, n_in, rtol=2.0 ** -10, atol=0)
        j0 += width


@pytest.mark.parametrize("bits,expect", [(2, 0.1175), (3, 0.0348), (4, 0.0095)])
def test_segment_distortion_tracks_its_rate(bits, expect):
    rng = np.random.default_rng(bits)
    d = 256
    rates = _rates(d, 11)
    perm, segs = tqk.segments(rates)
    s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x = rng.standard_normal((1500, d)).astype(np.float32)
    seg = tqk.encode_key(x, perm, segs, s)
    kh = tqk.decode_key(seg, perm, segs, s)
    j0 = 0
    for b, width in segs:
        if b == bits:
            idx = perm[j0:j0 + width]
            err = ((kh[:, idx] - x[:, idx]) ** 2).sum(-1) / (x[:, idx].astype(np.float64) ** 2).sum(-1)
            assert abs(err.mean() - expect) < 0.15 * expect
        j0 += width


@pytest.mark.parametrize("d", [128, 256])
def test_tqk_head_bytes(d):
    assert L.tqk_head_bytes(16, d) == 16 * accounting.tqk_token_head_bytes(
        d, seg_dims=(d // 4, d // 2, d // 4))
    assert accounting.tqk_token_head_bytes(128) == 104


@pytest.mark.parametrize("d", [128, 256])
def test_tqk_key_tile_bits_used_once(d):
    W_ = 3 * d // 128
    seen = set()
    for i in range(d // 4):
        pos = L.tqk_code_bit_positions(i, d)
        assert len(pos) == L.tqk_element_bits(i, d)
        for (w, p, cb) in pos:
            for l in range(64):
                key = L.word_byte_offset(l, w, W_) * 8 + p
                assert key not in seen
                seen.add(key)
    assert len(seen) == 16 * d * 3
    tok, dim = L.tqk_key_lane_map(d)
    assert np.array_equal(np.sort((tok * d + dim).ravel()), np.arange(16 * d))
    # a lane's element widths follow the segment of the coordinate it holds
    for i in range(d // 4):
        seg_bits = 2 if dim[0, i] < d // 4 else (3 if dim[0, i] < 3 * d // 4 else 4)
        assert L.tqk_element_bits(i, d) == seg_bits
        assert all((2 if dim[l, i] < d // 4 else (3 if dim[l, i] < 3 * d // 4 else 4)) == seg_bits
                   for l in range(64))


@pytest.mark.parametrize("d", [128, 256])
def test_tqk_vectorized_pack_matches_rule(d):
    rng = np.random.default_rng(d)
    c = np.zeros((2, 16, d), np.uint8)
    for j, b in ((slice(0, d // 4), 2), (slice(d // 4, 3 * d // 4), 3), (slice(3 * d // 4, d), 4)):
        c[:, :, j] = rng.integers(0, 1 << b, size=c[:, :, j].shape)
    t = L.tqk_pack_key_tiles(c)
    for k in range(2):
        assert np.array_equal(t[k], L.tqk_key_tile_pack_loop(c[k], d))
    assert np.array_equal(L.tqk_unpack_key_tiles(t, d), c)


def test_tqk_hand_placed_bits():
    d = 128
    # token 2, permuted dim 40 (3-bit segment): chunk 1 -> i // 8 = 1, lane
    # group (40 - 32) // 8 = 1 -> lane 2 + 16 = 18, element 8 + 0 = 8 ->
    # group 2 (first 3-bit group) slot 0: word 1 bits 0-2 of byte 0.
    # W = 3: word 1 is the second word of lane 18's 8-byte region -> byte 18 * 8 + 4
    c = np.zeros((1, 16, d), np.uint8)
    c[0, 2, 40] = 5
    t = L.tqk_pack_key_tiles(c)[0]
    assert {int(i): int(t[i]) for i in np.nonzero(t)[0]} == {18 * 8 + 4: 5}
    # token 7, permuted dim 125 (4-bit): chunk 3 -> i = 24 + 125 % 8 = 29, lane
    # group (125 - 96) // 8 = 3 -> lane 7 + 48 = 55; group 7, slot 1 -> word 0
    # bits 4-7 of byte 1
    c = np.zeros((1, 16, d), np.uint8)
    c[0, 7, 125] = 0xB
    t = L.tqk_pack_key_tiles(c)[0]
    assert {int(i): int(t[i]) for i in np.nonzero(t)[0]} == {55 * 8 + 1: 0xB0}
    # token 0, permuted dim 3 (2-bit): lane 0, element 3 -> group 0 slot 3:
    # word 1 bits 6-7 of byte 3
    c = np.zeros((1, 16, d), np.uint8)
    c[0, 0, 3] = 2
    t = L.tqk_pack_key_tiles(c)[0]
    assert {int(i): int(t[i]) for i in np.nonzero(t)[0]} == {0 * 8 + 4 + 3: 0x80}


def test_tqk_head_roundtrip():
    rng = np.random.default_rng(12)
    P, d = 32, 128
    rates = _rates(d, 3)
    perm, segs = tqk.segments(rates)
    k = rng.standard_normal((P, d)).astype(np.float32)
    v = rng.standard_normal((P, d)).astype(np.float32)
    sk = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    sv = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    blk = tqk.encode_page_head(k, v, sk, sv, rates)
    assert blk.size == tqk.head_bytes(P, d)
    kc, ksig, vc, vsig = L.tqk_unpack_head(blk, P, d)
    seg = tqk.encode_key(k, perm, segs, sk)
    assert np.array_equal(kc, tqk.codes_in_row(seg))
    assert np.array_equal(ksig, np.stack([s for _, s in seg]))
    vc2, vs2 = tq.tq_encode(v, sv, 3)
    assert np.array_equal(vc, vc2) and np.array_equal(vsig, vs2)
    # sigma block: K sigmas segment-major, then V sigmas, at the end of the block
    assert np.array_equal(blk[-8 * P:-2 * P].view("<f2").reshape(3, P), ksig)
    kh, vh = tqk.dequant_page_head(blk, P, d, sk, sv, rates)
    assert np.allclose(kh, tqk.decode_key(seg, perm, segs, sk), rtol=0, atol=0)
    assert np.allclose(vh, tq.tq_decode(vc2, vs2, sv, 3), rtol=0, atol=0)


def test_paged_reference_over_a_tqk_cache():
    """The paged walk (pools, tables, layout) gives the same attention as the
    plain definition over keys and values decoded straight from the codec."""
    from oracle import attention as A, cache as OC
    w = W.scaled(W.WORKLOADS["l70b"], batch=2, seq_len=300, recent_tokens=64, num_q_heads=8, num_kv_heads=2)
    plan = W.make_page_plan(w, 1)
    signs = W.make_signs(w, 1, 0)
    rates = W.make_tqk_rates(w, 1, 0)
    kv = {b: W.make_kv(w, 1, 0, b, int(plan.seq_lens[b])) for b in range(w.batch)}
    pools = OC.build_pools(w, plan, lambda b: kv[b], signs, tqk=rates)
    O, lse = A.paged_decode_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, W.make_q(w, 1, 0),
                                w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, signs, tqk=rates)
    q = W.bf16_to_f32(W.make_q(w, 1, 0)).astype(np.float64)
    from oracle import fp8
    for b in range(w.batch):
        K, V = kv[b]
        N = K.shape[0]
        Kh = np.zeros((N, 2, 128))
        Vh = np.zeros((N, 2, 128))
        for p in range((N + 31) // 32):
            sl = slice(32 * p, min(N, 32 * p + 32))
            for g in range(2):
                if plan.page_format[b, p] == W.FMT_FP8:
                    kc, ks = fp8.fp8_encode(K[sl, g])
                    vc, vs = fp8.fp8_encode(V[sl, g])
                    Kh[sl, g], Vh[sl, g] = fp8.fp8_decode(kc, ks), fp8.fp8_decode(vc, vs)
                else:
                    sk = tq.signs_from_bits(signs[g, 0], 128)
                    sv = tq.signs_from_bits(signs[g, 1], 128)
                    perm, segs = tqk.segments(rates[g])
                    Kh[sl, g] = tqk.decode_key(tqk.encode_key(K[sl, g], perm, segs, sk), perm, segs, sk)
                    vc, vsig = tq.tq_encode(V[sl, g], sv, 3)
                    Vh[sl, g] = tq.tq_decode(vc, vsig, sv, 3)
        Or, lr = A.attention_ref(q[b], Kh, Vh, w.sm_scale)
        assert np.allclose(O[b], Or, rtol=1e-12, atol=1e-12) and np.allclose(lse[b], lr, rtol=1e-12, atol=1e-12)
    assert (plan.page_format[:, :(300 + 31) // 32] == W.FMT_TQK).any()
