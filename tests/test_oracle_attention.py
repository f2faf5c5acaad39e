"""Pins of the attention reference: brute-force softmax, closed forms, the
Eq. 11-13 merge identity, and paged walking against direct (unpaged)
encode/decode of the same rows."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import cache, fp8, tq


def _brute(q, K, V, scale):
    """Pure-Python softmax attention, one q-head at a time (tiny inputs only)."""
    Hq, d = len(q), len(q[0])
    N, Hkv = len(K), len(K[0])
    G = Hq // Hkv
    O, lse = [], []
    for h in range(Hq):
        g = h // G
        s = [scale * sum(q[h][j] * K[i][g][j] for j in range(d)) for i in range(N)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        z = sum(e)
        O.append([sum(e[i] * V[i][g][j] for i in range(N)) / z for j in range(d)])
        lse.append(m + math.log(z))
    return np.array(O), np.array(lse)


def test_bruteforce_tiny():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((7, 2, 8))
    V = rng.standard_normal((7, 2, 8))
    O, lse = A.attention_ref(q, K, V, 0.3)
    Ob, lb = _brute(q.tolist(), K.tolist(), V.tolist(), 0.3)
    assert np.allclose(O, Ob, atol=1e-12) and np.allclose(lse, lb, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((9, 1, 16))
    V = rng.standard_normal((9, 1, 16))
    O, lse = A.attention_ref(np.zeros((3, 16)), K, V, 0.25)
    assert np.allclose(O, V[:, 0].mean(0)[None], atol=1e-12)
    assert np.allclose(lse, math.log(9), atol=1e-12)
    O, lse = A.attention_ref(rng.standard_normal((3, 16)), K[:1], V[:1], 0.25)
    assert np.allclose(O, V[0, 0][None], atol=1e-12)
    O, lse = A.attention_ref(rng.standard_normal((3, 16)), K[:0], V[:0], 0.25)
    assert (O == 0).all() and np.isneginf(lse).all()


def test_merge_equals_unpartitioned():
    """Minima-KV section 3.3: Eq. 11-13 over any partition = full attention."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((6, 32))
    K = 3 * rng.standard_normal((200, 1, 32))
    V = rng.standard_normal((200, 1, 32))
    O, lse = A.attention_ref(q, K, V, 1 / math.sqrt(32))
    for trial in range(5):
        lab = rng.integers(0, 4, size=200)
        parts = [A.partial_ref(q, K, V, 1 / math.sqrt(32), np.nonzero(lab == j)[0]) for j in range(4)]
        parts.append(A.partial_ref(q, K, V, 1 / math.sqrt(32), []))     # empty partition
        Om, lm = A.merge_ref(parts)
        assert np.allclose(Om, O, atol=1e-12) and np.allclose(lm, lse, atol=1e-12)
    Om, lm = A.merge_ref([A.partial_ref(q, K, V, 0.2, [])])
    assert (Om == 0).all() and np.isneginf(lm).all()


def _small(name, **over):
    return W.scaled(W.WORKLOADS[name], **over)


def test_paged_fp8_equals_direct_decode():
    w = _small("tiny", seq_len=100, recent_tokens=100 // 16 * 16 + 16, anchor_pages=1)
    plan = W.make_page_plan(w, seed=3)
    assert (plan.page_format[0, :7] == W.FMT_FP8).all()
    K, V = W.make_kv(w, 3, 0, 0, 100)
    signs = W.make_signs(w, 3, 0)
    pools = cache.build_pools(w, plan, lambda b: (K, V), signs)
    qb = W.make_q(w, 3, 0)
    O, lse = A.paged_decode_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, qb,
                                w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, signs)
    kc, ks = fp8.fp8_encode(K)
    vc, vs = fp8.fp8_encode(V)
    q = W.bf16_to_f32(qb)[0].astype(np.float64)
    O2, l2 = A.attention_ref(q, fp8.fp8_decode(kc, ks), fp8.fp8_decode(vc, vs), w.sm_scale)
    assert np.allclose(O[0], O2, atol=1e-12) and np.allclose(lse[0], l2, atol=1e-12)


@pytest.mark.parametrize("source", ["fp32", "fp8"])
def test_paged_mixed_equals_direct_decode(source):
    w = _small("tiny", seq_len=1000)        # partial last page: 1000 = 62*16 + 8
    plan = W.make_page_plan(w, seed=4)
    K, V = W.make_kv(w, 4, 0, 0, 1000)
    signs = W.make_signs(w, 4, 0)
    pools = cache.build_pools(w, plan, lambda b: (K, V), signs, stale_source=source)
    qb = W.make_q(w, 4, 0)
    O, lse = A.paged_decode_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, qb,
                                w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, signs)
    # direct: per token, FP8 or TQ3 by its page's tag, no layout involved
    sk = tq.signs_from_bits(signs[0, 0], 128)
    sv = tq.signs_from_bits(signs[0, 1], 128)
    Kh = np.zeros((1000, 1, 128))
    Vh = np.zeros((1000, 1, 128))
    for i in range(1000):
        f = plan.page_format[0, i // 16]
        for X, Xh, s in ((K, Kh, sk), (V, Vh, sv)):
            x = X[i:i + 1, 0]
            if f == W.FMT_FP8:
                c, sc = fp8.fp8_encode(x)
                Xh[i, 0] = fp8.fp8_decode(c, sc)[0]
            else:
                if source == "fp8":
                    c, sc = fp8.fp8_encode(x)
                    x = fp8.fp8_decode_f32(c, sc)
                c, sg = tq.tq_encode(x, s, 3)
                Xh[i, 0] = tq.tq_decode(c, sg, s, 3)[0]
    q = W.bf16_to_f32(qb)[0].astype(np.float64)
    O2, l2 = A.attention_ref(q, Kh, Vh, w.sm_scale)
    assert np.allclose(O[0], O2, atol=1e-12) and np.allclose(lse[0], l2, atol=1e-12)
    # the TQ3 result is close to exact attention over the fp32 rows
    O3, _ = A.attention_ref(q, K, V, w.sm_scale)
    assert np.abs(O[0] - O3).max() < 0.1


def test_duplicate_batch_parity():
    """Minima-KV appendix C: the same request twice in a batch gives identical
    outputs."""
    w = _small("tiny", batch=2, seq_len=300)
    plan = W.make_page_plan(w, seed=5)
    K, V = W.make_kv(w, 5, 0, 0, 300)
    signs = W.make_signs(w, 5, 0)
    pools = cache.build_pools(w, plan, lambda b: (K, V), signs)
    qb = W.make_q(w, 5, 0)
    qb[1] = qb[0]
    O, lse = A.paged_decode_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, qb,
                                w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, signs)
    assert np.array_equal(O[0], O[1]) and np.array_equal(lse[0], lse[1])


def test_paged_reference_head_subset_matches_full():
    """Restricting the paged reference to some KV heads gives their q-heads'
    outputs unchanged (the sampled full-size parity tests rely on it)."""
    import workloads as W
    from oracle import attention as A, cache as OC
    w = W.scaled(W.WORKLOADS["l27b"], seq_len=700, recent_tokens=128)
    plan = W.make_page_plan(w, 2)
    signs = W.make_signs(w, 2, 0)
    kv = W.make_kv(w, 2, 0, 0, 700)
    pools = OC.build_pools(w, plan, lambda b: kv, signs)
    q = W.make_q(w, 2, 0)
    O, L = A.paged_decode_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, q, w.sm_scale,
                              w.page_size, w.num_kv_heads, w.head_dim, signs)
    O2, L2 = A.paged_decode_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, q, w.sm_scale,
                                w.page_size, w.num_kv_heads, w.head_dim, signs, heads=[2])
    G = w.group
    assert np.allclose(O2[0, 2 * G:3 * G], O[0, 2 * G:3 * G], rtol=1e-12, atol=1e-12)
    assert np.allclose(L2[0, 2 * G:3 * G], L[0, 2 * G:3 * G], rtol=1e-12, atol=1e-12)
    assert np.all(O2[0, :2 * G] == 0) and np.all(np.isneginf(L2[0, :2 * G]))
