"""Pins of the oracle's page mass (Minima-KV Eq. 6-8) and running score (Eq. 9).

What fixes them from outside the Eq. 6-8 code: the plain global softmax over
the same scores summed per page (no partitions at all), the closed form of a
cache whose keys are all equal (uniform attention: mass = tokens in the page /
N, a partial last page included), the normalization sum_p q = 1, and the
limits beta = 0 (a = r) and beta = 1 (a unchanged) of the EWMA."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import cache as OC
from oracle import pagemass as PM


def _tiny(seq_len=300, seed=2, **over):
    w = W.scaled(W.WORKLOADS["tiny"], seq_len=seq_len, recent_tokens=64, **over)
    plan = W.make_page_plan(w, seed)
    signs = W.make_signs(w, seed, 0)
    q = W.make_q(w, seed, 0)
    kv = {b: W.make_kv(w, seed, 0, b, int(plan.seq_lens[b])) for b in range(w.batch)}
    pools = OC.build_pools(w, plan, lambda b: kv[b], signs)
    return w, plan, signs, q, pools


def test_page_mass_is_the_global_softmax_summed_per_page():
    w, plan, signs, q, pools = _tiny()
    got = PM.page_mass_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, q, w.sm_scale, w.page_size,
                           w.num_kv_heads, w.head_dim, signs)
    assert set(np.unique(plan.page_format[0][:(int(plan.seq_lens[0]) + 15) // 16])) == {0, 1}   # two partitions
    qf = (np.asarray(q, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    N = int(plan.seq_lens[0])
    K, _ = A.dequant_request(pools, plan.block_table[0], plan.page_format[0], N, w.page_size, w.num_kv_heads,
                             w.head_dim, signs)
    G = w.num_q_heads // w.num_kv_heads
    for h in range(w.num_q_heads):
        s = w.sm_scale * (K[:, h // G] @ qf[0, h])
        p = np.exp(s - s.max())
        p /= p.sum()
        ref = np.array([p[i:i + w.page_size].sum() for i in range(0, N, w.page_size)])
        np.testing.assert_allclose(got[0, h, :len(ref)], ref, rtol=1e-12, atol=1e-15)
        assert np.all(got[0, h, len(ref):] == 0)
        assert abs(got[0, h].sum() - 1.0) < 1e-12


def test_equal_keys_give_uniform_mass_with_a_partial_last_page():
    w = W.scaled(W.WORKLOADS["tiny"], seq_len=75, recent_tokens=32)
    plan = W.make_page_plan(w, 0)
    signs = W.make_signs(w, 0, 0)
    q = W.make_q(w, 0, 0)
    N = int(plan.seq_lens[0])
    plan.page_format[0, :] = 0                                 # FP8 everywhere: equal rows decode equal
    n_pages = (N + 15) // 16
    plan.block_table[0, :n_pages] = np.arange(n_pages)
    pool_pages = dict(plan.pool_pages)
    pool_pages[0] = max(pool_pages.get(0, 0), n_pages)
    plan = W.PagePlan(plan.seq_lens, plan.page_format, plan.block_table, pool_pages, plan.max_pages)
    row = np.random.default_rng(1).standard_normal((1, w.num_kv_heads, w.head_dim)).astype(np.float32)
    K = np.repeat(row, N, axis=0)
    V = np.random.default_rng(2).standard_normal((N, w.num_kv_heads, w.head_dim)).astype(np.float32)
    pools = OC.build_pools(w, plan, lambda b: (K, V), signs)
    got = PM.page_mass_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, q, w.sm_scale, w.page_size,
                           w.num_kv_heads, w.head_dim, signs)
    expect = np.array([16, 16, 16, 16, 11]) / 75.0             # 75 tokens: four full pages and 11
    for h in range(w.num_q_heads):
        np.testing.assert_allclose(got[0, h, :5], expect, rtol=1e-12)


def test_ewma_limits_and_normalization():
    rng = np.random.default_rng(4)
    B, Hq, MP, P = 3, 4, 6, 16
    qmass = rng.random((B, Hq, MP))
    seq = np.array([70, 0, 96])                                 # 5 pages, none, 6 pages
    a0 = rng.random((B, MP))
    r, a = PM.collect_ref(qmass, seq, P, [0, 2, 3], 0.0, a0)
    assert np.allclose(a[0, :5], r[0, :5]) and np.allclose(a[2], r[2])
    assert np.array_equal(a[0, 5:], a0[0, 5:]) and np.array_equal(a[1], a0[1])   # pages not live keep a
    assert abs(r[0].sum() - 1) < 1e-12 and abs(r[2].sum() - 1) < 1e-12 and r[1].sum() == 0
    ref0 = np.mean([qmass[0, h, :5] / qmass[0, h, :5].sum() for h in (0, 2, 3)], axis=0)
    np.testing.assert_allclose(r[0, :5], ref0, rtol=1e-14)
    _, a1 = PM.collect_ref(qmass, seq, P, [1], 1.0, a0)
    assert np.array_equal(a1, a0)
    _, ah = PM.collect_ref(qmass, seq, P, [1], 0.25, a0)
    rr, _ = PM.collect_ref(qmass, seq, P, [1], 0.0, a0)
    np.testing.assert_allclose(ah[2], 0.25 * a0[2] + 0.75 * rr[2], rtol=1e-14)


def test_empty_request_has_no_mass():
    w, plan, signs, q, pools = _tiny(seq_len=40)
    seq = plan.seq_lens.copy()
    seq[0] = 0
    got = PM.page_mass_ref(pools, plan.block_table, plan.page_format, seq, q, w.sm_scale, w.page_size,
                           w.num_kv_heads, w.head_dim, signs)
    assert not got.any()
