"""Pins of the oracle's chunked prefill (Block-GTQ appendix H.5).

What fixes it from outside the prefill function: a chunk of one token is a
decode step over N0 + 1 tokens (the decode reference is pinned against
brute-force softmax); causality (changing the K/V of later tokens leaves
earlier queries' outputs unchanged, and changes the later ones); and a
brute-force softmax over an explicit causal score matrix on a tiny cache."""
import math

import numpy as np

import workloads as W
from oracle import attention as A
from oracle import cache as OC
from oracle import prefill as PF


def _setup(seq_len=200, seed=3, **over):
    w = W.scaled(W.WORKLOADS["tiny"], seq_len=seq_len, recent_tokens=64, **over)
    plan = W.make_page_plan(w, seed)
    signs = W.make_signs(w, seed, 0)
    K, V = W.make_kv(w, seed, 0, 0, int(plan.seq_lens[0]))
    pools = OC.build_pools(w, plan, lambda b: (K, V), signs)
    return w, plan, signs, K, V, pools


def test_one_token_chunk_is_a_decode_step():
    w, plan, signs, K, V, pools = _setup()
    N = int(plan.seq_lens[0])
    q = W.make_q(w, 9, 0)                                      # [1, Hq, d]
    O, lse = PF.prefill_ref(pools, plan.block_table[0], plan.page_format[0], N - 1, q[0:1], w.sm_scale,
                            w.page_size, w.num_kv_heads, w.head_dim, signs)
    Od, ld = A.paged_decode_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, q, w.sm_scale,
                                w.page_size, w.num_kv_heads, w.head_dim, signs)
    np.testing.assert_allclose(O[0], Od[0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0], ld[0], rtol=1e-13)


def test_causality():
    w, plan, signs, K, V, pools = _setup(seq_len=160)
    N = int(plan.seq_lens[0])
    C = 4
    q = np.stack([W.make_q(w, 20 + c, 0)[0] for c in range(C)])      # [C, Hq, d]
    O, lse = PF.prefill_ref(pools, plan.block_table[0], plan.page_format[0], N - C, q, w.sm_scale, w.page_size,
                            w.num_kv_heads, w.head_dim, signs)
    K2, V2 = K.copy(), V.copy()
    K2[N - 1] *= -3.0                                          # the chunk's last token
    V2[N - 1] += 5.0
    pools2 = OC.build_pools(w, plan, lambda b: (K2, V2), signs)
    O2, lse2 = PF.prefill_ref(pools2, plan.block_table[0], plan.page_format[0], N - C, q, w.sm_scale, w.page_size,
                              w.num_kv_heads, w.head_dim, signs)
    assert np.array_equal(O[:C - 1], O2[:C - 1]) and np.array_equal(lse[:C - 1], lse2[:C - 1])
    assert not np.allclose(O[C - 1], O2[C - 1])


def test_bruteforce_causal_softmax():
    w, plan, signs, K, V, pools = _setup(seq_len=40)
    N = int(plan.seq_lens[0])
    C, Hq, Hkv = 5, w.num_q_heads, w.num_kv_heads
    G = Hq // Hkv
    q = np.stack([W.make_q(w, 30 + c, 0)[0] for c in range(C)])
    O, lse = PF.prefill_ref(pools, plan.block_table[0], plan.page_format[0], N - C, q, w.sm_scale, w.page_size,
                            Hkv, w.head_dim, signs)
    Kd, Vd = A.dequant_request(pools, plan.block_table[0], plan.page_format[0], N, w.page_size, Hkv, w.head_dim,
                               signs)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for c in range(C):
        for h in range(Hq):
            lim = N - C + c + 1
            s = [w.sm_scale * float(np.dot(qf[c, h], Kd[i, h // G])) for i in range(lim)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = sum(e)
            ref = sum(e[i] * Vd[i, h // G] for i in range(lim)) / tot
            np.testing.assert_allclose(O[c, h], ref, rtol=1e-12, atol=1e-14)
            assert abs(lse[c, h] - (m + math.log(tot))) < 1e-12
