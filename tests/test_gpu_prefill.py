"""GPU parity of chunked prefill (paged_prefill_attn_planned, Block-GTQ
appendix H.5) against the oracle's causal attention over its own encoding of
the same cache: every output element within 2e-3 + 1e-2 |ref|. A chunk of
one token must give the plain decode's output bit for bit."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import prefill as OP
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


def _prefill(case, lay, chunk, q_bits):
    torch = C.torch_mod()
    m = C.kvq()
    w = case.w
    bt, pf, sl = case.tables()
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    max_pages = bt.shape[1]
    plan_buf = torch.zeros(m.paged_decode_plan_bytes(lay.cache, B, max_pages), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(m.paged_prefill_attn_workspace_size(lay.cache, B, Hq, chunk, max_pages), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((B, chunk, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, chunk, Hq), float("nan"), dtype=torch.float32, device="cuda")
    q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).cuda().view(torch.bfloat16)
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf)
    m.paged_prefill_attn_planned(lay.cache, plan_buf, q, max_pages, w.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), plan_buf, ws


@pytest.mark.parametrize("name,over,chunk", [
    ("tiny", {"seq_len": 1000}, 4),                                     # G 4: 16 rows
    ("tiny", {"seq_len": 700, "num_q_heads": 1}, 16),                   # G 1: 16 tokens, 3 tiles of partial rows
    ("tiny", {"page_size": 32, "seq_len": 777}, 3),
    ("l27b", {"seq_len": 2500, "recent_tokens": 512}, 2),               # G 6: 12 rows
    ("serving", {"batch": 3, "seq_len_range": (2, 900)}, 4),            # ragged, a request shorter than most chunks
    ("l70b", {"batch": 2, "seq_len": 1500, "recent_tokens": 256, "num_q_heads": 16, "num_kv_heads": 2}, 2),
    # d 256 at page 32 with FP8 + TQ3 + TQ2, and grouped keys at page 16
    ("serving", {"head_dim": 256, "page_size": 32, "batch": 2, "seq_len_range": (300, 1500), "num_q_heads": 8,
                 "num_kv_heads": 2}, 4),
    ("l70b", {"page_size": 16, "batch": 2, "seq_len": 1300, "recent_tokens": 128, "num_q_heads": 16,
              "num_kv_heads": 2}, 2),
    # fractional-level Stale pages
    ("frac", {"batch": 2, "seq_len_range": (300, 1400)}, 4),
    ("frac", {"head_dim": 256, "page_size": 32, "batch": 2, "seq_len_range": (200, 1100), "num_q_heads": 8,
              "num_kv_heads": 2}, 3),
])
def test_prefill_parity(name, over, chunk):
    C.say(f"prefill {name} {over} chunk={chunk}")
    w = W.scaled(W.WORKLOADS[name], **over)
    case = C.Case(w, seed=13)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    C.assert_pools_equal(lay, pools, f"{name} pools")
    q = np.stack([np.stack([W.make_q(w, 100 + c, 0)[b] for c in range(chunk)]) for b in range(w.batch)])
    O, L, _, _ = _prefill(case, lay, chunk, q)                           # [B, C, Hq, d]
    for b in range(w.batch):
        N = int(case.plan.seq_lens[b])
        n0 = N - chunk
        if n0 < 0:
            # tokens at negative positions see nothing; the rest see 0 .. n0 + c
            for c in range(chunk):
                if n0 + c < 0:
                    assert np.all(O[b, c] == 0) and np.all(L[b, c] == -np.inf), f"request {b} token {c}"
            continue
        Oref, Lref = OP.prefill_ref(pools, case.plan.block_table[b], case.plan.page_format[b], n0, q[b],
                                    w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, case.signs,
                                    tqk=case.tqk_rates)
        C.assert_close(O[b], Oref, f"{name} prefill O request {b}")
        C.assert_close(L[b], Lref, f"{name} prefill lse request {b}")


def test_one_token_prefill_is_the_decode():
    torch = C.torch_mod()
    m = C.kvq()
    C.say("prefill chunk 1 = decode")
    w = W.scaled(W.WORKLOADS["l27b"], seq_len=3000, recent_tokens=512)
    case = C.Case(w, seed=2)
    lay = case.gpu_layer()
    O, L, plan_buf, ws = _prefill(case, lay, 1, case.q[:, None])
    Od, Ld = C.run_decode(case, lay, oneshot=False)
    assert np.array_equal(O[:, 0], Od) and np.array_equal(L[:, 0], Ld)


@pytest.mark.parametrize("name,over", [("canary", {"layers": 1}), ("serving", {})])
def test_last_chunk_token_is_the_decode_at_full_size(name, over):
    """At full size, in the benchmark's launch configuration: the chunk's last
    token sees every cached token, with the same tiles, masks and merge order
    as a decode step, so its rows equal the plain decode of the same query up
    to rounding (the deferred softmax rescale is decided over all rows of a
    wave, so the other tokens' rows can move its reference maximum)."""
    C.say(f"prefill full size {name}")
    w = W.scaled(W.WORKLOADS[name], **over)
    case = C.Case(w, seed=0)
    lay = case.gpu_layer()
    chunk = max(1, 16 // w.group)
    q = np.stack([np.stack([W.make_q(w, 200 + c, 0)[b] for c in range(chunk - 1)] + [case.q[b]])
                  for b in range(w.batch)])
    O, L, _, _ = _prefill(case, lay, chunk, q)
    Od, Ld = C.run_decode(case, lay, oneshot=False)
    C.assert_close(O[:, -1], Od, f"{name} last chunk token O")
    C.assert_close(L[:, -1], Ld, f"{name} last chunk token lse")
    assert np.isfinite(O).all() and np.isfinite(L).all()
    # sampled rows against the oracle: one KV head of two requests, rebuilt by
    # the oracle's own encoders
    g = 1
    sample = C.Case(w, seed=0, heads=[g], requests=[0, w.batch - 1])
    pools = sample.oracle_pools()
    G = w.group
    for b in sorted({0, w.batch - 1}):
        n0 = int(case.plan.seq_lens[b]) - chunk
        Oref, Lref = OP.prefill_ref(pools, case.plan.block_table[b], case.plan.page_format[b], n0, q[b], w.sm_scale,
                                    w.page_size, w.num_kv_heads, w.head_dim, case.signs, tqk=case.tqk_rates,
                                    heads=[g])
        hs = slice(g * G, (g + 1) * G)
        C.assert_close(O[b][:, hs], Oref[:, hs], f"{name} prefill O request {b} KV head {g} (oracle)")
        C.assert_close(L[b][:, hs], Lref[:, hs], f"{name} prefill lse request {b} KV head {g} (oracle)")


def test_requests_shorter_than_the_chunk():
    """N_b < C: the chunk's tokens at negative positions see nothing (O = 0,
    lse = -inf); the others see tokens 0 .. N_b - C + c."""
    C.say("prefill: requests shorter than the chunk")
    w = W.scaled(W.WORKLOADS["serving"], batch=4, seq_len_range=(1, 6), recent_tokens=16)
    case = C.Case(w, seed=8)
    case.plan.seq_lens[:] = np.array([1, 2, 3, 4], np.int32)[:w.batch]
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    chunk = 4
    q = np.stack([np.stack([W.make_q(w, 300 + c, 0)[b] for c in range(chunk)]) for b in range(w.batch)])
    O, L, _, _ = _prefill(case, lay, chunk, q)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for b in range(w.batch):
        N = int(case.plan.seq_lens[b])
        K, V = OA.dequant_request(pools, case.plan.block_table[b], case.plan.page_format[b], N, w.page_size,
                                  w.num_kv_heads, w.head_dim, case.signs)
        for c in range(chunk):
            lim = N - chunk + c + 1
            if lim <= 0:
                assert np.all(O[b, c] == 0) and np.all(L[b, c] == -np.inf), f"request {b} token {c}"
                continue
            Oref, Lref = OA.attention_ref(qf[b, c], K[:lim], V[:lim], w.sm_scale)
            C.assert_close(O[b, c], Oref, f"request {b} token {c} O")
            C.assert_close(L[b, c], Lref, f"request {b} token {c} lse")
