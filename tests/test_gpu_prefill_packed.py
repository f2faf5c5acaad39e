"""GPU parity of the packed chunked prefill (paged_prefill_attn_planned with
chunk x G > 16 query rows per KV head: 128-row query tiles, one launch per
format, Block-GTQ appendix H.5) against the oracle's causal attention over
its own encoding of the same cache: every output element within
2e-3 + 1e-2 |ref| (the scan's arithmetic is the decode's: f16 operands on
MFMA, fp32 accumulation and softmax)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import prefill as OP
from tests import gpu_common as C
from tests.test_gpu_prefill import _prefill

pytestmark = pytest.mark.gpu


def _chunk_q(w, chunk, seed):
    """bf16 bits uint16 [B, chunk, Hq, d], seeded N(0, 1)."""
    x = np.random.default_rng(seed).standard_normal((w.batch, chunk, w.num_q_heads, w.head_dim), dtype=np.float32)
    return W.bf16_round(x)


def _check_request(case, pools, O, L, q, b, chunk, what, heads=None, tokens=None):
    w = case.w
    N = int(case.plan.seq_lens[b])
    n_neg = max(0, chunk - N)                    # tokens at negative positions see nothing
    if n_neg:
        assert np.all(O[b, :n_neg] == 0) and np.all(L[b, :n_neg] == -np.inf), f"{what}: request {b} early tokens"
    if N == 0:
        return
    G = w.group
    hs = slice(None) if heads is None else np.concatenate([np.arange(g * G, (g + 1) * G) for g in heads])
    for cs in ([slice(n_neg, chunk)] if tokens is None else [slice(c, c + 1) for c in tokens if c >= n_neg]):
        n0 = N - chunk + cs.start
        Oref, Lref = OP.prefill_ref(pools, case.plan.block_table[b], case.plan.page_format[b], n0, q[b, cs],
                                    w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, case.signs,
                                    tqk=case.tqk_rates, heads=heads)
        C.assert_close(O[b, cs][:, hs], Oref[:, hs], f"{what}: request {b} tokens {cs.start}.. O")
        C.assert_close(L[b, cs][:, hs], Lref[:, hs], f"{what}: request {b} tokens {cs.start}.. lse")


@pytest.mark.parametrize("name,over,chunk", [
    # the canary layer shape (d 256, G 6) at reduced length: FP8 Recent +
    # Anchors + TQ3 Stale, chunks of 256 and 512 tokens (12 and 24 row tiles)
    ("canary", {"layers": 1, "batch": 1, "seq_len": 2600, "recent_tokens": 512, "anchor_pages": 3}, 256),
    ("canary", {"layers": 1, "batch": 2, "seq_len": 3000, "recent_tokens": 640, "anchor_pages": 4}, 512),
    # G 4, d 128, FP8 / TQ3 / TQ2 by importance, ragged lengths (one request
    # shorter than the chunk), both page sizes
    ("serving", {"batch": 3, "seq_len_range": (40, 1500)}, 64),
    ("serving", {"head_dim": 256, "page_size": 32, "batch": 2, "seq_len_range": (300, 1400), "num_q_heads": 8,
                 "num_kv_heads": 2}, 40),
    # grouped mixed-rate keys (G 8) and fractional-level pages
    ("l70b", {"batch": 1, "seq_len": 1500, "recent_tokens": 256, "num_q_heads": 16, "num_kv_heads": 2}, 100),
    ("frac", {"batch": 2, "seq_len_range": (200, 1300)}, 50),
    ("frac", {"head_dim": 256, "page_size": 32, "batch": 1, "seq_len_range": (700, 900), "num_q_heads": 8,
              "num_kv_heads": 2}, 33),
    # the smallest packed chunk: 3 tokens x G 6 = 18 rows, one partial tile
    ("l27b", {"seq_len": 1200, "recent_tokens": 256}, 3),
])
def test_packed_prefill_parity(name, over, chunk):
    C.say(f"packed prefill {name} {over} chunk={chunk}")
    w = W.scaled(W.WORKLOADS[name], **over)
    assert chunk * w.group > 16
    case = C.Case(w, seed=31)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    C.assert_pools_equal(lay, pools, f"{name} pools")
    q = _chunk_q(w, chunk, 7)
    O, L, _, _ = _prefill(case, lay, chunk, q)
    for b in range(w.batch):
        _check_request(case, pools, O, L, q, b, chunk, name)


def test_packed_prefill_route_counters_and_determinism():
    """Every visible (page, KV head) pair is counted once per format, and
    two calls give the same bits."""
    torch = C.torch_mod()
    m = C.kvq()
    C.say("packed prefill counters / determinism")
    w = W.scaled(W.WORKLOADS["serving"], batch=2, seq_len_range=(500, 900))
    case = C.Case(w, seed=5)
    lay = case.gpu_layer()
    chunk = 96
    q = _chunk_q(w, chunk, 3)
    bt, pf, sl = case.tables()
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    MP = bt.shape[1]
    plan = torch.zeros(m.paged_decode_plan_bytes(lay.cache, B, MP), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(m.paged_prefill_attn_workspace_size(lay.cache, B, Hq, chunk, MP), dtype=torch.uint8,
                     device="cuda")
    qd = torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).cuda().view(torch.bfloat16)
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan)
    outs = []
    ctr = torch.zeros(64, dtype=torch.uint8, device="cuda")
    for k in range(2):
        out = torch.full((B, chunk, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, chunk, Hq), float("nan"), dtype=torch.float32, device="cuda")
        m.paged_prefill_attn_planned(lay.cache, plan, qd, MP, w.sm_scale, out, lse, ws, ctr if k == 0 else None)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    cnt = m.read_counters(ctr)
    P = w.page_size
    for f, key in ((W.FMT_FP8, "pages_fp8"), (W.FMT_TQ3, "pages_tq3"), (W.FMT_TQ2, "pages_tq2")):
        # the last query row of a request sees all of its pages
        n = sum(int((case.plan.page_format[b, :(int(case.plan.seq_lens[b]) + P - 1) // P] == f).sum())
                for b in range(B))
        assert cnt[key] == w.num_kv_heads * n, key
    assert cnt["invalid_entries"] == 0


def test_packed_prefill_single_pool_needs_no_workspace():
    """A cache with one pool takes one launch and no workspace; a chunk of
    tokens on an all-FP8 cache matches the oracle."""
    m = C.kvq()
    C.say("packed prefill, FP8 only")
    w = W.scaled(W.WORKLOADS["tiny"], batch=2, seq_len=700, recent_tokens=4096, anchor_pages=0)
    case = C.Case(w, seed=2)
    assert set(f for f, n in case.plan.pool_pages.items() if n) == {W.FMT_FP8}
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    chunk = 70
    assert m.paged_prefill_attn_workspace_size(lay.cache, w.batch, w.num_q_heads, chunk, case.plan.max_pages) == 256
    q = _chunk_q(w, chunk, 11)
    O, L, _, _ = _prefill(case, lay, chunk, q)
    for b in range(w.batch):
        _check_request(case, pools, O, L, q, b, chunk, "fp8 only")


@pytest.mark.parametrize("name,chunk,heads,tokens", [
    # the full 2 x 59,008-token canary layer, a 4,096-token chunk in one call
    ("canary", 4096, [1], [0, 1531, 2047, 2048, 4095]),
    # the 64-request serving batch, a 256-token chunk per request
    ("serving", 256, [6], [0, 100, 255]),
])
def test_packed_prefill_full_size_sampled(name, chunk, heads, tokens):
    """At full size: every row finite, and sampled tokens of one KV head of
    the first and last request against the oracle (rebuilt for that head and
    those requests by the oracle's own encoders)."""
    C.say(f"packed prefill full size {name} chunk={chunk}")
    w = W.WORKLOADS[name]
    if w.layers > 1:
        w = W.scaled(w, layers=1)
    case = C.Case(w, seed=0)
    lay = case.gpu_layer()
    q = _chunk_q(w, chunk, 17)
    O, L, _, _ = _prefill(case, lay, chunk, q)
    assert np.isfinite(O).all()
    reqs = sorted({0, w.batch - 1})
    sample = C.Case(w, seed=0, heads=heads, requests=reqs)
    pools = sample.oracle_pools()
    for b in reqs:
        _check_request(sample, pools, O, L, q, b, chunk, f"{name} full size", heads=heads, tokens=tokens)
