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


def _f16_rounding_bound(pools, case, b, n0, qb, Oref, k_sigma=6.0):
    """First-order bound on |O_gpu - O_ref| from the scan's f16 operands, per
    element [C, Hq, d], for a chunk at positions n0 .. n0 + C - 1.

    The kernel rounds each element of the scaled rotated query and of a
    decoded key to f16 (unit roundoff u = 2^-11) before the MFMA; the d
    products' rounding errors are independent, so score j (log2 units) moves
    by delta_j with standard deviation c u |q| |k_j| sqrt(2 / (3 d)) (rotation
    keeps both norms), c = sm_scale log2 e. The softmax output then moves by
    ln 2 sum_j p_j delta_j (v_j - O), bounded here with k_sigma deviations per
    score, summed without cancellation, |v_j - O| taken exactly for the row's
    heaviest term and as |v_j| + |O| for the others. For ordinary keys this is below the
    fixed tolerance; for a key 40x louder than the rest it is what the f16
    operands cost while its weight is comparable to the others'."""
    w = case.w
    G, d, Hkv = w.group, w.head_dim, w.num_kv_heads
    chunk = qb.shape[0]
    K, V = OA.dequant_request(pools, case.plan.block_table[b], case.plan.page_format[b], n0 + chunk, w.page_size,
                              Hkv, d, case.signs, tqk=case.tqk_rates)
    qf = (np.asarray(qb, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    c = w.sm_scale * np.log2(np.e)
    sig = k_sigma * c * 2.0 ** -11 * np.sqrt(2.0 / (3.0 * d))
    hidden = np.arange(n0 + chunk)[None, None, :] > (n0 + np.arange(chunk))[:, None, None]
    out = np.zeros_like(Oref)
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        s = np.where(hidden, -np.inf, c * (qf[:, hs] @ K[:, g].T))
        p = np.exp2(s - s.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        wt = p * sig * np.linalg.norm(qf[:, hs], axis=-1)[..., None] * np.linalg.norm(K[:, g], axis=-1)
        Vg, Oh = V[:, g], Oref[:, hs]
        tri = wt @ np.abs(Vg) + np.abs(Oh) * wt.sum(-1, keepdims=True)
        # the row's heaviest key exactly: |v - O| is small where it dominates
        js = wt.argmax(-1)
        ws = np.take_along_axis(wt, js[..., None], -1)
        vs = Vg[js]
        out[:, hs] = np.log(2.0) * (tri - ws * (np.abs(vs) + np.abs(Oh)) + ws * np.abs(vs - Oh))
    return out


@pytest.mark.parametrize("name,over,chunk", [
    ("canary", {"layers": 1, "batch": 2, "seq_len": 2000, "recent_tokens": 512, "anchor_pages": 2}, 200),
    ("serving", {"batch": 2, "seq_len_range": (600, 900)}, 64),
    ("frac", {"batch": 2, "seq_len_range": (500, 800)}, 50),
    # grouped keys: their scan decodes the next step before computing the
    # current one, so its restart runs from a different point of the step
    ("l70b", {"batch": 2, "seq_len": 1500, "recent_tokens": 256, "num_q_heads": 16, "num_kv_heads": 2}, 100),
])
def test_packed_prefill_scores_past_the_reference(name, over, chunk):
    """One key per request made 40x louder, in the middle of its largest
    format run (even requests) or inside the chunk (odd ones): the scores of
    the rows that see it climb tens of log2 units past the reference each
    row took on its first pages, so the scans start again from their
    starting state with a larger one (Block-GTQ appendix H.5, online softmax
    over the prefix tiles). Tolerance: the fixed one plus the f16 operands'
    first-order bound, which only the rows that weigh the loud key raise."""
    C.say(f"packed prefill, climbing scores {name}")
    w = W.scaled(W.WORKLOADS[name], **over)
    case = C.Case(w, seed=13)
    for b in range(w.batch):
        K, V = case.kv(b)
        N = int(case.plan.seq_lens[b])
        assert N >= chunk
        if b % 2 == 0:
            t = C.loud_token(case.plan, b, w.page_size, C.request_formats(case.plan, b, w.page_size)[0])
        else:
            t = N - chunk // 2
        K[t] *= np.float32(40.0)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    q = _chunk_q(w, chunk, 19)
    O, L, _, _ = _prefill(case, lay, chunk, q)
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{name}: non-finite outputs"
    for b in range(w.batch):
        n0 = int(case.plan.seq_lens[b]) - chunk
        Oref, Lref = OP.prefill_ref(pools, case.plan.block_table[b], case.plan.page_format[b], n0, q[b], w.sm_scale,
                                    w.page_size, w.num_kv_heads, w.head_dim, case.signs, tqk=case.tqk_rates)
        extra = _f16_rounding_bound(pools, case, b, n0, q[b], Oref)
        C.assert_close(O[b], Oref, f"{name} climbing: request {b} O", atol=C.ATOL + extra)
        C.assert_close(L[b], Lref, f"{name} climbing: request {b} lse")
