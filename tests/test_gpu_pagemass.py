"""GPU parity of the direct page-mass collector (Minima-KV Eq. 6-9): the scored
decode (paged_decode_attn_scored) and page_mass_collect against the oracle's
Eq. 6-8 page mass over format partitions and its Eq. 9 running score.

Tolerance: a page's mass is e^{lambda - lse}, so a score error ds in the
kernel (fp16 rotated query and codes on MFMA, fp32 accumulation; bounded by
the attention tolerance 2e-3 + 1e-2 |ref|) becomes a relative error of about
|ds| in q. Elementwise |gpu - ref| <= 1e-6 + 2e-2 ref on r and a, and the
r of each request sums to 1 within 1e-4."""
import numpy as np
import pytest

import workloads as W
from oracle import pagemass as PM
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

RATOL, RRTOL = 1e-6, 2e-2


def _scored(case, lay):
    torch = C.torch_mod()
    m = C.kvq()
    w = case.w
    bt, pf, sl = case.tables()
    q = case.q_dev()
    B, Hq, P = w.batch, w.num_q_heads, w.page_size
    max_pages = bt.shape[1]
    plan_buf = torch.zeros(m.paged_decode_plan_bytes(lay.cache, B, max_pages), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(m.paged_decode_attn_planned_workspace_size(lay.cache, B, Hq, max_pages), dtype=torch.uint8,
                     device="cuda")
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf)
    out = torch.full((B, Hq, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    tlm = torch.full((B, Hq, max_pages, P // 16), 123.0, dtype=torch.float32, device="cuda")
    m.paged_decode_attn_scored(lay.cache, plan_buf, q, max_pages, w.sm_scale, out, lse, tlm, ws)
    m.paged_decode_attn_planned(lay.cache, plan_buf, q, max_pages, w.sm_scale, out2, lse2, ws)
    torch.cuda.synchronize()
    return out, lse, out2, lse2, tlm, sl


@pytest.mark.parametrize("name,over,beta,heads", [
    ("tiny", {"seq_len": 1000}, 0.0, None),
    ("tiny", {"page_size": 32, "seq_len": 777}, 0.9, [0, 3]),
    ("l27b", {"seq_len": 3000, "recent_tokens": 512}, 0.5, [0, 7, 11, 23]),
    ("serving", {"batch": 4, "seq_len_range": (1, 900)}, 0.75, None),
    ("l70b", {"batch": 2, "seq_len": 1500, "recent_tokens": 256, "num_q_heads": 16, "num_kv_heads": 2}, 0.3,
     [1, 2, 15]),
    ("serving", {"head_dim": 256, "page_size": 32, "batch": 3, "seq_len_range": (200, 1800), "num_q_heads": 8,
                 "num_kv_heads": 2}, 0.6, None),
    ("l70b", {"page_size": 16, "batch": 2, "seq_len": 1100, "recent_tokens": 128, "num_q_heads": 16,
              "num_kv_heads": 2}, 0.4, [0, 9]),
    ("frac", {"batch": 3, "seq_len_range": (100, 1500)}, 0.5, None),
])
def test_scored_decode_and_collect(name, over, beta, heads):
    torch = C.torch_mod()
    m = C.kvq()
    C.say(f"page mass {name} {over} beta={beta} heads={heads}")
    w = W.scaled(W.WORKLOADS[name], **over)
    case = C.Case(w, seed=21)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    C.assert_pools_equal(lay, pools, f"{name} pools")
    out, lse, out2, lse2, tlm, sl = _scored(case, lay)
    # the scored call's attention is the plain call's, bit for bit
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "scored decode changed the attention output"
    Oref, lref = case.oracle_attention(pools)
    C.assert_close(out.cpu().numpy(), Oref, f"{name} O (scored)")
    # every tile the scan reaches is written, tiles past N_b are -inf, and
    # each head's normalized masses sum to 1
    t = tlm.cpu().numpy().astype(np.float64)
    P = w.page_size
    for b in range(w.batch):
        n_tiles = (int(case.plan.seq_lens[b]) + 15) // 16
        rows = t[b].reshape(w.num_q_heads, -1)
        assert np.all(np.isfinite(rows[:, :n_tiles])), f"request {b}"
        assert np.all(rows[:, n_tiles:] == -np.inf), f"request {b} tail"
        np.testing.assert_allclose(np.exp(rows).sum(axis=1), 1.0, atol=1e-5)
    Hq = w.num_q_heads
    hs = list(range(Hq)) if heads is None else heads
    rng = np.random.default_rng(5)
    a0 = rng.random((w.batch, case.plan.max_pages)).astype(np.float32)
    score = torch.from_numpy(a0.copy()).cuda()
    r = torch.full_like(score, float("nan"))
    m.page_mass_collect(sl, tlm, hs, beta, score, r)
    torch.cuda.synchronize()
    qref = PM.page_mass_ref(pools, case.plan.block_table, case.plan.page_format, case.plan.seq_lens, case.q,
                            w.sm_scale, P, w.num_kv_heads, w.head_dim, case.signs, tqk=case.tqk_rates)
    rref, aref = PM.collect_ref(qref, case.plan.seq_lens, P, hs, beta, a0.astype(np.float64))
    rg, ag = r.cpu().numpy().astype(np.float64), score.cpu().numpy().astype(np.float64)
    for what, got, ref in (("r", rg, rref), ("a", ag, aref)):
        err = np.abs(got - ref)
        bad = err > RATOL + RRTOL * np.abs(ref)
        assert not bad.any(), f"{name} {what}: {bad.sum()} pages off, worst {err.max():.3e} at " \
                              f"{np.unravel_index(err.argmax(), err.shape)}"
    for b in range(w.batch):
        if int(case.plan.seq_lens[b]) > 0:
            assert abs(rg[b].sum() - 1.0) < 1e-4, f"request {b}: r sums to {rg[b].sum()}"


def test_collect_on_an_empty_request_and_no_heads():
    torch = C.torch_mod()
    m = C.kvq()
    C.say("page mass: empty request, no heads")
    w = W.scaled(W.WORKLOADS["serving"], batch=3, seq_len_range=(100, 400))
    case = C.Case(w, seed=4)
    case.plan.seq_lens[1] = 0
    lay = case.gpu_layer()
    out, lse, _, _, tlm, sl = _scored(case, lay)
    assert np.all(lse.cpu().numpy()[1] == -np.inf)
    assert np.all(tlm.cpu().numpy()[1] == -np.inf)
    a0 = np.random.default_rng(1).random((w.batch, case.plan.max_pages)).astype(np.float32)
    score = torch.from_numpy(a0.copy()).cuda()
    r = torch.full_like(score, float("nan"))
    m.page_mass_collect(sl, tlm, list(range(w.num_q_heads)), 0.5, score, r)
    m.page_mass_collect(sl, tlm, [], 0.5, score)            # no head set: nothing changes
    torch.cuda.synchronize()
    ag, rg = score.cpu().numpy(), r.cpu().numpy()
    assert np.array_equal(ag[1], a0[1]) and np.all(rg[1] == 0)
    assert not np.isnan(rg).any()
    for b in (0, 2):
        assert abs(rg[b].sum() - 1.0) < 1e-4


@pytest.mark.parametrize("name,over", [
    ("canary", {"layers": 1}),
    # G = 16 with 385-page items: the tile log-mass stage takes the scan's LDS
    # past 64 KB
    ("l70b", {"batch": 2, "num_q_heads": 128}),
])
def test_scored_decode_full_size_properties(name, over):
    """At full size, in the benchmark's launch configuration: the scored call's
    attention equals the plain call's bit for bit, every live tile holds a
    finite ln q~, tiles past N_b hold -inf, and each head's q~ sum to 1."""
    torch = C.torch_mod()
    C.say(f"scored full size {name} {over}")
    w = W.scaled(W.WORKLOADS[name], **over)
    case = C.Case(w, seed=0)
    lay = case.gpu_layer()
    out, lse, out2, lse2, tlm, sl = _scored(case, lay)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "scored decode changed the attention output"
    t = tlm.cpu().numpy().astype(np.float64)
    for b in range(w.batch):
        n_tiles = (int(case.plan.seq_lens[b]) + 15) // 16
        rows = t[b].reshape(w.num_q_heads, -1)
        assert np.all(np.isfinite(rows[:, :n_tiles])), f"request {b}"
        assert np.all(rows[:, n_tiles:] == -np.inf), f"request {b} tail"
        np.testing.assert_allclose(np.exp(rows).sum(axis=1), 1.0, atol=1e-4)
    # sampled heads against the oracle's Eq. 6-8 page mass (one KV head of one
    # request, rebuilt by the oracle's own encoders)
    g, b = 1, w.batch - 1
    sample = C.Case(w, seed=0, heads=[g], requests=[b])
    pools = sample.oracle_pools()
    qref = PM.page_mass_ref(pools, case.plan.block_table, case.plan.page_format, case.plan.seq_lens, case.q,
                            w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, case.signs, tqk=case.tqk_rates,
                            requests=[b], heads=[g])
    G, P = w.group, w.page_size
    n_pages = (int(case.plan.seq_lens[b]) + P - 1) // P
    for h in range(g * G, (g + 1) * G):
        page_mass = np.exp(t[b, h]).sum(axis=1)[:n_pages]         # sum over a page's tiles of q~
        ref = qref[b, h, :n_pages] / qref[b, h, :n_pages].sum()
        err = np.abs(page_mass - ref)
        assert not (err > RATOL + RRTOL * ref).any(), f"{name} head {h}: worst {err.max():.3e}"
