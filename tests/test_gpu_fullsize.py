"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one plan, then the planned decode call of one layer), on
sampled outputs: the oracle rebuilds only the sampled KV heads (and, for the
serving batch, requests) with its own encoders and computes their outputs one
request at a time in fp64.

Sizes: the canary (2 x 59,008 tokens, Hkv 4, d 256, FP8 + TQ3 demoted from
FP8), the 70B-class layer (4 x 131,072 tokens, Hkv 8, d 128, page 32, FP8 +
grouped mixed-rate keys), the serving batch (64 requests, FP8 + TQ3 + TQ2)
and the fractional-level batch (16 requests, FP8 + TQF6 + TQF5 demoted from
FP8).
"""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


def _run(name, heads, requests, stale):
    torch = C.torch_mod()
    m = C.kvq()
    w = W.WORKLOADS[name]
    if w.layers > 1:
        w = W.scaled(w, layers=1)
    C.say(f"full size {name}: heads {heads}, requests {requests}, stale from {stale}")
    case = C.Case(w, seed=0, stale_source=stale, heads=heads, requests=requests)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    if requests is None:   # every page of the sampled heads was encoded by both sides
        C.assert_pools_equal(lay, pools, f"{name} pools", heads=heads, P=w.page_size, d=w.head_dim,
                             Hkv=w.num_kv_heads)
    bt, pf, sl = case.tables()
    B, Hq, MP = w.batch, w.num_q_heads, bt.shape[1]
    plan = torch.empty(m.paged_decode_plan_bytes(lay.cache, B, MP), dtype=torch.uint8, device="cuda")
    ws = torch.empty(m.paged_decode_attn_planned_workspace_size(lay.cache, B, Hq, MP), dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan)
    m.paged_decode_attn_planned(lay.cache, plan, case.q_dev(), MP, w.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    O, L = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    Oref, Lref = case.oracle_attention(pools, requests=requests)
    G = w.group
    rq = range(B) if requests is None else requests
    for b in rq:
        for g in heads:
            hs = slice(g * G, (g + 1) * G)
            C.assert_close(O[b, hs], Oref[b, hs], f"{name} O request {b} KV head {g}")
            C.assert_close(L[b, hs], Lref[b, hs], f"{name} lse request {b} KV head {g}")


def test_canary_full_size_sampled():
    _run("canary", heads=[3], requests=None, stale="fp8")


def test_70b_class_layer_full_size_sampled():
    _run("l70b", heads=[5], requests=[2], stale="fp8")


def test_serving_batch_full_size_sampled():
    _run("serving", heads=[1], requests=[0, 37, 63], stale="fp32")


def test_fractional_level_batch_full_size_sampled():
    _run("frac", heads=[6], requests=[0, 15], stale="fp8")
