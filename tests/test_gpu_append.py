"""GPU parity of the fused append (paged_decode_attn_append, Minima-KV
algorithm 1 "Append" inside the decode launch).

The GPU cache holds N_b tokens; the call attends N_b + 1 (the cached ones and
the step's new token) and writes the new token's FP8 codes. The oracle builds
its cache from all N_b + 1 tokens with its own encoders (FP8 codes are per
token, so appending one token leaves every other byte as it was): pools
bit-exact after the call, O and lse within 2e-3 + 1e-2 |ref| of its fp64
attention over N_b + 1 tokens."""
import numpy as np
import pytest

import workloads as W
from oracle import cache as OC
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over,bf16", [
    ("tiny", {"seq_len": 1000}, False),                     # slot 7 of the last page
    ("tiny", {"page_size": 32, "seq_len": 641}, True),     # the new token opens page 20 (slot 0)
    ("l27b", {"seq_len": 2050, "recent_tokens": 512}, False),
    ("l70b", {"batch": 2, "seq_len": 1501, "recent_tokens": 256, "num_q_heads": 16, "num_kv_heads": 2}, True),
    ("canary", {"layers": 1, "seq_len": 3001, "recent_tokens": 512, "anchor_pages": 3}, False),
    ("serving", {"head_dim": 256, "page_size": 32, "batch": 3, "seq_len_range": (300, 1500), "num_q_heads": 8,
                 "num_kv_heads": 2, "importance_split": None, "recent_tokens": 256}, True),
    ("l70b", {"page_size": 16, "batch": 2, "seq_len": 901, "recent_tokens": 128, "num_q_heads": 16,
              "num_kv_heads": 2}, False),
])
def test_fused_append(name, over, bf16):
    torch = C.torch_mod()
    m = C.kvq()
    C.say(f"fused append {name} {over} bf16={bf16}")
    w1 = W.scaled(W.WORKLOADS[name], **over)                 # the cache after the append: N_b + 1 tokens
    seed = 17
    plan1 = W.make_page_plan(w1, seed)
    N1 = plan1.seq_lens.copy()
    P = w1.page_size
    kv_full = {b: W.make_kv(w1, seed, 0, b, int(N1[b])) for b in range(w1.batch)}
    if bf16:
        # the new token's rows are bf16: the oracle appends their exact values
        for b in range(w1.batch):
            K, V = kv_full[b]
            for X in (K, V):
                X[-1] = (X[-1].view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    case = C.Case(w1, seed=seed, plan=W.PagePlan(N1 - 1, plan1.page_format, plan1.block_table,
                                                  dict(plan1.pool_pages), plan1.max_pages))
    case._kv = {b: (kv_full[b][0][:-1], kv_full[b][1][:-1]) for b in range(w1.batch)}
    lay = case.gpu_layer()                                    # N_b tokens
    new_page = np.array([plan1.block_table[b, (N1[b] - 1) // P] for b in range(w1.batch)], np.int32)
    new_slot = ((N1 - 1) % P).astype(np.int32)
    assert all(plan1.page_format[b, (N1[b] - 1) // P] == 0 for b in range(w1.batch)), "Recent pages are FP8"
    rows = np.stack([np.stack([kv_full[b][0][-1], kv_full[b][1][-1]], axis=1) for b in range(w1.batch)])
    new_kv = torch.from_numpy(rows).cuda()                    # [B, Hkv, 2, d]
    if bf16:
        new_kv = new_kv.to(torch.bfloat16)
    bt, pf, sl = case.tables()                               # seq_lens = N_b
    B, Hq, d = w1.batch, w1.num_q_heads, w1.head_dim
    max_pages = bt.shape[1]
    plan_buf = torch.zeros(m.paged_decode_plan_bytes(lay.cache, B, max_pages), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(m.paged_decode_attn_planned_workspace_size(lay.cache, B, Hq, max_pages), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf)
    m.paged_decode_attn_append(lay.cache, plan_buf, case.q_dev(), max_pages, w1.sm_scale, new_kv,
                               torch.from_numpy(new_page).cuda(), torch.from_numpy(new_slot).cuda(), out, lse, ws)
    torch.cuda.synchronize()
    pools1 = OC.build_pools(w1, plan1, lambda b: kv_full[b], case.signs, tqk=case.tqk_rates)
    C.assert_pools_equal(lay, pools1, f"{name} pools after the fused append")
    ref = C.Case(w1, seed=seed, plan=plan1)
    ref._kv = kv_full
    Oref, lref = ref.oracle_attention(pools1)
    C.assert_close(out.cpu().numpy(), Oref, f"{name} O with the new token")
    C.assert_close(lse.cpu().numpy(), lref, f"{name} lse with the new token")


def test_fused_append_on_an_empty_cache_and_a_bad_slot():
    """N_b = 0: the output is the new token's decoded V and lse its score; a
    slot out of range is counted and not written, and the token still counts."""
    torch = C.torch_mod()
    m = C.kvq()
    from oracle import fp8 as OF
    from quantized_paged_kv_mixed_amd.paged import GpuLayer
    C.say("fused append: empty cache, bad slot")
    w = W.WORKLOADS["tiny"]
    Hkv, d, P, Hq = w.num_kv_heads, w.head_dim, w.page_size, w.num_q_heads
    lay = GpuLayer(Hkv, d, P, {0: 2}, W.make_signs(w, 0, 0))
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((2, Hkv, 2, d)).astype(np.float32)
    q = W.make_q(W.scaled(w, batch=2), 0, 0)
    bt = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    pf = torch.zeros((2, 1), dtype=torch.uint8, device="cuda")
    sl = torch.zeros(2, dtype=torch.int32, device="cuda")
    plan_buf = torch.zeros(m.paged_decode_plan_bytes(lay.cache, 2, 1), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(m.paged_decode_attn_planned_workspace_size(lay.cache, 2, Hq, 1), dtype=torch.uint8, device="cuda")
    cnt = torch.zeros(m.ctypes.sizeof(m.Counters), dtype=torch.uint8, device="cuda")
    out = torch.full((2, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((2, Hq), float("nan"), dtype=torch.float32, device="cuda")
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf)
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    m.paged_decode_attn_append(lay.cache, plan_buf, qd, 1, w.sm_scale, torch.from_numpy(rows).cuda(),
                               torch.tensor([1, 0], dtype=torch.int32, device="cuda"),
                               torch.tensor([5, P], dtype=torch.int32, device="cuda"), out, lse, ws, cnt)
    torch.cuda.synchronize()
    assert m.read_counters(cnt)["invalid_entries"] == 1
    pool = lay.pool_bytes(0)
    assert not pool[0].any(), "the bad slot must not be written"
    Kp = np.zeros((P, Hkv, d), np.float32)
    Vp = np.zeros((P, Hkv, d), np.float32)
    Kp[5], Vp[5] = rows[0, :, 0], rows[0, :, 1]
    C._cmp(pool[1], OC.encode_page(0, Kp, Vp, P, None), "page 1 after the append into slot 5")
    G = Hq // Hkv
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for b in range(2):
        kc, ks = OF.fp8_encode(rows[b, :, 0])
        vc, vs = OF.fp8_encode(rows[b, :, 1])
        khat, vhat = OF.fp8_decode(kc, ks), OF.fp8_decode(vc, vs)
        for h in range(Hq):
            C.assert_close(out.cpu().numpy()[b, h], vhat[h // G], f"request {b} head {h} O")
            s = w.sm_scale * float(qf[b, h] @ khat[h // G])
            C.assert_close(lse.cpu().numpy()[b, h], s, f"request {b} head {h} lse")
