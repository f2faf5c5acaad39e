"""The decode-step entry points inside a HIP graph: plan, chunked prefill,
scored decode, page-mass collector, decode with the fused append, plain
decode and promotion are captured once and replayed several times, with eager
work and synchronizations between replays; every replay must reproduce the
eager results bit for bit (the calls launch kernels only: no allocation, no
host synchronization, no memset nodes)."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


def test_step_entry_points_replay_in_a_graph():
    torch = C.torch_mod()
    m = C.kvq()
    C.say("graph capture of plan / prefill / scored / collect / append / planned / promote")
    w = W.scaled(W.WORKLOADS["l27b"], batch=2, seq_len=2000, recent_tokens=256)
    case = C.Case(w, seed=9)
    lay = case.gpu_layer()
    bt, pf, sl = case.tables()
    q = case.q_dev()
    B, Hq, d, P = w.batch, w.num_q_heads, w.head_dim, w.page_size
    max_pages = bt.shape[1]
    plan_buf = torch.zeros(m.paged_decode_plan_bytes(lay.cache, B, max_pages), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(m.paged_decode_attn_planned_workspace_size(lay.cache, B, Hq, max_pages), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda") for _ in range(3)]
    lses = [torch.zeros((B, Hq), dtype=torch.float32, device="cuda") for _ in range(3)]
    tlm = torch.zeros((B, Hq, max_pages, P // 16), dtype=torch.float32, device="cuda")
    a0 = torch.rand((B, max_pages), dtype=torch.float32, device="cuda")
    score = a0.clone()
    r = torch.zeros_like(score)
    used = set(int(x) for x in case.plan.block_table[case.plan.page_format == 0].ravel())
    free = [i for i in range(lay.pools[0].shape[0]) if i not in used]
    assert len(free) >= B + 2
    new_kv = torch.randn((B, w.num_kv_heads, 2, d), dtype=torch.float32, device="cuda")
    npg = torch.tensor(free[:B], dtype=torch.int32, device="cuda")
    nsl = torch.tensor([3, 0], dtype=torch.int32, device="cuda")
    tq_ids = [int(x) for x in case.plan.block_table[0][case.plan.page_format[0] == 1][:2]]
    psrc = torch.tensor(tq_ids, dtype=torch.int32, device="cuda")
    pdst = torch.tensor(free[B:B + 2], dtype=torch.int32, device="cuda")

    chunk = 16 // (Hq // w.num_kv_heads)
    qc = torch.randn((B, chunk, Hq, d), device="cuda").to(torch.bfloat16)
    outc = torch.zeros((B, chunk, Hq, d), dtype=torch.float32, device="cuda")
    lsec = torch.zeros((B, chunk, Hq), dtype=torch.float32, device="cuda")
    wsc = torch.zeros(m.paged_prefill_attn_workspace_size(lay.cache, B, Hq, chunk, max_pages), dtype=torch.uint8,
                      device="cuda")

    def step():
        m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf)
        m.paged_prefill_attn_planned(lay.cache, plan_buf, qc, max_pages, w.sm_scale, outc, lsec, wsc)
        m.paged_decode_attn_scored(lay.cache, plan_buf, q, max_pages, w.sm_scale, outs[0], lses[0], tlm, ws)
        m.page_mass_collect(sl, tlm, list(range(0, Hq, 3)), 0.8, score, r)
        m.paged_decode_attn_append(lay.cache, plan_buf, q, max_pages, w.sm_scale, new_kv, npg, nsl, outs[1],
                                   lses[1], ws)
        m.paged_decode_attn_planned(lay.cache, plan_buf, q, max_pages, w.sm_scale, outs[2], lses[2], ws)
        m.kv_promote_fp8(lay.cache, 1, psrc, pdst)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs + lses + [tlm, score, r, lay.pools[0], outc, lsec]]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        score.copy_(a0)
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    score.copy_(a0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for k in range(3):
        for t in outs + lses + [tlm, r, outc, lsec]:
            t.fill_(float("nan"))
        score.copy_(a0)
        junk = torch.randn(1 << 20, device="cuda").sum()          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outs + lses + [tlm, score, r, lay.pools[0], outc, lsec]
        names = ["out scored", "out append", "out planned", "lse scored", "lse append", "lse planned",
                 "tile log-mass", "score", "r", "FP8 pool", "out prefill", "lse prefill"]
        for name, a, b in zip(names, got, ref):
            assert torch.equal(a, b), f"replay {k}: {name} differs from the eager call"
        del junk
    # the three attention outputs: plain and scored agree; the append attends one more token
    assert torch.equal(outs[0], outs[2]) and not torch.equal(outs[1], outs[2])
