"""The entry point that allocates nothing (paged_decode_attn_noalloc): its
workspace is the library's fixed per-GPU array. Checked through the C ABI
against paged_decode_attn with a caller-owned workspace (the same kernels and
work split, so the outputs must be bitwise equal) and against the oracle
(|gpu - ref| <= 2e-3 + 1e-2 |ref|), on two calls in a row, the second with a
smaller input, so the array holds the first call's contents when the second
one starts."""
import ctypes

import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


def _both(case, lay):
    torch = C.torch_mod()
    m = C.kvq()
    w = case.w
    bt, pf, sl = case.tables()
    q = case.q_dev()
    B, Hq, MP = w.batch, w.num_q_heads, bt.shape[1]
    out = torch.full((B, Hq, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    ctr = torch.zeros(ctypes.sizeof(m.Counters), dtype=torch.uint8, device="cuda")
    st = m.lib.paged_decode_attn_noalloc(ctypes.byref(lay.cache), m._ptr(q), B, Hq, m._ptr(bt), m._ptr(pf), MP,
                                         m._ptr(sl), ctypes.c_float(w.sm_scale), m._ptr(out), m._ptr(lse),
                                         m._ptr(ctr), m._stream())
    assert st == 0, m.lib.kvq_last_error()
    torch.cuda.synchronize()
    O_na, L_na = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    O_ws, L_ws = C.run_decode(case, lay)                   # paged_decode_attn, its own workspace
    return O_na, L_na, O_ws, L_ws, m.read_counters(ctr)


def test_noalloc_matches_the_workspace_call_twice_larger_then_smaller():
    C.say("no-alloc decode: canary-shaped call, then a smaller one")
    first = C.Case(W.scaled(W.WORKLOADS["canary"], layers=1, seq_len=5000, recent_tokens=512, anchor_pages=4),
                   seed=31, stale_source="fp8")
    second = C.Case(W.scaled(W.WORKLOADS["serving"], batch=3, seq_len_range=(20, 700)), seed=32)
    for case in (first, second):
        lay = case.gpu_layer()
        O_na, L_na, O_ws, L_ws, cnt = _both(case, lay)
        assert np.array_equal(O_na, O_ws) and np.array_equal(L_na, L_ws), case.w.name
        Oref, Lref = case.oracle_attention(case.oracle_pools())
        C.assert_close(O_na, Oref, f"{case.w.name} no-alloc O")
        C.assert_close(L_na, Lref, f"{case.w.name} no-alloc lse")
        assert cnt["invalid_entries"] == 0 and cnt["fallbacks"] == 0


def test_noalloc_refuses_a_workspace_beyond_its_array():
    """A geometry whose one-call workspace exceeds the fixed array is refused
    before any launch (KVQ_ERR_UNSUPPORTED)."""
    m = C.kvq()
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 8, 256, 16
    c.fp8_pages, c.fp8_num_pages = 4096, 8            # never dereferenced: the call stops on the host
    B, Hq, MP = 256, 128, 8192
    assert m.lib.paged_decode_attn_workspace_size(B, Hq, MP, ctypes.byref(c)) > (32 << 20)
    st = m.lib.paged_decode_attn_noalloc(ctypes.byref(c), 4096, B, Hq, 4096, 4096, MP, 4096, ctypes.c_float(0.1),
                                         4096, None, None, None)
    assert st == -2 and b"fixed array" in m.lib.kvq_last_error()
