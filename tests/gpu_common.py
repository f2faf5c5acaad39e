"""Shared pieces of the GPU parity tests: build the same cache twice (the
oracle on the CPU, the HIP encoders on the GPU) from the same seeded rows."""
import os
import sys

import numpy as np

import workloads as W
from oracle import attention as A
from oracle import cache as OC

ATOL, RTOL = 2e-3, 1e-2   # |gpu - ref| <= ATOL + RTOL * |ref| (elementwise)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def kvq():
    import quantized_paged_kv_mixed_amd as m
    return m


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


class Case:
    """A workload instance: plan, rows, signs, q, and both caches."""

    def __init__(self, w, seed=0, layer=0, stale_source="fp32", requests=None, heads=None, plan=None):
        self.w, self.seed, self.layer = w, seed, layer
        self.plan = plan if plan is not None else W.make_page_plan(w, seed)
        self.signs = W.make_signs(w, seed, layer)
        self.q = W.make_q(w, seed, layer)
        self.stale_source = stale_source
        # grouped mixed-rate keys: block widths for the oracle, coordinate order for the library
        self.tqk_rates = W.make_tqk_rates(w, seed, layer) if w.tqk_rates else None
        self.tqk_perm = W.make_tqk_perm(w, seed, layer) if w.tqk_rates else None
        self._kv = {}
        self.requests, self.heads = requests, heads

    def kv(self, b):
        if b not in self._kv:
            n = int(self.plan.seq_lens[b])
            self._kv[b] = W.make_kv(self.w, self.seed, self.layer, b, n)
        return self._kv[b]

    def oracle_pools(self):
        return OC.build_pools(self.w, self.plan, self.kv, self.signs, self.stale_source, tqk=self.tqk_rates,
                              requests=self.requests, heads=self.heads)

    def gpu_layer(self):
        torch = torch_mod()
        from quantized_paged_kv_mixed_amd.paged import GpuLayer, build_layer
        w = self.w
        lay = GpuLayer(w.num_kv_heads, w.head_dim, w.page_size, self.plan.pool_pages, self.signs,
                       tqk_perm=self.tqk_perm)

        def kv_dev(b):
            K, V = self.kv(b)
            return torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()

        build_layer(lay, self.plan.page_format, self.plan.block_table, self.plan.seq_lens, kv_dev,
                    stale_source=self.stale_source)
        torch.cuda.synchronize()
        return lay

    def tables(self):
        torch = torch_mod()
        return (torch.from_numpy(self.plan.block_table).cuda(), torch.from_numpy(self.plan.page_format).cuda(),
                torch.from_numpy(self.plan.seq_lens).cuda())

    def q_dev(self):
        torch = torch_mod()
        return torch.from_numpy(self.q.view(np.int16)).cuda().view(torch.bfloat16)

    def oracle_attention(self, pools, requests=None):
        w = self.w
        return A.paged_decode_ref(pools, self.plan.block_table, self.plan.page_format, self.plan.seq_lens,
                                  self.q, w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, self.signs,
                                  requests=requests, tqk=self.tqk_rates, heads=self.heads)


def request_formats(plan, b, P):
    """The formats of request b's pages, with their page counts, largest first."""
    n = int(plan.seq_lens[b])
    f, c = np.unique(plan.page_format[b, :(n + P - 1) // P], return_counts=True)
    order = np.argsort(-c, kind="stable")
    return [int(x) for x in f[order]]


def loud_token(plan, b, P, fmt):
    """A token of the middle page of request b's pages of format fmt (at the
    page's middle offset, or the request's last token when that is earlier)."""
    n = int(plan.seq_lens[b])
    pages = np.flatnonzero(plan.page_format[b, :(n + P - 1) // P] == fmt)
    pg = int(pages[len(pages) // 2])
    return min(pg * P + P // 2, n - 1)


def run_decode(case, lay, oneshot=True, counters=None, out=None, lse=None, plan_buf=None, ws=None):
    torch = torch_mod()
    m = kvq()
    w = case.w
    bt, pf, sl = case.tables()
    q = case.q_dev()
    B, Hq = w.batch, w.num_q_heads
    max_pages = bt.shape[1]
    if out is None:
        out = torch.full((B, Hq, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    if lse is None:
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    if oneshot:
        n = m.paged_decode_attn_workspace_size(lay.cache, B, Hq, max_pages)
        if ws is None:
            ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        m.paged_decode_attn(lay.cache, q, bt, pf, sl, w.sm_scale, out, lse, ws, counters)
    else:
        if plan_buf is None:
            plan_buf = torch.zeros(m.paged_decode_plan_bytes(lay.cache, B, max_pages), dtype=torch.uint8,
                                   device="cuda")
        m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf, counters)
        if ws is None:
            ws = torch.zeros(m.paged_decode_attn_planned_workspace_size(lay.cache, B, Hq, max_pages), dtype=torch.uint8,
                             device="cuda")
        m.paged_decode_attn_planned(lay.cache, plan_buf, q, max_pages, w.sm_scale, out, lse, ws, counters)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def assert_close(got, ref, what, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(ref) & (got == ref)
    err = np.abs(got - ref)
    bad = ~both_inf & ~(err <= atol + rtol * np.abs(ref))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {got[tuple(i)]:.6g} ref {ref[tuple(i)]:.6g}" for i in idx)
        tol = f"{atol}" if np.isscalar(atol) else f"[{np.min(atol):.3g}, {np.max(atol):.3g}]"
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside |d| <= {tol} + {rtol}|ref|; "
                             f"max |d| {np.nanmax(np.where(both_inf, 0, err)):.3g}; {detail}")


def assert_pools_equal(gpu_layer, pools, what, heads=None, P=None, d=None, Hkv=None):
    from oracle.attention import head_block_bytes
    for f, ref in pools.items():
        got = gpu_layer.pool_bytes(f)
        assert got is not None and got.shape == ref.shape, f"{what}: pool {f} shape"
        if heads is not None:
            hb = head_block_bytes(f, P, d)
            for g in heads:
                a = got[:, g * hb:(g + 1) * hb]
                b = ref[:, g * hb:(g + 1) * hb]
                _cmp(a, b, f"{what} fmt {f} head {g}")
        else:
            _cmp(got, ref, f"{what} fmt {f}")


def _cmp(a, b, what):
    if not np.array_equal(a, b):
        diff = np.argwhere(a != b)
        raise AssertionError(f"{what}: {len(diff)} bytes differ, first at {diff[:4].tolist()} "
                             f"gpu {a[tuple(diff[0])]:#x} oracle {b[tuple(diff[0])]:#x}")
