"""Benchmark: mixed-format paged decode attention on one MI355X.

Workload (default "canary"): 2 requests x 59,008 cached tokens, 16
full-attention layers (Hq=24, Hkv=4, d=256), page 16 tokens; per request the
last 2,048 tokens and 8 Anchor pages (page 0 + 7 seeded) are FP8 E4M3 with
fp32 per-vector scales, every other page is TQ3. Shape from the Minima-KV
page, section 6.3 (the 2 x 59,008-token direct canary on the 16 full-attention
layers of a 4 KV-head, 256-dim model); inputs are seeded N(0,1) stand-ins.

Other workloads (--workload): l70b (grouped mixed-rate keys, d=128, page 32),
serving (64 ragged requests, FP8/TQ3/TQ2), l27b, tiny.

Setup (timed with HIP events, reported as encode tokens/s):
  * FP8 append (kv_encode_fp8) of every token of every layer;
  * demotion of every Stale page from FP8 (kv_encode_tq3 / _tq2 / _tqk).
Timed step: one decode step of the model's attention = paged_decode_plan
(format partition of the page table, shared by all layers) followed by one
paged_decode_attn_planned call per layer (16 for the canary), replayed as one
HIP graph.

Output: one JSON line on stdout. `value` is decode-attention KV GB/s over
the whole step (algorithmic KV bytes of the 16 layers / step time);
`roofline` prices the decode kernel alone (per-launch HIP-event durations);
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 / bf16 MFMA, published
# algorithmic bytes per (token, KV head): FP8, TQ3, TQ2, TQK (grouped keys + TQ3 values)
FMT_BYTES = {0: lambda d: 2 * d + 8, 1: lambda d: 2 * (3 * d // 8 + 2), 2: lambda d: 2 * (d // 4 + 2),
             3: lambda d: 2 * (3 * d // 8) + 8}
FMT_NAMES = {0: "FP8", 1: "TQ3", 2: "TQ2", 3: "TQK"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kv_bytes_per_layer(w, plan) -> int:
    """Algorithmic KV bytes one decode of one layer must read: per (token, KV
    head) 2d + 8 for FP8, 2 (3d/8 + 2) for TQ3, 2 (d/4 + 2) for TQ2 and
    2 (3d/8) + 8 for grouped keys (three K sigmas, one V sigma)."""
    total = 0
    for b in range(w.batch):
        N = int(plan.seq_lens[b])
        n_pages = (N + w.page_size - 1) // w.page_size
        for p in range(n_pages):
            toks = min(w.page_size, N - p * w.page_size)
            total += toks * w.num_kv_heads * FMT_BYTES[int(plan.page_format[b, p])](w.head_dim)
    return total


def build_layer(torch, m, w, plan, seed, layer, stage_pool):
    """Encode one layer's cache with the library's encoders: FP8 append of
    the Recent / Anchor tokens, and for every Stale page an FP8 append into a
    staging page followed by its demotion (TQ3, TQ2 or grouped keys). Returns
    the layer and the event-timed encode figures."""
    from quantized_paged_kv_mixed_amd import paged as PG
    P, Hkv, d, B = w.page_size, w.num_kv_heads, w.head_dim, w.batch
    signs = W.make_signs(w, seed, layer)
    perm = W.make_tqk_perm(w, seed, layer) if w.tqk_rates else None
    lay = PG.GpuLayer(Hkv, d, P, dict(plan.pool_pages), signs, tqk_perm=perm)
    stage_cache = m.make_cache(Hkv, d, P, stage_pool, None, None, lay.signs)
    demote_cache = m.make_cache(Hkv, d, P, stage_pool, lay.pools.get(1), lay.pools.get(2), lay.signs,
                                lay.pools.get(3), lay.perm)
    encoders = {1: m.kv_encode_tq3, 2: m.kv_encode_tq2, 3: m.kv_encode_tqk}
    t_fp8 = t_dem = 0.0
    n_fp8 = n_dem = 0
    b_fp8 = b_dem = 0          # algorithmic bytes: rows read + codes / scales written
    for b in range(B):
        N = int(plan.seq_lens[b])
        n_pages = (N + P - 1) // P
        K, V = W.make_kv(w, seed, layer, b, N)
        src_all = torch.from_numpy(np.stack([K, V], axis=2)).cuda()        # [N, Hkv, 2, d]
        del K, V
        fmt = plan.page_format[b, :n_pages]
        pid = plan.block_table[b, :n_pages]
        tok = np.arange(N)
        page_of = tok // P
        is_fp8 = fmt[page_of] == 0
        t8 = np.nonzero(is_fp8)[0]
        stale_pages = np.nonzero(fmt != 0)[0]
        ts = np.nonzero(~is_fp8)[0]
        stage_id = np.full(n_pages, -1, np.int64)
        stage_id[stale_pages] = np.arange(len(stale_pages))
        assert len(stale_pages) <= stage_pool.shape[0]
        jobs = [(lay.cache, t8, pid[page_of[t8]]), (stage_cache, ts, stage_id[page_of[ts]])]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for cache, toks, dpage in jobs:
            if len(toks) == 0:
                continue
            src = src_all[torch.from_numpy(toks).cuda()].contiguous()
            dp = torch.from_numpy(dpage.astype(np.int32)).cuda()
            ds = torch.from_numpy((toks % P).astype(np.int32)).cuda()
            e0.record()
            m.kv_encode_fp8(cache, src, dp, ds)
            e1.record()
            torch.cuda.synchronize()
            t_fp8 += e0.elapsed_time(e1) * 1e-3
            n_fp8 += len(toks)
            b_fp8 += len(toks) * Hkv * 2 * (4 * d + d + 4)
            del src
        for f, enc in encoders.items():
            pages = np.nonzero(fmt == f)[0]
            if not len(pages):
                continue
            sp = torch.from_numpy(stage_id[pages].astype(np.int32)).cuda()
            dp = torch.from_numpy(pid[pages].astype(np.int32)).cuda()
            valid = torch.from_numpy(np.minimum(P, N - pages * P).astype(np.int32)).cuda()
            e0.record()
            enc(demote_cache, m.SRC_FP8_PAGES, dp, src_page=sp, page_valid=valid)
            e1.record()
            torch.cuda.synchronize()
            t_dem += e0.elapsed_time(e1) * 1e-3
            nv = int(valid.sum().item())
            n_dem += nv
            b_dem += nv * Hkv * 2 * (d + 4) + len(pages) * m.page_bytes(f, Hkv, d, P)
        del src_all
    return lay, (n_fp8, t_fp8, n_dem, t_dem, b_fp8, b_dem)


def time_promote(torch, m, w, lay, plan, max_pages=4096, reps=5):
    """Promotion (kv_promote_fp8) of up to max_pages pages of each compressed
    pool of one layer into a scratch FP8 pool, HIP-event timed (mean of reps
    calls after one warm call): tokens per second, a token being all KV heads
    and both roles of one slot."""
    res = {}
    for f in (1, 2, 3):
        pool = lay.pools.get(f)
        if pool is None:
            continue
        n = int(min(max_pages, pool.shape[0]))
        scratch = torch.zeros((n, m.page_bytes(0, w.num_kv_heads, w.head_dim, w.page_size)), dtype=torch.uint8,
                              device="cuda")
        cache = m.make_cache(w.num_kv_heads, w.head_dim, w.page_size, scratch, lay.pools.get(1), lay.pools.get(2),
                             lay.signs, lay.pools.get(3), lay.perm)
        src = torch.arange(n, dtype=torch.int32, device="cuda")
        dst = torch.randperm(n, device="cuda").to(torch.int32)
        m.kv_promote_fp8(cache, f, src, dst)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            m.kv_promote_fp8(cache, f, src, dst)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        name = FMT_NAMES[f].lower()
        res[f"{name}_promote_tokens_per_s"] = round(n * w.page_size / t, 1)
        res[f"{name}_promote_pages"] = n
        moved = n * (m.page_bytes(f, w.num_kv_heads, w.head_dim, w.page_size) +
                     m.page_bytes(0, w.num_kv_heads, w.head_dim, w.page_size))
        res[f"{name}_promote_roofline"] = {"bound": "hbm", "bytes_per_page": moved // n,
                                            "achieved_GBps": round(moved / t / 1e9, 1),
                                            "frac": round(moved / t / 1e9 / HBM_PEAK_GBPS, 4)}
        del scratch
    return res


def time_entry_points(torch, m, w, lay, plan, plan_buf, q, bt, pf, sl, ws, reps=20):
    """One layer's scored decode (attention plus the tile log-mass of the
    page-mass collector), the collector itself over all q-heads, and the
    decode with the step's new token appended in the same launch (against an
    append launch followed by the plain call), each HIP-event timed over reps
    calls; the plain call's mean is the reference."""
    B, Hq, max_pages = w.batch, w.num_q_heads, plan.max_pages
    out = torch.empty((B, Hq, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    tlm = torch.empty((B, Hq, max_pages, w.page_size // 16), dtype=torch.float32, device="cuda")
    score = torch.zeros((B, max_pages), dtype=torch.float32, device="cuda")
    heads = list(range(Hq))
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    m.paged_decode_attn_scored(lay.cache, plan_buf, q, max_pages, w.sm_scale, out, lse, tlm, ws)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        m.paged_decode_attn_scored(lay.cache, plan_buf, q, max_pages, w.sm_scale, out, lse, tlm, ws)
    ev[1].record()
    for _ in range(reps):
        m.page_mass_collect(sl, tlm, heads, 0.9, score)
    ev[2].record()
    for _ in range(reps):
        m.paged_decode_attn_planned(lay.cache, plan_buf, q, max_pages, w.sm_scale, out, lse, ws)
    ev[3].record()
    torch.cuda.synchronize()
    us = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / reps for i in range(3)]
    res = {"scored_call_us": round(us[0], 2), "collect_us": round(us[1], 2), "plain_call_us": round(us[2], 2),
           "heads": Hq}
    # chunked prefill: each request's last C = 16 / G cached tokens as one
    # chunk (C x G rows share every tile), against the plain decode call
    G = Hq // w.num_kv_heads
    chunk = max(1, 16 // G)
    if chunk > 1:
        qc = torch.randn((B, chunk, Hq, w.head_dim), device="cuda").to(torch.bfloat16)
        outc = torch.empty((B, chunk, Hq, w.head_dim), dtype=torch.float32, device="cuda")
        lsec = torch.empty((B, chunk, Hq), dtype=torch.float32, device="cuda")
        wsc = torch.empty(m.paged_prefill_attn_workspace_size(lay.cache, B, Hq, chunk, max_pages), dtype=torch.uint8,
                          device="cuda")
        m.paged_prefill_attn_planned(lay.cache, plan_buf, qc, max_pages, w.sm_scale, outc, lsec, wsc)
        torch.cuda.synchronize()
        evp = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        evp[0].record()
        for _ in range(reps):
            m.paged_prefill_attn_planned(lay.cache, plan_buf, qc, max_pages, w.sm_scale, outc, lsec, wsc)
        evp[1].record()
        torch.cuda.synchronize()
        t = evp[0].elapsed_time(evp[1]) * 1e-3 / reps
        res["prefill_chunk"] = chunk
        res["prefill_call_us"] = round(t * 1e6, 2)
        res["prefill_tokens_per_s"] = round(B * chunk / t, 1)
    # the step's new token: fused into the decode launch, or appended by its
    # own launch before the plain call (into a free FP8 page, slot 0)
    used = set(int(x) for x in plan.block_table[plan.page_format == 0].ravel())
    free = [i for i in range(lay.pools[0].shape[0]) if i not in used]
    if len(free) >= B:
        new_kv = torch.randn((B, w.num_kv_heads, 2, w.head_dim), dtype=torch.float32, device="cuda")
        npg = torch.tensor(free[:B], dtype=torch.int32, device="cuda")
        nsl = torch.zeros(B, dtype=torch.int32, device="cuda")
        ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        m.paged_decode_attn_append(lay.cache, plan_buf, q, max_pages, w.sm_scale, new_kv, npg, nsl, out, lse, ws)
        torch.cuda.synchronize()
        ev2[0].record()
        for _ in range(reps):
            m.paged_decode_attn_append(lay.cache, plan_buf, q, max_pages, w.sm_scale, new_kv, npg, nsl, out, lse,
                                       ws)
        ev2[1].record()
        for _ in range(reps):
            m.kv_encode_fp8(lay.cache, new_kv, npg, nsl)
            m.paged_decode_attn_planned(lay.cache, plan_buf, q, max_pages, w.sm_scale, out, lse, ws)
        ev2[2].record()
        torch.cuda.synchronize()
        res["fused_append_call_us"] = round(ev2[0].elapsed_time(ev2[1]) * 1e3 / reps, 2)
        res["append_then_call_us"] = round(ev2[1].elapsed_time(ev2[2]) * 1e3 / reps, 2)
    return res


def time_packed_prefill(torch, m, w, lay, plan, plan_buf, chunk=8192, reps=3):
    """One layer's packed chunked prefill (Block-GTQ appendix H.5: the prompt
    goes through one layer at a time in 8192-token chunks): each request's
    last `chunk` cached tokens as the chunk, causal over everything before
    them, HIP-event timed over reps calls. Work: every visible (key, q-head)
    pair costs 2 d flops for QK^T and 2 d for PV on MFMA (f16 operands), so
    the roofline is dense fp16 MFMA."""
    B, Hq, d, max_pages = w.batch, w.num_q_heads, w.head_dim, plan.max_pages
    chunk = int(min(chunk, int(plan.seq_lens.min())))
    qc = torch.randn((B, chunk, Hq, d), device="cuda").to(torch.bfloat16)
    outc = torch.empty((B, chunk, Hq, d), dtype=torch.float32, device="cuda")
    lsec = torch.empty((B, chunk, Hq), dtype=torch.float32, device="cuda")
    wsc = torch.empty(m.paged_prefill_attn_workspace_size(lay.cache, B, Hq, chunk, max_pages), dtype=torch.uint8,
                      device="cuda")
    m.paged_prefill_attn_planned(lay.cache, plan_buf, qc, max_pages, w.sm_scale, outc, lsec, wsc)
    torch.cuda.synchronize()
    assert torch.isfinite(outc).all(), "packed prefill produced non-finite outputs"
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        m.paged_prefill_attn_planned(lay.cache, plan_buf, qc, max_pages, w.sm_scale, outc, lsec, wsc)
    ev[1].record()
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
    keys = 0
    for b in range(B):
        n0 = int(plan.seq_lens[b]) - chunk
        keys += chunk * n0 + chunk * (chunk + 1) // 2
    flops = keys * Hq * 4 * d
    tf = flops / t / 1e12
    fmts = [f for f in (1, 2, 3, 0) if (plan.page_format == f).any()]
    return {"chunk": chunk, "requests": B, "call_ms": round(t * 1e3, 3),
            "tokens_per_s": round(B * chunk / t, 1), "launches": len(fmts),
            "roofline": {"bound": "mfma", "kernel": f"prefill_kernel<{d}, fmt> (one launch per pool format)",
                         "achieved": round(tf, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "flops_per_call": int(flops),
                         "traffic": None}}


def ctypes_sizeof_counters(m):
    import ctypes
    return ctypes.sizeof(m.Counters)


def rate_accounting(w, plan, pools_bytes):
    """Rates of the cache as configured (Minima-KV Eq. 10; Block-GTQ appendix
    B.1's logical rate, effective rate and physical footprint), per layer.
    A scalar is one coordinate of one K or V vector of one live token."""
    d, H, P = w.head_dim, w.num_kv_heads, w.page_size
    tok = {f: 0 for f in FMT_NAMES}
    for b in range(w.batch):
        N = int(plan.seq_lens[b])
        for p in range((N + P - 1) // P):
            tok[int(plan.page_format[b, p])] += min(P, N - p * P)
    n = sum(tok.values())
    payload_bits = {0: 8.0, 1: 3.0, 2: 2.0, 3: 3.0}          # code bits per scalar (TQK keys average 3.0)
    frac = {f: tok[f] / n for f in tok}
    logical = sum(frac[f] * payload_bits[f] for f in tok)   # Eq. 10 with b_meta = 0
    eff_bytes = sum(tok[f] * H * FMT_BYTES[f](d) for f in tok)
    effective = 8.0 * eff_bytes / (n * H * 2 * d)
    bf16_bytes = n * H * 2 * d * 2
    return {
        "token_fraction": {FMT_NAMES[f].lower(): round(frac[f], 6) for f in tok if tok[f]},
        "b_eff_eq10_bits": round(logical, 4), "C_BF16_eq10": round(16.0 / logical, 4),
        "effective_rate_bits": round(effective, 4), "C_BF16_effective": round(16.0 / effective, 4),
        "compression_vs_bf16_bytes": round(bf16_bytes / eff_bytes, 4),
        "compression_vs_fp8_bytes": round((bf16_bytes / 2) / eff_bytes, 4),
        "kv_bytes_per_token_all_layers": round(eff_bytes * w.layers / n, 1),
        "physical_pool_bytes_per_layer": int(pools_bytes),
        "physical_bytes_per_token_all_layers": round(pools_bytes * w.layers / n, 1),
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def decode_source_hash():
    """Hash of the sources that fix a decode call's kernels and work split
    (the scan/merge kernels and the item sizing)."""
    import hashlib
    h = hashlib.sha256()
    for part in ("decode.hip", "kvq_internal.h"):
        h.update(open(os.path.join(ROOT, "quantized_paged_kv_mixed_amd", "csrc", part), "rb").read())
    return h.hexdigest()[:16]


def scan_kernel_name(d):
    """The scan kernel of a plain decode call (its merge kernel follows)."""
    return f"decode_kernel<{d}, false, false>"


def measured_traffic(workload, d):
    """(scan kernel HBM bytes per launch, call bytes, counter GB/s of the scan
    kernel, its rocprofv3 average) from the committed counter summary, only
    if it was taken on the current decode source (else Nones)."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    none = (None, None, None, None)
    try:
        rec = json.load(open(path))
        h = decode_source_hash()
    except (OSError, ValueError):
        return none
    if rec.get("decode_source_sha256_16") != h:
        return none
    k = rec.get("kernels", {}).get(scan_kernel_name(d), {})
    scan = sum(k[c]["bytes"] for c in ("FETCH_SIZE", "WRITE_SIZE") if c in k) or None
    return (None if scan is None else int(round(scan)), int(round(rec["decode_call_hbm_bytes"])),
            k.get("counter_GBps"), k.get("trace_average_us"))


def cpu_baseline(w, plan, seed, token_heads=240_000):
    """The oracle (as it stands) on a bounded sample of the same workload:
    request 0 of layer 0 with every cached token and the workload's own
    page-format mix, for the first KV heads (as many as keep tokens x heads
    near `token_heads`) and their q-heads. The oracle builds that cache with
    its own encoders (FP8 append, demotion from FP8; reported, not the value);
    its fp64 decode is the value."""
    from threadpoolctl import threadpool_info
    from oracle import attention as OA
    from oracle import cache as OC
    P = w.page_size
    N = int(plan.seq_lens[0])
    n_pages = (N + P - 1) // P
    H = int(min(w.num_kv_heads, max(1, token_heads // max(N, 1))))
    w1 = W.scaled(w, batch=1, num_kv_heads=H, num_q_heads=w.group * H)
    sub = W.PagePlan(plan.seq_lens[:1].copy(), plan.page_format[:1, :n_pages].copy(),
                     plan.block_table[:1, :n_pages].copy(), dict(plan.pool_pages), n_pages)
    K, V = W.make_kv(w, seed, 0, 0, N)
    K, V = np.ascontiguousarray(K[:, :H]), np.ascontiguousarray(V[:, :H])
    signs = W.make_signs(w, seed, 0)[:H]
    rates = W.make_tqk_rates(w, seed, 0)[:H] if w.tqk_rates else None
    t0 = time.perf_counter()
    pools = OC.build_pools(w1, sub, lambda b: (K, V), signs, "fp8", tqk=rates)
    t_build = time.perf_counter() - t0
    q = W.make_q(w, seed, 0)[:1, :w.group * H]
    t0 = time.perf_counter()
    OA.paged_decode_ref(pools, sub.block_table, sub.page_format, sub.seq_lens, q, w.sm_scale, P, H,
                        w.head_dim, signs, tqk=rates)
    t_dec = time.perf_counter() - t0
    nbytes = kv_bytes_per_layer(w1, sub)
    threads = [i.get("num_threads", 1) for i in threadpool_info()]
    return {
        "value": round(nbytes / t_dec / 1e9, 5), "unit": "GB/s", "cores": int(max(threads) if threads else 1),
        "kind": "oracle",
        "sample": f"oracle fp64 decode of request 0, layer 0, KV heads 0..{H - 1} with their {w.group * H} "
                  f"q-heads over all {N} tokens ({nbytes} algorithmic KV bytes) in {t_dec:.2f} s; the oracle "
                  f"encoders built that cache (FP8 append + demotion) in {t_build:.1f} s = "
                  f"{N * H / t_build:.0f} token-heads/s",
        "cpu_model": cpu_model(),
        "os_cpu_count": os.cpu_count(),
        **l27b_oracle_decode(seed),
    }


def l27b_oracle_decode(seed):
    """The oracle's fp64 decode of the 27B-layer shape (1 x 16,384 tokens, 4
    KV heads x 256, 24 q-heads, FP8 Recent 1,024 + 4 Anchors, the rest TQ3),
    with its own encoders building that cache first."""
    from oracle import attention as OA
    from oracle import cache as OC
    w = W.WORKLOADS["l27b"]
    plan = W.make_page_plan(w, seed)
    t0 = time.perf_counter()
    pools = OC.build_pools(w, plan, lambda b: W.make_kv(w, seed, 0, b, int(plan.seq_lens[b])),
                           W.make_signs(w, seed, 0), "fp8")
    t_build = time.perf_counter() - t0
    t0 = time.perf_counter()
    OA.paged_decode_ref(pools, plan.block_table, plan.page_format, plan.seq_lens, W.make_q(w, seed, 0),
                        w.sm_scale, w.page_size, w.num_kv_heads, w.head_dim, W.make_signs(w, seed, 0))
    t_dec = time.perf_counter() - t0
    nbytes = kv_bytes_per_layer(w, plan)
    return {"l27b_oracle_decode_s": round(t_dec, 3), "l27b_oracle_decode_GBps": round(nbytes / t_dec / 1e9, 5),
            "l27b_oracle_build_s": round(t_build, 2), "l27b_kv_bytes": nbytes}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="canary", choices=sorted(W.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-entry-points", action="store_true",
                    help="skip the timings of the other entry points (promotion, scored, prefill, fused append)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path has no multi-GPU part (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_paged_kv_mixed_amd as m
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = W.WORKLOADS[args.workload]
    if args.layers:
        w = W.scaled(w, layers=args.layers)
    plan = W.make_page_plan(w, args.seed)
    B, Hq, d, L = w.batch, w.num_q_heads, w.head_dim, w.layers
    log(f"[bench] workload {w.name}: B={B} Hq={Hq} Hkv={w.num_kv_heads} d={d} P={w.page_size} layers={L} "
        f"tokens={plan.seq_lens.tolist()[:4]}")

    # ---- setup: encode every layer's cache with the library ----
    n_stage = int(max(((plan.page_format[b] != 0) & (plan.page_format[b] != 255)).sum() for b in range(B)))
    stage_pool = torch.zeros((max(1, n_stage), m.page_bytes(0, w.num_kv_heads, d, w.page_size)),
                             dtype=torch.uint8, device="cuda")
    layers = []
    enc = np.zeros(6)
    t_setup = time.perf_counter()
    for li in range(L):
        lay, e = build_layer(torch, m, w, plan, args.seed, li, stage_pool)
        layers.append(lay)
        enc += np.array(e, dtype=np.float64)
        log(f"[bench] layer {li} encoded ({time.perf_counter() - t_setup:.1f} s)")
    del stage_pool
    torch.cuda.empty_cache()

    # ---- decode state ----
    bt = torch.from_numpy(plan.block_table).cuda()
    pf = torch.from_numpy(plan.page_format).cuda()
    sl = torch.from_numpy(plan.seq_lens).cuda()
    max_pages = plan.max_pages
    qs = [torch.from_numpy(W.make_q(w, args.seed, li).view(np.int16)).cuda().view(torch.bfloat16) for li in range(L)]
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device="cuda") for _ in range(L)]
    lses = [torch.empty((B, Hq), dtype=torch.float32, device="cuda") for _ in range(L)]
    c0 = layers[0].cache
    plan_buf = torch.zeros(m.paged_decode_plan_bytes(c0, B, max_pages), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(m.paged_decode_attn_planned_workspace_size(c0, B, Hq, max_pages), dtype=torch.uint8, device="cuda")

    def step():
        m.paged_decode_plan(c0, bt, pf, sl, plan_buf)
        for li in range(L):
            m.paged_decode_attn_planned(layers[li].cache, plan_buf, qs[li], max_pages, w.sm_scale, outs[li],
                                        lses[li], ws)

    # eager run first (also the reference for the graph replays)
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    for li in range(L):
        assert torch.equal(outs[li], ref[li]), f"graph replay differs from the eager call on layer {li}"

    # ---- timed region: K graph replays of the whole step ----
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for k in range(args.steps):
        g.replay()
        evs[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(args.steps)])
    for li in range(L):
        assert torch.equal(outs[li], ref[li]), f"timed replays changed layer {li}'s output"

    # ---- the same step issued call by call on the stream (no graph) ----
    # A bounded spin kernel first lets the host queue every launch before the
    # GPU reaches them, so the events time the GPU's own back-to-back work.
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)
    sev[0].record()
    for k in range(args.steps):
        step()
        sev[k + 1].record()
    torch.cuda.synchronize()
    eager_us = np.array([sev[k].elapsed_time(sev[k + 1]) * 1e3 for k in range(args.steps)])
    for li in range(L):
        assert torch.equal(outs[li], ref[li]), f"stream-issued steps changed layer {li}'s output"

    # ---- per-launch decode durations (HIP events on the launch stream) ----
    # A bounded spin kernel first lets the host queue every launch before the
    # GPU reaches them, so each event pair brackets one kernel and no host gap.
    # The library records a third event between the scan and the merge
    # kernel of each call (kvq_set_scan_end_event), so the scan kernel, the
    # dominant one, is timed alone on the stream it runs on.
    n_launch = args.steps * L
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * n_launch)]
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for e in kev[1::3]:
        e.record()                                   # creates the HIP event the library records
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)
    for k in range(args.steps):
        pev[2 * k].record()
        m.paged_decode_plan(c0, bt, pf, sl, plan_buf)
        pev[2 * k + 1].record()
        for li in range(L):
            i = k * L + li
            kev[3 * i].record()
            m.set_scan_end_event(kev[3 * i + 1])
            m.paged_decode_attn_planned(layers[li].cache, plan_buf, qs[li], max_pages, w.sm_scale, outs[li],
                                        lses[li], ws)
            kev[3 * i + 2].record()
    m.set_scan_end_event(None)
    torch.cuda.synchronize()
    dec_us = np.array([kev[3 * i].elapsed_time(kev[3 * i + 2]) * 1e3 for i in range(n_launch)])
    scan_us = np.array([kev[3 * i].elapsed_time(kev[3 * i + 1]) * 1e3 for i in range(n_launch)])
    merge_us = np.array([kev[3 * i + 1].elapsed_time(kev[3 * i + 2]) * 1e3 for i in range(n_launch)])
    plan_us = np.array([pev[2 * k].elapsed_time(pev[2 * k + 1]) * 1e3 for k in range(args.steps)])

    # ---- route counters of one step (Minima-KV section 3.3 and Table 4) ----
    ctr = torch.zeros(ctypes_sizeof_counters(m), dtype=torch.uint8, device="cuda")
    m.paged_decode_plan(c0, bt, pf, sl, plan_buf, ctr)
    for li in range(L):
        m.paged_decode_attn_planned(layers[li].cache, plan_buf, qs[li], max_pages, w.sm_scale, outs[li], lses[li],
                                    ws, ctr)
    torch.cuda.synchronize()
    step_counters = m.read_counters(ctr)
    for li in range(L):
        assert torch.equal(outs[li], ref[li]), f"the counted step changed layer {li}'s output"

    # ---- a plain device copy of known size, for the achievable bandwidth ----
    nbytes_copy = 1 << 30
    a = torch.empty(nbytes_copy // 4, dtype=torch.float32, device="cuda")
    bcopy = torch.empty_like(a)
    bcopy.copy_(a)
    c_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    c_ev[0].record()
    for _ in range(10):
        bcopy.copy_(a)
    c_ev[1].record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes_copy * 10 / (c_ev[0].elapsed_time(c_ev[1]) * 1e-3) / 1e9
    del a, bcopy

    prom, scored, prefill = {}, {}, {}
    if not args.no_entry_points:
        prom = time_promote(torch, m, w, layers[0], plan)
        scored = time_entry_points(torch, m, w, layers[0], plan, plan_buf, qs[0], bt, pf, sl, ws)
        m.paged_decode_plan(c0, bt, pf, sl, plan_buf)
        prefill = time_packed_prefill(torch, m, w, layers[0], plan, plan_buf)

    layer_bytes = kv_bytes_per_layer(w, plan)
    step_bytes = layer_bytes * L
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9
    kern_mean = float(dec_us.mean())
    scan_mean = float(scan_us.mean())
    achieved = layer_bytes / (scan_mean * 1e-6) / 1e9
    call_achieved = layer_bytes / (kern_mean * 1e-6) / 1e9
    traffic_scan, traffic_call, counter_gbps, rocprof_scan_us = measured_traffic(w.name, d)
    pool_bytes = sum(int(t.numel()) for t in layers[0].pools.values())
    n_fp8, t_fp8, n_dem, t_dem, b_fp8, b_dem = enc
    present = [f for f in (0, 1, 2, 3) if (plan.page_format == f).any()]
    stale = "/".join(FMT_NAMES[f] for f in present if f != 0) or "none"
    metric = ("decode-attn KV GB/s (% HBM peak) + \u00b5s/step, 2\u00d759,008-token FP8/TQ3 cache"
              if w.name == "canary" else f"decode-attn KV GB/s (% HBM peak) + \u00b5s/step, {w.name} workload")
    rec = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {B} requests x {int(plan.seq_lens.max())} tokens (lengths "
                        f"{int(plan.seq_lens.min())}..{int(plan.seq_lens.max())}), {L} layers, Hq={Hq}, "
                        f"Hkv={w.num_kv_heads}, d={d}, page {w.page_size}; "
                        + (f"FP8/TQ3/TQ2 by seeded page-importance rank {w.importance_split}"
                           if w.importance_split else
                           f"FP8 Recent {w.recent_tokens} tokens + {w.anchor_pages} Anchor pages, {stale} Stale")
                        + f"; seeded N(0,1) K/V" + (", per-RoPE-block variance" if w.block_var_range else "")
                        + ", bf16 q",
            "batch": B, "layers": L, "seq_len": int(plan.seq_lens.max()), "num_q_heads": Hq,
            "num_kv_heads": w.num_kv_heads, "head_dim": d, "page_size": w.page_size,
            **{f"pages_{FMT_NAMES[f].lower()}": int((plan.page_format == f).sum()) for f in present},
            "seed": args.seed,
        },
        "us_per_step": {"wall_mean": round(ms_per_step * 1e3, 2), "median": round(float(np.median(step_us)), 2),
                        "min": round(float(step_us.min()), 2), "p95": round(float(np.percentile(step_us, 95)), 2)},
        "us_per_step_stream": {"mean": round(float(eager_us.mean()), 2), "median": round(float(np.median(eager_us)), 2),
                               "min": round(float(eager_us.min()), 2)},
        "hbm_frac_of_step": round(value / HBM_PEAK_GBPS, 4),
        "kv_bytes_per_layer": layer_bytes,
        "kv_bytes_per_step": step_bytes,
        "roofline": {
            "bound": "hbm", "kernel": f"{scan_kernel_name(d)} (the scan of one paged_decode_attn_planned call)",
            "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_scan,
            "kernel_us": {"mean": round(scan_mean, 3), "median": round(float(np.median(scan_us)), 3),
                          "min": round(float(scan_us.min()), 3), "launches": int(n_launch)},
            "algorithmic_bytes_per_launch": layer_bytes,
            "counter_GBps": None if counter_gbps is None else round(counter_gbps, 1),
            "counter_frac": None if counter_gbps is None else round(counter_gbps / HBM_PEAK_GBPS, 4),
            "rocprof_kernel_us": None if rocprof_scan_us is None else round(rocprof_scan_us, 3),
            "whole_call": {"kernels": f"{scan_kernel_name(d)} + merge_kernel<{d}, false, false>",
                           "us_mean": round(kern_mean, 3), "achieved": round(call_achieved, 2),
                           "frac": round(call_achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_call,
                           "merge_us_mean": round(float(merge_us.mean()), 3)},
        },
        "route_counters_per_step": step_counters,
        "rates": rate_accounting(w, plan, pool_bytes),
        "plan_kernel_us": round(float(plan_us.mean()), 3),
        "page_mass": scored,
        "packed_prefill": prefill,
        "copy_GBps": round(copy_gbps, 1),
        "encode": {
            "fp8_append_tokens_per_s": round(n_fp8 / t_fp8, 1) if t_fp8 else None,
            f"{stale.lower().replace('/', '_')}_demote_tokens_per_s": round(n_dem / t_dem, 1) if t_dem else None,
            "fp8_append_tokens": int(n_fp8), f"{stale.lower().replace('/', '_')}_demote_tokens": int(n_dem),
            "demote_roofline": {"bound": "hbm",
                                "kernel": ("encode_tqk_tiles_kernel" if 3 in present else "encode_tq_tiles_kernel")
                                          + " (FP8 pages -> TQ pages)",
                                "bytes_per_token": round(b_dem / n_dem, 1) if n_dem else None,
                                "achieved_GBps": round(b_dem / t_dem / 1e9, 1) if t_dem else None,
                                "frac": round(b_dem / t_dem / 1e9 / HBM_PEAK_GBPS, 4) if t_dem else None},
            "fp8_append_roofline": {"bound": "hbm", "bytes_per_token": round(b_fp8 / n_fp8, 1) if n_fp8 else None,
                                    "achieved_GBps": round(b_fp8 / t_fp8 / 1e9, 1) if t_fp8 else None,
                                    "frac": round(b_fp8 / t_fp8 / 1e9 / HBM_PEAK_GBPS, 4) if t_fp8 else None},
            **prom,
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline(w, plan, args.seed)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
