"""Host-side logic of the benchmark (no GPU): the one-GPU contract, the
algorithmic bytes it prices the roofline with, and the gate that reports
counter traffic only for the decode source the counters were taken on."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W
from oracle import accounting as acc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name", ["tiny", "l27b", "canary", "serving"])
def test_bench_bytes_match_the_oracle_accounting(name):
    """The benchmark counts the tokens of a partial last page only; the
    accounting function counts whole pages. They agree exactly when every
    request ends on a page boundary, and differ by the missing slots otherwise."""
    w = W.WORKLOADS[name]
    plan = W.make_page_plan(w, 0)
    got = bench.kv_bytes_per_layer(w, plan)
    whole = acc.decode_kv_bytes(plan.page_format, plan.seq_lens, w.page_size, w.num_kv_heads, w.head_dim)
    missing = 0
    for b in range(w.batch):
        N = int(plan.seq_lens[b])
        tail = (-N) % w.page_size
        if tail:
            f = int(plan.page_format[b, (N - 1) // w.page_size])
            missing += tail * w.num_kv_heads * acc.token_head_bytes(f, w.head_dim)
    assert got == whole - missing
    if name == "canary":
        assert got == 98164736                      # 2 x 59,008 tokens end on a page boundary


def test_grouped_key_bytes_use_three_key_sigmas():
    w = W.WORKLOADS["l70b"]
    plan = W.make_page_plan(w, 0)
    assert bench.kv_bytes_per_layer(w, plan) == 457179136
    assert bench.FMT_BYTES[3](128) == acc.tqk_token_head_bytes(128) == 104


def test_traffic_is_reported_only_for_the_profiled_source(monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "decode_canary_traffic.json")))
    k = rec["kernels"].get(bench.scan_kernel_name(256), {})     # absent if the kernels were renamed since
    scan = sum(k[c]["bytes"] for c in ("FETCH_SIZE", "WRITE_SIZE") if c in k) or None
    scan = None if scan is None else int(round(scan))
    call = int(round(rec["decode_call_hbm_bytes"]))
    if rec["decode_source_sha256_16"] == bench.decode_source_hash():
        assert bench.measured_traffic("canary", 256)[:2] == (scan, call)
    else:                                       # the kernels changed since the counters were taken
        assert bench.measured_traffic("canary", 256) == (None, None, None, None)
    monkeypatch.setattr(bench, "decode_source_hash", lambda: rec["decode_source_sha256_16"])
    assert bench.measured_traffic("canary", 256)[:2] == (scan, call)
    # once the decode source changes, the record no longer counts
    monkeypatch.setattr(bench, "decode_source_hash", lambda: "f" * 16)
    assert bench.measured_traffic("canary", 256) == (None, None, None, None)


def test_rate_accounting_of_the_canary():
    """b_eff and compression of the canary's page mix: FP8 = 136 of 3,688
    pages per request at 8 bits (+ an fp32 scale per 256-vector), TQ3 the
    rest at 3 bits (+ an fp16 sigma), Minima-KV Eq. 10."""
    w = W.WORKLOADS["canary"]
    plan = W.make_page_plan(w, 0)
    r = bench.rate_accounting(w, plan, 0)
    p8 = 136 / 3688
    assert abs(r["b_eff_eq10_bits"] - round(8 * p8 + 3 * (1 - p8), 4)) < 1e-4
    eff = p8 * 8 * 520 / 512 + (1 - p8) * 8 * 196 / 512
    assert abs(r["effective_rate_bits"] - eff) < 1e-3
    assert abs(r["compression_vs_bf16_bytes"] - 16 / eff) < 1e-3
    assert abs(r["kv_bytes_per_token_all_layers"] - 16 * 4 * (p8 * 520 + (1 - p8) * 196)) < 0.1
