"""Pins of the byte accounting against numbers printed on the pages."""
import math

import numpy as np

import workloads as W
from oracle import accounting as acc
from tests.golden_io import load

GIB = 2.0 ** 30


def test_minima_kv_eq1_to_3_and_table2():
    g = load("minima_kv_printed.txt")
    L, H, d = int(g["L_f"]), int(g["H_kv"]), int(g["d_h"])
    assert acc.kv_bytes_per_token(L, H, d, 2) == g["bf16_bytes_per_token"]
    assert acc.kv_bytes_per_token(L, H, d, 1) == g["fp8_bytes_per_token"]
    assert acc.kv_bytes_per_token(L, H, d, 2) * 32768 / GIB == g["bf16_gib_32k"]
    assert acc.kv_bytes_per_token(L, H, d, 2) * 131072 / GIB == g["bf16_gib_128k"]
    agg = g["aggregate_kib_per_token"] * 1024
    for key in ("table2_8K", "table2_32K", "table2_128K", "table2_262144", "table2_1000000"):
        T, bf, f8, mk = g[key]
        nd = 2 if T == 1000000 else 3
        assert round(acc.kv_bytes_per_token(L, H, d, 2) * T / GIB, nd) == bf
        assert round(acc.kv_bytes_per_token(L, H, d, 1) * T / GIB, nd) == f8
        assert round(agg * T / GIB, nd) == mk
    bits = agg * 8 / (2 * L * H * d)
    assert round(bits, 2) == g["aggregate_bits_per_scalar"]
    assert round(16 / bits, 3) == g["aggregate_x_bf16"]
    assert round(8 / bits, 3) == g["aggregate_x_fp8"]
    assert round(acc.c_bf16(acc.b_eff(0, 0, 1, bits)), 3) == g["aggregate_x_bf16"]


def test_minima_kv_canary_numbers():
    g = load("minima_kv_printed.txt")
    assert round(g["canary_full_bytes"] / g["canary_compressed_bytes"], 4) == g["canary_ratio"]
    tps_c = g["canary_counted_tokens"] / g["canary_control_wall_s"]
    tps_m = g["canary_counted_tokens"] / g["canary_minima_wall_s"]
    assert round(tps_c, 3) == g["canary_control_tps"] and round(tps_m, 3) == g["canary_minima_tps"]
    assert round(tps_m / tps_c, 4) == g["canary_tps_ratio"]
    # 477,102,080 = BF16 bytes of one full-attention layer (4 KV heads x 256 x
    # 2 roles x 2 B = 4,096 B/token) over the 65 complete 1,792-token blocks of
    # the two requests (2 x floor(59,008 / 1,792) + 1 = 65); a reading, not a
    # statement of the page
    per_tok_layer = acc.kv_bytes_per_token(1, int(g["H_kv"]), int(g["d_h"]), 2)
    assert per_tok_layer == 4096
    assert g["canary_full_bytes"] == 65 * int(g["canary_block_tokens"]) * per_tok_layer
    assert 2 * (int(g["canary_prompt_tokens"]) // int(g["canary_block_tokens"])) + 1 == 65


def test_minima_kv_eq14_table5():
    g = load("minima_kv_printed.txt")
    M, Wt, D = g["eq14_M_gib"], g["eq14_W_gib"], g["eq14_D_gib"]
    for key in ("table5_8K", "table5_16K", "table5_32K", "table5_64K", "table5_128K", "table5_262K"):
        T, bf, f8, mk = g[key]
        kb = acc.kv_bytes_per_token(16, 4, 256, 2) * T / GIB
        assert acc.capacity(M, Wt, D, kb) == bf
        assert acc.capacity(M, Wt, D, kb / 2) == f8
        assert acc.capacity(M, Wt, D, kb / g["eq14_minima_x_bf16"]) == mk


def test_block_gtq_footprint():
    g = load("block_gtq_printed.txt")
    d = int(g["head_dim"])
    assert 2 * d * 3 // 8 == g["ideal_k3v3_bytes"]
    assert acc.tq_nibble_token_head_bytes(d) == g["uniform_tq_mse_bytes"]
    assert 2 * d * 2 == g["fp16_bytes"]
    assert round(g["fp16_bytes"] / g["uniform_tq_mse_bytes"], 2) == g["uniform_x_fp16"]
    assert round(g["fp16_bytes"] / g["block_gtq_bytes"], 2) == g["block_gtq_x_fp16"]
    per_tok = lambda b: b * g["kv_heads"] * g["layers"]
    assert round(per_tok(g["fp16_bytes"]) * 131072 / 1e9, 2) == g["fp16_resident_gb_128k"]
    assert round(per_tok(g["fp16_bytes"]) * 2 ** 20 / 1e9, 2) == g["fp16_resident_gb_1m"]
    assert round(per_tok(g["block_gtq_bytes"]) * 131072 / 1e9, 2) == g["block_gtq_resident_gb_128k"]
    assert round(per_tok(g["block_gtq_bytes"]) * 2 ** 20 / 1e9, 2) == g["block_gtq_resident_gb_1m"]


def test_workload_decode_bytes():
    """Algorithmic bytes per decode step of the named workloads."""
    w = W.WORKLOADS["tiny"]
    p = W.make_page_plan(w, 0)
    assert (p.page_format[0] == W.FMT_FP8).sum() == 17
    assert acc.decode_kv_bytes(p.page_format, p.seq_lens, 16, 1, 128) == 17 * 16 * 264 + 47 * 16 * 100 == 147008
    w = W.WORKLOADS["l27b"]
    p = W.make_page_plan(w, 0)
    assert (p.page_format[0] == W.FMT_FP8).sum() == 68
    assert acc.decode_kv_bytes(p.page_format, p.seq_lens, 16, 4, 256) == 14255104
    w = W.WORKLOADS["canary"]
    p = W.make_page_plan(w, 0)
    assert ((p.page_format == W.FMT_FP8).sum(1) == 136).all()
    assert acc.decode_kv_bytes(p.page_format, p.seq_lens, 16, 4, 256) == 98164736
    assert acc.tqk_token_head_bytes(128) == 104
