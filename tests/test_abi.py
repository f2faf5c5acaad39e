"""The C-ABI library loads and exports every function include/kvq.h
declares; host-side validation fails closed without touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")
LIB = os.path.join(ROOT, "quantized_paged_kv_mixed_amd", "libkvq.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(LIB), "libkvq.so is not built (__graft_entry__.build())"
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    d = _declared()
    for name in ("kv_encode_fp8", "kv_encode_tq3", "kv_encode_tqk", "kv_promote_fp8", "paged_decode_attn",
                 "paged_decode_plan", "paged_decode_attn_scored", "page_mass_collect", "paged_decode_attn_append",
                 "paged_prefill_attn_planned", "paged_prefill_attn_workspace_size",
                 "paged_decode_attn_planned", "kvq_status_string"):
        assert name in d, name


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for name in _declared():
        assert name in exported, f"{name} declared in kvq.h but not exported"
        assert hasattr(lib, name)


def test_host_helpers(lib):
    lib.kvq_status_string.restype = ctypes.c_char_p
    assert lib.kvq_status_string(0) == b"ok"
    assert lib.kvq_status_string(-2) == b"unsupported geometry"
    lib.kvq_page_bytes.restype = ctypes.c_size_t
    assert lib.kvq_page_bytes(0, 4, 256, 16) == 4 * 16 * 520
    assert lib.kvq_page_bytes(1, 4, 256, 16) == 4 * 16 * 196
    assert lib.kvq_page_bytes(2, 8, 128, 16) == 8 * 16 * 68
    assert lib.kvq_page_bytes(1, 4, 96, 16) == 0
    lib.kvq_abi_version.restype = ctypes.c_int32
    assert lib.kvq_abi_version() == 10
    assert lib.kvq_page_bytes(3, 8, 128, 32) == 8 * 32 * 104
    assert lib.kvq_page_bytes(3, 8, 256, 32) == 0           # grouped keys: head_dim 128 only


def test_fail_closed_without_launch():
    """Unsupported or invalid arguments return an error before any HIP call
    (these calls run on a machine with no GPU)."""
    import quantized_paged_kv_mixed_amd as m
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 4, 96, 16
    st = m.lib.kv_encode_fp8(ctypes.byref(c), None, 0, 1, None, None, None)
    assert st == -2 and b"head_dim" in m.lib.kvq_last_error()
    c.head_dim, c.page_size = 256, 8
    assert m.lib.paged_decode_plan(ctypes.byref(c), 1, None, None, 4, None, None, 0, None, None) == -2
    c.page_size = 16
    c.tq3_num_pages = 10                      # pages but no pointer
    assert m.lib.kv_encode_tq3(ctypes.byref(c), 0, None, None, 1, None, None, None) == -1
    c.tq3_num_pages = 0
    c.fp8_pages, c.fp8_num_pages = 4096, 3    # fake non-null address, never dereferenced
    assert m.lib.kv_encode_fp8(ctypes.byref(c), None, 0, 5, None, None, None) == -1
    # GQA group too large / Hq not a multiple of Hkv
    assert m.lib.paged_decode_attn_planned(ctypes.byref(c), None, 0, None, 1, 72, 8, ctypes.c_float(0.1),
                                           None, None, None, 0, None, None) == -2
    assert m.lib.paged_decode_attn_planned(ctypes.byref(c), None, 0, None, 1, 6, 8, ctypes.c_float(0.1),
                                           None, None, None, 0, None, None) == -2
    # workspace too small
    assert m.lib.paged_decode_attn_planned(ctypes.byref(c), 256, 1 << 30, 256, 1, 24, 8, ctypes.c_float(0.1),
                                           256, None, 256, 16, None, None) == -1
    assert b"workspace" in m.lib.kvq_last_error()
    # plan buffer shorter than this geometry's plan
    nplan = m.paged_decode_plan_bytes(c, 1, 8)
    nws = m.lib.paged_decode_attn_planned_workspace_size(1, 24, 8, ctypes.byref(c))
    for call in (m.lib.paged_decode_attn_planned, m.lib.paged_decode_attn_scored):
        extra = (256,) if call is m.lib.paged_decode_attn_scored else ()
        assert call(ctypes.byref(c), 256, nplan - 1, 256, 1, 24, 8, ctypes.c_float(0.1), 256, 256, *extra,
                    256, nws, None, None) == -1
        assert b"plan buffer" in m.lib.kvq_last_error()
    assert m.lib.paged_prefill_attn_planned(ctypes.byref(c), 256, nplan - 1, 256, 1, 8, 2, 8, ctypes.c_float(0.1),
                                            256, None, 256, 1 << 30, None, None) == -1
    assert b"plan buffer" in m.lib.kvq_last_error()
    # empty work is fine
    assert m.lib.kv_encode_fp8(ctypes.byref(c), None, 0, 0, None, None, None) == 0
    c.num_kv_heads, c.head_dim, c.page_size = 4, 256, 16
    assert m.paged_decode_plan_bytes(c, 2, 3688) > 8 * 2 * 3688


def test_tqk_fails_closed():
    """Grouped-key pools need head_dim 128 and a coordinate order; errors
    come back before any launch (fake addresses are never dereferenced)."""
    import quantized_paged_kv_mixed_amd as m
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 2, 128, 32
    c.tqk_pages, c.tqk_num_pages = 4096, 4
    assert m.lib.kv_encode_tqk(ctypes.byref(c), 0, 4096, None, 1, 4096, None, None) == -1   # no signs
    c.rot_signs = 4096
    assert m.lib.kv_encode_tqk(ctypes.byref(c), 0, 4096, None, 1, 4096, None, None) == -1   # no order
    assert b"tqk_perm" in m.lib.kvq_last_error()
    c.tqk_perm = 4098                                                                     # misaligned
    assert m.lib.kv_encode_tqk(ctypes.byref(c), 0, 4096, None, 1, 4096, None, None) == -1
    c.tqk_perm = 4096
    c.head_dim = 256
    assert m.lib.kv_encode_tqk(ctypes.byref(c), 0, 4096, None, 1, 4096, None, None) == -2
    assert m.lib.paged_decode_plan(ctypes.byref(c), 1, 4096, 4096, 4, 4096, 4096, 1 << 20, None, None) == -2
    assert m.page_bytes(m.FMT_TQK, 2, 128, 32) == 2 * 32 * 104
    assert ctypes.sizeof(m.LayerCache) == 128 and ctypes.sizeof(m.Counters) == 64


def test_binding_structs_match_the_header(tmp_path):
    """The ctypes mirrors have the C sizes and field offsets of kvq.h."""
    import quantized_paged_kv_mixed_amd as m
    src = tmp_path / "sz.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kvq.h"\nint main(void) {\n'
                   'printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(kvq_layer_cache), sizeof(kvq_counters),\n'
                   'offsetof(kvq_layer_cache, rot_signs), offsetof(kvq_layer_cache, tqk_perm),\n'
                   'offsetof(kvq_counters, pages_tqk), offsetof(kvq_layer_cache, tqf5_pages),\n'
                   'offsetof(kvq_layer_cache, tqf6_num_pages), offsetof(kvq_counters, pages_tqf6));\n'
                   'return 0;\n}\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [ctypes.sizeof(m.LayerCache), ctypes.sizeof(m.Counters), m.LayerCache.rot_signs.offset,
                   m.LayerCache.tqk_perm.offset, m.Counters.pages_tqk.offset, m.LayerCache.tqf5_pages.offset,
                   m.LayerCache.tqf6_num_pages.offset, m.Counters.pages_tqf6.offset]


def test_promote_fails_closed():
    """Promotion needs a compressed source format, a non-empty source pool
    and an FP8 destination pool; errors come back before any launch."""
    import quantized_paged_kv_mixed_amd as m
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 4, 256, 16
    c.tq3_pages, c.tq3_num_pages, c.rot_signs = 4096, 8, 4096
    assert m.lib.kv_promote_fp8(ctypes.byref(c), m.FMT_FP8, 4096, 1, 4096, None) == -1     # FP8 is not compressed
    assert m.lib.kv_promote_fp8(ctypes.byref(c), 7, 4096, 1, 4096, None) == -1
    assert m.lib.kv_promote_fp8(ctypes.byref(c), m.FMT_TQ3, 4096, 1, 4096, None) == -1     # no FP8 pool
    assert b"FP8" in m.lib.kvq_last_error()
    c.fp8_pages, c.fp8_num_pages = 8192, 8
    assert m.lib.kv_promote_fp8(ctypes.byref(c), m.FMT_TQ2, 4096, 1, 4096, None) == -1     # empty TQ2 pool
    assert m.lib.kv_promote_fp8(ctypes.byref(c), m.FMT_TQ3, None, 1, 4096, None) == -1     # no source ids
    assert m.lib.kv_promote_fp8(ctypes.byref(c), m.FMT_TQ3, 4096, -1, 4096, None) == -1
    assert m.lib.kv_promote_fp8(ctypes.byref(c), m.FMT_TQ3, 4096, 0, 4096, None) == 0      # nothing to do
    c.page_size = 8
    assert m.lib.kv_promote_fp8(ctypes.byref(c), m.FMT_TQ3, 4096, 1, 4096, None) == -2


def test_scored_decode_and_collect_fail_closed():
    """The scored decode needs its tile log-mass and lse outputs; the
    collector checks its head set, beta and pointers before any launch."""
    import quantized_paged_kv_mixed_amd as m
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 4, 256, 16
    c.fp8_pages, c.fp8_num_pages = 4096, 8
    assert m.lib.paged_decode_attn_scored(ctypes.byref(c), 4096, 1 << 30, 4096, 1, 24, 8, 0.06, 4096, 4096, None,
                                          4096, 1 << 30, None, None) == -1
    assert b"tile_lmass" in m.lib.kvq_last_error()
    assert m.lib.paged_decode_attn_scored(ctypes.byref(c), 4096, 1 << 30, 4096, 1, 24, 8, 0.06, 4096, None, 4096,
                                          4096, 1 << 30, None, None) == -1
    H = (ctypes.c_int32 * 3)(0, 5, 23)
    Hp = ctypes.cast(H, ctypes.c_void_p)
    call = lambda hs, n, beta, P=16, score=4096: m.lib.page_mass_collect(2, 24, 8, P, 4096, 4096, hs, n, beta,
                                                                      score, None, None)
    assert call(Hp, 3, 1.5) == -1                              # beta outside [0, 1]
    assert call(Hp, 3, -0.1) == -1
    assert call(None, 3, 0.5) == -1                            # no head set
    assert call(Hp, 3, 0.5, P=8) == -2
    assert call(Hp, 3, 0.5, score=None) == -1
    assert call(Hp, 257, 0.5) == -2                            # more heads than one call takes
    bad = (ctypes.c_int32 * 2)(0, 24)                          # q-head 24 of 24
    assert call(ctypes.cast(bad, ctypes.c_void_p), 2, 0.5) == -1
    assert b"head 24" in m.lib.kvq_last_error()
    assert m.lib.page_mass_collect(0, 24, 8, 16, None, None, Hp, 3, 0.5, None, None, None) == 0


def test_fused_append_fails_closed():
    """The fused append needs its new-token rows, destinations and an FP8
    pool; errors come back before any launch."""
    import quantized_paged_kv_mixed_amd as m
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 4, 256, 16
    c.tq3_pages, c.tq3_num_pages, c.rot_signs = 4096, 8, 4096
    args = lambda kv, pg, sl, bf=0: (ctypes.byref(c), 4096, 1 << 30, 4096, 1, 24, 8, 0.06, kv, bf, pg, sl, 4096,
                                     4096, 4096, 1 << 30, None, None)
    assert m.lib.paged_decode_attn_append(*args(None, 4096, 4096)) == -1
    assert m.lib.paged_decode_attn_append(*args(4096, None, 4096)) == -1
    assert m.lib.paged_decode_attn_append(*args(4098, 4096, 4096)) == -1          # float rows misaligned
    assert m.lib.paged_decode_attn_append(*args(4096, 4096, 4096)) == -1          # no FP8 pool
    assert b"FP8 pool" in m.lib.kvq_last_error()


def test_prefill_fails_closed():
    """A chunk must be at least one token. Up to 16 rows (chunk x GQA group)
    the decode scan serves the chunk and its workspace is the decode's; past
    that the packed prefill checks its own arguments (alignment, the running
    state's workspace when more than one pool is present, the grid) before any
    launch."""
    import quantized_paged_kv_mixed_amd as m
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 4, 256, 16
    c.fp8_pages, c.fp8_num_pages = 4096, 8
    call = lambda chunk, out=4096, ws_bytes=1 << 30, batch=1: m.lib.paged_prefill_attn_planned(
        ctypes.byref(c), 4096, 1 << 30, 4096, batch, 24, chunk, 8, 0.06, out, None, 4096, ws_bytes, None, None)
    assert call(0) == -1
    assert m.lib.paged_prefill_attn_workspace_size(2, 24, 2, 8, ctypes.byref(c)) == \
        m.lib.paged_decode_attn_planned_workspace_size(2, 48, 8, ctypes.byref(c))
    # packed (3 x 6 rows): one pool needs no workspace
    assert m.lib.paged_prefill_attn_workspace_size(2, 24, 3, 8, ctypes.byref(c)) == 256
    assert call(3, out=4100) == -1                          # out must be 16-byte aligned
    assert b"misaligned" in m.lib.kvq_last_error()
    assert call(3, batch=70000) == -2
    # two pools: the running state between the launches
    c.tq3_pages, c.tq3_num_pages, c.rot_signs = 8192, 8, 4096
    rows = 2 * 3 * 24
    need = ((rows * 256 * 4 + 255) // 256) * 256 + rows * 8
    assert m.lib.paged_prefill_attn_workspace_size(2, 24, 3, 8, ctypes.byref(c)) == need
    assert call(3, ws_bytes=1000) == -1
    assert b"workspace" in m.lib.kvq_last_error()


def test_one_call_workspace_is_plan_plus_partials():
    """paged_decode_attn_workspace_size sizes the one-call paged_decode_attn:
    the plan rounded up to 256 bytes, then the planned call's partials."""
    import quantized_paged_kv_mixed_amd as m
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 4, 256, 16
    for B, Hq, MP in ((2, 24, 3688), (1, 4, 1), (64, 32, 2048)):
        plan = m.lib.paged_decode_plan_bytes(B, MP, ctypes.byref(c))
        part = m.lib.paged_decode_attn_planned_workspace_size(B, Hq, MP, ctypes.byref(c))
        assert plan > 0 and part > 0
        assert m.lib.paged_decode_attn_workspace_size(B, Hq, MP, ctypes.byref(c)) == ((plan + 255) // 256) * 256 + part
        assert m.paged_decode_attn_workspace_size(c, B, Hq, MP) == ((plan + 255) // 256) * 256 + part
    # a workspace one byte short is refused before any launch
    need = m.lib.paged_decode_attn_workspace_size(1, 24, 8, ctypes.byref(c))
    c.fp8_pages, c.fp8_num_pages = 4096, 8
    st = m.lib.paged_decode_attn(ctypes.byref(c), 4096, 1, 24, 4096, 4096, 8, 4096, ctypes.c_float(0.1), 4096, None,
                                 4096, need - 1, None, None)
    assert st == -1 and b"workspace" in m.lib.kvq_last_error()


def test_counters_follow_the_boundary_order():
    """kvq_counters: pages per format (FP8, TQ3, TQ2, TQK), then
    invalid_entries and fallbacks, then the fractional-level formats."""
    import quantized_paged_kv_mixed_amd as m
    names = [f[0] for f in m.Counters._fields_]
    assert names == ["pages_fp8", "pages_tq3", "pages_tq2", "pages_tqk", "invalid_entries", "fallbacks",
                     "pages_tqf5", "pages_tqf6"]
    assert [m.Counters.__dict__[n].offset for n in names] == [0, 8, 16, 24, 32, 40, 48, 56]
    assert names == m.COUNTER_FIELDS


@pytest.mark.parametrize("fmt,levels", [(4, 5), (5, 6)])
@pytest.mark.parametrize("d,P", [(128, 16), (128, 32), (256, 16), (256, 32)])
def test_fractional_page_bytes_follow_the_row_bitstreams(fmt, levels, d, P):
    """A fractional-level head block is P key rows and P value rows of
    row_bytes(d, L) each plus two fp16 sigma per token: the library's page
    size is the oracle's byte accounting, and a fractional pool without
    rotation signs is refused before any launch."""
    import quantized_paged_kv_mixed_amd as m
    from oracle import tqf
    R = tqf.row_bytes(d, levels)
    assert m.page_bytes(fmt, 3, d, P) == 3 * P * (2 * R + 4)
    c = m.LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = 3, d, P
    setattr(c, f"tqf{levels}_pages", 4096)
    setattr(c, f"tqf{levels}_num_pages", 4)
    enc = m.lib.kv_encode_tqf5 if levels == 5 else m.lib.kv_encode_tqf6
    assert enc(ctypes.byref(c), 0, 4096, None, 1, 4096, None, None) == -1              # no signs
    c.rot_signs = 4096
    setattr(c, f"tqf{levels}_pages", None)
    assert enc(ctypes.byref(c), 0, 4096, None, 1, 4096, None, None) == -1              # pages but no pointer
