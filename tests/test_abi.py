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
    for name in ("kv_encode_fp8", "kv_encode_tq3", "paged_decode_attn", "paged_decode_plan",
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
    assert lib.kvq_abi_version() == 2


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
    assert m.lib.paged_decode_attn_planned(ctypes.byref(c), None, None, 1, 72, 8, ctypes.c_float(0.1),
                                           None, None, None, 0, None, None) == -2
    assert m.lib.paged_decode_attn_planned(ctypes.byref(c), None, None, 1, 6, 8, ctypes.c_float(0.1),
                                           None, None, None, 0, None, None) == -2
    # workspace too small
    assert m.lib.paged_decode_attn_planned(ctypes.byref(c), 256, 256, 1, 24, 8, ctypes.c_float(0.1),
                                           256, None, 256, 16, None, None) == -1
    assert b"workspace" in m.lib.kvq_last_error()
    # empty work is fine
    assert m.lib.kv_encode_fp8(ctypes.byref(c), None, 0, 0, None, None, None) == 0
    c.num_kv_heads, c.head_dim, c.page_size = 4, 256, 16
    assert m.paged_decode_plan_bytes(c, 2, 3688) > 8 * 2 * 3688
