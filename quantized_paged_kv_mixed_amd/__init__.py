"""Mixed-format (FP8 / TQ) paged KV decode attention for MI355X (gfx950).

Thin ctypes binding of libkvq.so (include/kvq.h): argument marshalling only.
Every step of the path runs in the library's HIP kernels; torch supplies
device memory and the current stream. If the library is not built this
module raises at import: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "FMT_FP8", "FMT_TQ3", "FMT_TQ2", "FMT_TQK", "FMT_TQF5", "FMT_TQF6", "SRC_F32_ROWS", "SRC_FP8_PAGES", "KvqError",
    "LayerCache", "Counters", "lib", "page_bytes", "kv_encode_fp8", "kv_encode_tq3", "kv_encode_tq2",
    "kv_encode_tqk", "kv_encode_tqf5", "kv_encode_tqf6", "kv_promote_fp8",
    "paged_decode_plan_bytes", "paged_decode_plan", "paged_decode_attn_planned_workspace_size",
    "paged_decode_attn_planned", "paged_decode_attn_workspace_size", "paged_decode_attn",
    "paged_decode_attn_scored", "page_mass_collect", "paged_decode_attn_append",
    "paged_prefill_attn_workspace_size", "paged_prefill_attn_planned", "paged_decode_attn_noalloc",
]

FMT_FP8, FMT_TQ3, FMT_TQ2, FMT_TQK, FMT_TQF5, FMT_TQF6 = 0, 1, 2, 3, 4, 5
SRC_F32_ROWS, SRC_FP8_PAGES = 0, 1
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")


class KvqError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"kvq status {status}: {detail}")
        self.status = status


class LayerCache(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("fp8_pages", ctypes.c_void_p), ("fp8_num_pages", ctypes.c_int64),
        ("tq3_pages", ctypes.c_void_p), ("tq3_num_pages", ctypes.c_int64),
        ("tq2_pages", ctypes.c_void_p), ("tq2_num_pages", ctypes.c_int64),
        ("rot_signs", ctypes.c_void_p),
        ("tqk_pages", ctypes.c_void_p), ("tqk_num_pages", ctypes.c_int64),
        ("tqk_perm", ctypes.c_void_p),
        ("tqf5_pages", ctypes.c_void_p), ("tqf5_num_pages", ctypes.c_int64),
        ("tqf6_pages", ctypes.c_void_p), ("tqf6_num_pages", ctypes.c_int64),
    ]


class Counters(ctypes.Structure):
    _fields_ = [("pages_fp8", ctypes.c_uint64), ("pages_tq3", ctypes.c_uint64), ("pages_tq2", ctypes.c_uint64),
                ("pages_tqk", ctypes.c_uint64), ("invalid_entries", ctypes.c_uint64),
                ("fallbacks", ctypes.c_uint64), ("pages_tqf5", ctypes.c_uint64), ("pages_tqf6", ctypes.c_uint64)]


COUNTER_FIELDS = ["pages_fp8", "pages_tq3", "pages_tq2", "pages_tqk", "invalid_entries", "fallbacks", "pages_tqf5",
                  "pages_tqf6"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    CP = ctypes.POINTER(LayerCache)
    sig = {
        "kvq_status_string": (ctypes.c_char_p, [I32]),
        "kvq_last_error": (ctypes.c_char_p, []),
        "kvq_abi_version": (I32, []),
        "kvq_set_scan_end_event": (None, [P]),
        "kvq_page_bytes": (SZ, [I32, I32, I32, I32]),
        "kv_encode_fp8": (I32, [CP, P, I32, I64, P, P, P]),
        "kv_encode_tq3": (I32, [CP, I32, P, P, I64, P, P, P]),
        "kv_encode_tq2": (I32, [CP, I32, P, P, I64, P, P, P]),
        "kv_encode_tqk": (I32, [CP, I32, P, P, I64, P, P, P]),
        "kv_encode_tqf5": (I32, [CP, I32, P, P, I64, P, P, P]),
        "kv_encode_tqf6": (I32, [CP, I32, P, P, I64, P, P, P]),
        "kv_promote_fp8": (I32, [CP, I32, P, I64, P, P]),
        "paged_decode_plan_bytes": (SZ, [I32, I32, CP]),
        "paged_decode_plan": (I32, [CP, I32, P, P, I32, P, P, SZ, P, P]),
        "paged_decode_attn_planned_workspace_size": (SZ, [I32, I32, I32, CP]),
        "paged_decode_attn_planned": (I32, [CP, P, SZ, P, I32, I32, I32, F32, P, P, P, SZ, P, P]),
        "paged_decode_attn_scored": (I32, [CP, P, SZ, P, I32, I32, I32, F32, P, P, P, P, SZ, P, P]),
        "page_mass_collect": (I32, [I32, I32, I32, I32, P, P, P, I32, F32, P, P, P]),
        "paged_decode_attn_append": (I32, [CP, P, SZ, P, I32, I32, I32, F32, P, I32, P, P, P, P, P, SZ, P, P]),
        "paged_prefill_attn_workspace_size": (SZ, [I32, I32, I32, I32, CP]),
        "paged_prefill_attn_planned": (I32, [CP, P, SZ, P, I32, I32, I32, I32, F32, P, P, P, SZ, P, P]),
        "paged_decode_attn_workspace_size": (SZ, [I32, I32, I32, CP]),
        "paged_decode_attn": (I32, [CP, P, I32, I32, P, P, I32, P, F32, P, P, P, SZ, P, P]),
        "paged_decode_attn_noalloc": (I32, [CP, P, I32, I32, P, P, I32, P, F32, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def _check(status: int):
    if status != 0:
        raise KvqError(status, lib.kvq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def set_scan_end_event(event):
    """Measurement hook: record `event` (a torch.cuda.Event that has been
    recorded once, so its HIP event exists) between the scan and merge
    kernels of every decode call on this thread; None turns it off."""
    lib.kvq_set_scan_end_event(None if event is None else ctypes.c_void_p(event.cuda_event))


def page_bytes(fmt: int, num_kv_heads: int, head_dim: int, page_size: int) -> int:
    return int(lib.kvq_page_bytes(fmt, num_kv_heads, head_dim, page_size))


def make_cache(num_kv_heads, head_dim, page_size, fp8_pool=None, tq3_pool=None, tq2_pool=None, rot_signs=None,
               tqk_pool=None, tqk_perm=None, tqf5_pool=None, tqf6_pool=None):
    """Describe one layer's pools (uint8 tensors [pages, page bytes]), signs
    (int32 tensor [Hkv, 2, d/32] holding the uint32 sign words) and the key
    coordinate order of grouped mixed-rate pages (int16 tensor [Hkv, d]
    holding the uint16 entries)."""
    c = LayerCache()
    c.num_kv_heads, c.head_dim, c.page_size = num_kv_heads, head_dim, page_size
    for name, t in (("fp8", fp8_pool), ("tq3", tq3_pool), ("tq2", tq2_pool), ("tqk", tqk_pool),
                    ("tqf5", tqf5_pool), ("tqf6", tqf6_pool)):
        setattr(c, f"{name}_pages", None if t is None else t.data_ptr())
        setattr(c, f"{name}_num_pages", 0 if t is None else t.shape[0])
    c.rot_signs = None if rot_signs is None else rot_signs.data_ptr()
    c.tqk_perm = None if tqk_perm is None else tqk_perm.data_ptr()
    c._keep = (fp8_pool, tq3_pool, tq2_pool, rot_signs, tqk_pool, tqk_perm, tqf5_pool, tqf6_pool)
    return c


def kv_encode_fp8(cache, src, dst_page, dst_slot):
    bf = 1 if src.dtype == torch.bfloat16 else 0
    _check(lib.kv_encode_fp8(ctypes.byref(cache), _ptr(src), bf, src.shape[0], _ptr(dst_page), _ptr(dst_slot),
                             _stream()))


def _encode_tq(fn, cache, src_kind, dst_page, src=None, src_page=None, page_valid=None):
    _check(fn(ctypes.byref(cache), src_kind, _ptr(src), _ptr(src_page), dst_page.shape[0], _ptr(dst_page),
              _ptr(page_valid), _stream()))


def kv_encode_tq3(cache, src_kind, dst_page, src=None, src_page=None, page_valid=None):
    _encode_tq(lib.kv_encode_tq3, cache, src_kind, dst_page, src, src_page, page_valid)


def kv_encode_tq2(cache, src_kind, dst_page, src=None, src_page=None, page_valid=None):
    _encode_tq(lib.kv_encode_tq2, cache, src_kind, dst_page, src, src_page, page_valid)


def kv_encode_tqk(cache, src_kind, dst_page, src=None, src_page=None, page_valid=None):
    _encode_tq(lib.kv_encode_tqk, cache, src_kind, dst_page, src, src_page, page_valid)


def kv_encode_tqf5(cache, src_kind, dst_page, src=None, src_page=None, page_valid=None):
    _encode_tq(lib.kv_encode_tqf5, cache, src_kind, dst_page, src, src_page, page_valid)


def kv_encode_tqf6(cache, src_kind, dst_page, src=None, src_page=None, page_valid=None):
    _encode_tq(lib.kv_encode_tqf6, cache, src_kind, dst_page, src, src_page, page_valid)


def kv_promote_fp8(cache, src_format, src_page, dst_page):
    """Rebuild pages of a compressed pool (src_format) into FP8 pages."""
    _check(lib.kv_promote_fp8(ctypes.byref(cache), src_format, _ptr(src_page), src_page.shape[0], _ptr(dst_page),
                              _stream()))


def paged_decode_plan_bytes(cache, batch, max_pages) -> int:
    return int(lib.paged_decode_plan_bytes(batch, max_pages, ctypes.byref(cache)))


def paged_decode_plan(cache, block_table, page_format, seq_lens, plan, counters=None):
    B, max_pages = block_table.shape
    _check(lib.paged_decode_plan(ctypes.byref(cache), B, _ptr(block_table), _ptr(page_format), max_pages,
                                 _ptr(seq_lens), _ptr(plan), plan.numel() * plan.element_size(), _ptr(counters),
                                 _stream()))


def _nbytes(t):
    return t.numel() * t.element_size()


def paged_decode_attn_planned_workspace_size(cache, batch, num_q_heads, max_pages) -> int:
    """Workspace of paged_decode_attn_planned (partials only)."""
    return int(lib.paged_decode_attn_planned_workspace_size(batch, num_q_heads, max_pages, ctypes.byref(cache)))


def paged_decode_attn_workspace_size(cache, batch, num_q_heads, max_pages) -> int:
    """Workspace of the one-call paged_decode_attn (plan + partials)."""
    return int(lib.paged_decode_attn_workspace_size(batch, num_q_heads, max_pages, ctypes.byref(cache)))


def paged_decode_attn_planned(cache, plan, q, max_pages, sm_scale, out, lse, workspace, counters=None):
    B, Hq, _ = q.shape
    _check(lib.paged_decode_attn_planned(ctypes.byref(cache), _ptr(plan), _nbytes(plan), _ptr(q), B, Hq, max_pages,
                                         float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(counters), _stream()))


def paged_decode_attn_scored(cache, plan, q, max_pages, sm_scale, out, lse, tile_lmass, workspace, counters=None):
    """paged_decode_attn_planned that also writes ln q~ per 16-token tile,
    tile_lmass [B, Hq, max_pages, P/16] (float32)."""
    B, Hq, _ = q.shape
    _check(lib.paged_decode_attn_scored(ctypes.byref(cache), _ptr(plan), _nbytes(plan), _ptr(q), B, Hq, max_pages,
                                        float(sm_scale), _ptr(out), _ptr(lse), _ptr(tile_lmass), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(counters), _stream()))


def paged_decode_attn_append(cache, plan, q, max_pages, sm_scale, new_kv, new_page, new_slot, out, lse, workspace,
                             counters=None):
    """Planned decode over the cached tokens plus the step's new token
    (new_kv [B, Hkv, 2, d] float32 or bf16), which is also FP8-appended at
    (new_page[b], new_slot[b])."""
    B, Hq, _ = q.shape
    bf = 1 if new_kv.dtype == torch.bfloat16 else 0
    _check(lib.paged_decode_attn_append(ctypes.byref(cache), _ptr(plan), _nbytes(plan), _ptr(q), B, Hq, max_pages,
                                        float(sm_scale), _ptr(new_kv), bf, _ptr(new_page), _ptr(new_slot),
                                        _ptr(out), _ptr(lse), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(counters), _stream()))


def paged_prefill_attn_workspace_size(cache, batch, num_q_heads, chunk, max_pages) -> int:
    return int(lib.paged_prefill_attn_workspace_size(batch, num_q_heads, chunk, max_pages, ctypes.byref(cache)))


def paged_prefill_attn_planned(cache, plan, q, max_pages, sm_scale, out, lse, workspace, counters=None):
    """Causal attention of each request's next C tokens (q [B, C, Hq, d] bf16,
    already appended to the cache) -> out [B, C, Hq, d], lse [B, C, Hq]."""
    B, C, Hq, _ = q.shape
    _check(lib.paged_prefill_attn_planned(ctypes.byref(cache), _ptr(plan), _nbytes(plan), _ptr(q), B, Hq, C, max_pages,
                                          float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _ptr(counters), _stream()))


def page_mass_collect(seq_lens, tile_lmass, heads, beta, score, r_out=None):
    """Running page score (Eq. 8-9) from a scored decode; `heads` is a host
    sequence of q-head ids, score [B, max_pages] float32 is updated in place."""
    B, Hq, max_pages, T = tile_lmass.shape
    hs = (ctypes.c_int32 * max(1, len(heads)))(*[int(h) for h in heads])
    _check(lib.page_mass_collect(B, Hq, max_pages, 16 * T, _ptr(seq_lens), _ptr(tile_lmass),
                                 ctypes.cast(hs, ctypes.c_void_p), len(heads), float(beta), _ptr(score),
                                 _ptr(r_out), _stream()))


def paged_decode_attn(cache, q, block_table, page_format, seq_lens, sm_scale, out, lse, workspace, counters=None):
    B, Hq, _ = q.shape
    max_pages = block_table.shape[1]
    _check(lib.paged_decode_attn(ctypes.byref(cache), _ptr(q), B, Hq, _ptr(block_table), _ptr(page_format),
                                 max_pages, _ptr(seq_lens), float(sm_scale), _ptr(out), _ptr(lse),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(counters),
                                 _stream()))


def paged_decode_attn_noalloc(cache, q, block_table, page_format, seq_lens, sm_scale, out, lse, counters=None):
    """paged_decode_attn with the library's fixed per-GPU workspace array
    (nothing is allocated)."""
    B, Hq, _ = q.shape
    max_pages = block_table.shape[1]
    _check(lib.paged_decode_attn_noalloc(ctypes.byref(cache), _ptr(q), B, Hq, _ptr(block_table), _ptr(page_format),
                                         max_pages, _ptr(seq_lens), float(sm_scale), _ptr(out), _ptr(lse),
                                         _ptr(counters), _stream()))


def read_counters(counters_tensor) -> dict:
    """Counters live in a uint8 device tensor of ctypes.sizeof(Counters) bytes."""
    raw = counters_tensor.cpu().numpy().tobytes()
    c = Counters.from_buffer_copy(raw)
    return {k: int(getattr(c, k)) for k in COUNTER_FIELDS}
