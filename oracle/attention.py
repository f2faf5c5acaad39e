"""Reference decode attention over a paged mixed-format cache (fp64).

Minima-KV, section 3.3: for one query tile the runtime partitions logical
pages by format; partition j yields a partial maximum m_j, exponential sum
l_j and normalized partial output O_j = l_j^-1 sum_{i in j} e^{s_i - m_j} v_i;
Eq. 11-13 merge them (m = max_j m_j, l = sum_j e^{m_j - m} l_j,
O = sum_j e^{m_j - m} l_j O_j / l), which is algebraically the same as
attention over the concatenated logical cache up to codec error and rounding.

The oracle therefore computes the plain definition: softmax attention in fp64
over every cached token of the request, in logical order, using each page's
own dequantized K and V (FP8: value * scale; TQ: sigma * R^T c). The query is
the bf16 query widened exactly. GQA maps q-head h to KV head h // (Hq / Hkv);
sm_scale is an argument (1/sqrt(d) in every workload). A request with no
tokens gives O = 0 and lse = -inf.
"""
from __future__ import annotations

import math

import numpy as np

from . import fp8 as _fp8
from . import layout as _layout
from . import tq as _tq

FMT_FP8, FMT_TQ3, FMT_TQ2, FMT_TQK, FMT_TQF5, FMT_TQF6 = 0, 1, 2, 3, 4, 5
TQ_BITS = {FMT_TQ3: 3, FMT_TQ2: 2}
TQF_LEVELS = {FMT_TQF5: 5, FMT_TQF6: 6}     # fractional-level TQ (SemKV section 4.1)


def attention_ref(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float):
    """q [Hq, d]; K, V [N, Hkv, d] -> (O [Hq, d], lse [Hq]) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, d = q.shape
    N, Hkv, _ = K.shape
    G = Hq // Hkv
    O = np.zeros((Hq, d))
    lse = np.full(Hq, -np.inf)
    if N == 0:
        return O, lse
    for h in range(Hq):
        g = h // G
        s = sm_scale * (K[:, g, :] @ q[h])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        O[h] = (e @ V[:, g, :]) / l
        lse[h] = m + math.log(l)
    return O, lse


def partial_ref(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float, idx):
    """(m, l, O_bar) of one partition (Minima-KV Eq. 6 and section 3.3)."""
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    idx = np.asarray(idx, dtype=np.int64)
    m = np.full(Hq, -np.inf)
    l = np.zeros(Hq)
    Ob = np.zeros((Hq, d))
    if idx.size == 0:
        return m, l, Ob
    for h in range(Hq):
        g = h // G
        s = sm_scale * (np.asarray(K, dtype=np.float64)[idx, g, :] @ q[h])
        m[h] = s.max()
        e = np.exp(s - m[h])
        l[h] = e.sum()
        Ob[h] = (e @ np.asarray(V, dtype=np.float64)[idx, g, :]) / l[h]
    return m, l, Ob


def merge_ref(parts):
    """Minima-KV Eq. 11-13 over partials [(m [H], l [H], O_bar [H, d])].
    Empty partials (m = -inf, l = 0) contribute nothing. Returns (O, lse)."""
    ms = np.stack([p[0] for p in parts])
    ls = np.stack([p[1] for p in parts])
    Os = np.stack([p[2] for p in parts])
    m = ms.max(axis=0)                                           # Eq. 11
    with np.errstate(invalid="ignore"):
        wgt = np.where(ls > 0, np.exp(ms - m[None, :]), 0.0)
    l = (wgt * ls).sum(axis=0)                                    # Eq. 12
    num = ((wgt * ls)[:, :, None] * Os).sum(axis=0)
    O = np.where(l[:, None] > 0, num / np.where(l > 0, l, 1.0)[:, None], 0.0)   # Eq. 13
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, lse


# --------------------------------------------------------------------------
# paged cache walking
# --------------------------------------------------------------------------
def dequant_page_head(fmt: int, blk: np.ndarray, P: int, d: int, signs_k, signs_v, tqk=None):
    """Dequantized K, V [P, d] (fp64) of one head block of one page."""
    if fmt == FMT_FP8:
        kc, vc, ks, vs = _layout.fp8_unpack_head(blk, P, d)
        return _fp8.fp8_decode(kc, ks), _fp8.fp8_decode(vc, vs)
    if fmt in TQ_BITS:
        b = TQ_BITS[fmt]
        kc, vc, ksig, vsig = _layout.tq_unpack_head(blk, P, d, b)
        return _tq.tq_decode(kc, ksig, signs_k, b), _tq.tq_decode(vc, vsig, signs_v, b)
    if fmt == FMT_TQK:
        from . import tqk as _tqk
        return _tqk.dequant_page_head(blk, P, d, signs_k, signs_v, tqk)
    if fmt in TQF_LEVELS:
        from . import tqf as _tqf
        L = TQF_LEVELS[fmt]
        kc, vc, ksig, vsig = _layout.tqf_unpack_head(blk, P, d, L)
        return _tqf.decode(kc, ksig, signs_k, L), _tqf.decode(vc, vsig, signs_v, L)
    raise ValueError(f"unknown format tag {fmt}")


def head_block_bytes(fmt: int, P: int, d: int) -> int:
    if fmt == FMT_FP8:
        return _layout.fp8_head_bytes(P, d)
    if fmt in TQ_BITS:
        return _layout.tq_head_bytes(P, d, TQ_BITS[fmt])
    if fmt == FMT_TQK:
        from . import tqk as _tqk
        return _tqk.head_bytes(P, d)
    if fmt in TQF_LEVELS:
        return _layout.tqf_head_bytes(P, d, TQF_LEVELS[fmt])
    raise ValueError(fmt)


def dequant_request(pools, block_table_row, format_row, seq_len: int, P: int, Hkv: int, d: int,
                    signs_words, heads=None, tqk=None):
    """Dequantized K, V [N, Hkv, d] of one request in logical order.
    `signs_words` uint32 [Hkv, 2, d/32]; `heads` restricts the KV heads filled."""
    N = int(seq_len)
    n_pages = (N + P - 1) // P
    heads = range(Hkv) if heads is None else heads
    K = np.zeros((n_pages * P, Hkv, d))
    V = np.zeros((n_pages * P, Hkv, d))
    for p in range(n_pages):
        f = int(format_row[p])
        pid = int(block_table_row[p])
        hb = head_block_bytes(f, P, d)
        page = pools[f][pid]
        for g in heads:
            blk = page[g * hb:(g + 1) * hb]
            sk = _tq.signs_from_bits(signs_words[g, 0], d)
            sv = _tq.signs_from_bits(signs_words[g, 1], d)
            k, v = dequant_page_head(f, blk, P, d, sk, sv, None if tqk is None else tqk[g])
            K[p * P:(p + 1) * P, g] = k
            V[p * P:(p + 1) * P, g] = v
    return K[:N], V[:N]


def paged_decode_ref(pools, block_table, page_format, seq_lens, q_bits, sm_scale: float,
                     P: int, Hkv: int, d: int, signs_words, requests=None, tqk=None, heads=None):
    """O [B, Hq, d], lse [B, Hq] for the requests listed (all by default);
    with `heads`, only the q-heads of those KV heads are computed (the rest
    stay O = 0, lse = -inf). q_bits: bf16 bit patterns uint16 [B, Hq, d]."""
    q = (np.asarray(q_bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    B, Hq, _ = q.shape
    O = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    G = Hq // Hkv
    for b in (range(B) if requests is None else requests):
        K, V = dequant_request(pools, block_table[b], page_format[b], int(seq_lens[b]), P, Hkv, d,
                               signs_words, heads=heads, tqk=tqk)
        if heads is None:
            O[b], lse[b] = attention_ref(q[b], K, V, sm_scale)
            continue
        for g in heads:
            hs = slice(g * G, (g + 1) * G)
            O[b, hs], lse[b, hs] = attention_ref(q[b, hs], K[:, g:g + 1], V[:, g:g + 1], sm_scale)
    return O, lse
