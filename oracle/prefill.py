"""Chunked prefill attention over a paged mixed-format cache (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Block-GTQ (paperpeel 2606.24033) appendix H.5 ("packed chunked prefill"):
a chunk of new tokens attends causally to the compressed cache and to the
chunk itself, with an online softmax and no decoded copy of the cache. The
plain definition computed here: the chunk's own K/V are already appended to
the cache (FP8 Recent pages, as every new token is), so query token c of a
chunk starting at position N0 attends to cache tokens 0 .. N0 + c, in fp64,
each page read through its own format's dequantization (oracle.attention).

Readings fixed here: the chunk is one request's next C tokens; query head h
reads KV head h // (Hq / Hkv); sm_scale is an argument; q is bf16 widened
exactly.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_ref, dequant_request


def prefill_ref(pools, block_table_row, format_row, n0: int, q_bits, sm_scale: float, P: int, Hkv: int, d: int,
                signs_words, tqk=None, heads=None):
    """q_bits uint16 [C, Hq, d] (bf16 bits) of the tokens at positions
    n0 .. n0 + C - 1 -> (O [C, Hq, d], lse [C, Hq]) in fp64. `heads` limits
    the work to the q-heads of the listed KV heads (the others stay O = 0,
    lse = -inf)."""
    q = (np.asarray(q_bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    C, Hq = q.shape[0], q.shape[1]
    G = Hq // Hkv
    K, V = dequant_request(pools, block_table_row, format_row, n0 + C, P, Hkv, d, signs_words, heads=heads, tqk=tqk)
    O = np.zeros(q.shape)
    lse = np.full(q.shape[:2], -np.inf)
    for c in range(C):
        if heads is None:
            O[c], lse[c] = attention_ref(q[c], K[:n0 + c + 1], V[:n0 + c + 1], sm_scale)
            continue
        for g in heads:
            hs = slice(g * G, (g + 1) * G)
            O[c, hs], lse[c, hs] = attention_ref(q[c, hs], K[:n0 + c + 1, g:g + 1], V[:n0 + c + 1, g:g + 1],
                                                 sm_scale)
    return O, lse
