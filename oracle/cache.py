"""Build a whole paged cache (pools and tables) the way the encoders must.

Minima-KV, algorithm 1 (Append, Retier) and section 4.3: new KV is written
to FP8 Recent pages; eligible old pages are converted FP8 -> TQ3 in batches
by normalize-rotate-pack; the conversion never changes the logical mapping.
Readings fixed here: a demoted page is encoded from the fp32 rows an FP8 page
decodes to, x = fp32(value(e) * scale); the small parity workloads may also
encode Stale pages straight from fp32 rows. Slots of a partial last page that
hold no token are all-zero (codes 0, scale/sigma 0).
"""
from __future__ import annotations

import numpy as np

from . import fp8 as _fp8
from . import layout as _layout
from . import tq as _tq
from .attention import FMT_FP8, FMT_TQ2, FMT_TQ3, FMT_TQK, TQ_BITS, TQF_LEVELS, head_block_bytes


def encode_page(fmt: int, Kp: np.ndarray, Vp: np.ndarray, n_valid: int, signs_words,
                stale_source: str = "fp32", tqk=None, heads=None) -> np.ndarray:
    """One page (all KV heads). Kp, Vp float32 [P, Hkv, d] -> page bytes.
    `heads` restricts the encoded KV heads (other head blocks stay zero)."""
    P, Hkv, d = Kp.shape
    Kp = np.array(Kp, dtype=np.float32)
    Vp = np.array(Vp, dtype=np.float32)
    Kp[n_valid:] = 0
    Vp[n_valid:] = 0
    blocks = []
    for g in range(Hkv):
        if heads is not None and g not in heads:
            blocks.append(np.zeros(head_block_bytes(fmt, P, d), np.uint8))
            continue
        k, v = Kp[:, g, :], Vp[:, g, :]
        if fmt == FMT_FP8:
            kc, ks = _fp8.fp8_encode(k)
            vc, vs = _fp8.fp8_encode(v)
            blocks.append(_layout.fp8_pack_head(kc, vc, ks, vs))
            continue
        if stale_source == "fp8":
            kc8, ks8 = _fp8.fp8_encode(k)
            vc8, vs8 = _fp8.fp8_encode(v)
            k = _fp8.fp8_decode_f32(kc8, ks8)
            v = _fp8.fp8_decode_f32(vc8, vs8)
        sk = _tq.signs_from_bits(signs_words[g, 0], d)
        sv = _tq.signs_from_bits(signs_words[g, 1], d)
        if fmt in TQ_BITS:
            b = TQ_BITS[fmt]
            kc, ksig = _tq.tq_encode(k, sk, b)
            vc, vsig = _tq.tq_encode(v, sv, b)
            blocks.append(_layout.tq_pack_head(kc, vc, ksig, vsig, b))
        elif fmt == FMT_TQK:
            from . import tqk as _tqk
            blocks.append(_tqk.encode_page_head(k, v, sk, sv, tqk[g]))
        elif fmt in TQF_LEVELS:
            from . import tqf as _tqf
            L = TQF_LEVELS[fmt]
            kc, ksig = _tqf.encode(k, sk, L)
            vc, vsig = _tqf.encode(v, sv, L)
            blocks.append(_layout.tqf_pack_head(kc, vc, ksig, vsig, L))
        else:
            raise ValueError(fmt)
    return np.concatenate(blocks)


def build_pools(w, plan, kv_of_request, signs_words, stale_source: str = "fp32", tqk=None,
                requests=None, heads=None):
    """Pools {format: uint8 [pool pages, page bytes]} holding every page of the
    plan (or of the listed requests / KV heads only; the rest stays zero).
    kv_of_request(b) -> (K, V) float32 [N_b, Hkv, d]."""
    P, Hkv, d = w.page_size, w.num_kv_heads, w.head_dim
    pools = {}
    for f, n in plan.pool_pages.items():
        if n:
            pools[f] = np.zeros((n, Hkv * head_block_bytes(f, P, d)), dtype=np.uint8)
    for b in (range(plan.seq_lens.shape[0]) if requests is None else requests):
        N = int(plan.seq_lens[b])
        if N == 0:
            continue
        K, V = kv_of_request(b)
        n_pages = (N + P - 1) // P
        for p in range(n_pages):
            f = int(plan.page_format[b, p])
            pid = int(plan.block_table[b, p])
            nv = min(P, N - p * P)
            Kp = np.zeros((P, Hkv, d), dtype=np.float32)
            Vp = np.zeros((P, Hkv, d), dtype=np.float32)
            Kp[:nv] = K[p * P:p * P + nv]
            Vp[:nv] = V[p * P:p * P + nv]
            pools[f][pid] = encode_page(f, Kp, Vp, nv, signs_words, stale_source, tqk, heads)
    return pools
