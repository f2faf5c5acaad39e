"""Build a paged mixed-format layer cache on the GPU with the library's own
encoders (Minima-KV algorithm 1: Append writes FP8 pages; Retier converts
eligible pages to TQ in batches; section 4.3).

Everything here is plumbing around the C ABI: torch allocates the pools and
tables, the HIP encoders write every byte.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import (FMT_FP8, FMT_TQ2, FMT_TQ3, FMT_TQF5, FMT_TQF6, FMT_TQK, SRC_F32_ROWS, SRC_FP8_PAGES, Counters,
               kv_encode_fp8, kv_encode_tq2, kv_encode_tq3, kv_encode_tqf5, kv_encode_tqf6, kv_encode_tqk, make_cache,
               page_bytes)

_TQ_ENCODERS = {FMT_TQ3: kv_encode_tq3, FMT_TQ2: kv_encode_tq2, FMT_TQK: kv_encode_tqk, FMT_TQF5: kv_encode_tqf5,
                FMT_TQF6: kv_encode_tqf6}


class GpuLayer:
    """One layer's pools on a device plus its cache descriptor."""

    def __init__(self, num_kv_heads, head_dim, page_size, pool_pages: dict, signs_words: np.ndarray, device="cuda",
                 tqk_perm: np.ndarray = None):
        self.Hkv, self.d, self.P = num_kv_heads, head_dim, page_size
        self.device = device
        self.pools = {}
        for f in (FMT_FP8, FMT_TQ3, FMT_TQ2, FMT_TQK, FMT_TQF5, FMT_TQF6):
            n = int(pool_pages.get(f, 0))
            if n:
                self.pools[f] = torch.zeros((n, page_bytes(f, num_kv_heads, head_dim, page_size)),
                                            dtype=torch.uint8, device=device)
        self.signs = torch.from_numpy(np.ascontiguousarray(signs_words).view(np.int32)).to(device)
        self.perm = None
        if tqk_perm is not None:
            self.perm = torch.from_numpy(np.ascontiguousarray(tqk_perm, dtype=np.uint16).view(np.int16)).to(device)
        self.cache = make_cache(num_kv_heads, head_dim, page_size, self.pools.get(FMT_FP8),
                                self.pools.get(FMT_TQ3), self.pools.get(FMT_TQ2), self.signs,
                                self.pools.get(FMT_TQK), self.perm, self.pools.get(FMT_TQF5),
                                self.pools.get(FMT_TQF6))

    def pool_bytes(self, fmt):
        return self.pools[fmt].cpu().numpy() if fmt in self.pools else None


def _page_rows(K, V, P, pages, n_tokens):
    """float32 [n, P, Hkv, 2, d] rows of the listed logical pages (zero padded)
    and the number of filled slots per page."""
    Hkv, d = K.shape[1], K.shape[2]
    rows = torch.zeros((len(pages), P, Hkv, 2, d), dtype=torch.float32, device=K.device)
    valid = []
    for i, p in enumerate(pages):
        t0 = p * P
        nv = min(P, n_tokens - t0)
        rows[i, :nv, :, 0] = K[t0:t0 + nv]
        rows[i, :nv, :, 1] = V[t0:t0 + nv]
        valid.append(nv)
    return rows, torch.tensor(valid, dtype=torch.int32, device=K.device)


def build_layer(layer: GpuLayer, page_format: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                kv_of_request, stale_source: str = "fp32", staging_pages: int = 0, chunk_pages: int = 4096):
    """Encode every page of every request.

    kv_of_request(b) -> (K, V) float32 device tensors [N_b, Hkv, d].
    FP8 pages are appended token by token. Stale pages (any TQ format) are encoded
    straight from fp32 rows (stale_source="fp32") or, as a demotion, first
    appended to a staging FP8 pool and converted from there ("fp8")."""
    P, Hkv, d, dev = layer.P, layer.Hkv, layer.d, layer.device
    stage = None
    if stale_source == "fp8":
        n_stage = max(1, staging_pages or chunk_pages)
        stage = GpuLayer(Hkv, d, P, {FMT_FP8: n_stage}, np.zeros((Hkv, 2, d // 32), np.uint32), dev)
    for b in range(len(seq_lens)):
        N = int(seq_lens[b])
        if N == 0:
            continue
        K, V = kv_of_request(b)
        n_pages = (N + P - 1) // P
        fmt = page_format[b, :n_pages]
        pid = block_table[b, :n_pages]
        # FP8 Recent / Anchor pages: per-token append
        fp8_pages = np.nonzero(fmt == FMT_FP8)[0]
        if len(fp8_pages):
            tok = np.concatenate([np.arange(p * P, min(N, p * P + P)) for p in fp8_pages])
            src = torch.stack([K[tok], V[tok]], dim=2).contiguous()      # [n, Hkv, 2, d]
            dpage = torch.from_numpy(pid[tok // P].astype(np.int32)).to(dev)
            dslot = torch.from_numpy((tok % P).astype(np.int32)).to(dev)
            kv_encode_fp8(layer.cache, src, dpage, dslot)
        for f, enc in _TQ_ENCODERS.items():
            pages = np.nonzero(fmt == f)[0]
            for c0 in range(0, len(pages), chunk_pages):
                chunk = pages[c0:c0 + chunk_pages]
                rows, valid = _page_rows(K, V, P, chunk, N)
                dst = torch.from_numpy(pid[chunk].astype(np.int32)).to(dev)
                if stale_source == "fp32":
                    enc(layer.cache, SRC_F32_ROWS, dst, src=rows, page_valid=valid)
                else:
                    # Append into staging FP8 pages, then convert them (Retier)
                    n = len(chunk)
                    assert n <= stage.pools[FMT_FP8].shape[0]
                    flat = rows.reshape(n * P, Hkv, 2, d)
                    keep = (torch.arange(P, device=dev)[None, :] < valid[:, None]).reshape(-1)
                    tok_idx = torch.nonzero(keep).squeeze(1)
                    spage = (tok_idx // P).to(torch.int32)
                    sslot = (tok_idx % P).to(torch.int32)
                    stage.pools[FMT_FP8].zero_()
                    kv_encode_fp8(stage.cache, flat[tok_idx].contiguous(), spage, sslot)
                    src_ids = torch.arange(n, dtype=torch.int32, device=dev)
                    demote = make_cache(Hkv, d, P, stage.pools[FMT_FP8], layer.pools.get(FMT_TQ3),
                                        layer.pools.get(FMT_TQ2), layer.signs, layer.pools.get(FMT_TQK),
                                        layer.perm, layer.pools.get(FMT_TQF5), layer.pools.get(FMT_TQF6))
                    enc(demote, SRC_FP8_PAGES, dst, src_page=src_ids, page_valid=valid)
    return layer


def new_counters(device="cuda"):
    return torch.zeros(ctypes.sizeof(Counters), dtype=torch.uint8, device=device)
