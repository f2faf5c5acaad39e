"""Seeded synthetic inputs for mixed-format paged decode attention.

This module only draws random numbers and lays out page tables. It holds none
of the method's arithmetic (no codec, no rotation, no attention): both the CPU
oracle and the HIP path consume what it returns.

Workloads (shapes and value distributions follow the Minima-KV page, section
4.1 and section 6.3, and the Block-GTQ page, appendix I.4; the lengths and the
per-page format mixes are the five named workloads below):

  tiny       1 layer, B=1, Hq=4, Hkv=1, d=128, N=1,024, page 16. FP8 = page 0
             (sink) + the last 256 tokens; the rest TQ3.
  l27b       Qwen3.6-27B full-attention layer shape: B=1, Hq=24, Hkv=4, d=256,
             N=16,384, page 16; FP8 = the last 1,024 tokens + 4 Anchor pages
             (page 0 + 3 seeded); the rest TQ3; 2% outlier channels x8.
  canary     2 requests x 59,008 tokens, 16 layers, Hq=24, Hkv=4, d=256, page
             16; per request FP8 = the last 2,048 tokens + 8 Anchor pages
             (page 0 + 7 seeded); the rest TQ3.
  l70b       B=4, Hq=64, Hkv=8, d=128, N=131,072, page 32; the last 4,096
             tokens FP8, the rest TQK (grouped mixed-rate keys); per (KV head,
             RoPE block) variance log-uniform in [1e-3, 1e1].
  serving    B=64, N_b ~ U{4,096..32,768}, Hq=32, Hkv=8, d=128, page 16; per
             request FP8 / TQ3 / TQ2 by seeded page-importance rank
             (floor(0.2 P_b) / floor(0.7 P_b) - floor(0.2 P_b) / rest).
  frac       fractional-level Stale pages (SemKV section 4.1 bit widths
             log2 6 and log2 5): B=16, N_b ~ U{4,096..16,384}, Hq=32, Hkv=8,
             d=128, page 16; per request FP8 / TQF6 / TQF5 by seeded
             page-importance rank (floor(0.2 P_b) / floor(0.5 P_b) -
             floor(0.2 P_b) / rest).

Every array comes from numpy PCG64 keyed by
SeedSequence([seed, workload id, layer, request, stream]).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

FMT_FP8 = 0
FMT_TQ3 = 1
FMT_TQ2 = 2
FMT_TQK = 3
FMT_TQF5 = 4
FMT_TQF6 = 5
ALL_FORMATS = (FMT_FP8, FMT_TQ3, FMT_TQ2, FMT_TQK, FMT_TQF5, FMT_TQF6)
FMT_NAMES = {FMT_FP8: "fp8", FMT_TQ3: "tq3", FMT_TQ2: "tq2", FMT_TQK: "tqk", FMT_TQF5: "tqf5", FMT_TQF6: "tqf6"}

# stream ids inside the seed sequence
_S_LENGTHS, _S_FORMAT, _S_TABLE, _S_K, _S_V, _S_Q, _S_SIGNS, _S_OUTLIER, _S_VAR, _S_RATES = range(10)

_WORKLOAD_IDS = {"tiny": 1, "l27b": 2, "canary": 3, "l70b": 4, "serving": 5, "frac": 6}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    # fixed length for every request, or None for seeded lengths
    seq_len: Optional[int]
    seq_len_range: Optional[tuple] = None
    recent_tokens: int = 0          # FP8 Recent window (tokens, page aligned)
    anchor_pages: int = 0           # FP8 Anchors incl. the sink page 0
    outlier_frac: float = 0.0       # fraction of channels scaled by outlier_gain
    outlier_gain: float = 1.0
    stale_format: int = FMT_TQ3
    importance_split: Optional[tuple] = None  # (fp8 frac, fp8+mid frac) -> low rest
    split_formats: tuple = (FMT_TQ3, FMT_TQ2)  # (mid, low) formats of an importance split
    block_var_range: Optional[tuple] = None   # per-RoPE-block variance range
    tqk_rates: Optional[tuple] = None         # (#2-bit, #3-bit, #4-bit) blocks
    pool_slack: float = 0.25

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 1, 4, 1, 128, 16, 1024, recent_tokens=256, anchor_pages=1),
    "l27b": Workload("l27b", 1, 1, 24, 4, 256, 16, 16384, recent_tokens=1024, anchor_pages=4,
                     outlier_frac=0.02, outlier_gain=8.0),
    "canary": Workload("canary", 16, 2, 24, 4, 256, 16, 59008, recent_tokens=2048, anchor_pages=8),
    "l70b": Workload("l70b", 1, 4, 64, 8, 128, 32, 131072, recent_tokens=4096, anchor_pages=0,
                     stale_format=FMT_TQK, block_var_range=(1e-3, 1e1), tqk_rates=(16, 32, 16)),
    "serving": Workload("serving", 1, 64, 32, 8, 128, 16, None, seq_len_range=(4096, 32768),
                        importance_split=(0.2, 0.7)),
    "frac": Workload("frac", 1, 16, 32, 8, 128, 16, None, seq_len_range=(4096, 16384),
                     importance_split=(0.2, 0.5), split_formats=(FMT_TQF6, FMT_TQF5)),
}


def rng(seed: int, workload: str, layer: int, request: int, stream: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), _WORKLOAD_IDS.get(workload, 99), int(layer), int(request), int(stream)])
    return np.random.Generator(np.random.PCG64(ss))


def scaled(w: Workload, **over) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    return dataclasses.replace(w, **over)


# --------------------------------------------------------------------------
# page tables
# --------------------------------------------------------------------------
@dataclasses.dataclass
class PagePlan:
    seq_lens: np.ndarray        # int32 [B]
    page_format: np.ndarray     # uint8 [B, max_pages] (255 beyond a request's pages)
    block_table: np.ndarray     # int32 [B, max_pages] (-1 beyond a request's pages)
    pool_pages: Dict[int, int]  # format -> pool size (pages), with slack
    max_pages: int


def _formats_for_request(w: Workload, n_pages: int, seed: int, b: int) -> np.ndarray:
    fmt = np.full(n_pages, w.stale_format, dtype=np.uint8)
    if w.importance_split is not None:
        # seeded importance u_p ~ U(0,1), ranked descending (SemKV top-r floor rule)
        r = rng(seed, w.name, 0, b, _S_FORMAT)
        u = r.random(n_pages)
        order = np.argsort(-u, kind="stable")
        n8 = int(np.floor(w.importance_split[0] * n_pages))
        n83 = int(np.floor(w.importance_split[1] * n_pages))
        mid, low = w.split_formats
        fmt[:] = low
        fmt[order[:n8]] = FMT_FP8
        fmt[order[n8:n83]] = mid
        return fmt
    n_recent = min(n_pages, w.recent_tokens // w.page_size)
    if n_recent:
        fmt[n_pages - n_recent:] = FMT_FP8
    if w.anchor_pages > 0 and n_pages > 0:
        fmt[0] = FMT_FP8  # sink
        cand = np.arange(1, n_pages - n_recent)
        k = min(len(cand), w.anchor_pages - 1)
        if k > 0:
            r = rng(seed, w.name, 0, b, _S_FORMAT)
            fmt[r.choice(cand, size=k, replace=False)] = FMT_FP8
    return fmt


def make_page_plan(w: Workload, seed: int = 0) -> PagePlan:
    B, P = w.batch, w.page_size
    if w.seq_len is not None:
        lens = np.full(B, w.seq_len, dtype=np.int32)
    else:
        lo, hi = w.seq_len_range
        lens = rng(seed, w.name, 0, 0, _S_LENGTHS).integers(lo, hi + 1, size=B).astype(np.int32)
    npages = (lens.astype(np.int64) + P - 1) // P
    max_pages = int(npages.max()) if B else 0
    fmt = np.full((B, max_pages), 255, dtype=np.uint8)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    for b in range(B):
        fmt[b, :npages[b]] = _formats_for_request(w, int(npages[b]), seed, b)
    pools = {}
    for f in ALL_FORMATS:
        used = int((fmt == f).sum())
        size = int(np.ceil(used * (1.0 + w.pool_slack))) if used else 0
        pools[f] = size
        if used == 0:
            continue
        # one shared, fragmented pool per format: a seeded permutation of its ids
        ids = rng(seed, w.name, 0, f, _S_TABLE).permutation(size)[:used].astype(np.int32)
        k = 0
        for b in range(B):
            sel = np.nonzero(fmt[b, :npages[b]] == f)[0]
            table[b, sel] = ids[k:k + len(sel)]
            k += len(sel)
    return PagePlan(lens, fmt, table, pools, max_pages)


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------
def make_kv(w: Workload, seed: int, layer: int, request: int, n_tokens: int):
    """K, V float32 [n_tokens, Hkv, d] for one request of one layer."""
    H, d = w.num_kv_heads, w.head_dim
    out = []
    for role, stream in ((0, _S_K), (1, _S_V)):
        x = rng(seed, w.name, layer, request, stream).standard_normal((n_tokens, H, d), dtype=np.float32)
        if w.outlier_frac > 0:
            n_out = int(round(w.outlier_frac * d))
            r = rng(seed, w.name, layer, 1000 + role, _S_OUTLIER)
            for h in range(H):
                ch = r.choice(d, size=n_out, replace=False)
                x[:, h, ch] *= np.float32(w.outlier_gain)
        if w.block_var_range is not None:
            lo, hi = np.log(w.block_var_range[0]), np.log(w.block_var_range[1])
            r = rng(seed, w.name, layer, 1000 + role, _S_VAR)
            var = np.exp(r.uniform(lo, hi, size=(H, d // 2)))
            std = np.sqrt(var).astype(np.float32)
            x *= np.repeat(std, 2, axis=1)[None, :, :]
        out.append(x)
    return out[0], out[1]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def make_q(w: Workload, seed: int, layer: int):
    """q as bf16 bit patterns uint16 [B, Hq, d] (drawn N(0,1))."""
    x = rng(seed, w.name, layer, 0, _S_Q).standard_normal((w.batch, w.num_q_heads, w.head_dim), dtype=np.float32)
    return bf16_round(x)


def make_signs(w: Workload, seed: int, layer: int) -> np.ndarray:
    """Rotation sign bits uint32 [Hkv, 2, d/32]; bit j of word j//32 set means -1.

    Role 0 is K, role 1 is V. For grouped keys each segment gets its own draw
    (they are concatenated in segment order, so one word array still covers d)."""
    H, d = w.num_kv_heads, w.head_dim
    words = np.zeros((H, 2, d // 32), dtype=np.uint32)
    for h in range(H):
        for role in range(2):
            bits = rng(seed, w.name, layer, 2000 + 2 * h + role, _S_SIGNS).integers(0, 2, size=d)
            for j in range(d):
                if bits[j]:
                    words[h, role, j // 32] |= np.uint32(1 << (j % 32))
    return words


def make_tqk_rates(w: Workload, seed: int, layer: int) -> np.ndarray:
    """Per (KV head, RoPE block) key bit width, int8 [Hkv, d/2] with exactly
    n2/n3/n4 blocks at 2/3/4 bits, seeded placement."""
    n2, n3, n4 = w.tqk_rates
    H, nb = w.num_kv_heads, w.head_dim // 2
    assert n2 + n3 + n4 == nb
    rates = np.zeros((H, nb), dtype=np.int8)
    for h in range(H):
        perm = rng(seed, w.name, layer, 3000 + h, _S_RATES).permutation(nb)
        rates[h, perm[:n2]] = 2
        rates[h, perm[n2:n2 + n3]] = 3
        rates[h, perm[n2 + n3:]] = 4
    return rates


def make_tqk_perm(w: Workload, seed: int, layer: int) -> np.ndarray:
    """Key coordinate order of the grouped mixed-rate layout, uint16 [Hkv, d]:
    entry j is the original coordinate stored at position j. The RoPE blocks
    of make_tqk_rates are taken by width (2, 3, then 4 bits), ascending block
    index inside a width, each block giving coordinates 2i, 2i + 1."""
    rates = make_tqk_rates(w, seed, layer)
    out = np.zeros((w.num_kv_heads, w.head_dim), dtype=np.uint16)
    for h in range(w.num_kv_heads):
        order = np.argsort(rates[h], kind="stable")
        out[h] = np.stack([2 * order, 2 * order + 1], axis=1).reshape(-1)
    return out


def stale_demote_sources(plan: PagePlan, fmt: int):
    """(request, logical page) pairs of every page tagged `fmt`, in request order."""
    out: List[tuple] = []
    for b in range(plan.seq_lens.shape[0]):
        for p in np.nonzero(plan.page_format[b] == fmt)[0]:
            out.append((b, int(p)))
    return out
