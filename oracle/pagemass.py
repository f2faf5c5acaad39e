"""Attention page mass of a mixed-format decode step, and its running score.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Minima-KV (arxiv 2608.23834), section 3.1, Eq. 6-9, and section 4.2: page
mass taken from format-specific partitions must be normalized by the same
global softmax as the attention output. For query head h, partition j
reports m_j = max_{i in j} s_i and l_j = sum_{i in j} e^{s_i - m_j} (Eq. 6);
with m = max_j m_j and l = sum_j e^{m_j - m} l_j, the local mass of page p in
partition j and the partition's global weight are

    rho_p^(j) = l_j^-1 sum_{i in p} e^{s_i - m_j}      (Eq. 7)
    w_j       = e^{m_j - m} l_j / l                      (Eq. 8)

and q_{h,p} = w_{j(p)} rho_p^(j(p)) is the globally normalized page mass. The
collector conditions on page-addressable mass: q~_{h,p} = q_{h,p} / sum_p'
q_{h,p'}. Over a sampled head set H: r_p = |H|^-1 sum_{h in H} q~_{h,p}, and
the running score is a_p <- beta a_p + (1 - beta) r_p (Eq. 9).

Readings fixed here (the pages leave them open):
  * the partitions are the format classes of the request (its FP8 pages,
    its TQ3 pages, ...), as in the mixed-format decode of section 3.3;
  * scores s_i are the decode's own: sm_scale * q_h . k_hat_i over the
    dequantized cache, the bf16 query widened exactly, in fp64;
  * "page" is a logical page of the request; there is no learned sink state
    in these caches, so the normalization by sum_p' q only removes rounding;
  * pages at or past ceil(N_b / P) are not live: their r and a are left out
    (a stays as it was); a request with no tokens updates nothing.
"""
from __future__ import annotations

import numpy as np

from .attention import dequant_request


def page_mass_ref(pools, block_table, page_format, seq_lens, q_bits, sm_scale: float, P: int, Hkv: int, d: int,
                  signs_words, tqk=None, requests=None, heads=None):
    """q [B, Hq, max_pages] (fp64): the globally normalized page mass of
    Eq. 6-8, partitions = format classes. Pages that are not live are 0.
    `heads` limits the work to the q-heads of the listed KV heads."""
    q = (np.asarray(q_bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    B, Hq, _ = q.shape
    max_pages = block_table.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, max_pages))
    for b in (range(B) if requests is None else requests):
        N = int(seq_lens[b])
        if N == 0:
            continue
        K, _ = dequant_request(pools, block_table[b], page_format[b], N, P, Hkv, d, signs_words, heads=heads, tqk=tqk)
        n_pages = (N + P - 1) // P
        page_of = np.arange(N) // P
        fmt_of = np.asarray(page_format[b][:n_pages])[page_of]
        for h in (range(Hq) if heads is None else [g * G + n for g in heads for n in range(G)]):
            s = sm_scale * (K[:, h // G, :] @ q[b, h])
            parts = {}
            for f in np.unique(fmt_of):                                  # Eq. 6 per partition
                idx = np.nonzero(fmt_of == f)[0]
                m_j = s[idx].max()
                parts[int(f)] = (idx, m_j, np.exp(s[idx] - m_j).sum())
            m = max(m_j for _, m_j, _ in parts.values())
            l = sum(np.exp(m_j - m) * l_j for _, m_j, l_j in parts.values())
            for f, (idx, m_j, l_j) in parts.items():
                w_j = np.exp(m_j - m) * l_j / l                           # Eq. 8
                e = np.exp(s[idx] - m_j)
                rho = np.zeros(n_pages)
                np.add.at(rho, page_of[idx], e)                           # Eq. 7, before 1 / l_j
                pages = np.unique(page_of[idx])
                out[b, h, pages] = w_j * rho[pages] / l_j
    return out


def collect_ref(qmass, seq_lens, P: int, heads, beta: float, a_prev):
    """(r [B, max_pages], a [B, max_pages]) of Eq. 9 from the page mass q
    [B, Hq, max_pages]: per head q~ = q / sum_p q over the live pages, r the
    mean over `heads`, a = beta a_prev + (1 - beta) r on live pages (others
    keep a_prev, r = 0 there)."""
    qmass = np.asarray(qmass, dtype=np.float64)
    B, _, max_pages = qmass.shape
    r = np.zeros((B, max_pages))
    a = np.array(a_prev, dtype=np.float64, copy=True)
    heads = list(heads)
    for b in range(B):
        n_pages = (int(seq_lens[b]) + P - 1) // P
        if n_pages == 0 or not heads:
            continue
        for h in heads:
            qh = qmass[b, h, :n_pages]
            tot = qh.sum()
            if tot > 0:
                r[b, :n_pages] += qh / tot
        r[b, :n_pages] /= len(heads)
        a[b, :n_pages] = beta * a[b, :n_pages] + (1.0 - beta) * r[b, :n_pages]
    return r, a
