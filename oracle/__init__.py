"""CPU oracle for mixed-format (FP8 / TQ) paged decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg call it.
It shares no code, header, table or constant generator with the HIP library.

What it computes (each function cites the passage it follows):
  fp8.py        OCP E4M3 ("e4m3fn") per-token-per-head scaled codes for Recent
                and Anchor pages (Minima-KV, section 3.1 "Recent", section 4.1).
  tq.py         TurboQuant-MSE-style codes for Stale pages: per-vector norm,
                seeded Hadamard-sign rotation, Gaussian Lloyd-Max scalar
                codebook, one fp16 norm correction per vector (Minima-KV
                section 3.1 "Stale" and section 4.3; Block-GTQ appendix B.1).
  tqk.py        grouped mixed-rate keys: RoPE blocks of equal width form one
                segment, each segment a TQ codec with its own signs and fp16
                norm; uniform TQ3 values (Block-GTQ appendix A.7, B.1, H.1-H.2).
  layout.py     the byte layout of one page of each format (the pages only say
                "packed next to the page"; this build fixes one dense layout).
  attention.py  full-softmax attention over the dequantized logical cache in
                fp64, which the mixed-format merge reaches exactly up to codec
                and rounding error (Minima-KV section 3.3, Eq. 11-13), plus the
                literal Eq. 11-13 merge of partials.
  accounting.py the byte formulas (Minima-KV Eq. 1-3 and 10; Block-GTQ B.1).
  cache.py      builds a whole paged cache (pools + tables) from fp32 K/V.
  promote.py    promotion of a compressed page back into an FP8 page: the TQ
                decode evaluated in fp32 in a fixed order, then the FP8 codec
                (Minima-KV algorithm 1 "Promote", figure 2).
  pagemass.py   the attention page mass of Eq. 6-8 over format partitions and
                the running page score of Eq. 9 (Minima-KV section 3.1).
  prefill.py    causal attention of a chunk of new tokens over the cache
                (Block-GTQ appendix H.5), in fp64.
  tqf.py        fractional-level TQ codes (5 or 6 levels) and their mixed-
                radix packing (SemKV section 4.1); no kernel uses it yet.

Precision: encoders run every step in IEEE fp32 round-to-nearest-even with no
fused multiply-add (numpy float32 scalar/array ops), which fixes the codes
bit for bit; attention and decoding run in fp64.

Pins: every function here is checked in tests/test_oracle_*.py against values
fixed outside this package (the pages' printed numbers, the OCP FP8 table,
Max's 1960 Gaussian quantizer table, dense Hadamard products, brute-force
softmax, a decimal square root, closed forms of constant code rows and of
equal keys). The TQ encoder has no worked example on the pages; it is pinned by
brute-force nearest-centroid search and closed-form special cases instead.
"""
