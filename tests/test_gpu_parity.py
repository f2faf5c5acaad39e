"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Encoders: pool bytes bit-exact. Decode: every output element within
|gpu - ref| <= 2e-3 + 1e-2 |ref| of the oracle's fp64 attention over its own
dequantized cache (the same bytes, checked bitwise first).
"""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


def _case(name, stale="fp32", seed=0, **over):
    w = W.scaled(W.WORKLOADS[name], **over) if over else W.WORKLOADS[name]
    return C.Case(w, seed=seed, stale_source=stale)


# ---------------------------------------------------------------- encoders
@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("tiny", {"page_size": 32, "seq_len": 1000}),
    # three KV heads: a wave's consecutive (token, head, role) vectors cross
    # tokens mid-wave, and the token count leaves a partial last wave
    ("tiny", {"batch": 2, "seq_len": 777, "num_kv_heads": 3, "num_q_heads": 6}),
    ("l27b", {"seq_len": 2048, "recent_tokens": 256}),
    ("serving", {"batch": 3, "seq_len_range": (40, 700)}),
    ("l70b", {"batch": 2, "seq_len": 1500, "recent_tokens": 256, "num_q_heads": 16, "num_kv_heads": 2}),
    # fractional-level Stale pages (TQF6 / TQF5) at d 128 page 16 and d 256 page 32
    ("frac", {"batch": 3, "seq_len_range": (40, 900)}),
    ("frac", {"head_dim": 256, "page_size": 32, "batch": 2, "seq_len_range": (300, 1200), "num_q_heads": 8,
              "num_kv_heads": 2}),
])
@pytest.mark.parametrize("stale", ["fp32", "fp8"])
def test_encoders_bitexact(name, over, stale):
    C.say(f"encode {name} {over} {stale}")
    case = _case(name, stale, seed=11, **over)
    lay = case.gpu_layer()
    C.assert_pools_equal(lay, case.oracle_pools(), f"{name}/{stale}")


def test_fp8_encode_edge_rows_and_bf16():
    torch = C.torch_mod()
    m = C.kvq()
    from oracle import fp8 as OF, layout as OL
    from quantized_paged_kv_mixed_amd.paged import GpuLayer
    C.say("fp8 edge rows")
    rng = np.random.default_rng(5)
    Hkv, d, P = 2, 128, 16
    n = 32
    x = rng.standard_normal((n, Hkv, 2, d)).astype(np.float32)
    x[0] = 0                                           # zero rows
    x[1, 0, 0, :] = 0
    x[1, 0, 0, 7] = -3.0                               # single spike
    x[2] *= 1e-30                                      # tiny values -> subnormal codes
    x[3] *= 1e30
    x[4, :, :, ::2] = 0                                # ties / signed zeros
    x[5] = np.round(x[5] * 4) / 4
    # scattered slots (token by token), slots in order (V codes of four
    # aligned slots stored as words), and in order from slot 2 (groups of four
    # tokens are misaligned or straddle pages, so they go token by token)
    layouts = {
        "scattered": (np.arange(n) // P,
                      np.concatenate([np.random.default_rng(1 + k).permutation(P) for k in range(2)])),
        "in order": (np.arange(n) // P, np.arange(n) % P),
        "from slot 2": ((np.arange(n) + 2) // P, (np.arange(n) + 2) % P),
    }
    for bf16 in (False, True):
        src = x
        if bf16:
            src = W.bf16_to_f32(W.bf16_round(x)).reshape(x.shape)
        for lname, (page, slot) in layouts.items():
            n_pages = int(page.max()) + 1
            lay = GpuLayer(Hkv, d, P, {0: n_pages}, np.zeros((Hkv, 2, d // 32), np.uint32))
            t = torch.from_numpy(src).cuda()
            if bf16:
                t = torch.from_numpy(W.bf16_round(x).view(np.int16)).cuda().view(torch.bfloat16)
            m.kv_encode_fp8(lay.cache, t, torch.from_numpy(page.astype(np.int32)).cuda(),
                            torch.from_numpy(slot.astype(np.int32)).cuda())
            torch.cuda.synchronize()
            ref = np.zeros((n_pages, Hkv * OL.fp8_head_bytes(P, d)), np.uint8)
            for pg in range(n_pages):
                blocks = []
                for g in range(Hkv):
                    kc = np.zeros((P, d), np.uint8); vc = np.zeros((P, d), np.uint8)
                    ks = np.zeros(P, np.float32); vs = np.zeros(P, np.float32)
                    for i in np.nonzero(page == pg)[0]:
                        s = slot[i]
                        kc[s], ks[s] = OF.fp8_encode(src[i, g, 0])
                        vc[s], vs[s] = OF.fp8_encode(src[i, g, 1])
                    blocks.append(OL.fp8_pack_head(kc, vc, ks, vs))
                ref[pg] = np.concatenate(blocks)
            C._cmp(lay.pool_bytes(0), ref, f"fp8 edge rows bf16={bf16} {lname}")


def test_tq_encode_edge_vectors():
    torch = C.torch_mod()
    m = C.kvq()
    from oracle import layout as OL, tq as OT
    from quantized_paged_kv_mixed_amd.paged import GpuLayer
    C.say("tq edge vectors")
    rng = np.random.default_rng(6)
    for d in (128, 256):
        Hkv, P = 1, 16
        rows = rng.standard_normal((3, P, Hkv, 2, d)).astype(np.float32)
        rows[0, 0] = 0                                 # zero vector
        rows[0, 1] = 0
        rows[0, 1, 0, 0, 3] = 2.5                      # spike
        rows[0, 2, 0, 1, :2] = 1.0                     # lands on the zero threshold
        rows[0, 2, 0, 1, 2:] = 0
        rows[1] *= 1e-20                               # tiny norms
        rows[2, 3] *= 1e15
        signs = W.make_signs(W.scaled(W.WORKLOADS["tiny"], head_dim=d), 3, 0)[:1]
        valid = np.array([P, 9, P], np.int32)
        for bits, f in ((3, 1), (2, 2)):
            lay = GpuLayer(Hkv, d, P, {f: 3}, signs)
            enc = m.kv_encode_tq3 if bits == 3 else m.kv_encode_tq2
            enc(lay.cache, m.SRC_F32_ROWS, torch.arange(3, dtype=torch.int32).cuda().flip(0),
                src=torch.from_numpy(rows).cuda(), page_valid=torch.from_numpy(valid).cuda())
            torch.cuda.synchronize()
            got = lay.pool_bytes(f)
            sk = OT.signs_from_bits(signs[0, 0], d)
            sv = OT.signs_from_bits(signs[0, 1], d)
            for i in range(3):
                x = rows[i].copy()
                x[valid[i]:] = 0
                kc, ksig = OT.tq_encode(x[:, 0, 0], sk, bits)
                vc, vsig = OT.tq_encode(x[:, 0, 1], sv, bits)
                ref = OL.tq_pack_head(kc, vc, ksig, vsig, bits)
                C._cmp(got[2 - i], ref, f"tq{bits} d={d} page {i}")


def test_tqf_encode_edge_vectors():
    """Fractional-level encode of the edge rows of the uniform formats (zero
    rows, a spike, a coordinate on a threshold, tiny and huge norms, a partial
    page) at both head dims, bit-exact against the oracle's row bitstreams."""
    torch = C.torch_mod()
    m = C.kvq()
    from oracle import layout as OL, tq as OT, tqf as OF
    from quantized_paged_kv_mixed_amd.paged import GpuLayer
    C.say("tqf edge vectors")
    rng = np.random.default_rng(16)
    for d in (128, 256):
        Hkv, P = 1, 16
        rows = rng.standard_normal((3, P, Hkv, 2, d)).astype(np.float32)
        rows[0, 0] = 0
        rows[0, 1] = 0
        rows[0, 1, 0, 0, 7] = -1.5
        rows[0, 2, 0, 1, :2] = 1.0
        rows[0, 2, 0, 1, 2:] = 0
        rows[1] *= 1e-20
        rows[2, 5] *= 1e15
        signs = W.make_signs(W.scaled(W.WORKLOADS["tiny"], head_dim=d), 7, 0)[:1]
        valid = np.array([P, 11, P], np.int32)
        for levels, f, enc in ((5, m.FMT_TQF5, m.kv_encode_tqf5), (6, m.FMT_TQF6, m.kv_encode_tqf6)):
            lay = GpuLayer(Hkv, d, P, {f: 3}, signs)
            enc(lay.cache, m.SRC_F32_ROWS, torch.arange(3, dtype=torch.int32).cuda().flip(0),
                src=torch.from_numpy(rows).cuda(), page_valid=torch.from_numpy(valid).cuda())
            torch.cuda.synchronize()
            got = lay.pool_bytes(f)
            sk = OT.signs_from_bits(signs[0, 0], d)
            sv = OT.signs_from_bits(signs[0, 1], d)
            for i in range(3):
                x = rows[i].copy()
                x[valid[i]:] = 0
                kc, ksig = OF.encode(x[:, 0, 0], sk, levels)
                vc, vsig = OF.encode(x[:, 0, 1], sv, levels)
                ref = OL.tqf_pack_head(kc, vc, ksig, vsig, levels)
                C._cmp(got[2 - i], ref, f"tqf{levels} d={d} page {i}")


def test_tqk_encode_edge_vectors():
    """Grouped keys: whole-zero rows, one zero segment, spikes, tiny and huge
    norms, a partial last page; bit-exact against the oracle."""
    torch = C.torch_mod()
    m = C.kvq()
    from oracle import layout as OL, tq as OT, tqk as OK
    from quantized_paged_kv_mixed_amd.paged import GpuLayer
    C.say("tqk edge vectors")
    rng = np.random.default_rng(16)
    w = W.scaled(W.WORKLOADS["l70b"], num_kv_heads=2, num_q_heads=4)
    d, P, Hkv = 128, 32, 2
    rates = W.make_tqk_rates(w, 2, 0)
    perm = W.make_tqk_perm(w, 2, 0)
    signs = W.make_signs(w, 2, 0)
    rows = rng.standard_normal((3, P, Hkv, 2, d)).astype(np.float32)
    rows[0, 0] = 0                                          # zero key and value
    p0, segs0 = OK.segments(rates[0])
    rows[0, 1, 0, 0, p0[:32]] = 0                           # the 2-bit segment of head 0 is zero
    rows[0, 2, 1, 0, :] = 0
    rows[0, 2, 1, 0, 5] = -4.0                              # spike
    rows[1] *= 1e-20
    rows[2, 4] *= 1e15
    valid = np.array([P, 17, P], np.int32)
    lay = GpuLayer(Hkv, d, P, {W.FMT_TQK: 3}, signs, tqk_perm=perm)
    m.kv_encode_tqk(lay.cache, m.SRC_F32_ROWS, torch.tensor([2, 0, 1], dtype=torch.int32).cuda(),
                    src=torch.from_numpy(rows).cuda(), page_valid=torch.from_numpy(valid).cuda())
    torch.cuda.synchronize()
    got = lay.pool_bytes(W.FMT_TQK)
    hb = OL.tqk_head_bytes(P, d)
    for i, dst in enumerate([2, 0, 1]):
        x = rows[i].copy()
        x[valid[i]:] = 0
        for g in range(Hkv):
            sk = OT.signs_from_bits(signs[g, 0], d)
            sv = OT.signs_from_bits(signs[g, 1], d)
            ref = OK.encode_page_head(x[:, g, 0], x[:, g, 1], sk, sv, rates[g])
            C._cmp(got[dst, g * hb:(g + 1) * hb], ref, f"tqk page {i} head {g}")


# ---------------------------------------------------------------- plan
def test_plan_entries_match_compaction():
    torch = C.torch_mod()
    m = C.kvq()
    C.say("plan compaction")
    case = _case("serving", seed=3, batch=5, seq_len_range=(200, 600))
    lay = case.gpu_layer()
    plan = case.plan
    pf = plan.page_format.copy()
    bt = plan.block_table.copy()
    # plant bad entries: unknown tag, id past the pool, negative id
    pf[1, 0] = 9
    bt[2, 1] = lay.pools[pf[2, 1]].shape[0] + 5 if pf[2, 1] in lay.pools else 10 ** 6
    bt[3, 0] = -4
    B, MP = bt.shape
    nb = m.paged_decode_plan_bytes(lay.cache, B, MP)
    buf = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    ctr = torch.zeros(64, dtype=torch.uint8, device="cuda")
    m.paged_decode_plan(lay.cache, torch.from_numpy(bt).cuda(), torch.from_numpy(pf).cuda(),
                        torch.from_numpy(plan.seq_lens).cuda(), buf, ctr)
    torch.cuda.synchronize()
    raw = buf.cpu().numpy()
    # expected: per request, per format in tag order, (logical page, id) in logical order
    o = 64
    seq = raw[o:o + 4 * B].view(np.int32); o += 4 * B; o = (o + 15) & ~15
    NF = m.FMT_TQF6 + 1                           # format tags of the boundary
    counts = raw[o:o + 4 * NF * B].view(np.int32).reshape(B, NF); o += 4 * NF * B; o = (o + 15) & ~15
    o += 16 * B                                   # per-request item ranges
    ent = raw[o:o + 8 * B * MP].view(np.int32).reshape(B, MP, 2)
    pools = {f: lay.pools[f].shape[0] for f in lay.pools}
    n_bad = 0
    for b in range(B):
        n_pages = (int(plan.seq_lens[b]) + 15) // 16
        assert seq[b] == plan.seq_lens[b]
        exp = []
        for f in range(NF):
            lst = [(p, int(bt[b, p])) for p in range(n_pages)
                   if pf[b, p] == f and 0 <= bt[b, p] < pools.get(f, 0)]
            assert counts[b, f] == len(lst)
            exp += lst
        n_bad += n_pages - len(exp)
        assert [tuple(e) for e in ent[b, :len(exp)].tolist()] == exp
    assert m.read_counters(ctr)["invalid_entries"] == n_bad == 3


# ---------------------------------------------------------------- decode
DECODE_CASES = [
    ("tiny", {}, "fp32"),
    ("tiny", {"seq_len": 1000}, "fp8"),                       # ragged tail
    ("tiny", {"page_size": 32, "seq_len": 777}, "fp32"),
    ("l27b", {}, "fp32"),                                      # the 27B layer, full size
    ("canary", {"seq_len": 4100, "layers": 1}, "fp8"),
    ("serving", {"batch": 6, "seq_len_range": (1, 3000)}, "fp32"),
    ("l70b", {"batch": 2, "seq_len": 3000, "recent_tokens": 512, "num_q_heads": 16, "num_kv_heads": 2}, "fp32"),
    ("l70b", {"seq_len": 4000, "recent_tokens": 1024}, "fp8"),          # the 70B-class shape, short
    ("l70b", {"batch": 3, "seq_len": 999, "recent_tokens": 96, "num_kv_heads": 4, "num_q_heads": 20}, "fp32"),
    # GQA groups whose staged rows exceed the merge's LDS: the workgroup merge runs in dim chunks
    ("l27b", {"batch": 2, "seq_len": 2000, "recent_tokens": 256, "num_q_heads": 32, "num_kv_heads": 4}, "fp32"),
    ("tiny", {"batch": 2, "seq_len": 1500, "num_q_heads": 16, "num_kv_heads": 1}, "fp8"),
    ("tiny", {"batch": 2, "seq_len": 777, "num_kv_heads": 3, "num_q_heads": 6}, "fp8"),   # three KV heads
    # about 64 items per request: the merge takes its partial rows in several chunks
    ("tiny", {"seq_len": 33000, "recent_tokens": 512}, "fp8"),
    # every (head_dim, page_size, format) the header accepts: d 256 at page 32
    # (FP8 + TQ3 + TQ2), TQ2 at d 256 with a 16-head group (the merge's D/4
    # dim chunks), grouped keys at page 16, FP8 + TQ3 at d 256 / page 32
    ("serving", {"head_dim": 256, "page_size": 32, "batch": 3, "seq_len_range": (300, 2600), "num_q_heads": 12,
                 "num_kv_heads": 2}, "fp8"),
    ("serving", {"head_dim": 256, "batch": 3, "seq_len_range": (100, 2000), "num_q_heads": 32, "num_kv_heads": 2},
     "fp32"),
    ("l70b", {"page_size": 16, "batch": 2, "seq_len": 2100, "recent_tokens": 256, "num_q_heads": 16,
              "num_kv_heads": 2}, "fp8"),
    ("l27b", {"page_size": 32, "seq_len": 3000, "recent_tokens": 512, "anchor_pages": 3}, "fp32"),
    # FP8 + TQF6 + TQF5 by page importance: ragged lengths, both page sizes and
    # head dims, GQA groups 4 to 8
    ("frac", {"batch": 4, "seq_len_range": (1, 2500)}, "fp32"),
    ("frac", {"batch": 3, "seq_len_range": (200, 1800), "page_size": 32}, "fp8"),
    ("frac", {"head_dim": 256, "batch": 2, "seq_len_range": (300, 2200), "num_q_heads": 16, "num_kv_heads": 2},
     "fp32"),
    ("frac", {"head_dim": 256, "page_size": 32, "batch": 2, "seq_len_range": (500, 2000), "num_q_heads": 16,
              "num_kv_heads": 4}, "fp8"),
]


@pytest.mark.parametrize("name,over,stale", DECODE_CASES)
def test_decode_parity(name, over, stale):
    C.say(f"decode {name} {over} {stale}")
    case = _case(name, stale, seed=21, **over)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    C.assert_pools_equal(lay, pools, f"{name} pools")
    O, lse = C.run_decode(case, lay)
    Oref, lref = case.oracle_attention(pools)
    C.assert_close(O, Oref, f"{name} O")
    C.assert_close(lse, lref, f"{name} lse")
    O2, l2 = C.run_decode(case, lay, oneshot=False)
    assert np.array_equal(O, O2) and np.array_equal(lse, l2), "planned and one-shot differ"


@pytest.mark.parametrize("name,over", [
    ("canary", {"layers": 1, "batch": 2, "seq_len": 7000, "recent_tokens": 640, "anchor_pages": 2}),
    ("serving", {"batch": 3, "seq_len_range": (700, 1600)}),
    ("frac", {"batch": 3, "seq_len_range": (600, 1200)}),
])
def test_decode_scores_far_above_the_earlier_pages(name, over):
    """Block-GTQ appendix H.3, fp32 online-softmax statistics: in request b
    one key of a page of its (b mod n)-th format is made 40x louder, so its
    score stands tens of log2 units above the maxima of the pages scanned
    before it and that format's split must lift its running maximum (over all
    four lane groups of an MFMA column) before taking exponentials. One loud
    key per request dominates its heads outright, which keeps the share of
    the f16 query rounding (about |s| 2^-12 per score) small."""
    C.say(f"decode loud keys {name} {over}")
    case = _case(name, "fp32", seed=23, **over)
    w = case.w
    for b in range(w.batch):
        K, _ = case.kv(b)
        fmts = C.request_formats(case.plan, b, w.page_size)
        K[C.loud_token(case.plan, b, w.page_size, fmts[b % len(fmts)])] *= np.float32(40.0)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    O, lse = C.run_decode(case, lay)
    assert np.isfinite(O).all() and np.isfinite(lse).all(), f"{name}: non-finite outputs"
    Oref, lref = case.oracle_attention(pools)
    C.assert_close(O, Oref, f"{name} loud O")
    C.assert_close(lse, lref, f"{name} loud lse")


def test_decode_single_format_and_empty_requests():
    C.say("decode single-format / empty / seq 1")
    w = W.scaled(W.WORKLOADS["serving"], batch=5, seq_len_range=(400, 400), num_q_heads=16, num_kv_heads=4)
    plan = W.make_page_plan(w, 4)
    plan.seq_lens[:] = [0, 1, 17, 400, 230]
    n_pages = (plan.seq_lens + 15) // 16
    plan.page_format[0, :] = 255
    plan.page_format[3, :n_pages[3]] = W.FMT_FP8                 # all FP8
    plan.page_format[4, :n_pages[4]] = W.FMT_TQ3                 # all TQ3
    for b in range(5):
        plan.page_format[b, n_pages[b]:] = 255
    # re-assign ids so every used page has a home in its pool
    rng = np.random.default_rng(0)
    for f in (0, 1, 2):
        used = [(b, p) for b in range(5) for p in range(n_pages[b]) if plan.page_format[b, p] == f]
        plan.pool_pages[f] = len(used) + 3
        ids = rng.permutation(len(used) + 3)[:len(used)]
        for (b, p), i in zip(used, ids):
            plan.block_table[b, p] = i
    case = C.Case(w, seed=4, plan=plan)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    C.assert_pools_equal(lay, pools, "edge pools")
    torch = C.torch_mod()
    ctr = torch.zeros(64, dtype=torch.uint8, device="cuda")
    O, lse = C.run_decode(case, lay, counters=ctr)
    Oref, lref = case.oracle_attention(pools)
    assert np.all(O[0] == 0) and np.all(np.isneginf(lse[0]))
    C.assert_close(O, Oref, "edge O")
    C.assert_close(lse, lref, "edge lse")
    cnt = C.kvq().read_counters(ctr)
    Hkv = w.num_kv_heads
    for f, key in ((0, "pages_fp8"), (1, "pages_tq3"), (2, "pages_tq2")):
        assert cnt[key] == Hkv * int(sum((plan.page_format[b, :n_pages[b]] == f).sum() for b in range(5)))
    assert cnt["fallbacks"] == 0 and cnt["invalid_entries"] == 0


def test_fractional_level_route_counters():
    """Every (page, KV head) pair of a fractional-level page is counted under
    its own format."""
    torch = C.torch_mod()
    C.say("decode route counters, fractional levels")
    w = W.scaled(W.WORKLOADS["frac"], batch=3, seq_len_range=(100, 1500))
    case = C.Case(w, seed=9)
    lay = case.gpu_layer()
    ctr = torch.zeros(64, dtype=torch.uint8, device="cuda")
    C.run_decode(case, lay, counters=ctr)
    cnt = C.kvq().read_counters(ctr)
    plan, P = case.plan, w.page_size
    n_pages = (plan.seq_lens + P - 1) // P
    for f, key in ((W.FMT_FP8, "pages_fp8"), (W.FMT_TQF5, "pages_tqf5"), (W.FMT_TQF6, "pages_tqf6")):
        used = int(sum((plan.page_format[b, :n_pages[b]] == f).sum() for b in range(w.batch)))
        assert used > 0 and cnt[key] == w.num_kv_heads * used, key
    assert cnt["pages_tq3"] == cnt["pages_tq2"] == cnt["invalid_entries"] == 0


def test_duplicate_batch_and_determinism():
    """Minima-KV appendix C: the same request twice in a batch gives the same
    tokens; the fixed reduction order makes repeated calls bitwise equal."""
    C.say("duplicate batch")
    w1 = W.scaled(W.WORKLOADS["l27b"], batch=1, seq_len=3000, recent_tokens=512)
    p1 = W.make_page_plan(w1, 8)
    w = W.scaled(w1, batch=2)
    bt = np.concatenate([p1.block_table, p1.block_table], 0)
    for f, n in p1.pool_pages.items():           # second copy lives after the first in each pool
        sel = p1.page_format[0] == f
        bt[1, sel] += n
    plan = W.PagePlan(np.concatenate([p1.seq_lens, p1.seq_lens]), np.concatenate([p1.page_format] * 2, 0),
                      bt, {f: 2 * n for f, n in p1.pool_pages.items()}, p1.max_pages)
    case = C.Case(w, seed=8, plan=plan)
    K, V = case.kv(0)
    case._kv[1] = (K, V)
    case.q[1] = case.q[0]
    lay = case.gpu_layer()
    O, lse = C.run_decode(case, lay)
    # the two requests have different physical pages but identical contents
    assert np.array_equal(O[0], O[1]) and np.array_equal(lse[0], lse[1])
    for _ in range(3):
        O2, l2 = C.run_decode(case, lay)
        assert np.array_equal(O, O2) and np.array_equal(lse, l2)


def test_masked_invalid_entries():
    C.say("invalid entries masked")
    torch = C.torch_mod()
    case = _case("tiny", seed=9)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    bt = case.plan.block_table.copy()
    pf = case.plan.page_format.copy()
    pf[0, 5] = 200                       # unknown tag -> page 5 dropped
    ctr = torch.zeros(64, dtype=torch.uint8, device="cuda")
    orig = (case.plan.block_table, case.plan.page_format)
    case.plan.block_table, case.plan.page_format = bt, pf
    O, lse = C.run_decode(case, lay, counters=ctr)
    case.plan.block_table, case.plan.page_format = orig
    # oracle: attention over the request without page 5's tokens
    from oracle import attention as A
    w = case.w
    Kh, Vh = A.dequant_request(pools, orig[0][0], orig[1][0], 1024, 16, 1, 128, case.signs)
    keep = np.r_[0:80, 96:1024]
    q = W.bf16_to_f32(case.q)[0].astype(np.float64)
    Oref, lref = A.attention_ref(q, Kh[keep], Vh[keep], w.sm_scale)
    C.assert_close(O[0], Oref, "masked O")
    C.assert_close(lse[0], lref, "masked lse")
    assert C.kvq().read_counters(ctr)["invalid_entries"] == 1


def test_reused_plan_and_workspace_across_calls():
    """Several layers' calls share one plan and one workspace, both filled
    with garbage before the plan is built: each call, with its own query and
    cache, matches the oracle."""
    torch = C.torch_mod()
    m = C.kvq()
    C.say("reused plan / workspace")
    w = W.scaled(W.WORKLOADS["l27b"], batch=3, seq_len=2500, recent_tokens=256)
    plan = W.make_page_plan(w, 12)
    cases = [C.Case(w, seed=12, layer=li, plan=plan) for li in range(3)]
    lays = [c.gpu_layer() for c in cases]
    bt, pf, sl = cases[0].tables()
    B, Hq, MP = w.batch, w.num_q_heads, bt.shape[1]
    plan_buf = torch.full((m.paged_decode_plan_bytes(lays[0].cache, B, MP),), 0xA5, dtype=torch.uint8, device="cuda")
    ws = torch.full((m.paged_decode_attn_planned_workspace_size(lays[0].cache, B, Hq, MP),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    m.paged_decode_plan(lays[0].cache, bt, pf, sl, plan_buf)
    for rep in range(2):
        for li in (2, 0, 1):
            out = torch.full((B, Hq, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
            lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
            m.paged_decode_attn_planned(lays[li].cache, plan_buf, cases[li].q_dev(), MP, w.sm_scale, out, lse, ws)
            torch.cuda.synchronize()
            Oref, lref = cases[li].oracle_attention(cases[li].oracle_pools())
            C.assert_close(out.cpu().numpy(), Oref, f"call {rep}/{li} O")
            C.assert_close(lse.cpu().numpy(), lref, f"call {rep}/{li} lse")


def test_plan_for_another_geometry_poisons_the_outputs():
    """A plan built for another batch or max_pages (same buffer size or
    larger) is refused on the device: every out and lse element is NaN and
    invalid_entries counts the call once; nothing is read past the plan."""
    torch = C.torch_mod()
    m = C.kvq()
    C.say("plan geometry mismatch")
    case = _case("serving", seed=5, batch=3, seq_len_range=(100, 600))
    lay = case.gpu_layer()
    bt, pf, sl = case.tables()
    B, Hq, MP = case.w.batch, case.w.num_q_heads, bt.shape[1]
    # plan for the first two requests only, in a buffer big enough for three
    plan_buf = torch.zeros(m.paged_decode_plan_bytes(lay.cache, B, MP), dtype=torch.uint8, device="cuda")
    m.paged_decode_plan(lay.cache, bt[:2].contiguous(), pf[:2].contiguous(), sl[:2].contiguous(), plan_buf)
    ws = torch.zeros(m.paged_decode_attn_planned_workspace_size(lay.cache, B, Hq, MP), dtype=torch.uint8,
                     device="cuda")
    ctr = torch.zeros(64, dtype=torch.uint8, device="cuda")
    out = torch.zeros((B, Hq, case.w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    m.paged_decode_attn_planned(lay.cache, plan_buf, case.q_dev(), MP, case.w.sm_scale, out, lse, ws, ctr)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all()
    cnt = m.read_counters(ctr)
    assert cnt["invalid_entries"] == 1 and cnt["pages_tq3"] == 0 and cnt["pages_fp8"] == 0
    # the same buffer re-planned for this geometry works again
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf)
    m.paged_decode_attn_planned(lay.cache, plan_buf, case.q_dev(), MP, case.w.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    Oref, lref = case.oracle_attention(case.oracle_pools())
    C.assert_close(out.cpu().numpy(), Oref, "re-planned O")


def test_decode_masks_ids_outside_a_smaller_pool():
    """The plan is built against the full pools; the decode call names a TQ3
    pool of fewer pages (same allocation, so even a broken check stays in
    mapped memory). Entries whose id is outside the smaller pool are masked
    and counted once per KV head; the result is the oracle's attention over
    the remaining tokens."""
    torch = C.torch_mod()
    m = C.kvq()
    C.say("ids outside a smaller pool")
    case = _case("l27b", seed=6, seq_len=2000, recent_tokens=256, num_q_heads=8, num_kv_heads=2)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    plan = case.plan
    n3 = plan.pool_pages[W.FMT_TQ3]
    cut = n3 // 2
    small = m.make_cache(lay.Hkv, lay.d, lay.P, lay.pools[W.FMT_FP8], lay.pools[W.FMT_TQ3][:cut], None, lay.signs)
    bt, pf, sl = case.tables()
    B, Hq, MP = case.w.batch, case.w.num_q_heads, bt.shape[1]
    plan_buf = torch.zeros(m.paged_decode_plan_bytes(lay.cache, B, MP), dtype=torch.uint8, device="cuda")
    m.paged_decode_plan(lay.cache, bt, pf, sl, plan_buf)
    ws = torch.zeros(m.paged_decode_attn_planned_workspace_size(lay.cache, B, Hq, MP), dtype=torch.uint8,
                     device="cuda")
    ctr = torch.zeros(64, dtype=torch.uint8, device="cuda")
    out = torch.full((B, Hq, case.w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    m.paged_decode_attn_planned(small, plan_buf, case.q_dev(), MP, case.w.sm_scale, out, lse, ws, ctr)
    torch.cuda.synchronize()
    N = int(plan.seq_lens[0])
    n_pages = (N + 15) // 16
    drop = [p for p in range(n_pages) if plan.page_format[0, p] == W.FMT_TQ3 and plan.block_table[0, p] >= cut]
    assert drop, "the cut must drop some pages"
    assert m.read_counters(ctr)["invalid_entries"] == len(drop) * case.w.num_kv_heads
    from oracle import attention as A
    K, V = A.dequant_request(pools, plan.block_table[0], plan.page_format[0], N, 16, case.w.num_kv_heads,
                             case.w.head_dim, case.signs)
    keep = np.setdiff1d(np.arange(N), np.concatenate([np.arange(p * 16, min(N, p * 16 + 16)) for p in drop]))
    q = W.bf16_to_f32(case.q)[0].astype(np.float64)
    Oref, lref = A.attention_ref(q, K[keep], V[keep], case.w.sm_scale)
    C.assert_close(out.cpu().numpy()[0], Oref, "smaller pool O")
    C.assert_close(lse.cpu().numpy()[0], lref, "smaller pool lse")


def test_one_call_with_exactly_the_declared_workspace():
    """paged_decode_attn with a workspace of exactly
    paged_decode_attn_workspace_size bytes (filled with garbage): KVQ_OK and
    oracle parity."""
    torch = C.torch_mod()
    m = C.kvq()
    C.say("one call, exact workspace")
    case = _case("canary", "fp8", seed=7, seq_len=2100, layers=1, recent_tokens=256, anchor_pages=3)
    lay = case.gpu_layer()
    bt = case.tables()[0]
    n = m.paged_decode_attn_workspace_size(lay.cache, case.w.batch, case.w.num_q_heads, bt.shape[1])
    ws = torch.full((n,), 0xC3, dtype=torch.uint8, device="cuda")
    O, lse = C.run_decode(case, lay, ws=ws)
    Oref, lref = case.oracle_attention(case.oracle_pools())
    C.assert_close(O, Oref, "exact-workspace O")
    C.assert_close(lse, lref, "exact-workspace lse")
