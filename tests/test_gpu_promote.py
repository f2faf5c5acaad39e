"""GPU parity of promotion (kv_promote_fp8): compressed pages rebuilt into FP8
pages, bit-exact against the oracle's promotion of its own encoding of the
same seeded rows (Minima-KV algorithm 1, "Promote")."""
import numpy as np
import pytest

import workloads as W
from oracle import promote as OP
from oracle.attention import FMT_FP8, FMT_TQ2, FMT_TQ3, FMT_TQF5, FMT_TQF6, FMT_TQK
from oracle.cache import encode_page
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

FILL = 0xA5   # destination bytes a skipped page must keep


def _rows(rng, n, P, Hkv, d):
    rows = rng.standard_normal((n, P, Hkv, 2, d)).astype(np.float32)
    rows[0, 0] = 0                                  # zero vectors
    rows[0, 1, :, 0, :] = 0
    rows[0, 1, :, 0, 5] = -3.0                      # spike
    rows[1] *= 1e-20                                # tiny norms (subnormal-range sigmas)
    rows[2, 3] *= 1e4
    rows[n - 1, :, 0] *= np.float32(8.0)            # a loud head
    return rows


@pytest.mark.parametrize("fmt,d,P,Hkv", [
    (FMT_TQ3, 256, 16, 4), (FMT_TQ3, 128, 32, 2), (FMT_TQ2, 128, 16, 2), (FMT_TQ2, 256, 32, 1),
    (FMT_TQK, 128, 32, 2), (FMT_TQK, 128, 16, 3),
    (FMT_TQF5, 128, 16, 2), (FMT_TQF5, 256, 32, 1), (FMT_TQF6, 128, 32, 2), (FMT_TQF6, 256, 16, 3),
])
def test_promote_bitexact(fmt, d, P, Hkv):
    torch = C.torch_mod()
    m = C.kvq()
    from quantized_paged_kv_mixed_amd.paged import GpuLayer
    C.say(f"promote fmt={fmt} d={d} P={P} Hkv={Hkv}")
    n = 7
    rng = np.random.default_rng(100 * fmt + d + P)
    base = W.WORKLOADS["l70b"] if fmt == FMT_TQK else W.WORKLOADS["tiny"]
    w = W.scaled(base, head_dim=d, num_kv_heads=Hkv, num_q_heads=Hkv, page_size=P)
    signs = W.make_signs(w, 5, 0)
    rates = W.make_tqk_rates(w, 5, 0) if fmt == FMT_TQK else None
    perm = W.make_tqk_perm(w, 5, 0) if fmt == FMT_TQK else None
    rows = _rows(rng, n, P, Hkv, d)
    valid = np.full(n, P, np.int32)
    valid[3] = P - 5                                   # a partial last page
    valid[4] = 1
    n_fp8 = n + 3
    lay = GpuLayer(Hkv, d, P, {fmt: n, FMT_FP8: n_fp8}, signs, tqk_perm=perm)
    lay.pools[FMT_FP8].fill_(FILL)
    enc = {FMT_TQ3: m.kv_encode_tq3, FMT_TQ2: m.kv_encode_tq2, FMT_TQK: m.kv_encode_tqk, FMT_TQF5: m.kv_encode_tqf5,
           FMT_TQF6: m.kv_encode_tqf6}[fmt]
    enc(lay.cache, m.SRC_F32_ROWS, torch.arange(n, dtype=torch.int32).cuda(), src=torch.from_numpy(rows).cuda(),
        page_valid=torch.from_numpy(valid).cuda())
    # sources in a shuffled order into scattered FP8 pages; the last two
    # entries are out of range on one side and must be skipped
    src_ids = rng.permutation(n).astype(np.int32)
    dst_ids = rng.permutation(n_fp8)[:n].astype(np.int32)
    src_call = np.concatenate([src_ids, [n, 0]]).astype(np.int32)
    dst_call = np.concatenate([dst_ids, [dst_ids[0], n_fp8 + 4]]).astype(np.int32)
    dst_call[n] = [i for i in range(n_fp8) if i not in dst_ids][0]       # a free page, src out of range
    m.kv_promote_fp8(lay.cache, fmt, torch.from_numpy(src_call).cuda(), torch.from_numpy(dst_call).cuda())
    torch.cuda.synchronize()

    got_tq = lay.pool_bytes(fmt)
    got_fp8 = lay.pool_bytes(FMT_FP8)
    written = set()
    for i in range(n):
        page = encode_page(fmt, rows[i, :, :, 0], rows[i, :, :, 1], int(valid[i]), signs, tqk=rates)
        C._cmp(got_tq[i], page, f"source page {i}")
    for src, dst in zip(src_ids, dst_ids):
        page = encode_page(fmt, rows[src, :, :, 0], rows[src, :, :, 1], int(valid[src]), signs, tqk=rates)
        ref = OP.promote_page(fmt, page, Hkv, P, d, signs, tqk=rates)
        C._cmp(got_fp8[dst], ref, f"promoted page {src} -> {dst}")
        written.add(int(dst))
    for j in range(n_fp8):
        if j not in written:
            assert np.all(got_fp8[j] == FILL), f"FP8 page {j} was not a destination but changed"


def test_promote_then_decode_reads_the_fp8_page():
    """A promoted page serves decode as an FP8 page: the table entry is
    switched to the new FP8 page and the attention matches the oracle's over
    its own promoted bytes."""
    torch = C.torch_mod()
    m = C.kvq()
    C.say("promote then decode")
    w = W.scaled(W.WORKLOADS["tiny"], seq_len=700)
    case = C.Case(w, seed=3)
    lay = case.gpu_layer()
    pools = case.oracle_pools()
    C.assert_pools_equal(lay, pools, "tiny pools")
    plan = case.plan
    b = 0
    tq_pages = [p for p in range((int(plan.seq_lens[b]) + w.page_size - 1) // w.page_size)
                if plan.page_format[b, p] == FMT_TQ3][:5]
    n8 = lay.pools[FMT_FP8].shape[0]
    free = sorted(set(range(n8)) - set(int(x) for x in plan.block_table[b][plan.page_format[b] == FMT_FP8]))
    assert len(free) >= len(tq_pages), "the workload keeps slack in the FP8 pool"
    src = np.array([plan.block_table[b, p] for p in tq_pages], np.int32)
    dst = np.array(free[:len(tq_pages)], np.int32)
    m.kv_promote_fp8(lay.cache, FMT_TQ3, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    # oracle: its own promotion of its own TQ3 pages
    for s, t in zip(src, dst):
        pools[FMT_FP8][t] = OP.promote_page(FMT_TQ3, pools[FMT_TQ3][s], w.num_kv_heads, w.page_size, w.head_dim,
                                            case.signs)
    for p, t in zip(tq_pages, dst):
        plan.block_table[b, p] = t
        plan.page_format[b, p] = FMT_FP8
    torch.cuda.synchronize()
    C._cmp(lay.pool_bytes(FMT_FP8), pools[FMT_FP8], "FP8 pool after promotion")
    O, lse = C.run_decode(case, lay)
    Oref, lref = case.oracle_attention(pools)
    C.assert_close(O, Oref, "O after promotion")
    C.assert_close(lse, lref, "lse after promotion")
