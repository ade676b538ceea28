"""Prefill, extend and decode rows on one task map (query-block segments):
the GPU map bit for bit against the oracle's assign, and the attention of the
packed queries against the fp64 oracle under the parity bar.

The mixed batch of the vLLM post's Table 4 shapes -- one request extending an
8K context by 8K new tokens beside 63 decode rows, 64/8 heads -- runs at full
size: every decode row and sampled rows of the extend, plus the partial-free
rows of small mixes in full.
"""
import numpy as np
import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa
from load_balanced_split_assign_amd import workload as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def varlen_batch(seqlens, qlens, Hq=8, Hkv=1, seed=70, gen_device="cpu"):
    b = wl.make_batch(seqlens=seqlens, qlens=qlens, num_heads=Hq, num_kv_heads=Hkv, kv_dtype="bf16", seed=seed,
                      tail="nan", device=gen_device)
    for k, v in list(b.items()):
        if isinstance(v, torch.Tensor):
            b[k] = v.to("cuda:0")
    b["total_q"] = int(sum(qlens))
    return b


def plan(batch, P, F=0):
    return lbsa.plan_varlen(batch["seqlens"], batch["qlens"], batch["num_heads"], batch["num_kv_heads"],
                            batch["max_pages"], P, F, total_q=batch["total_q"])


def attend(batch, tm, P):
    return lbsa.attend_varlen(batch["q"], batch["k_cache"], batch["v_cache"], batch["page_table"], tm, P,
                              batch["softmax_scale"], batch["B"])


def expected_extras(o, sl, ql, P):
    """GPU-only arrays of the map, from the oracle's map and the lengths."""
    nq = [-(-q // lbsa.QBLOCK) for q in ql]
    qbase = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qstart = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    bdb = np.asarray(o["bin_desc_begin"], np.int64)
    def slot_of(d):
        j = int(np.searchsorted(bdb[:P], d, side="right") - 1)     # the bin holding descriptor d
        return 2 * j + (0 if bdb[j] == d else 1)
    slot0 = [slot_of(d0) for d0 in o["seg_first_desc"]]
    desc_slot = [slot_of(d) for d in range(len(o["desc"]))]
    # claim order: 8 groups of consecutive bins, each by decreasing length
    # class (the tile count below 8, then four classes per power of two: the
    # octave and the two bits below its leading one), equal classes by
    # decreasing descriptor index
    def length_class(d):
        n = int(o["desc"][d][4] - o["desc"][d][3])
        if n < 8:
            return n
        e = n.bit_length() - 1
        return min(8 + 4 * (e - 3) + ((n >> (e - 2)) & 3), 63)
    order = []
    for x in range(8):
        lo, hi = int(bdb[x * P // 8]), int(bdb[(x + 1) * P // 8])
        order += sorted(range(lo, hi), key=lambda d: (-length_class(d), -d))
    blk_req = np.repeat(np.arange(len(ql)), nq).astype(np.int32)
    blk_k = np.concatenate([np.arange(n) for n in nq]).astype(np.int32)
    return dict(qbase=qbase, qstart=qstart, slot0=np.asarray(slot0, np.int32), blk_req=blk_req, blk_k=blk_k,
                desc_slot=np.asarray(desc_slot, np.int32), claim_order=np.asarray(order, np.int32))


def assert_same_varlen_map(oracle_mod, sl, ql, Hkv, P, F, mp, what=""):
    sl_t = torch.tensor(sl, dtype=torch.int32, device="cuda:0")
    ql_t = torch.tensor(ql, dtype=torch.int32, device="cuda:0")
    tm = lbsa.plan_varlen(sl_t, ql_t, 8 * Hkv, Hkv, mp, P, F, total_q=int(sum(ql)))
    g = lbsa.read_varlen_task_map(tm, len(sl), Hkv, P, int(sum(ql)))
    o = oracle_mod.assign_varlen(np.asarray(sl, np.int32), np.asarray(ql, np.int32), 8 * Hkv, Hkv, P, F or 2, mp,
                                 lbsa.QBLOCK)
    ctx = str((what, len(sl), Hkv, P, F))
    np.testing.assert_array_equal(g["header"], o["header"], err_msg=ctx)
    np.testing.assert_array_equal(g["bin_desc_begin"], o["bin_desc_begin"], err_msg=ctx)
    np.testing.assert_array_equal(g["desc"][:, :5], o["desc"], err_msg=ctx)
    np.testing.assert_array_equal(g["seg_first_desc"], o["seg_first_desc"], err_msg=ctx)
    np.testing.assert_array_equal(g["seg_num_chunks"], o["seg_num_chunks"], err_msg=ctx)
    if len(o["desc"]):
        b = o["desc"][:, 1]
        qs = np.concatenate([[0], np.cumsum(ql)])
        np.testing.assert_array_equal(g["desc"][:, 5], np.asarray(sl)[b], err_msg=ctx)
        np.testing.assert_array_equal(g["desc"][:, 6], np.asarray(ql)[b], err_msg=ctx)
        np.testing.assert_array_equal(g["desc"][:, 7], qs[b], err_msg=ctx)
    if o["error"] == 0:
        e = expected_extras(o, sl, ql, P)
        np.testing.assert_array_equal(g["seg_slot0"], e["slot0"], err_msg=ctx)
        np.testing.assert_array_equal(g["desc_slot"], e["desc_slot"], err_msg=ctx)
        np.testing.assert_array_equal(g["claim_order"], e["claim_order"], err_msg=ctx)
        np.testing.assert_array_equal(g["blk_req"], e["blk_req"], err_msg=ctx)
        np.testing.assert_array_equal(g["blk_k"], e["blk_k"], err_msg=ctx)
        np.testing.assert_array_equal(g["qbase"], e["qbase"], err_msg=ctx)
        np.testing.assert_array_equal(g["qstart"], e["qstart"], err_msg=ctx)
    return g


def test_worked_example_map(oracle_mod):
    g = assert_same_varlen_map(oracle_mod, [100, 50], [20, 1], 1, 4, 2, 4)
    assert g["QB"] == lbsa.QBLOCK == 24
    assert g["Ndesc"] == 2 and g["NQ"] == 2        # one block per request, 3 tiles in one bin (F = 2)


def test_mixed_extend_map_bitexact(oracle_mod):
    sl, ql = wl.mixed_extend_lengths()
    mp = max((L + 63) // 64 for L in sl)
    for P in (256, 512, 1000):
        for F in (0, 1, 3):
            assert_same_varlen_map(oracle_mod, sl, ql, 8, P, F, mp, "mixed extend")


def test_random_varlen_maps_bitexact(oracle_mod):
    rng = np.random.default_rng(77)
    for it in range(120):
        B = int(rng.integers(1, 40))
        Hkv = int(rng.choice([1, 2, 8]))
        sl = rng.integers(1, 3000, B)
        kind = rng.integers(0, 3, B)                      # decode row, extend, prefill
        ql = np.where(kind == 0, 1, np.where(kind == 1, np.maximum(1, (sl * rng.random(B)).astype(int)), sl))
        if B + ql.sum() // 16 > 1500:
            continue
        P = int(rng.choice([1, 7, 64, 256, 512, 2048]))
        F = int(rng.integers(0, 4))
        mp = int(max(1, (sl.max() + 63) // 64) + rng.integers(0, 3))
        assert_same_varlen_map(oracle_mod, sl.tolist(), ql.tolist(), Hkv, P, F, mp, f"random {it}")


def test_maps_near_the_lds_limit(oracle_mod):
    """The single assign workgroup keeps its prefixes in up to 144 KiB of LDS:
    an 88000-token prefill and a mix of long extends, 8 KV heads, bit-exact
    against the oracle; then the prefill's attention on sampled rows."""
    for sl, ql in [([88000], [88000]), ([40000, 30000, 45000, 9000], [30000, 30000, 27000, 1])]:
        mp = max(-(-x // 64) for x in sl)
        assert_same_varlen_map(oracle_mod, sl, ql, 8, 512, 0, mp, "near the LDS limit")
    b = wl.make_batch(seqlens=[88000], qlens=[88000], num_heads=64, num_kv_heads=8, kv_dtype="bf16", seed=78,
                      tail="nan", device="cuda:0")
    b["total_q"] = 88000
    P = lbsa.varlen_default_workgroups(0)
    out = H.out_np(attend(b, plan(b, P), P))
    rows = [(t, hq) for t in (0, 23, 24, 30001, 87999) for hq in (0, 9, 63)]
    bc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in b.items()}
    ref, _ = oracle_mod.attention_varlen_rows(bc, rows)
    got = np.stack([out[t, hq] for t, hq in rows])
    H.check(b, got, ref, "88000-token prefill, sampled rows")


def test_one_query_per_request_gives_the_decode_map(oracle_mod):
    w = wl.WORKLOADS["tp8_share"]
    sl = wl.draw_seqlens(w, torch.Generator().manual_seed(w.seed)).tolist()
    mp = max((L + 63) // 64 for L in sl)
    g = assert_same_varlen_map(oracle_mod, sl, [1] * len(sl), 1, 256, 0, mp, "q = 1")
    d = lbsa.read_task_map(lbsa.plan(torch.tensor(sl, dtype=torch.int32, device="cuda:0"), 8, 1, mp, 256), len(sl), 1,
                           256)
    np.testing.assert_array_equal(g["desc"][:, [0, 1, 3, 4]], d["desc"])
    np.testing.assert_array_equal(g["bin_desc_begin"], d["bin_desc_begin"])


def test_bad_lengths_set_the_error_word_and_nan_rows(oracle_mod):
    for sl, ql in (([100, 50], [101, 1]), ([100, 50], [20, 1])):
        b = varlen_batch([100, 50], [20, 1], seed=71)
        b["seqlens"] = torch.tensor(sl, dtype=torch.int32, device="cuda:0")
        b["qlens"] = torch.tensor(ql, dtype=torch.int32, device="cuda:0")
        if ql == [20, 1]:
            b["total_q"] = 22                                 # disagrees with the device lengths
            b["q"] = torch.zeros((22, 8, 128), dtype=torch.bfloat16, device="cuda:0")
        tm = plan(b, 8)
        m = lbsa.read_varlen_task_map(tm, 2, 1, 8, b["total_q"])
        assert m["error"] == 1 and m["Ndesc"] == 0
        out = H.out_np(attend(b, tm, 8))
        assert np.isnan(out).all()


SMALL_MIXES = {
    "extend+decode": ([1000, 300, 64, 4097, 130], [300, 1, 1, 1, 130]),
    "prefills": ([37, 64, 65, 200, 1000], [37, 64, 65, 200, 1000]),
    "extends": ([2000, 777, 129], [1500, 700, 16]),
}


@pytest.mark.parametrize("name", list(SMALL_MIXES))
@pytest.mark.parametrize("P,F", [(1, 0), (13, 1), (100, 2), (0, 0)])
def test_small_mixes_full_parity(oracle_mod, name, P, F):
    """Every row against the oracle, with P from one bin (nothing cut) to many
    (most segments cut into several chunks), 16 query / 2 KV heads."""
    sl, ql = SMALL_MIXES[name]
    b = varlen_batch(sl, ql, Hq=16, Hkv=2, seed=72)
    P = P or lbsa.varlen_default_workgroups(0)
    tm = plan(b, P, F)
    m = lbsa.read_varlen_task_map(tm, b["B"], 2, P, b["total_q"])
    out = attend(b, tm, P)
    ref, _ = oracle_mod.attention_varlen(b)
    H.check(b, H.out_np(out), ref, f"{name} P={P} F={F} (cut segments: {int((m['seg_num_chunks'] > 1).sum())})")


def test_many_chunk_segments_merged_in_the_split_kernel(oracle_mod):
    """A decode row of 128 tiles spread over dozens of bins (more chunks than
    the merge loads at once) beside a prefill cut at many bin edges: every
    row against the oracle."""
    b = varlen_batch([8192, 200, 3000], [1, 200, 40], Hq=8, Hkv=1, seed=74)
    P = 64
    tm = plan(b, P, 1)
    m = lbsa.read_varlen_task_map(tm, b["B"], 1, P, b["total_q"])
    assert m["seg_num_chunks"].max() > 16 and (m["seg_num_chunks"] > 1).sum() >= 4
    out = attend(b, tm, P)
    ref, _ = oracle_mod.attention_varlen(b)
    H.check(b, H.out_np(out), ref, f"many-chunk segments (max {int(m['seg_num_chunks'].max())} chunks)")


def test_repeated_calls_on_one_workspace_are_bit_identical(oracle_mod):
    """The counters are cleared by every call, and the result does not depend on
    which workgroup claims which descriptor: three calls on one workspace, with
    another map's call in between, give the same bits."""
    b = varlen_batch([2000, 777, 129, 4000], [1500, 700, 16, 1], Hq=16, Hkv=2, seed=75)
    P = 100
    tm = plan(b, P, 1)
    ws = torch.empty(lbsa.varlen_workspace_bytes(16, 2, P), dtype=torch.uint8, device="cuda:0")
    run = lambda: lbsa.attend_varlen(b["q"], b["k_cache"], b["v_cache"], b["page_table"], tm, P, b["softmax_scale"],
                                     b["B"], workspace=ws)
    first = run().clone()
    second = run().clone()
    other = varlen_batch([300, 64], [30, 64], Hq=16, Hkv=2, seed=76)
    lbsa.attend_varlen(other["q"], other["k_cache"], other["v_cache"], other["page_table"], plan(other, P), P,
                       other["softmax_scale"], other["B"], workspace=ws)
    third = run().clone()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), second.view(torch.int16))
    assert torch.equal(first.view(torch.int16), third.view(torch.int16))
    ref, _ = oracle_mod.attention_varlen(b)
    H.check(b, H.out_np(first), ref, "repeated calls")


def test_decode_rows_match_the_decode_path(oracle_mod):
    """q = 1 everywhere: the query-block path agrees with lbsa_decode within the bar
    (both against the oracle)."""
    b = varlen_batch([900, 33, 2000, 5000, 64, 1], [1] * 6, Hq=64, Hkv=8, seed=73)
    P = 256
    out = H.out_np(attend(b, plan(b, P), P))
    d = dict(b)
    d["qlens"] = None
    ref, _ = oracle_mod.attention(d)
    H.check(b, out, ref, "decode rows through query blocks")
    dec = H.out_np(H.decode(d, H.plan(d, P), P))
    H.check(b, dec, ref, "decode rows through lbsa_decode")


def test_mixed_extend_full_size_sampled_parity(oracle_mod):
    """One 8K extend of an 8K context plus 63 decode rows (64/8 heads): every
    decode row and 48 positions x 64 heads of the extend against the oracle."""
    b = wl.make_mixed_extend_batch(tail="nan", device="cuda:0")
    b["total_q"] = int(b["qlens"].sum())
    P = lbsa.varlen_default_workgroups(0)
    tm = plan(b, P)
    m = lbsa.read_varlen_task_map(tm, b["B"], 8, P, b["total_q"])
    assert m["error"] == 0 and (m["seg_num_chunks"] > 1).any()
    out = H.out_np(attend(b, tm, P))
    eq = int(b["qlens"][0])
    rng = np.random.default_rng(5)
    pos = np.unique(np.concatenate([[0, 23, 24, 4095, eq - 1], rng.integers(0, eq, 43)]))
    rows = [(int(t), hq) for t in pos for hq in range(64)] + [(eq + i, hq) for i in range(63) for hq in range(64)]
    bc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in b.items()}
    ref, _ = oracle_mod.attention_varlen_rows(bc, rows)
    got = np.stack([out[t, hq] for t, hq in rows])
    H.check(b, got, ref, f"mixed extend: {len(pos)} extend positions + 63 decode rows, all heads")


def test_varlen_auto_workgroups_rule():
    """A quarter of the resident bins once the batch has 4 segments (KV heads x
    query blocks) per resident workgroup, else one bin per resident workgroup."""
    res = lbsa.varlen_default_workgroups(0)
    qb = lbsa.QBLOCK
    enough = -(-4 * res // 8) * qb                      # one request, 8 KV heads: 4 res segments
    assert lbsa.varlen_auto_workgroups([enough], 8) == -(-res // 4)
    assert lbsa.varlen_auto_workgroups([enough - qb], 8) == res
    _, ql = wl.mixed_extend_lengths()
    nq = sum(-(-q // qb) for q in ql)
    assert lbsa.varlen_auto_workgroups(ql, 8) == (-(-res // 4) if 8 * nq >= 4 * res else res)
    assert lbsa.varlen_auto_workgroups([0, -5, 1], 1) == res   # q out of range counts no block
