"""CPU pins of the oracle's prefill / extend path on the task map (reading Q1):
query-block segments in the assign, attention of packed per-request queries,
and query-block partials.

The assign is pinned by a hand-derived example, by its reduction to the decode
map when every request brings one query, by a brute force that rebuilds the map
tile by tile from the rule, and by its error cases.  The attention is pinned by
torch's scaled_dot_product_attention in float64 with an explicit causal mask
per request, and by the uniform-q_len oracle on equal lengths; the partials by
merging every segment's chunks back into the unsplit rows.
"""
import json
import os

import numpy as np
import pytest
import torch

from load_balanced_split_assign_amd import workload as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "assign_varlen_worked_example.json")


def brute_force_map(seqlens, qlens, Hkv, P, F, QB):
    """The map rebuilt tile by tile from the rule (reading Q1 with R1): list every
    (h, b, k, t) in walk order, put global tile x in the bin whose balanced range
    holds it, and cut a descriptor wherever the segment or the bin changes."""
    tiles = []
    nq = [-(-q // QB) for q in qlens]
    for h in range(Hkv):
        for b, (L, q) in enumerate(zip(seqlens, qlens)):
            for k in range(nq[b]):
                seen = L - q + min(q, QB * (k + 1))          # tokens the block's last query sees
                for t in range(-(-seen // 64)):
                    tiles.append((h, b, k, t))
    T = len(tiles)
    if T == 0:
        return dict(T=0, K=0, desc=[], bin_desc_begin=[0] * (P + 1))
    K = min(P, max(1, T // F))
    sizes = [T // K + (1 if j < T % K else 0) for j in range(K)]
    bin_of = [j for j in range(K) for _ in range(sizes[j])]
    desc, begin = [], [None] * (P + 1)
    for x, (h, b, k, t) in enumerate(tiles):
        j = bin_of[x]
        if begin[j] is None:
            begin[j] = len(desc)
        if desc and desc[-1][:3] == [h, b, k] and desc[-1][4] == t and bin_of[x - 1] == j:
            desc[-1][4] = t + 1
        else:
            desc.append([h, b, k, t, t + 1])
    for j in range(P + 1):
        if begin[j] is None:
            begin[j] = len(desc)
    return dict(T=T, K=K, desc=desc, bin_desc_begin=begin)


def test_worked_example_from_the_golden_file(oracle_mod):
    g = json.load(open(GOLDEN))
    i, e = g["inputs"], g["expected"]
    m = oracle_mod.assign_varlen(i["seqlens"], i["qlens"], i["num_heads"], i["num_kv_heads"], i["P"], i["F"],
                                 i["max_pages"], i["QB"])
    np.testing.assert_array_equal(m["header"], e["header"])
    np.testing.assert_array_equal(m["bin_desc_begin"], e["bin_desc_begin"])
    np.testing.assert_array_equal(m["desc"], e["desc"])
    np.testing.assert_array_equal(m["seg_first_desc"], e["seg_first_desc"])
    np.testing.assert_array_equal(m["seg_num_chunks"], e["seg_num_chunks"])


def test_one_query_per_request_is_the_decode_map(oracle_mod):
    rng = np.random.default_rng(11)
    for _ in range(60):
        B = int(rng.integers(1, 30))
        Hkv = int(rng.choice([1, 2, 8]))
        sl = rng.integers(1, 3000, B).astype(np.int32)
        P, F = int(rng.integers(1, 300)), int(rng.integers(1, 4))
        mp = int(max(1, (sl.max() + 63) // 64))
        d = oracle_mod.assign(sl, 8 * Hkv, Hkv, P, F, mp)
        v = oracle_mod.assign_varlen(sl, np.ones(B, np.int32), 8 * Hkv, Hkv, P, F, mp)
        np.testing.assert_array_equal(v["header"][:14], d["header"][:14])
        np.testing.assert_array_equal(v["bin_desc_begin"], d["bin_desc_begin"])
        np.testing.assert_array_equal(v["desc"][:, [0, 1, 3, 4]], d["desc"])
        assert (v["desc"][:, 2] == 0).all()
        np.testing.assert_array_equal(v["seg_first_desc"], d["seg_first_desc"])   # s = h*B + b: NQ = B
        np.testing.assert_array_equal(v["seg_num_chunks"], d["seg_num_chunks"])


@pytest.mark.parametrize("QB", [4, 16, 24])
def test_brute_force_small_cases(oracle_mod, QB):
    rng = np.random.default_rng(12 + QB)
    cases = 0
    for L0 in (1, 63, 64, 65, 130):
        for q0 in sorted({1, min(L0, 5), min(L0, 17), L0}):
            for L1, q1 in ((40, 1), (200, 37), (64, 64)):
                for Hkv in (1, 2):
                    for P in (1, 2, 3, 5, 7):
                        F = int(rng.integers(1, 4))
                        sl, ql = [L0, L1], [q0, q1]
                        m = oracle_mod.assign_varlen(sl, ql, 8 * Hkv, Hkv, P, F, 4, QB)
                        bf = brute_force_map(sl, ql, Hkv, P, F, QB)
                        assert m["T"] == bf["T"] and m["K"] == bf["K"], (sl, ql, Hkv, P, F)
                        np.testing.assert_array_equal(m["desc"].reshape(-1, 5), np.asarray(bf["desc"]).reshape(-1, 5))
                        np.testing.assert_array_equal(m["bin_desc_begin"], bf["bin_desc_begin"])
                        # chunk counts per segment, segments in (h, b, k) order
                        segs = [(h, b, k) for h in range(Hkv) for b in range(2) for k in range(-(-ql[b] // QB))]
                        counts = [sum(1 for d in bf["desc"] if tuple(d[:3]) == s) for s in segs]
                        np.testing.assert_array_equal(m["seg_num_chunks"], counts)
                        np.testing.assert_array_equal(m["seg_first_desc"], np.cumsum([0] + counts[:-1]))
                        cases += 1
    assert cases > 200


def test_prefill_segments_follow_the_causal_extent(oracle_mod):
    """q = L (a prefill of 1000 tokens), one KV head, enough bins for every tile:
    block k spans ceil(min(1000, 16 (k + 1)) / 64) tiles."""
    m = oracle_mod.assign_varlen([1000], [1000], 8, 1, 100000, 1, 16)
    nq = -(-1000 // 16)
    assert m["NQ"] == nq and m["Ndesc"] == m["T"]                     # one tile per bin
    per_block = np.bincount(m["desc"][:, 2], minlength=nq)
    np.testing.assert_array_equal(per_block, [-(-min(1000, 16 * (k + 1)) // 64) for k in range(nq)])


@pytest.mark.parametrize("sl,ql", [([100, 50], [101, 1]), ([100, 50], [0, 1]), ([-1, 50], [1, 1]),
                                   ([300, 50], [1, 1])])
def test_bad_lengths_set_the_error_word(oracle_mod, sl, ql):
    m = oracle_mod.assign_varlen(sl, ql, 8, 1, 8, 2, 4)
    assert m["error"] == 1 and m["T"] == 0 and m["Ndesc"] == 0


def _sdpa_rows(batch, oracle_mod):
    """Per request: dense fp64 K/V, the request's packed queries, an explicit
    causal mask (query i sees tokens <= L - q + i), torch SDPA."""
    outs = []
    qs = 0
    q = oracle_mod.bf16_values(batch["q"].view(torch.int16))
    Hq, Hkv = batch["num_heads"], batch["num_kv_heads"]
    for b in range(batch["B"]):
        L, n = int(batch["seqlens"][b]), int(batch["qlens"][b])
        pages = batch["page_table"][b, : (L + 63) // 64].numpy()
        k = oracle_mod.bf16_values(batch["k_cache"].view(torch.int16)[pages]).reshape(-1, Hkv, 128)[:L]
        v = oracle_mod.bf16_values(batch["v_cache"].view(torch.int16)[pages]).reshape(-1, Hkv, 128)[:L]
        kk = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1)).permute(1, 0, 2)      # [Hq, L, D]
        vv = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1)).permute(1, 0, 2)
        qq = torch.from_numpy(q[qs: qs + n]).permute(1, 0, 2)                          # [Hq, n, D]
        mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                                             scale=batch["softmax_scale"])
        outs.append(o.permute(1, 0, 2).numpy())
        qs += n
    return np.concatenate(outs)


def test_varlen_attention_matches_sdpa_with_causal_masks(oracle_mod):
    batch = wl.make_batch(seqlens=[100, 50, 130, 64], qlens=[20, 1, 130, 64], num_heads=16, num_kv_heads=2,
                          kv_dtype="bf16", seed=60, tail="normal")
    out, lse = oracle_mod.attention_varlen(batch)
    ref = _sdpa_rows(batch, oracle_mod)
    assert out.shape == ref.shape == (20 + 1 + 130 + 64, 16, 128)
    assert np.abs(out - ref).max() < 1e-12


def test_varlen_attention_equals_uniform_q_len_layout(oracle_mod):
    """Every request with q = 3: the packed rows are the [B][3] rows of the M1 oracle."""
    kw = dict(seqlens=[70, 3, 200], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=61, tail="nan")
    packed = wl.make_batch(**kw, qlens=[3, 3, 3])
    uniform = dict(packed)
    uniform["q"] = packed["q"].reshape(3, 3, 8, 128)
    uniform["qlens"] = None
    a, la = oracle_mod.attention_varlen(packed)
    u, lu = oracle_mod.attention(uniform)
    np.testing.assert_array_equal(a.reshape(3, 3, 8, 128), u)
    np.testing.assert_array_equal(la.reshape(3, 3, 8), lu)


def test_varlen_partials_merge_back_and_pad_empty(oracle_mod):
    """Every segment's chunks (a small P cuts most segments) merge to the unsplit
    rows; rows of block positions past q_b are empty."""
    sl, ql = [300, 50, 1000, 40], [37, 1, 1000, 40]
    batch = wl.make_batch(seqlens=sl, qlens=ql, num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=62,
                          tail="nan")
    m = oracle_mod.assign_varlen(sl, ql, 16, 2, 37, 1, 16)
    po, pl = oracle_mod.partials_varlen(batch, m["desc"])
    full, _ = oracle_mod.attention_varlen(batch)
    qstart = np.concatenate([[0], np.cumsum(ql)])
    nq = [-(-q // 16) for q in ql]
    qbase = np.concatenate([[0], np.cumsum(nq)])
    checked = 0
    for s in range(2 * m["NQ"]):
        h, rest = divmod(s, m["NQ"])
        b = int(np.searchsorted(qbase, rest, side="right") - 1)
        k = rest - qbase[b]
        d0, n = m["seg_first_desc"][s], m["seg_num_chunks"][s]
        for p in range(16):
            for g in range(8):
                row = p * 8 + g
                o, lse = oracle_mod.merge(po[d0:d0 + n, row], pl[d0:d0 + n, row])
                i = 16 * k + p
                if i >= ql[b]:
                    assert (po[d0:d0 + n, row] == 0).all() and np.isneginf(pl[d0:d0 + n, row]).all()
                    continue
                assert np.abs(o - full[qstart[b] + i, h * 8 + g]).max() < 1e-12
                checked += 1
    assert checked == sum(ql) * 16
