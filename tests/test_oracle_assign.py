"""Pins of the oracle's assign (task-map builder).

The rule is the "Assign" bullet of the HPC-Ops vLLM integration post (section
"The solution: a per-step, load-balanced decode scheduler") and the paragraph
"Scheduling around live KV work" of the SGLang post: 64-token tiles, head-major
and batch-minor traversal, a per-workgroup budget of total tiles / workgroups,
fill a bucket then spill into the next, a minimum-work floor.  Reading taken
for the budget: K = min(P, max(1, floor(T/F))) active bins, the first T mod K
filled to ceil(T/K), the rest to floor(T/K).

Pins, none of which reuse the oracle's code:
* hand-derived task maps (tests/golden/assign_worked_examples.json);
* an independent brute force (explicit tile list, cumulative bin bounds,
  maximal runs), exhaustive over small inputs and randomised beyond;
* the invariants the method promises: exact cover, each bin one contiguous
  range, bin sizes within one tile, the floor, max bin = ceil(T/P) when the
  floor does not bind, the chunk-count bound.
"""
import bisect
import itertools
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "assign_worked_examples.json")


def brute_force(seqlens, Hkv, P, F, max_pages):
    """Independent construction of the task map on tiny inputs."""
    B = len(seqlens)
    if any(L < 0 or L > max_pages * 64 for L in seqlens):
        return dict(T=0, K=0, q=0, r=0, error=1, desc=[], bin_desc_begin=[0] * (P + 1),
                    seg_num_chunks=[0] * (Hkv * B), seg_first_desc=[0] * (Hkv * B))
    n = [(L + 63) // 64 for L in seqlens]
    tiles = [(h, b, t) for h in range(Hkv) for b in range(B) for t in range(n[b])]
    T = len(tiles)
    if T == 0:
        K = q = r = 0
        sizes = []
    else:
        K = min(P, max(1, T // F))
        q, r = divmod(T, K)
        sizes = [q + 1] * r + [q] * (K - r)
    ends = list(itertools.accumulate(sizes))
    desc, desc_bin = [], []
    for g, (h, b, t) in enumerate(tiles):
        j = bisect.bisect_right(ends, g)
        if desc and desc_bin[-1] == j and desc[-1][0] == h and desc[-1][1] == b:
            desc[-1][3] = t + 1
        else:
            desc.append([h, b, t, t + 1])
            desc_bin.append(j)
    bdb = [sum(1 for x in desc_bin if x < j) for j in range(P + 1)]
    snc = [sum(1 for d in desc if d[0] == h and d[1] == b) for h in range(Hkv) for b in range(B)]
    sfd = [sum(snc[:s]) for s in range(Hkv * B)]
    return dict(T=T, K=K, q=q, r=r, error=0, desc=desc, bin_desc_begin=bdb,
                seg_num_chunks=snc, seg_first_desc=sfd)


def check_invariants(m, seqlens, Hkv, P, F):
    B = len(seqlens)
    n = [(L + 63) // 64 for L in seqlens]
    T = Hkv * sum(n)
    assert m["T"] == T
    desc = m["desc"]
    nd = len(desc)
    assert m["Ndesc"] == nd
    # exact cover, in head-major batch-minor order, no empty descriptor
    covered = [(h, b, t) for (h, b, t0, t1) in desc for t in range(t0, t1)]
    expected = [(h, b, t) for h in range(Hkv) for b in range(B) for t in range(n[b])]
    assert covered == expected
    assert all(t1 > t0 for (_, _, t0, t1) in desc)
    if T == 0:
        assert m["K"] == 0 and nd == 0
        assert list(m["bin_desc_begin"]) == [0] * (P + 1)
        return
    K = m["K"]
    assert K == min(P, max(1, T // F))
    bdb = list(m["bin_desc_begin"])
    assert bdb[0] == 0 and all(x == nd for x in bdb[K:])
    sizes = [sum(d[3] - d[2] for d in desc[bdb[j]:bdb[j + 1]]) for j in range(K)]
    assert sum(sizes) == T
    assert max(sizes) - min(sizes) <= 1                      # balanced within one tile
    assert sizes == sorted(sizes, reverse=True)               # fill first, then spill
    if T >= F:
        assert min(sizes) >= F                                # the minimum-work floor
    if T // F >= P:                                           # floor does not bind
        assert max(sizes) == -(-T // P)                       # budget = ceil(T / P)
    # within a bin, descriptors follow each other in traversal order
    for j in range(K):
        for a, b2 in zip(desc[bdb[j]:bdb[j + 1]], desc[bdb[j] + 1:bdb[j + 1]]):
            assert (a[0], a[1]) < (b2[0], b2[1]) and b2[2] == 0
    snc = list(m["seg_num_chunks"])
    assert sum(snc) == nd <= Hkv * B + K - 1
    sfd = list(m["seg_first_desc"])
    for s in range(Hkv * B):
        h, b = divmod(s, B)
        for k in range(snc[s]):
            assert tuple(desc[sfd[s] + k][:2]) == (h, b)


def _as_lists(m):
    return dict(m, desc=m["desc"].tolist(), bin_desc_begin=m["bin_desc_begin"].tolist(),
                seg_num_chunks=m["seg_num_chunks"].tolist(), seg_first_desc=m["seg_first_desc"].tolist())


def test_worked_examples(oracle_mod):
    for ex in json.load(open(GOLDEN))["examples"]:
        m = _as_lists(oracle_mod.assign(ex["seqlens"], ex["num_heads"], ex["num_kv_heads"],
                                        ex["P"], ex["F"], ex["max_pages"]))
        e = ex["expect"]
        for key in ("T", "K", "q", "r", "Ndesc", "N", "error"):
            assert m[key] == e[key], (ex["name"], key)
        if "desc" in e:
            assert m["desc"] == e["desc"], ex["name"]
        if "bin_desc_begin" in e:
            assert m["bin_desc_begin"] == e["bin_desc_begin"]
        if "bin_desc_begin_prefix" in e:
            k = len(e["bin_desc_begin_prefix"])
            assert m["bin_desc_begin"][:k] == e["bin_desc_begin_prefix"]
            assert all(x == e["bin_desc_begin_rest"] for x in m["bin_desc_begin"][k:])
        if "desc_16_17" in e:
            assert m["desc"][16:18] == e["desc_16_17"] and m["desc"][-1] == e["desc_last"]
        assert m["seg_num_chunks"] == e["seg_num_chunks"]
        assert m["seg_first_desc"] == e["seg_first_desc"]
        assert m["header"][5] == ex["P"] and m["header"][6] == ex["F"]
        assert m["header"][13] == 64


def test_floor_limits_chunks_per_head(oracle_mod):
    """Batch-1 200-token run: at most 4 chunks per head, exactly 2 with the floor."""
    for P in (256, 512, 768, 1024, 2048):
        m = oracle_mod.assign([200], 64, 8, P, 2, 4)
        assert m["K"] == 16 and list(m["seg_num_chunks"]) == [2] * 8
        m1 = oracle_mod.assign([200], 64, 8, P, 1, 4)
        assert list(m1["seg_num_chunks"]) == [4] * 8


@pytest.mark.parametrize("Hkv", [1, 2])
def test_brute_force_exhaustive_small(oracle_mod, Hkv):
    lengths = [0, 1, 63, 64, 65, 128, 200]
    for B in (1, 2, 3):
        for sl in itertools.product(lengths, repeat=B):
            for P in range(1, 10):
                for F in (1, 2, 3):
                    m = _as_lists(oracle_mod.assign(list(sl), Hkv * 2, Hkv, P, F, 4))
                    bf = brute_force(list(sl), Hkv, P, F, 4)
                    for key in ("T", "K", "q", "r", "error", "desc", "bin_desc_begin",
                                "seg_num_chunks", "seg_first_desc"):
                        assert m[key] == bf[key], (sl, Hkv, P, F, key)
                    check_invariants(m, list(sl), Hkv, P, F)


def test_brute_force_random(oracle_mod):
    rng = np.random.default_rng(1234)
    for _ in range(300):
        B = int(rng.integers(1, 12))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        sl = [int(x) for x in rng.integers(0, 3000, B)]
        if rng.random() < 0.3:
            sl[int(rng.integers(0, B))] = int(rng.integers(3000, 40000))
        P = int(rng.integers(1, 300))
        F = int(rng.integers(1, 6))
        mp = max(1, max((L + 63) // 64 for L in sl))
        m = _as_lists(oracle_mod.assign(sl, Hkv * 8, Hkv, P, F, mp))
        bf = brute_force(sl, Hkv, P, F, mp)
        for key in ("T", "K", "q", "r", "desc", "bin_desc_begin", "seg_num_chunks", "seg_first_desc"):
            assert m[key] == bf[key], (sl, Hkv, P, F, key)
        check_invariants(m, sl, Hkv, P, F)


def test_invalid_lengths_give_empty_map_with_error(oracle_mod):
    for sl in ([5, -1, 7], [5, 64 * 3 + 1]):
        m = oracle_mod.assign(sl, 8, 1, 16, 2, 3)
        assert m["error"] == 1 and m["T"] == 0 and m["K"] == 0 and m["Ndesc"] == 0
        assert list(m["bin_desc_begin"]) == [0] * 17
        assert list(m["seg_num_chunks"]) == [0] * len(sl)


def test_all_empty_batch(oracle_mod):
    m = oracle_mod.assign([0, 0, 0], 64, 8, 100, 2, 1)
    assert m["error"] == 0 and m["T"] == 0 and m["K"] == 0 and m["Ndesc"] == 0


def test_rejects_bad_arguments(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.assign([10], 12, 8, 4, 2, 1)   # Hq not a multiple of Hkv
    with pytest.raises(ValueError):
        oracle_mod.assign([10], 8, 1, 0, 2, 1)    # no bins
