"""GPU assign kernel vs the oracle's assign: the task map must be bit-exact.

Compared: header words 0..13, bin CSR (P + 1 entries), descriptors [0, Ndesc),
per-segment first descriptor and chunk count, the length copy, the per-bin
head records (expected values built from the oracle's descriptors and CSR), and
the combine's list of long segments (more than 8 chunks, header word 14),
built here from the oracle's chunk counts.  Slots of the descriptor array past
Ndesc are unspecified and not compared.
"""
import numpy as np
import pytest
import torch

from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa
from load_balanced_split_assign_amd import workload as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def gpu_map(seqlens, Hq, Hkv, P, F, max_pages):
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda:0")
    tm = lbsa.plan(sl, Hq, Hkv, max_pages, P, F)
    torch.cuda.synchronize()
    return lbsa.read_task_map(tm, len(seqlens), Hkv, P)


def assert_same_map(oracle_mod, seqlens, Hq, Hkv, P, F, max_pages, what=""):
    g = gpu_map(seqlens, Hq, Hkv, P, F, max_pages)
    o = oracle_mod.assign(np.asarray(seqlens, np.int32), Hq, Hkv, P, F or 2, max_pages)
    ctx = (what, len(seqlens), Hkv, P, F)
    np.testing.assert_array_equal(g["header"][:14], o["header"][:14], err_msg=str(ctx))
    np.testing.assert_array_equal(g["bin_desc_begin"], o["bin_desc_begin"], err_msg=str(ctx))
    np.testing.assert_array_equal(g["desc"], o["desc"], err_msg=str(ctx))
    np.testing.assert_array_equal(g["seg_first_desc"], o["seg_first_desc"], err_msg=str(ctx))
    np.testing.assert_array_equal(g["seg_num_chunks"], o["seg_num_chunks"], err_msg=str(ctx))
    np.testing.assert_array_equal(g["seqlens"], np.asarray(seqlens, np.int32), err_msg=str(ctx))
    sl = np.asarray(seqlens, np.int32)
    np.testing.assert_array_equal(g["bin_head"], expected_bin_head(o, P, sl), err_msg=str(ctx))
    np.testing.assert_array_equal(g["desc_len"], sl[np.asarray(o["desc"], np.int64)[:, 1]] if len(o["desc"]) else
                                  np.zeros(0, np.int32), err_msg=str(ctx))
    want = expected_long_segments(o)
    assert g["nlong"] == len(want), ctx
    np.testing.assert_array_equal(g["long_seg"], want, err_msg=str(ctx))
    return g


def expected_long_segments(o):
    """(segment, first descriptor, chunks, 0) of each segment with more than
    lbsa.LONG_SEGMENT_CHUNKS chunks in the oracle's map, in segment order."""
    snc = np.asarray(o["seg_num_chunks"], np.int64)
    sfd = np.asarray(o["seg_first_desc"], np.int64)
    s = np.nonzero(snc > lbsa.LONG_SEGMENT_CHUNKS)[0]
    return np.stack([s, sfd[s], snc[s], np.zeros_like(s)], axis=1).astype(np.int32).reshape(-1, 4)


def expected_bin_head(o, P, seqlens):
    """Head record of each bin from the oracle's map: first descriptor of the
    bin (zeros if none), its index, the bin's descriptor count, the length of
    the descriptor's request, 0."""
    bdb = np.asarray(o["bin_desc_begin"], np.int64)
    head = np.zeros((P, 8), np.int32)
    for j in range(P):
        d0, d1 = int(bdb[j]), int(bdb[j + 1])
        head[j, 4] = d0
        head[j, 5] = d1 - d0
        if d1 > d0:
            head[j, :4] = o["desc"][d0]
            head[j, 6] = seqlens[o["desc"][d0][1]]
    return head


@pytest.mark.parametrize("name", ["tiny", "tp8_share", "skewed", "fp8", "long", "floor",
                                  "t3_64x0.5K", "t3_1x128K+31x4K"])
def test_workload_maps_bitexact(oracle_mod, name):
    w = wl.WORKLOADS[name]
    sl = wl.draw_seqlens(w, torch.Generator().manual_seed(w.seed)).tolist()
    mp = max(1, max((L + 63) // 64 for L in sl))
    Ps = [w.num_workgroups] if w.num_workgroups else [256, 512, 768, 1024, 2048, lbsa.default_workgroups(0, w.kv_dtype)]
    for P in Ps:
        for F in (0, 1, 3):
            g = assert_same_map(oracle_mod, sl, w.num_heads, w.num_kv_heads, P, F, mp, name)
    if name == "floor":   # batch-1, 200 tokens: the floor caps every head at 2 chunks (<= 4)
        assert g["K"] < P and (g["seg_num_chunks"] <= 4).all()


def test_random_maps_bitexact(oracle_mod):
    rng = np.random.default_rng(2024)
    for it in range(150):
        B = int(rng.integers(1, 400))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        if 2 * B + 1 + Hkv * B + 1 > 16384:
            B = 16382 // (Hkv + 2)
        sl = rng.integers(0, 5000, B)
        sl[rng.random(B) < 0.1] = 0
        sl[rng.random(B) < 0.1] = 64 * rng.integers(1, 40)
        if rng.random() < 0.3:
            sl[int(rng.integers(0, B))] = int(rng.integers(50000, 300000))
        mp = max(1, int((sl.max() + 63) // 64) + int(rng.integers(0, 3)))
        P = int(rng.choice([1, 2, 3, 17, 255, 256, 257, 512, 1000, 1536, 4096]))
        F = int(rng.integers(0, 6))
        assert_same_map(oracle_mod, sl.astype(np.int32).tolist(), 8 * Hkv, Hkv, P, F, mp, f"random {it}")


def test_large_batch_and_segment_count(oracle_mod):
    rng = np.random.default_rng(7)
    sl = rng.integers(0, 3000, 1630).astype(np.int32).tolist()       # 2*1630 + 13040 + 2 ints of LDS
    assert_same_map(oracle_mod, sl, 64, 8, 1024, 0, 47, "B=1630 Hkv=8")
    sl = rng.integers(1, 9000, 5400).astype(np.int32).tolist()       # Hkv = 1, batch 5400
    assert_same_map(oracle_mod, sl, 8, 1, 2048, 0, 141, "B=5400 Hkv=1")


def test_bad_lengths_set_error_and_empty_map(oracle_mod):
    for sl in ([10, -5, 70], [10, 64 * 4 + 1, 70]):
        g = assert_same_map(oracle_mod, sl, 8, 1, 16, 0, 4, "bad")
        assert g["error"] == 1 and g["Ndesc"] == 0 and (g["bin_desc_begin"] == 0).all()


def test_all_empty(oracle_mod):
    g = assert_same_map(oracle_mod, [0, 0, 0, 0], 64, 8, 512, 0, 2, "empty")
    assert g["T"] == 0 and g["K"] == 0 and g["Ndesc"] == 0


def test_map_is_deterministic():
    sl = list(range(0, 5000, 37))
    a = gpu_map(sl, 64, 8, 777, 2, 79)
    b = gpu_map(sl, 64, 8, 777, 2, 79)
    for k in ("header", "bin_desc_begin", "desc", "seg_first_desc", "seg_num_chunks"):
        np.testing.assert_array_equal(a[k], b[k])
