"""GPU split + combine vs the fp64 oracle, and properties of the path.

Tolerances: max |out - oracle| <= 2e-2 for bf16 KV and <= 6e-2 for fp8-e4m3 KV
(bf16 output); partials: O within the same bound, LSE within 1e-3.  Every
input comes from the seeded generator with NaN in the tail slots of each last
page, so a masked token that leaks shows up as NaN.
"""
import numpy as np
import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa

pytestmark = [pytest.mark.gpu, requires_gpu]


def check_full(oracle_mod, batch, out, what):
    ref, _ = oracle_mod.attention(batch)
    return H.check(batch, H.out_np(out), ref, what)


def check_rows(oracle_mod, batch, out, rows, what):
    ref, _ = oracle_mod.attention_rows(batch, rows)
    got = H.out_np(out)[rows[:, 0], rows[:, 1]]
    return H.check(batch, got, ref, what)


@pytest.mark.parametrize("name", ["tiny", "floor", "t3_32x0.125K+32x4K", "t3_1x64K+15x4K"])
def test_small_workloads_full_parity(oracle_mod, name):
    batch = H.batch_on_gpu(name)
    P = H.workgroups(batch)
    tm = H.plan(batch, P)
    out = H.decode(batch, tm, P)
    check_full(oracle_mod, batch, out, name)


def test_tp8_share_full_parity(oracle_mod):
    batch = H.batch_on_gpu("tp8_share")
    P = H.workgroups(batch)
    out = H.decode(batch, H.plan(batch, P), P)
    check_full(oracle_mod, batch, out, "tp8_share")


@pytest.mark.parametrize("name", ["skewed", "fp8", "long"])
def test_large_workloads_full_parity(oracle_mod, name):
    """Every row of the full-size batches (skewed: 4096 rows, 10.4M token-rows,
    its 131072-token request spread over many bins; fp8: 4096 rows; long: 512 rows
    of 64K-256K tokens) against the fp64 oracle, under both bounds."""
    batch = H.batch_on_gpu(name, gen_device="cuda:0")
    P = H.workgroups(batch)
    out = H.decode(batch, H.plan(batch, P), P)
    check_full(oracle_mod, batch, out, name)


def test_long_partials_of_sampled_descriptors(oracle_mod):
    """Config 5 at full size: partial O and LSE of 20 sampled descriptors (the first
    and last of the map, the longest, and random ones) against oracle_partials."""
    batch = H.batch_on_gpu("long", gen_device="cuda:0")
    P = H.workgroups(batch)
    tm = H.plan(batch, P)
    ws = H.decode_split(batch, tm, P)
    m = lbsa.read_task_map(tm, batch["B"], batch["num_kv_heads"], P)
    nd = m["Ndesc"]
    po, pl = lbsa.read_partials(ws, batch["B"], batch["num_heads"], batch["num_kv_heads"], P, nd)
    rng = np.random.default_rng(7)
    span = m["desc"][:, 3] - m["desc"][:, 2]
    pick = sorted({0, nd - 1, int(np.argmax(span)), *rng.choice(nd, 17, replace=False).tolist()})
    ro, rl = oracle_mod.partials(batch, m["desc"][pick])
    H.check(batch, po[pick], ro, f"long partial O ({len(pick)} descriptors)")
    assert np.abs(pl[pick] - rl).max() <= H.LSE_TOL


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_partials_match_oracle(oracle_mod, kv):
    batch = H.batch_on_gpu(dict(seqlens=[37, 64, 1000, 4097, 1, 130], num_heads=16, num_kv_heads=2,
                                kv_dtype=kv, seed=21))
    P = 29
    tm = H.plan(batch, P)
    ws = H.decode_split(batch, tm, P)
    m = lbsa.read_task_map(tm, batch["B"], batch["num_kv_heads"], P)
    po, pl = lbsa.read_partials(ws, batch["B"], batch["num_heads"], batch["num_kv_heads"], P, m["Ndesc"])
    ro, rl = oracle_mod.partials(batch, m["desc"])
    assert np.isfinite(pl).all()
    H.check(batch, po, ro, f"partials {kv}")
    assert np.abs(pl - rl).max() <= H.LSE_TOL


@pytest.mark.parametrize("P", [1, 3, 64, 1000, 4096])
@pytest.mark.parametrize("F", [0, 1, 5])
def test_any_workgroup_count_and_floor(oracle_mod, P, F):
    batch = H.batch_on_gpu(dict(seqlens=[5, 3000, 64, 700, 0, 129], num_heads=16, num_kv_heads=2,
                                kv_dtype="bf16", seed=22))
    out = H.decode(batch, H.plan(batch, P, F), P)
    check_full(oracle_mod, batch, out, (P, F))


def test_fp8_mixed_lengths(oracle_mod):
    batch = H.batch_on_gpu(dict(seqlens=[1, 63, 64, 65, 2047, 5000, 130, 17], num_heads=64, num_kv_heads=8,
                                kv_dtype="fp8", seed=23))
    P = H.workgroups(batch)
    out = H.decode(batch, H.plan(batch, P), P)
    check_full(oracle_mod, batch, out, "fp8 mixed")


def test_empty_requests_give_zero_rows(oracle_mod):
    batch = H.batch_on_gpu(dict(seqlens=[0, 100, 0, 7], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=24))
    P = 40
    out = H.decode(batch, H.plan(batch, P), P)
    got = H.out_np(out)
    assert (got[0] == 0).all() and (got[2] == 0).all()
    check_full(oracle_mod, batch, out, "empty rows")


def test_deterministic_and_workspace_fully_overwritten():
    batch = H.batch_on_gpu("tp8_share")
    P = H.workgroups(batch)
    tm = H.plan(batch, P)
    ws = torch.full((lbsa.workspace_bytes(batch["B"], 8, 1, P) // 4,), float("nan"), device="cuda:0")
    a = H.decode(batch, tm, P, workspace=ws.view(torch.uint8)).clone()
    ws.fill_(float("nan"))
    b = H.decode(batch, tm, P, workspace=ws.view(torch.uint8)).clone()
    c = H.decode(batch, tm, P).clone()
    torch.cuda.synchronize()
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_page_permutation_invariance():
    batch = H.batch_on_gpu(dict(seqlens=[300, 4097, 64, 1], num_heads=16, num_kv_heads=2, kv_dtype="fp8",
                                seed=25))
    P = 50
    tm = H.plan(batch, P)
    a = H.decode(batch, tm, P).clone()
    perm = torch.randperm(batch["num_pages"], generator=torch.Generator().manual_seed(5)).to("cuda:0")
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel(), device="cuda:0")
    b2 = dict(batch)
    for k in ("k_cache", "v_cache", "k_scale", "v_scale"):
        b2[k] = batch[k][perm].contiguous()
    pt = batch["page_table"].clone()
    m = pt >= 0
    pt[m] = inv[pt[m].long()].to(torch.int32)
    b2["page_table"] = pt
    b = H.decode(b2, tm, P)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_map_reused_across_layers(oracle_mod):
    """One plan per step, many layers: two layers with different K/V."""
    l1 = H.batch_on_gpu(dict(seqlens=[900, 33, 2000], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=26))
    l2 = H.batch_on_gpu(dict(seqlens=[900, 33, 2000], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=27))
    P = 70
    tm = H.plan(l1, P)
    o1 = H.decode(l1, tm, P).clone()
    o2 = H.decode(l2, tm, P).clone()
    check_full(oracle_mod, l1, o1, "layer 1")
    check_full(oracle_mod, l2, o2, "layer 2")


def test_bad_page_id_poisons_only_its_rows():
    batch = H.batch_on_gpu(dict(seqlens=[200, 300, 100], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=28))
    batch["page_table"][1, 2] = batch["num_pages"] + 5          # out of range: never read
    P = 9
    out = H.out_np(H.decode(batch, H.plan(batch, P), P))
    assert np.isnan(out[1]).all()
    assert np.isfinite(out[0]).all() and np.isfinite(out[2]).all()


def test_bad_length_gives_error_flag_and_nan_output():
    """A length outside [0, max_pages * 64] sets the map's error word; the map is
    empty and the decode writes NaN in every row (never plausible zeros)."""
    batch = H.batch_on_gpu(dict(seqlens=[200, 300], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=29))
    batch["seqlens"][1] = 64 * batch["max_pages"] + 1
    P = 9
    tm = H.plan(batch, P)
    out = H.out_np(H.decode(batch, tm, P))
    assert lbsa.read_task_map(tm, 2, 1, P)["error"] == 1
    assert np.isnan(out).all()
    ws = H.decode_split(batch, tm, P)
    out2 = H.out_np(lbsa.decode_combine(2, 8, 1, P, tm, ws))
    assert np.isnan(out2).all()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("q_len", [1, 2])
def test_direct_rows_match_split_then_combine(kv, q_len):
    """lbsa_decode writes a single-chunk segment's rows from the split kernel;
    split + combine (all partials written and merged) gives the same bits."""
    batch = H.batch_on_gpu(dict(seqlens=[1, 64, 65, 300, 2000, 9000, 0, 130, 4097, 17], num_heads=64,
                                num_kv_heads=8, kv_dtype=kv, seed=31, q_len=q_len))
    P = 96
    tm = H.plan(batch, P)
    m = lbsa.read_task_map(tm, batch["B"], 8, P)
    single = int((m["seg_num_chunks"] == 1).sum())
    assert single > 0 and int((m["seg_num_chunks"] > 1).sum()) > 0
    a = H.decode(batch, tm, P)
    ws = H.decode_split(batch, tm, P)
    b = lbsa.decode_combine(batch["B"], 64, 8, P, tm, ws, q_len=q_len)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.reshape(a.shape).view(torch.int16))


@pytest.mark.parametrize("n", [2, 15, 16, 17, 63, 64, 65, 300])
def test_combine_of_n_chunks(oracle_mod, n):
    """One request of n tiles on P = n bins with floor 1: its segment is cut into
    n one-tile chunks (the combine's slices take 64 per round trip: 63, 64 and 65
    straddle that)."""
    batch = H.batch_on_gpu(dict(seqlens=[64 * n - 5], num_heads=8, num_kv_heads=1, kv_dtype="bf16",
                                seed=40 + n))
    tm = H.plan(batch, n, F=1)
    assert int(lbsa.read_task_map(tm, 1, 1, n)["seg_num_chunks"][0]) == n
    check_full(oracle_mod, batch, H.decode(batch, tm, n), f"{n} chunks")


def test_many_cut_segments_two_query_tokens(oracle_mod):
    """fp8, two query tokens, two KV heads: a 400-tile request cut into about 360
    chunks per head beside short, empty and mid-size requests."""
    batch = H.batch_on_gpu(dict(seqlens=[64 * 400, 100, 2600, 0, 7000], num_heads=16, num_kv_heads=2,
                                kv_dtype="fp8", seed=48, q_len=2))
    P = 1000
    tm = H.plan(batch, P, F=1)
    assert int(lbsa.read_task_map(tm, 5, 2, P)["seg_num_chunks"].max()) > 256
    check_full(oracle_mod, batch, H.decode(batch, tm, P), "many cut segments")


def test_all_requests_empty_gives_zero_rows():
    """T = 0: no bins and no descriptors; every row is 0, whatever out held."""
    batch = H.batch_on_gpu(dict(seqlens=[0, 0, 0], num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=50))
    P = 32
    out = H.decode(batch, H.plan(batch, P), P, out=torch.full((3, 16, 128), float("nan"), dtype=torch.bfloat16,
                                                                device="cuda:0"))
    assert (H.out_np(out) == 0).all()


def test_mismatched_map_poisons_output():
    batch = H.batch_on_gpu(dict(seqlens=[200, 300], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=30))
    tm = H.plan(batch, 16)
    big = torch.zeros(lbsa.task_map_bytes(2, 1, 32), dtype=torch.uint8, device="cuda:0")
    big[:tm.numel()] = tm                                          # map built for P = 16, used with P = 32
    out = H.out_np(H.decode(batch, big, 32))
    assert np.isnan(out).all()


def test_auto_workgroups_rule():
    """lbsa_auto_workgroups: the resident count, doubled for batches of several KV
    heads with at least 32 tiles per resident workgroup."""
    for kv in ("bf16", "fp8"):
        res = lbsa.default_workgroups(0, kv)
        assert lbsa.auto_workgroups([64 * 32] * res, 1, kv) == res                 # one KV head: never doubled
        assert lbsa.auto_workgroups([64 * 32] * (res // 8), 8, kv) == 2 * res      # exactly 32 tiles each
        assert lbsa.auto_workgroups([64 * 31] * (res // 8), 8, kv) == res          # 31 tiles each
        assert lbsa.auto_workgroups([], 8, kv) == res


@pytest.mark.parametrize("q_len", [1, 2])
def test_combine_segment_forms(oracle_mod, q_len):
    """The combine's two forms side by side: segments of 0, 1 and 2..8 chunks
    (merged whole, one workgroup per segment; a single chunk written by the
    split kernel) and of 9 and 11 (one workgroup per output row, from the map's
    long-segment list); every row against the oracle, both query counts."""
    sl = [4629, 3196, 4561, 120, 2544, 1590, 553, 3552, 5776, 1142, 255, 0]
    batch = H.batch_on_gpu(dict(seqlens=sl, num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=61, q_len=q_len))
    P = 96
    tm = H.plan(batch, P, 1)
    m = lbsa.read_task_map(tm, len(sl), 2, P)
    snc = m["seg_num_chunks"]
    assert {0, 1, 8, 9}.issubset(set(snc.tolist()))
    assert m["nlong"] == int((snc > lbsa.LONG_SEGMENT_CHUNKS).sum()) > 0
    out = H.decode(batch, tm, P)
    check_full(oracle_mod, batch, out, ("combine segment forms", q_len))


def test_combine_long_list_at_its_bound(oracle_mod):
    """One request, 8 KV heads, 72 bins of 2 tiles: every head's segment has 9
    chunks, so the long-segment list is full ((8 + 72) / 9 = 8 records)."""
    batch = H.batch_on_gpu(dict(seqlens=[1152], num_heads=64, num_kv_heads=8, kv_dtype="bf16", seed=62))
    P = 72
    tm = H.plan(batch, P, 1)
    m = lbsa.read_task_map(tm, 1, 8, P)
    assert (m["seg_num_chunks"] == 9).all() and m["nlong"] == (8 + P) // 9 == 8
    check_full(oracle_mod, batch, H.decode(batch, tm, P), "long list at its bound")


def test_combine_row_of_hundreds_of_chunks(oracle_mod):
    """One 100000-token request over 512 bins, 8 query heads on one KV head: each
    output row merges 512 chunks, four rounds of the long form's loads."""
    batch = H.batch_on_gpu(dict(seqlens=[100000], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=63))
    P = 512
    tm = H.plan(batch, P, 1)
    m = lbsa.read_task_map(tm, 1, 1, P)
    assert int(m["seg_num_chunks"][0]) == 512 and m["nlong"] == 1
    check_full(oracle_mod, batch, H.decode(batch, tm, P), "512-chunk rows")
