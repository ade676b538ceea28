"""Pins of the oracle's fp64 attention, partials and merge.

Decode attention computes plain softmax attention of one query token per head
over the live KV of its request (vLLM post, "The challenge: mixed-length decode
in every batch"); split-KV chunks carry a partial output with its log-sum-exp
and a combine merges them "under the correct global softmax normalisation"
(SGLang post, "Scheduling around live KV work"; vLLM post, bullet "Compute and
combine").

Pins, independent of the oracle's code:
* torch's scaled_dot_product_attention in fp64 on K/V gathered here through the
  page table with torch indexing (library routine), GQA by repeat_interleave;
* torch.logsumexp of the gathered scores for the LSE;
* closed forms: one token gives v_0, constant V gives that constant, q = 0 gives
  the mean of V;
* merging ANY contiguous partition of a request's tiles equals the unsplit
  result (fp64, 1e-12), and the merge of the oracle's own task map equals it;
* invariance under a different physical page permutation (bit-identical).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from load_balanced_split_assign_amd import workload as wl


def gather_dense(batch, b):
    """K, V of request b as fp64 [Hkv, L, D], dequantised with torch."""
    L = int(batch["seqlens"][b])
    t = torch.arange(L)
    pages = batch["page_table"][b, t // 64].long()
    slots = t % 64
    k = batch["k_cache"][pages, slots]                   # [L, Hkv, D]
    v = batch["v_cache"][pages, slots]
    k = k.to(torch.float64)
    v = v.to(torch.float64)
    if batch["kv_dtype"] == "fp8":
        ks = batch["k_scale"][pages, :, slots].to(torch.float64)   # [L, Hkv]
        vs = batch["v_scale"][pages, :, slots].to(torch.float64)
        k = k * ks[..., None]
        v = v * vs[..., None]
    return k.permute(1, 0, 2), v.permute(1, 0, 2)


def q_dense(batch, b):
    q = batch["q"][b].to(torch.float64)                  # [Hq, D]
    if batch["kv_dtype"] == "fp8":
        q = q * batch["q_scale"][b].to(torch.float64)[:, None]
    return q


def sdpa_reference(batch):
    """Library-routine reference: (out [B,Hq,D], lse [B,Hq]) in fp64."""
    B, Hq, Hkv = batch["B"], batch["num_heads"], batch["num_kv_heads"]
    G = Hq // Hkv
    outs, lses = [], []
    for b in range(B):
        L = int(batch["seqlens"][b])
        if L == 0:
            outs.append(torch.zeros(Hq, batch["head_dim"], dtype=torch.float64))
            lses.append(torch.full((Hq,), -math.inf, dtype=torch.float64))
            continue
        k, v = gather_dense(batch, b)
        k = k.repeat_interleave(G, dim=0)                # [Hq, L, D]
        v = v.repeat_interleave(G, dim=0)
        q = q_dense(batch, b)[:, None, :]                # [Hq, 1, D]
        o = F.scaled_dot_product_attention(q, k, v, scale=batch["softmax_scale"])
        s = (q @ k.transpose(1, 2))[:, 0, :] * batch["softmax_scale"]
        outs.append(o[:, 0, :])
        lses.append(torch.logsumexp(s, dim=-1))
    return torch.stack(outs).numpy(), torch.stack(lses).numpy()


CASES = [
    ("bf16_gqa8", dict(seqlens=[37, 64, 1000, 130], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=3)),
    ("bf16_64_8", dict(seqlens=[1, 65, 300], num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=4)),
    ("fp8_gqa8", dict(seqlens=[200, 64, 129], num_heads=8, num_kv_heads=1, kv_dtype="fp8", seed=5)),
    ("fp8_2kv", dict(seqlens=[77, 500], num_heads=16, num_kv_heads=2, kv_dtype="fp8", seed=6)),
    ("with_empty", dict(seqlens=[0, 100, 0, 3], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=7)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_attention_matches_sdpa(oracle_mod, name, kw):
    batch = wl.make_batch(**kw, tail="nan")
    out, lse = oracle_mod.attention(batch)
    ref_out, ref_lse = sdpa_reference(batch)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-12)


def test_single_token_gives_v0(oracle_mod):
    batch = wl.make_batch(seqlens=[1, 1], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=11)
    out, lse = oracle_mod.attention(batch)
    for b in range(2):
        _, v = gather_dense(batch, b)
        np.testing.assert_array_equal(out[b], np.repeat(v[:, 0, :].numpy(), 8, axis=0))
        k, _ = gather_dense(batch, b)
        s = (q_dense(batch, b) @ k[0, 0]).numpy() * batch["softmax_scale"]
        np.testing.assert_allclose(lse[b], s, atol=1e-12)     # ln(exp(s)) = s


def test_constant_v_gives_constant(oracle_mod):
    batch = wl.make_batch(seqlens=[333, 64], num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=12,
                          tail="normal")
    batch["v_cache"][:] = 0.375
    out, _ = oracle_mod.attention(batch)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-15)


def test_zero_query_gives_mean_of_v(oracle_mod):
    batch = wl.make_batch(seqlens=[90, 257], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=13)
    batch["q"][:] = 0
    out, lse = oracle_mod.attention(batch)
    for b in range(2):
        _, v = gather_dense(batch, b)
        np.testing.assert_allclose(out[b], np.repeat(v.mean(dim=1).numpy(), 8, axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[b], math.log(int(batch["seqlens"][b])), atol=1e-13)


def test_empty_request_gives_zero(oracle_mod):
    batch = wl.make_batch(seqlens=[0, 5], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=14)
    out, lse = oracle_mod.attention(batch)
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()


def test_any_contiguous_partition_merges_to_unsplit(oracle_mod):
    rng = np.random.default_rng(7)
    for kv_dtype in ("bf16", "fp8"):
        batch = wl.make_batch(seqlens=[700, 64, 1], num_heads=16, num_kv_heads=2, kv_dtype=kv_dtype, seed=15)
        out, lse = oracle_mod.attention(batch)
        G = 8
        for b, L in enumerate([700, 64, 1]):
            n = (L + 63) // 64
            for _ in range(6):
                cuts = sorted(set(rng.integers(1, n, size=rng.integers(0, n)).tolist())) if n > 1 else []
                bounds = [0] + cuts + [n]
                for h in range(2):
                    desc = [[h, b, t0, t1] for t0, t1 in zip(bounds[:-1], bounds[1:])]
                    po, pl = oracle_mod.partials(batch, desc)
                    for g in range(G):
                        m, ml = oracle_mod.merge(po[:, g, :], pl[:, g])
                        np.testing.assert_allclose(m, out[b, h * G + g], rtol=0, atol=1e-12)
                        assert abs(ml - lse[b, h * G + g]) < 1e-12


def test_single_tile_descriptor_equals_unsplit(oracle_mod):
    batch = wl.make_batch(seqlens=[50, 64], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=16)
    out, lse = oracle_mod.attention(batch)
    po, pl = oracle_mod.partials(batch, [[0, 0, 0, 1], [0, 1, 0, 1]])
    np.testing.assert_array_equal(po, out)
    np.testing.assert_array_equal(pl, lse)


def test_merge_of_task_map_equals_unsplit(oracle_mod):
    for name in ("tiny",):
        batch = wl.make_batch(name)
        m = oracle_mod.assign(batch["seqlens"], batch["num_heads"], batch["num_kv_heads"],
                              batch["num_workgroups"], 2, batch["max_pages"])
        out, lse = oracle_mod.attention(batch)
        po, pl = oracle_mod.partials(batch, m["desc"])
        G = batch["num_heads"] // batch["num_kv_heads"]
        for s in range(batch["num_kv_heads"] * batch["B"]):
            h, b = divmod(s, batch["B"])
            d0, n = int(m["seg_first_desc"][s]), int(m["seg_num_chunks"][s])
            for g in range(G):
                o, l = oracle_mod.merge(po[d0:d0 + n, g], pl[d0:d0 + n, g])
                np.testing.assert_allclose(o, out[b, h * G + g], rtol=0, atol=1e-12)
                assert abs(l - lse[b, h * G + g]) < 1e-12


def test_merge_closed_forms(oracle_mod):
    o = np.array([[1.0, 2.0], [3.0, 5.0]])
    m, l = oracle_mod.merge(o, np.array([0.0, 0.0]))             # equal weights
    np.testing.assert_allclose(m, [2.0, 3.5], atol=1e-15)
    assert abs(l - math.log(2.0)) < 1e-15
    m, l = oracle_mod.merge(o, np.array([0.0, -math.inf]))       # an empty chunk
    np.testing.assert_array_equal(m, [1.0, 2.0])
    m, l = oracle_mod.merge(o, np.array([math.log(3.0), 0.0]))   # weights 3 : 1
    np.testing.assert_allclose(m, [1.5, 2.75], atol=1e-15)
    m, l = oracle_mod.merge(np.zeros((0, 2)), np.zeros(0))
    assert (m == 0).all() and l == -math.inf


def test_page_permutation_invariance(oracle_mod):
    batch = wl.make_batch(seqlens=[300, 129, 64], num_heads=16, num_kv_heads=2, kv_dtype="fp8", seed=17)
    out, lse = oracle_mod.attention(batch)
    # move every physical page to a new slot and rewrite the page table
    perm = torch.randperm(batch["num_pages"], generator=torch.Generator().manual_seed(99))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    b2 = dict(batch)
    b2["k_cache"] = batch["k_cache"][perm].contiguous()
    b2["v_cache"] = batch["v_cache"][perm].contiguous()
    b2["k_scale"] = batch["k_scale"][perm].contiguous()
    b2["v_scale"] = batch["v_scale"][perm].contiguous()
    pt = batch["page_table"].clone()
    pt[pt >= 0] = inv[pt[pt >= 0].long()].to(torch.int32)
    b2["page_table"] = pt
    out2, lse2 = oracle_mod.attention(b2)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_nan_tail_never_leaks(oracle_mod):
    batch = wl.make_batch(seqlens=[1, 63, 65], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=18,
                          tail="nan")
    out, lse = oracle_mod.attention(batch)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_bad_page_is_reported(oracle_mod):
    batch = wl.make_batch(seqlens=[70], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=19)
    batch["page_table"][0, 1] = batch["num_pages"]
    with pytest.raises(ValueError):
        oracle_mod.attention(batch)
