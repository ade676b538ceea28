"""Pins of the oracle's multi-token decode (q_len query tokens per request).

Hy3 serves with a multi-token-prediction layer for speculative decoding (vLLM
post, the model paragraph "A Quick Word on Hy3-series models"); verifying its
draft tokens is a decode step with q_len > 1 new tokens per request.  Reading
M1: the q_len new tokens are the last q_len of the request's L cached tokens,
and query i (position L - q_len + i) sees tokens [0, L - q_len + i] -- causal
among the new tokens.  A query that sees no token gives 0 (LSE -inf).

Pins, independent of the oracle's code:
* torch's scaled_dot_product_attention in fp64 with an explicit boolean mask
  built here from M1, on K/V gathered with torch indexing, and torch.logsumexp
  of the masked scores;
* the last query sees the whole request: it equals one-token decode of the same
  query; query 0 of q_len = 2 equals one-token decode over L - 1 tokens;
* the partials of a task map (any split of the tiles, including chunks a query
  does not reach) merge back to the unsplit result.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from load_balanced_split_assign_amd import workload as wl
from test_oracle_attention import gather_dense


def q_dense_multi(batch, b):
    q = batch["q"][b].to(torch.float64)                              # [q_len, Hq, D]
    if batch["kv_dtype"] == "fp8":
        q = q * batch["q_scale"][b].to(torch.float64)[..., None]
    return q


def masked_sdpa_reference(batch):
    """(out [B, q_len, Hq, D], lse [B, q_len, Hq]) in fp64 from SDPA with the M1 mask."""
    B, Hq, Hkv, QL, D = batch["B"], batch["num_heads"], batch["num_kv_heads"], batch["q_len"], batch["head_dim"]
    G = Hq // Hkv
    out = torch.zeros((B, QL, Hq, D), dtype=torch.float64)
    lse = torch.full((B, QL, Hq), -math.inf, dtype=torch.float64)
    for b in range(B):
        L = int(batch["seqlens"][b])
        if L == 0:
            continue
        k, v = gather_dense(batch, b)
        k = k.repeat_interleave(G, dim=0)                            # [Hq, L, D]
        v = v.repeat_interleave(G, dim=0)
        q = q_dense_multi(batch, b).permute(1, 0, 2)                 # [Hq, q_len, D]
        pos = torch.arange(L)
        last = L - QL + torch.arange(QL)                             # last visible token of query i
        mask = pos[None, :] <= last[:, None]                         # [q_len, L]
        live = mask.any(dim=1)                                       # queries that see something
        if not live.any():
            continue
        o = F.scaled_dot_product_attention(q[:, live], k, v, attn_mask=mask[live], scale=batch["softmax_scale"])
        s = (q @ k.transpose(1, 2)) * batch["softmax_scale"]         # [Hq, q_len, L]
        s = s.masked_fill(~mask[None], -math.inf)
        out[b, live] = o.permute(1, 0, 2)
        lse[b, live] = torch.logsumexp(s[:, live], dim=-1).permute(1, 0)
    return out.numpy(), lse.numpy()


CASES = [
    ("bf16_q2", dict(seqlens=[2, 63, 64, 65, 200], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=40, q_len=2)),
    ("fp8_q2", dict(seqlens=[129, 64, 3], num_heads=16, num_kv_heads=2, kv_dtype="fp8", seed=41, q_len=2)),
    ("bf16_q3_short", dict(seqlens=[1, 2, 3, 70], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=42, q_len=3)),
    ("bf16_q4_empty", dict(seqlens=[0, 500], num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=43, q_len=4)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_multitoken_matches_masked_sdpa(oracle_mod, name, kw):
    batch = wl.make_batch(**kw, tail="nan")
    assert batch["q"].shape[1] == kw["q_len"]
    out, lse = oracle_mod.attention(batch)
    ref_out, ref_lse = masked_sdpa_reference(batch)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-13, atol=1e-12)


def test_queries_that_see_nothing_give_zero(oracle_mod):
    # L = 1 with q_len = 3: queries 0 and 1 see no token, query 2 sees token 0
    batch = wl.make_batch(seqlens=[1], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=44, q_len=3)
    out, lse = oracle_mod.attention(batch)
    assert (out[0, :2] == 0).all() and np.isneginf(lse[0, :2]).all()
    _, v = gather_dense(batch, 0)
    np.testing.assert_array_equal(out[0, 2], np.repeat(v[:, 0, :].numpy(), 8, axis=0))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_last_query_is_one_token_decode_and_first_is_shorter(oracle_mod, kv_dtype):
    sl = [1, 64, 65, 130, 999]
    multi = wl.make_batch(seqlens=sl, num_heads=16, num_kv_heads=2, kv_dtype=kv_dtype, seed=45, q_len=2,
                          tail="normal")
    out, lse = oracle_mod.attention(multi)
    for i, lengths in ((1, sl), (0, [max(0, x - 1) for x in sl])):
        single = dict(multi)
        single["q"] = multi["q"][:, i].contiguous()
        single["q_scale"] = None if multi["q_scale"] is None else multi["q_scale"][:, i].contiguous()
        single["seqlens"] = torch.tensor(lengths, dtype=torch.int32)
        o1, l1 = oracle_mod.attention(single)
        np.testing.assert_allclose(out[:, i], o1, rtol=0, atol=1e-13)
        np.testing.assert_array_equal(lse[:, i], l1)


def test_partials_of_a_task_map_merge_to_unsplit(oracle_mod):
    sl = [65, 64, 700, 2]
    batch = wl.make_batch(seqlens=sl, num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=46, q_len=2)
    out, lse = oracle_mod.attention(batch)
    m = oracle_mod.assign(sl, 16, 2, P=30, F=1, max_pages=batch["max_pages"])   # one tile per bin
    po, pl = oracle_mod.partials(batch, m["desc"])                       # [n, 2*8, D]
    assert po.shape[1] == 16
    # request 0 (L = 65) has a one-token last tile that its query 0 does not reach
    assert np.isneginf(pl).any()
    for b in range(len(sl)):
        for h in range(2):
            s = h * len(sl) + b
            d0, n = m["seg_first_desc"][s], m["seg_num_chunks"][s]
            for qi in range(2):
                for g in range(8):
                    row = qi * 8 + g
                    o, l = oracle_mod.merge(po[d0:d0 + n, row], pl[d0:d0 + n, row])
                    np.testing.assert_allclose(o, out[b, qi, h * 8 + g], rtol=0, atol=1e-12)
                    if np.isfinite(lse[b, qi, h * 8 + g]):
                        assert abs(l - lse[b, qi, h * 8 + g]) < 1e-12
                    else:
                        assert np.isneginf(l)


def test_rows_sample_matches_full(oracle_mod):
    batch = wl.make_batch(seqlens=[90, 3, 257], num_heads=16, num_kv_heads=2, kv_dtype="fp8", seed=47, q_len=2)
    out, lse = oracle_mod.attention(batch)
    rows = [(0, 0), (0, 17), (1, 31), (2, 16), (2, 5)]                   # j = query * Hq + head
    o, l = oracle_mod.attention_rows(batch, rows)
    for k, (b, j) in enumerate(rows):
        np.testing.assert_array_equal(o[k], out[b, j // 16, j % 16])
        assert l[k] == lse[b, j // 16, j % 16]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prefill_and_extend_match_masked_sdpa(oracle_mod, kv_dtype):
    """Prefill (q_len = L: plain causal attention) and extend (q_len < L) are
    the same rule at larger q_len."""
    for seed, sl, ql in ((48, [130, 130], 130), (49, [300, 77], 77), (50, [64, 200], 64)):
        batch = wl.make_batch(seqlens=sl, num_heads=16, num_kv_heads=2, kv_dtype=kv_dtype, seed=seed, q_len=ql,
                              tail="nan")
        out, lse = oracle_mod.attention(batch)
        ref_out, ref_lse = masked_sdpa_reference(batch)
        np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
        fin = np.isfinite(ref_lse)
        np.testing.assert_array_equal(np.isfinite(lse), fin)
        np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-13, atol=1e-12)


def test_prefill_is_torch_causal_attention(oracle_mod):
    """q_len = L: the first query sees only token 0, the mask is torch's own
    is_causal (top-left aligned, which coincides with M1 when q_len = L)."""
    batch = wl.make_batch(seqlens=[96], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=51, q_len=96)
    out, _ = oracle_mod.attention(batch)
    k, v = gather_dense(batch, 0)
    q = q_dense_multi(batch, 0).permute(1, 0, 2)                        # [Hq, 96, D]
    ref = F.scaled_dot_product_attention(q, k.repeat_interleave(8, 0), v.repeat_interleave(8, 0), is_causal=True,
                                         scale=batch["softmax_scale"])
    np.testing.assert_allclose(out[0], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(out[0, 0], np.repeat(v[:, 0, :].numpy(), 8, axis=0))
