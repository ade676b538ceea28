"""GPU prefill / extend attention vs the fp64 oracle.

Prefill and extend are causal attention of each request's q_len new tokens
(the last q_len of its L cached tokens) over the paged cache; the vLLM post's
Table 4 measures the backend on such shapes.  Tolerance: max |out - oracle|
<= 2e-2 (bf16 KV, bf16 output), as for decode.  Inputs carry NaN in every
tail slot past L of each last page, so a leak past a request's length shows.
The query-block width CB (1, 2 or 3 MFMA column blocks per wave, 8, 16 or 24
query positions per workgroup) is chosen on the host from the grid size; the
shapes below reach all three, the widest with a ragged last block.
"""
import numpy as np
import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa
from load_balanced_split_assign_amd import workload as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def run(batch):
    out = lbsa.prefill(batch["q"], batch["k_cache"], batch["v_cache"], batch["page_table"], batch["seqlens"],
                       batch["softmax_scale"])
    return H.out_np(out)


def cb_of(B, Hkv, QL):
    """The host's choice of column blocks per wave (mirrors the launch rule)."""
    if B * Hkv * -(-QL // 24) >= 1024:
        return 3
    return 2 if B * Hkv * -(-QL // 16) >= 512 else 1


CASES = [
    # (seqlens, q_len, Hq, Hkv): prefill (L = q_len), extend (L > q_len), short and ragged
    ([1], 1, 8, 1),
    ([5, 64, 65], 5, 8, 1),
    ([130, 130], 130, 16, 2),
    ([700, 300, 64], 64, 16, 2),
    ([2048], 1000, 64, 8),
    ([77, 200, 513, 1024], 77, 64, 8),
]


@pytest.mark.parametrize("sl,ql,Hq,Hkv", CASES)
def test_prefill_matches_oracle(oracle_mod, sl, ql, Hq, Hkv):
    batch = H.batch_on_gpu(dict(seqlens=sl, num_heads=Hq, num_kv_heads=Hkv, kv_dtype="bf16", seed=90 + ql,
                                q_len=ql))
    got = run(batch)
    ref, _ = oracle_mod.attention(batch)
    assert got.shape == ref.shape
    H.check(batch, got, ref, ("prefill", ql, Hq, Hkv))


@pytest.mark.parametrize("B,Hkv,QL,expect_cb", [(4, 8, 770, 3), (2, 8, 770, 2), (4, 8, 256, 2), (8, 8, 100, 1), (2, 2, 96, 1)])
def test_prefill_each_block_width(oracle_mod, B, Hkv, QL, expect_cb):
    assert cb_of(B, Hkv, QL) == expect_cb
    sl = [QL + 37 * i for i in range(B)]                      # extend with different prefixes
    batch = H.batch_on_gpu(dict(seqlens=sl, num_heads=8 * Hkv, num_kv_heads=Hkv, kv_dtype="bf16", seed=95,
                                q_len=QL), gen_device="cuda:0")
    got = run(batch)
    ref, _ = oracle_mod.attention(batch)
    H.check(batch, got, ref, ("prefill block width", B, Hkv, QL))


def test_queries_that_see_nothing_and_empty_requests(oracle_mod):
    # L < q_len: the first q_len - L queries see no token (zero rows); L = 0: all zero
    batch = H.batch_on_gpu(dict(seqlens=[3, 0, 40], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=97,
                                q_len=8))
    got = run(batch)
    ref, _ = oracle_mod.attention(batch)
    assert (got[0, :5] == 0).all() and (got[1] == 0).all()
    H.check(batch, got, ref, "prefill empty queries")


def test_one_token_prefill_equals_decode(oracle_mod):
    """q_len = 1 prefill is decode: it agrees with the split + combine path."""
    batch = H.batch_on_gpu(dict(seqlens=[1, 100, 4097, 64], num_heads=64, num_kv_heads=8, kv_dtype="bf16",
                                seed=98, q_len=1))
    P = H.workgroups(batch)
    dec = H.out_np(H.decode(batch, H.plan(batch, P), P))
    pre = lbsa.prefill(batch["q"].unsqueeze(1).contiguous(), batch["k_cache"], batch["v_cache"],
                       batch["page_table"], batch["seqlens"], batch["softmax_scale"])
    assert np.abs(H.out_np(pre)[:, 0] - dec).max() <= 1e-2


@pytest.mark.parametrize("name", [n for n, v in wl.TABLE4.items() if v[0] != "decode"])
def test_table4_shapes_sampled(oracle_mod, name):
    batch = wl.make_table4_batch(name, tail="nan", device="cuda:0")
    got = run(batch)
    assert np.isfinite(got).all()
    B, QL, Hq = batch["B"], batch["q_len"], batch["num_heads"]
    rng = np.random.default_rng(7)
    # first, last and random queries, heads across group boundaries
    qs = sorted({0, QL - 1, *rng.integers(0, QL, 4).tolist()})
    rows = np.array([(b, qi * Hq + hq) for b in range(B) for qi in qs for hq in range(Hq)], np.int32)
    ref, _ = oracle_mod.attention_rows(batch, rows)
    sub = got.reshape(B, QL * Hq, 128)[rows[:, 0], rows[:, 1]]
    H.check(batch, sub, ref, ("table4", name))


def test_bad_page_poisons_the_queries_that_read_it():
    """Request 1's second page id is out of range: its queries 64.. (which see
    that page) come out NaN; nothing is read out of bounds, request 0 and the
    queries that never reach the page are untouched."""
    batch = H.batch_on_gpu(dict(seqlens=[100, 100], num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=99,
                                q_len=100))
    batch["page_table"][1, 1] = 10 ** 6
    got = run(batch)
    assert np.isfinite(got[0]).all() and np.isfinite(got[1, :64]).all()
    assert np.isnan(got[1, 64:]).all()
