"""GPU multi-token decode (2 query tokens per request, causal among them) vs
the fp64 oracle.

The two new tokens of a request are its last two cached tokens; query 0 sees
tokens [0, L - 2], query 1 sees [0, L - 1] (reading M1, Hy3's MTP speculative
layer in the vLLM post's model paragraph).  Tolerances are the decode path's:
max |out - oracle| <= 2e-2 (bf16 KV), 6e-2 (fp8 KV); partial LSE within 1e-3.
Inputs carry NaN in every tail slot past L, so a token leaking past a query's
limit into a real row would show.
"""
import numpy as np
import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa

pytestmark = [pytest.mark.gpu, requires_gpu]

EDGE = [1, 2, 17, 63, 64, 65, 66, 81, 128, 129, 1000, 4097]   # 17, 81: a wave whose only live token is the last


def check_full(oracle_mod, batch, out, what):
    ref, _ = oracle_mod.attention(batch)
    got = H.out_np(out)
    assert got.shape == ref.shape, what
    return H.check(batch, got, ref, what)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("heads", [(8, 1), (64, 8)])
@pytest.mark.parametrize("P,F", [(None, 0), (7, 1), (300, 1)])
def test_two_token_decode_matches_oracle(oracle_mod, kv_dtype, heads, P, F):
    batch = H.batch_on_gpu(dict(seqlens=EDGE, num_heads=heads[0], num_kv_heads=heads[1], kv_dtype=kv_dtype,
                                seed=60 + heads[1], q_len=2))
    P = H.workgroups(batch, P)
    out = H.decode(batch, H.plan(batch, P, F), P)
    assert tuple(out.shape) == (len(EDGE), 2, heads[0], 128)
    check_full(oracle_mod, batch, out, (kv_dtype, heads, P))
    # L = 1: query 0 sees no token, its row is zero
    assert (out[0, 0] == 0).all()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_two_token_partials_match_oracle(oracle_mod, kv_dtype):
    """One-tile bins: the last tile of L = 65 holds only the token query 0 does
    not see, so that partial row is empty (O = 0, LSE = -inf), not NaN."""
    sl = [65, 64, 700, 2, 130]
    batch = H.batch_on_gpu(dict(seqlens=sl, num_heads=16, num_kv_heads=2, kv_dtype=kv_dtype, seed=66, q_len=2))
    P = 64
    tm = H.plan(batch, P, F=1)
    ws = H.decode_split(batch, tm, P)
    m = lbsa.read_task_map(tm, batch["B"], 2, P)
    po, pl = lbsa.read_partials(ws, batch["B"], 16, 2, P, m["Ndesc"], q_len=2)
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in batch.items()}
    ro, rl = oracle_mod.partials(cpu, m["desc"])
    empty = np.isneginf(rl)
    assert empty.any()
    np.testing.assert_array_equal(np.isneginf(pl), empty)
    assert (po[empty] == 0).all()
    H.check(batch, po[~empty], ro[~empty], f"two-token partials {kv_dtype}")
    assert np.abs(pl[~empty] - rl[~empty]).max() <= H.LSE_TOL


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S", [1, 3, 8])
def test_two_token_static_matches_oracle(oracle_mod, kv_dtype, S):
    batch = H.batch_on_gpu(dict(seqlens=EDGE, num_heads=16, num_kv_heads=2, kv_dtype=kv_dtype, seed=67,
                                q_len=2))
    out = H.decode_static(batch, S)
    check_full(oracle_mod, batch, out, (kv_dtype, S))


def test_two_token_tp8_share_full_parity(oracle_mod):
    batch = H.batch_on_gpu("tp8_share")
    batch = H.batch_on_gpu(dict(seqlens=batch["seqlens"].cpu().tolist(), num_heads=8, num_kv_heads=1,
                                kv_dtype="bf16", seed=68, q_len=2))
    P = H.workgroups(batch)
    out = H.decode(batch, H.plan(batch, P), P)
    check_full(oracle_mod, batch, out, "tp8_share q_len 2")


def test_two_token_fp8_workload_full_parity(oracle_mod):
    """The fp8 workload's lengths at q_len 2: all 8192 rows against the oracle."""
    b1 = H.batch_on_gpu("fp8", gen_device="cuda:0")
    sl = b1["seqlens"].cpu().tolist()
    del b1
    batch = H.batch_on_gpu(dict(seqlens=sl, num_heads=64, num_kv_heads=8, kv_dtype="fp8", seed=69, q_len=2),
                           gen_device="cuda:0")
    P = H.workgroups(batch)
    out = H.decode(batch, H.plan(batch, P), P)
    check_full(oracle_mod, batch, out, "fp8 workload q_len 2")


def test_empty_request_and_q_len_one_agree(oracle_mod):
    """An empty request gives zero rows for both queries; the second query of a
    two-token decode equals one-token decode of that query over the same cache."""
    sl = [0, 77, 3000, 64]
    batch = H.batch_on_gpu(dict(seqlens=sl, num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=70, q_len=2))
    P = H.workgroups(batch)
    tm = H.plan(batch, P)
    out = H.out_np(H.decode(batch, tm, P))
    assert (out[0] == 0).all()
    one = dict(batch)
    one["q"] = batch["q"][:, 1].contiguous()
    out1 = H.out_np(H.decode(one, tm, P))
    assert np.abs(out[:, 1] - out1).max() <= 1e-2
