"""Static split-KV baseline kernel vs the fp64 oracle (the bar of tests/parity.py)."""
import numpy as np
import pytest

import _gpu_helpers as H
from _gpu_helpers import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("S", [1, 2, 3, 16, 64])
def test_static_matches_oracle(oracle_mod, S):
    batch = H.batch_on_gpu(dict(seqlens=[1, 63, 64, 65, 2047, 5000, 0, 17], num_heads=16, num_kv_heads=2,
                                kv_dtype="bf16", seed=31))
    out = H.out_np(H.decode_static(batch, S))
    ref, _ = oracle_mod.attention(batch)
    H.check(batch, out, ref, f"static S={S}")
    assert (out[6] == 0).all()


@pytest.mark.parametrize("S", [1, 4])
def test_static_fp8(oracle_mod, S):
    batch = H.batch_on_gpu(dict(seqlens=[100, 3000, 64, 9], num_heads=64, num_kv_heads=8, kv_dtype="fp8",
                                seed=32))
    out = H.out_np(H.decode_static(batch, S))
    ref, _ = oracle_mod.attention(batch)
    H.check(batch, out, ref, f"static fp8 S={S}")


def test_static_skewed_full_parity(oracle_mod):
    batch = H.batch_on_gpu("skewed", gen_device="cuda:0")
    out = H.decode_static(batch, 8)
    ref, _ = oracle_mod.attention(batch)
    H.check(batch, H.out_np(out), ref, "static skewed S=8")


def test_static_and_dynamic_agree_bitwise_when_unsplit():
    """With one split per request and one chunk per segment both paths run the
    same tile sequence per request, so their outputs are identical."""
    batch = H.batch_on_gpu(dict(seqlens=[640, 64, 128], num_heads=8, num_kv_heads=1, kv_dtype="bf16",
                                seed=33))
    P = 1
    a = H.out_np(H.decode(batch, H.plan(batch, P, 1000), P))
    b = H.out_np(H.decode_static(batch, 1))
    np.testing.assert_array_equal(a, b)
