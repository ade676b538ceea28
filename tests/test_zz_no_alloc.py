"""lbsa_decode_noalloc (the decode entry point with no workspace argument, its
partials in the library's static device array) against lbsa_decode on the same
inputs and task map: identical bits, on two calls in a row, the second with a
smaller batch (the array keeps the first call's partials, which the second
must not read).  Also the host-side rejection of a shape whose partials do not
fit the array."""
import ctypes

import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa

pytestmark = [pytest.mark.gpu, requires_gpu]


def _both(batch, P):
    tm = H.plan(batch, P)
    ref = H.decode(batch, tm, P).clone()
    got = lbsa.decode_noalloc(batch["q"], batch["k_cache"], batch["v_cache"], batch["page_table"], tm, P,
                              batch["softmax_scale"], q_scale=batch["q_scale"], k_scale=batch["k_scale"],
                              v_scale=batch["v_scale"])
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_matches_decode_on_two_calls(kv):
    big = H.batch_on_gpu(dict(seqlens=[5000, 64, 1, 30000, 777, 0, 4097, 12000], num_heads=64, num_kv_heads=8,
                              kv_dtype=kv, seed=111))
    small = H.batch_on_gpu(dict(seqlens=[300, 65, 2000], num_heads=64, num_kv_heads=8, kv_dtype=kv, seed=112))
    P = H.workgroups(big)
    for batch in (big, small):
        ref, got = _both(batch, P)
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_noalloc_two_token_decode_matches():
    batch = H.batch_on_gpu(dict(seqlens=[1, 2, 700, 9000, 64], num_heads=16, num_kv_heads=2, kv_dtype="bf16",
                                seed=113, q_len=2))
    ref, got = _both(batch, 50)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_noalloc_rejects_partials_beyond_the_array():
    """batch 512 x 8 KV heads with P = 4096 needs 8192 partial slots (33.8 MB at
    q_len 1): refused on the host, nothing launched."""
    need = lbsa.workspace_bytes(512, 64, 8, 4096)
    assert need > lbsa.NOALLOC_SCRATCH_BYTES
    vp = ctypes.c_void_p
    fake = vp(1 << 20)
    st = lbsa.lib().lbsa_decode_noalloc(fake, None, fake, fake, None, None, lbsa.KV_BF16, fake, 512, 1, 64, 8, 128,
                                       64, 16, 1000, 4096, 0.088, fake, 1 << 24, fake, None)
    assert st == lbsa.ERR_UNSUPPORTED
