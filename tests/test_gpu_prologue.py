"""GPU fused prologue (QK-Norm -> RoPE -> Q out, K/V into the paged cache) vs
the fp64 prologue oracle.

Tolerances, derived from the output formats:
* bf16 outputs: |gpu - ref| <= 2^-7 |ref| (one bf16 step, which allows for a
  rounding decision that flips between fp32 and fp64) + 1e-5 of the head's
  largest magnitude (fp32 arithmetic);
* fp8 outputs: scales within 1e-5 relative; dequantised values within one e4m3
  step, 2^-3 |ref| + scale * 2^-8;
* V is a copy: bit-exact in bf16; in fp8 its codes dequantise within the
  same bound as Q and K;
* cache rows that no token maps to are untouched, bit for bit.
"""
import numpy as np
import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa
from load_balanced_split_assign_amd import workload as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def run_gpu(inp):
    g = {k: (v.to("cuda:0").clone() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    q, qs = lbsa.prologue(g["qkv"], g["positions"], g["slot_mapping"], g["q_weight"], g["k_weight"],
                          g["num_heads"], g["num_kv_heads"], g["k_cache"], g["v_cache"], rope_theta=g["theta"],
                          eps=g["eps"], k_scale=g["k_scale"], v_scale=g["v_scale"])
    torch.cuda.synchronize()
    return q.cpu(), (None if qs is None else qs.cpu()), g


def values(t):
    if t.dtype == torch.bfloat16:
        return t.float().double().numpy()
    return t.view(torch.uint8).numpy()


def check_bf16(got, ref, what):
    tol = np.abs(ref) * 2.0 ** -7 + 1e-5 * np.abs(ref).max(axis=-1, keepdims=True) + 1e-30
    err = np.abs(got - ref)
    assert (err <= tol).all(), (what, float((err - tol).max()))


def check_fp8(oracle_mod, codes, scale, ref, what):
    amax = np.abs(ref).max(axis=-1)
    ref_scale = np.where(amax > 0, amax / 448.0, 1.0)
    np.testing.assert_allclose(scale, ref_scale, rtol=1e-5, err_msg=what)
    deq = oracle_mod.e4m3_values(codes) * scale[..., None]
    bound = np.abs(ref) * 2.0 ** -3 + scale[..., None] * 2.0 ** -8
    assert (np.abs(deq - ref) <= bound).all(), what
    live = amax > 0      # the largest magnitude of each head lands on +-448
    am = np.abs(ref).argmax(axis=-1)
    top = np.take_along_axis(codes, am[..., None], axis=-1)[..., 0]
    assert ((top[live] & 0x7F) == 0x7E).all(), what
    assert ((codes[~live] & 0x7F) == 0).all(), what    # +0 or -0


def check(oracle_mod, inp):
    T, Hq, Hkv = inp["tokens"], inp["num_heads"], inp["num_kv_heads"]
    q_ref, k_ref, v_ref = oracle_mod.prologue(inp["qkv"], inp["positions"], inp["q_weight"].double().numpy(),
                                              inp["k_weight"].double().numpy(), Hq, Hkv, inp["theta"], inp["eps"])
    q, qs, g = run_gpu(inp)
    slots = inp["slot_mapping"].numpy()
    live = (slots >= 0) & (slots < inp["num_pages"] * 64)
    page, row = slots // 64, slots % 64
    fp8 = inp["kv_dtype"] == "fp8"
    if fp8:
        check_fp8(oracle_mod, values(q), qs.double().numpy(), q_ref, "q")
    else:
        check_bf16(values(q), q_ref, "q")
    for name, ref, sc in (("k", k_ref, "k_scale"), ("v", v_ref, "v_scale")):
        before = inp[name + "_cache"]
        after = g[name + "_cache"].cpu()
        # rows no token maps to are untouched
        mask = torch.ones(before.shape[:2], dtype=torch.bool)
        mask[page[live], row[live]] = False
        assert torch.equal(before.view(torch.uint8 if fp8 else torch.int16)[mask],
                           after.view(torch.uint8 if fp8 else torch.int16)[mask]), name
        got = after[page[live], row[live]]                              # [n, Hkv, 128]
        if fp8:
            sc_got = g[sc].cpu()[page[live], :, row[live]].double().numpy()   # [n, Hkv]
            check_fp8(oracle_mod, values(got), sc_got, ref[live], name)
            sc_mask = mask.unsqueeze(1).expand(-1, Hkv, -1)
            assert torch.equal(inp[sc][sc_mask], g[sc].cpu()[sc_mask]), name + " scales"
        elif name == "v":
            np.testing.assert_array_equal(values(got), ref[live])        # a copy
        else:
            check_bf16(values(got), ref[live], name)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("T,Hq,Hkv", [(1, 8, 1), (37, 8, 1), (100, 64, 8), (513, 16, 2)])
def test_prologue_matches_oracle(oracle_mod, kv_dtype, T, Hq, Hkv):
    inp = wl.make_prologue_inputs(T, Hq, Hkv, kv_dtype, seed=T + Hq, padding=min(3, T // 10),
                                  zero_heads=min(4, T))
    check(oracle_mod, inp)


@pytest.mark.parametrize("name", list(wl.PROLOGUE_WORKLOADS))
def test_prologue_workloads(oracle_mod, name):
    inp = wl.make_prologue_inputs(**wl.PROLOGUE_WORKLOADS[name])
    if inp["tokens"] > 1024:     # full-size prefill: the oracle checks a sample of tokens
        keep = torch.randperm(inp["tokens"], generator=torch.Generator().manual_seed(0))[:384]
        sub = dict(inp)
        for k in ("qkv", "positions", "slot_mapping"):
            sub[k] = inp[k][keep]
        sub["tokens"] = len(keep)
        check(oracle_mod, sub)
    else:
        check(oracle_mod, inp)


def test_prologue_zero_tokens_is_a_no_op():
    inp = wl.make_prologue_inputs(4, 8, 1, "bf16", seed=3)
    g = {k: (v.to("cuda:0").clone() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    empty = g["qkv"][:0]
    q, _ = lbsa.prologue(empty, g["positions"][:0], g["slot_mapping"][:0], g["q_weight"], g["k_weight"], 8, 1,
                         g["k_cache"], g["v_cache"])
    torch.cuda.synchronize()
    assert q.shape[0] == 0 and torch.equal(g["k_cache"].cpu().view(torch.int16), inp["k_cache"].view(torch.int16))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prologue_feeds_decode(oracle_mod, kv_dtype):
    """Decode step end to end: the prologue writes each request's newest token
    (position L_b - 1) into the paged cache and emits Q; decode then reads
    them.  The oracle attends over the caches and Q the GPU produced."""
    batch = H.batch_on_gpu(dict(seqlens=[1, 63, 64, 65, 700, 3000], num_heads=64, num_kv_heads=8,
                                kv_dtype=kv_dtype, seed=51))
    B, Hq, Hkv = batch["B"], batch["num_heads"], batch["num_kv_heads"]
    # unit magnitudes: V of the new token is N(0, 1) like the rest of the cache, so
    # the decode tolerances (absolute, for O(1) outputs) apply
    inp = wl.make_prologue_inputs(B, Hq, Hkv, kv_dtype, seed=52, magnitude=1.0)
    sl = batch["seqlens"].cpu().long()
    pt = batch["page_table"].cpu().long()
    pos = sl - 1
    slots = pt[torch.arange(B), pos // 64] * 64 + pos % 64
    dev = lambda x: x.to("cuda:0")  # noqa: E731
    q, qs = lbsa.prologue(dev(inp["qkv"]), dev(pos.to(torch.int32)), dev(slots), dev(inp["q_weight"]),
                          dev(inp["k_weight"]), Hq, Hkv, batch["k_cache"], batch["v_cache"],
                          k_scale=batch["k_scale"], v_scale=batch["v_scale"])
    batch["q"], batch["q_scale"] = q, qs
    P = H.workgroups(batch)
    out = H.decode(batch, H.plan(batch, P), P)
    torch.cuda.synchronize()
    ref, _ = oracle_mod.attention(batch)
    H.check(batch, H.out_np(out), ref, f"prologue -> decode {kv_dtype}")
    # the written K row of each request is the rotated, normalised key
    _, k_ref, _ = oracle_mod.prologue(inp["qkv"], pos.to(torch.int32), inp["q_weight"].double().numpy(),
                                      inp["k_weight"].double().numpy(), Hq, Hkv, inp["theta"], inp["eps"])
    krow = batch["k_cache"].cpu()[pt[torch.arange(B), pos // 64], pos % 64]
    if kv_dtype == "bf16":
        check_bf16(values(krow), k_ref, "k")
    else:
        ks = batch["k_scale"].cpu()[pt[torch.arange(B), pos // 64], :, pos % 64].double().numpy()
        check_fp8(oracle_mod, values(krow), ks, k_ref, "k")
