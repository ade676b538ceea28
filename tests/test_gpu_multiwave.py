"""Task maps with more bins than the device holds workgroups at once (P a
multiple of compute units x occupancy): the split grid then runs in several
waves of workgroups.  Checked against the fp64 oracle (the bar of
tests/parity.py) and for run-to-run bit equality, and the map's reserved
header word stays zero.
"""
import numpy as np
import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa

pytestmark = [pytest.mark.gpu, requires_gpu]

HDR_RESERVED = (15,)


def resident(batch):
    return lbsa.default_workgroups(0, batch["kv_dtype"], batch.get("q_len", 1))


def reserved_words(tm):
    h = tm[:64].cpu().numpy().view(np.int32)
    return tuple(int(h[i]) for i in HDR_RESERVED)


def check(oracle_mod, batch, out, what=""):
    ref, _ = oracle_mod.attention(batch)
    return H.check(batch, H.out_np(out), ref, what)


@pytest.mark.parametrize("mult", [2, 3, 4])
def test_multiwave_matches_oracle_and_repeats(oracle_mod, mult):
    batch = H.batch_on_gpu(dict(seqlens=[3000, 64, 1, 9000, 700, 0, 129, 40000, 2222, 513],
                                num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=41))
    P = mult * resident(batch)
    tm = H.plan(batch, P)
    assert reserved_words(tm) == (0,)
    outs = []
    for _ in range(3):
        outs.append(H.decode(batch, tm, P).clone())
        torch.cuda.synchronize()
        assert reserved_words(tm) == (0,)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    check(oracle_mod, batch, outs[0], f"multiwave x{mult}")


def test_multiwave_fp8(oracle_mod):
    batch = H.batch_on_gpu(dict(seqlens=[5000, 17, 64, 20000, 333, 4096], num_heads=8, num_kv_heads=1,
                                kv_dtype="fp8", seed=42))
    P = 4 * resident(batch)
    tm = H.plan(batch, P)
    out = H.decode(batch, tm, P)
    torch.cuda.synchronize()
    assert reserved_words(tm) == (0,)
    check(oracle_mod, batch, out, "multiwave fp8")


@pytest.mark.parametrize("name", ["tp8_share", "skewed"])
def test_multiwave_full_size(oracle_mod, name):
    batch = H.batch_on_gpu(name)
    G = resident(batch)
    ref, _ = oracle_mod.attention(batch)
    for P in (2 * G, 4 * G):
        tm = H.plan(batch, P)
        out = H.decode(batch, tm, P)
        torch.cuda.synchronize()
        assert reserved_words(tm) == (0,), (name, P)
        H.check(batch, H.out_np(out), ref, (name, P))


def test_multiwave_partials_repeat_bitwise():
    """The same map decoded twice gives bit-identical partials, and every
    descriptor slot is written (the workspace starts as NaN bytes)."""
    batch = H.batch_on_gpu(dict(seqlens=[7000, 100, 2500, 64, 12000], num_heads=8, num_kv_heads=1,
                                kv_dtype="bf16", seed=43))
    P = 3 * resident(batch)
    tm = H.plan(batch, P)
    m = lbsa.read_task_map(tm, batch["B"], batch["num_kv_heads"], P)
    ws = torch.full((lbsa.workspace_bytes(batch["B"], batch["num_heads"], batch["num_kv_heads"], P),),
                    255, dtype=torch.uint8, device="cuda:0")
    H.decode_split(batch, tm, P, workspace=ws)
    torch.cuda.synchronize()
    p1 = lbsa.read_partials(ws, batch["B"], batch["num_heads"], batch["num_kv_heads"], P, m["Ndesc"])
    ws.fill_(0)
    H.decode_split(batch, tm, P, workspace=ws)
    torch.cuda.synchronize()
    p2 = lbsa.read_partials(ws, batch["B"], batch["num_heads"], batch["num_kv_heads"], P, m["Ndesc"])
    for a, b in zip(p1, p2):
        assert np.isfinite(a).all()
        assert np.array_equal(a.view(np.int32), b.view(np.int32))
    assert reserved_words(tm) == (0,)
