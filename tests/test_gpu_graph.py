"""The plan + decode sequence is graph-capturable (no allocation, no host sync,
no memset in the library): replays of a captured graph, interleaved with eager
work and synchronisations, give exactly the eager result every time."""
import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graph_replays_match_eager(kv):
    batch = H.batch_on_gpu(dict(seqlens=[5, 3000, 64, 700, 0, 129, 4097], num_heads=16, num_kv_heads=2,
                                kv_dtype=kv, seed=41))
    P = 37
    B, Hq, Hkv = batch["B"], batch["num_heads"], batch["num_kv_heads"]
    tm = torch.empty(lbsa.task_map_bytes(B, Hkv, P), dtype=torch.uint8, device="cuda:0")
    ws = torch.empty(lbsa.workspace_bytes(B, Hq, Hkv, P), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda:0")

    def step():
        lbsa.plan(batch["seqlens"], Hq, Hkv, batch["max_pages"], P, task_map=tm)
        H.decode(batch, tm, P, workspace=ws, out=out)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.fill_(float("nan"))          # eager work between replays
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"


def test_varlen_graph_replays_match_eager():
    """Prefill / extend / decode rows on the task map: plan_varlen + attend_varlen
    (the counter-clearing kernel, the split kernel with its in-kernel merges)
    captured once; before every replay the workspace is filled with garbage,
    so the claim and arrival counters must be cleared inside the graph."""
    from load_balanced_split_assign_amd import workload as wl
    sl, ql = [2000, 777, 129, 4000], [1500, 700, 16, 1]
    b = wl.make_batch(seqlens=sl, qlens=ql, num_heads=16, num_kv_heads=2, kv_dtype="bf16", seed=42, device="cpu")
    b = {k: (v.to("cuda:0") if isinstance(v, torch.Tensor) else v) for k, v in b.items()}
    tq, P = sum(ql), 100
    tm = torch.empty(lbsa.varlen_task_map_bytes(b["B"], 2, P, tq), dtype=torch.uint8, device="cuda:0")
    ws = torch.empty(lbsa.varlen_workspace_bytes(16, 2, P), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(b["q"])

    def step():
        lbsa.plan_varlen(b["seqlens"], b["qlens"], 16, 2, b["max_pages"], P, 1, total_q=tq, task_map=tm)
        lbsa.attend_varlen(b["q"], b["k_cache"], b["v_cache"], b["page_table"], tm, P, b["softmax_scale"], b["B"],
                           workspace=ws, out=out)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    m = lbsa.read_varlen_task_map(tm, b["B"], 2, P, tq)
    assert (m["seg_num_chunks"] > 1).sum() >= 2            # the merges run inside the graph too
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
