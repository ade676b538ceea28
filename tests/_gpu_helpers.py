"""Shared helpers of the GPU parity tests (inputs from the seeded generator,
results through the C ABI binding, expectations from the CPU oracle)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from load_balanced_split_assign_amd import lbsa
from load_balanced_split_assign_amd import workload as wl

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")

BF16_TOL = 2e-2     # max |out - oracle| for bf16 KV
FP8_TOL = 6e-2      # max |out - oracle| for fp8-e4m3 KV
LSE_TOL = 1e-3      # |partial LSE - oracle| (natural log)


def tol(batch) -> float:
    return FP8_TOL if batch["kv_dtype"] == "fp8" else BF16_TOL


def batch_on_gpu(name_or_kw, tail="nan", gen_device="cpu"):
    """Seeded batch; generated on `gen_device`, always returned on cuda:0."""
    if isinstance(name_or_kw, str):
        b = wl.make_batch(name_or_kw, tail=tail, device=gen_device)
    else:
        b = wl.make_batch(**name_or_kw, tail=tail, device=gen_device)
    for k, v in list(b.items()):
        if isinstance(v, torch.Tensor):
            b[k] = v.to("cuda:0")
    return b


def workgroups(batch, P=None) -> int:
    if P:
        return int(P)
    if batch.get("num_workgroups"):
        return int(batch["num_workgroups"])
    return lbsa.default_workgroups(0, batch["kv_dtype"], batch.get("q_len", 1))


def plan(batch, P, F=0):
    return lbsa.plan(batch["seqlens"], batch["num_heads"], batch["num_kv_heads"], batch["max_pages"], P, F)


def decode(batch, task_map, P, **kw):
    return lbsa.decode(batch["q"], batch["k_cache"], batch["v_cache"], batch["page_table"], task_map, P,
                       batch["softmax_scale"], q_scale=batch["q_scale"], k_scale=batch["k_scale"],
                       v_scale=batch["v_scale"], **kw)


def decode_split(batch, task_map, P, **kw):
    return lbsa.decode_split(batch["q"], batch["k_cache"], batch["v_cache"], batch["page_table"], task_map, P,
                             batch["softmax_scale"], q_scale=batch["q_scale"], k_scale=batch["k_scale"],
                             v_scale=batch["v_scale"], **kw)


def decode_static(batch, S, **kw):
    return lbsa.decode_static(batch["q"], batch["k_cache"], batch["v_cache"], batch["page_table"],
                              batch["seqlens"], S, batch["softmax_scale"], q_scale=batch["q_scale"],
                              k_scale=batch["k_scale"], v_scale=batch["v_scale"], **kw)


def out_np(out: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def sample_rows(batch, n_requests=6, heads=(0, 7, 8, 63), seed=0):
    """(request, query head) rows for sampled parity at full size: the longest
    and shortest requests plus random ones, heads across group boundaries."""
    sl = batch["seqlens"].cpu().numpy()
    rng = np.random.default_rng(seed)
    reqs = {int(np.argmax(sl)), int(np.argmin(sl))}
    while len(reqs) < min(n_requests, len(sl)):
        reqs.add(int(rng.integers(0, len(sl))))
    hq = [h for h in heads if h < batch["num_heads"]]
    return np.array([(b, h) for b in sorted(reqs) for h in hq], np.int32)
