"""Shared helpers of the GPU parity tests (inputs from the seeded generator,
results through the C ABI binding, expectations from the CPU oracle)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from load_balanced_split_assign_amd import lbsa
from load_balanced_split_assign_amd import workload as wl

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")

from parity import BF16_TOL, FP8_TOL, LSE_TOL, REL_TOL, assert_parity  # noqa: F401  (the bar, tests/parity.py)


def tol(batch) -> float:
    return FP8_TOL if batch["kv_dtype"] == "fp8" else BF16_TOL


def check(batch, got, ref, what=""):
    """Both bounds of the bar on every row (absolute, and relative to the row's
    largest oracle entry); prints the figures so a run shows the margins."""
    err, ratio = assert_parity(got, ref, tol(batch), REL_TOL, what)
    print(f"parity {what}: max abs err {err:.2e}, worst row ratio {ratio:.2e}", flush=True)
    return err


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


def plan(batch, P, F=0, **kw):
    return lbsa.plan(batch["seqlens"], batch["num_heads"], batch["num_kv_heads"], batch["max_pages"], P, F, **kw)


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
