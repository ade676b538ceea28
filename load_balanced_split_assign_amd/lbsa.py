"""Thin ctypes binding of liblbsa.so (see include/lbsa.h for the C ABI).

Argument marshalling only: every step of the path (assign, split, combine and
the static baseline) runs in the library's HIP kernels.  PyTorch provides the
device memory and the stream.  If the shared library is missing this module
raises at first use -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblbsa.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_HIP = 0, -1, -2, -3
NOALLOC_SCRATCH_BYTES = 16 << 20      # LBSA_NOALLOC_SCRATCH_BYTES
KV_BF16, KV_FP8_E4M3 = 0, 1
PAGE_SIZE, HEAD_DIM, GROUP, DEFAULT_MIN_TILES = 64, 128, 8, 2
HEADER_FIELDS = ("T", "K", "q", "r", "Ndesc", "P", "F", "B", "Hq", "Hkv",
                 "error", "N", "max_pages", "page_size")
# a decode segment with more chunks than this is listed in the map's long_seg
# records and merged one output row per combine workgroup
LONG_SEGMENT_CHUNKS = 8

_lib = None


class LbsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


class _MapLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("header", "bin_desc_begin", "desc", "seg_first_desc", "seg_num_chunks", "seqlens", "bin_head",
                 "desc_len", "long_seg", "total")]


class _VarlenMapLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("header", "bin_desc_begin", "desc", "desc_slot", "claim_order", "seg_first_desc", "seg_num_chunks",
                 "seg_slot0", "blk_req", "blk_k", "qbase", "qstart", "seqlens", "qlens", "total")]


class _WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("part_lse", "part_o", "total")]


def lib() -> ctypes.CDLL:
    """The loaded liblbsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m load_balanced_split_assign_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        f32 = ctypes.c_float
        L.lbsa_status_string.argtypes = [ctypes.c_int]
        L.lbsa_status_string.restype = ctypes.c_char_p
        L.lbsa_version.restype = ctypes.c_int
        L.lbsa_default_workgroups.argtypes = [ctypes.c_int, i32, i32, ctypes.POINTER(i32)]
        L.lbsa_auto_workgroups.argtypes = [ctypes.c_int, i32, i32, i32, i64, ctypes.POINTER(i32)]
        L.lbsa_task_map_layout_get.argtypes = [i32, i32, i32, ctypes.POINTER(_MapLayout)]
        L.lbsa_task_map_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.lbsa_workspace_layout_get.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(_WsLayout)]
        L.lbsa_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.lbsa_static_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.lbsa_plan.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
        attn = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, i64, i32, f32, vp, sz, vp,
                sz]
        L.lbsa_decode.argtypes = attn + [vp, vp]
        L.lbsa_decode_noalloc.argtypes = attn[:-2] + [vp, vp]
        L.lbsa_decode_split.argtypes = attn + [vp]
        L.lbsa_decode_combine.argtypes = [i32, i32, i32, i32, i32, i32, vp, sz, vp, sz, vp, vp]
        L.lbsa_decode_static.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i32, i64, i32, f32, vp, sz, vp, vp]
        L.lbsa_prefill.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, f32, vp, vp]
        L.lbsa_varlen_task_map_layout_get.argtypes = [i32, i32, i32, i64, ctypes.POINTER(_VarlenMapLayout)]
        L.lbsa_varlen_task_map_bytes.argtypes = [i32, i32, i32, i64, ctypes.POINTER(sz)]
        L.lbsa_varlen_workspace_bytes.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.lbsa_varlen_default_workgroups.argtypes = [ctypes.c_int, ctypes.POINTER(i32)]
        L.lbsa_varlen_auto_workgroups.argtypes = [ctypes.c_int, ctypes.POINTER(i32), i32, i32, ctypes.POINTER(i32)]
        L.lbsa_plan_varlen.argtypes = [vp, vp, i32, i32, i32, i32, i32, i64, i32, i32, vp, sz, vp]
        L.lbsa_attend_varlen.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, i64, i32, f32, vp, sz,
                                         vp, sz, vp, vp]
        L.lbsa_router_split_weights.argtypes = [vp, i32, i32, vp, vp, vp]
        L.lbsa_router_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.lbsa_router_gemm.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
        L.lbsa_time_next_kernel.argtypes = [vp, vp]
        L.lbsa_time_next_kernels.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.lbsa_prologue.argtypes = [vp, vp, vp, vp, vp, ctypes.c_double, f32, i32, i32, i32, i32, i32, i32,
                                    vp, vp, vp, vp, vp, vp, i64, vp]
        for fn in ("lbsa_default_workgroups", "lbsa_auto_workgroups", "lbsa_task_map_layout_get", "lbsa_task_map_bytes", "lbsa_prologue",
                   "lbsa_workspace_layout_get", "lbsa_workspace_bytes", "lbsa_static_workspace_bytes",
                   "lbsa_plan", "lbsa_decode", "lbsa_decode_noalloc", "lbsa_decode_split", "lbsa_decode_combine",
                   "lbsa_decode_static", "lbsa_prefill", "lbsa_router_split_weights",
                   "lbsa_router_workspace_bytes", "lbsa_router_gemm", "lbsa_time_next_kernel",
                   "lbsa_time_next_kernels", "lbsa_varlen_task_map_layout_get", "lbsa_varlen_task_map_bytes",
                   "lbsa_varlen_workspace_bytes", "lbsa_varlen_default_workgroups", "lbsa_varlen_auto_workgroups",
                   "lbsa_plan_varlen",
                   "lbsa_attend_varlen"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lbsa_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise LbsaError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def kv_dtype_code(kv_dtype: str) -> int:
    return {"bf16": KV_BF16, "fp8": KV_FP8_E4M3}[kv_dtype]


# ---------------------------------------------------------------------------
# sizes and layouts
# ---------------------------------------------------------------------------

def _event_handle(ev):
    """hipEvent_t of a torch.cuda.Event (None stays None).  torch creates an
    event at its first record: an event never recorded is recorded once here,
    on the current stream, to create it."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def time_next_kernel(start=None, stop=None) -> None:
    """Arm the library's kernel timing hook: the next kernel that this thread
    launches through the library stamps `start` and `stop` (torch.cuda.Event
    with enable_timing=True) at its own start and end, so
    start.elapsed_time(stop) is that kernel's duration without a dispatch
    gap.  (None, None) disarms."""
    _check("lbsa_time_next_kernel", lib().lbsa_time_next_kernel(_event_handle(start), _event_handle(stop)))


def time_next_kernels(pairs) -> None:
    """Arm the hook for the next len(pairs) launches, in order: launch i stamps
    pairs[i] = (start, stop).  An empty list disarms."""
    n = len(pairs)
    starts = (ctypes.c_void_p * max(1, n))(*[_event_handle(a) for a, _ in pairs])
    stops = (ctypes.c_void_p * max(1, n))(*[_event_handle(b) for _, b in pairs])
    _check("lbsa_time_next_kernels", lib().lbsa_time_next_kernels(n, starts, stops))


def default_workgroups(device: int = 0, kv_dtype: str = "bf16", q_len: int = 1) -> int:
    out = ctypes.c_int32()
    _check("lbsa_default_workgroups", lib().lbsa_default_workgroups(int(device), kv_dtype_code(kv_dtype),
                                                                    int(q_len), ctypes.byref(out)))
    return int(out.value)


def auto_workgroups(seqlens, num_kv_heads: int, kv_dtype: str = "bf16", q_len: int = 1, device: int = 0) -> int:
    """lbsa_auto_workgroups for host-side lengths (a sequence of ints)."""
    total_tiles = int(num_kv_heads) * sum(-(-int(x) // 64) for x in seqlens if int(x) > 0)
    out = ctypes.c_int32()
    _check("lbsa_auto_workgroups", lib().lbsa_auto_workgroups(int(device), kv_dtype_code(kv_dtype), int(q_len),
                                                              int(num_kv_heads), total_tiles, ctypes.byref(out)))
    return int(out.value)


def task_map_layout(batch: int, num_kv_heads: int, P: int) -> dict:
    m = _MapLayout()
    _check("lbsa_task_map_layout_get", lib().lbsa_task_map_layout_get(batch, num_kv_heads, P, ctypes.byref(m)))
    return {n: int(getattr(m, n)) for n, _ in m._fields_}


def task_map_bytes(batch: int, num_kv_heads: int, P: int) -> int:
    out = ctypes.c_size_t()
    _check("lbsa_task_map_bytes", lib().lbsa_task_map_bytes(batch, num_kv_heads, P, ctypes.byref(out)))
    return int(out.value)


def workspace_layout(batch: int, num_heads: int, num_kv_heads: int, P: int, head_dim: int = HEAD_DIM,
                     q_len: int = 1) -> dict:
    w = _WsLayout()
    _check("lbsa_workspace_layout_get",
           lib().lbsa_workspace_layout_get(batch, q_len, num_heads, num_kv_heads, head_dim, P, ctypes.byref(w)))
    return {n: int(getattr(w, n)) for n, _ in w._fields_}


def workspace_bytes(batch: int, num_heads: int, num_kv_heads: int, P: int, head_dim: int = HEAD_DIM,
                    q_len: int = 1) -> int:
    out = ctypes.c_size_t()
    _check("lbsa_workspace_bytes",
           lib().lbsa_workspace_bytes(batch, q_len, num_heads, num_kv_heads, head_dim, P, ctypes.byref(out)))
    return int(out.value)


def static_workspace_bytes(batch: int, num_heads: int, num_kv_heads: int, num_splits: int,
                           head_dim: int = HEAD_DIM, q_len: int = 1) -> int:
    out = ctypes.c_size_t()
    _check("lbsa_static_workspace_bytes",
           lib().lbsa_static_workspace_bytes(batch, q_len, num_heads, num_kv_heads, head_dim, num_splits,
                                             ctypes.byref(out)))
    return int(out.value)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def plan(seqlens: torch.Tensor, num_heads: int, num_kv_heads: int, max_pages: int, num_workgroups: int,
         min_tiles_per_bin: int = 0, page_size: int = PAGE_SIZE, task_map: torch.Tensor | None = None):
    """Run the assign kernel; returns the task map (uint8 device tensor)."""
    B = int(seqlens.numel())
    nbytes = task_map_bytes(B, num_kv_heads, num_workgroups)
    if task_map is None:
        task_map = torch.empty(nbytes, dtype=torch.uint8, device=seqlens.device)
    assert seqlens.dtype == torch.int32 and seqlens.is_contiguous()
    _check("lbsa_plan", lib().lbsa_plan(_ptr(seqlens), B, num_heads, num_kv_heads, page_size, max_pages,
                                        num_workgroups, min_tiles_per_bin, _ptr(task_map),
                                        task_map.numel() * task_map.element_size(), _stream(seqlens.device)))
    return task_map


def _attn_args(q, q_scale, k_cache, v_cache, k_scale, v_scale, page_table):
    """Checks the decode tensors against each other (the C ABI takes no sizes for
    the scales, so a mis-sized tensor here would mean reads out of bounds) and
    returns the leading C arguments and (B, q_len, Hq, Hkv, D)."""
    fp8 = k_cache.dtype == torch.float8_e4m3fn
    if fp8:
        assert q.dtype == torch.float8_e4m3fn and v_cache.dtype == torch.float8_e4m3fn
        assert q_scale is not None and k_scale is not None and v_scale is not None
    else:
        assert q.dtype == torch.bfloat16 and k_cache.dtype == torch.bfloat16 and v_cache.dtype == torch.bfloat16
    dev = q.device
    for t in (q, k_cache, v_cache, page_table, q_scale, k_scale, v_scale):
        assert t is None or (t.is_contiguous() and t.device == dev)
    # q [B, Hq, D]: one query token per request; [B, q_len, Hq, D]: multi-token decode
    if q.dim() == 3:
        (B, Hq, D), QL = q.shape, 1
    else:
        B, QL, Hq, D = q.shape
    num_pages, page, Hkv, D2 = k_cache.shape
    assert page == PAGE_SIZE and D2 == D and tuple(v_cache.shape) == tuple(k_cache.shape)
    assert page_table.dtype == torch.int32 and page_table.dim() == 2 and page_table.shape[0] == B
    if fp8:
        assert q_scale.dtype == torch.float32 and q_scale.numel() == B * QL * Hq
        for sc in (k_scale, v_scale):
            assert sc.dtype == torch.float32 and sc.numel() == num_pages * Hkv * PAGE_SIZE
    return [_ptr(q), _ptr(q_scale) if fp8 else None, _ptr(k_cache), _ptr(v_cache),
            _ptr(k_scale) if fp8 else None, _ptr(v_scale) if fp8 else None,
            KV_FP8_E4M3 if fp8 else KV_BF16, _ptr(page_table), B, QL, Hq, Hkv, D, page,
            int(page_table.shape[1]), int(num_pages)], (B, QL, Hq, Hkv, D)


def _check_out(out, q):
    """A caller's output tensor: bf16, contiguous, on q's device, shaped like q."""
    assert out.dtype == torch.bfloat16 and out.is_contiguous() and out.device == q.device
    assert tuple(out.shape) == tuple(q.shape), (tuple(out.shape), tuple(q.shape))


def _check_bytes(buf, device, what):
    """A caller's byte buffer (workspace, task map): uint8, contiguous, on `device`."""
    assert buf.dtype == torch.uint8 and buf.is_contiguous() and buf.device == device, what


def decode(q, k_cache, v_cache, page_table, task_map, num_workgroups: int, softmax_scale: float,
           q_scale=None, k_scale=None, v_scale=None, workspace=None, out=None):
    """Split + combine with a task map from :func:`plan`; returns bf16 shaped like q."""
    args, (B, QL, Hq, Hkv, D) = _attn_args(q, q_scale, k_cache, v_cache, k_scale, v_scale, page_table)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(B, Hq, Hkv, num_workgroups, D, QL), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=q.device)
    _check_out(out, q)
    _check_bytes(workspace, q.device, "workspace")
    _check_bytes(task_map, q.device, "task map")
    _check("lbsa_decode", lib().lbsa_decode(*args, num_workgroups, float(softmax_scale), _ptr(task_map),
                                            task_map.numel(), _ptr(workspace), workspace.numel(), _ptr(out),
                                            _stream(q.device)))
    return out


def decode_noalloc(q, k_cache, v_cache, page_table, task_map, num_workgroups: int, softmax_scale: float,
                   q_scale=None, k_scale=None, v_scale=None, out=None):
    """lbsa_decode_noalloc: split + combine with the partials in the library's
    own device scratch array (no workspace; calls on one GPU must not overlap).
    With `out` given, nothing is allocated on this path either."""
    args, (B, QL, Hq, Hkv, D) = _attn_args(q, q_scale, k_cache, v_cache, k_scale, v_scale, page_table)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=q.device)
    _check_out(out, q)
    _check_bytes(task_map, q.device, "task map")
    _check("lbsa_decode_noalloc", lib().lbsa_decode_noalloc(*args, num_workgroups, float(softmax_scale),
                                                            _ptr(task_map), task_map.numel(), _ptr(out),
                                                            _stream(q.device)))
    return out


def decode_split(q, k_cache, v_cache, page_table, task_map, num_workgroups: int, softmax_scale: float,
                 q_scale=None, k_scale=None, v_scale=None, workspace=None):
    """Split kernel only; returns the workspace holding the partials."""
    args, (B, QL, Hq, Hkv, D) = _attn_args(q, q_scale, k_cache, v_cache, k_scale, v_scale, page_table)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(B, Hq, Hkv, num_workgroups, D, QL), dtype=torch.uint8,
                                device=q.device)
    _check_bytes(workspace, q.device, "workspace")
    _check_bytes(task_map, q.device, "task map")
    _check("lbsa_decode_split", lib().lbsa_decode_split(*args, num_workgroups, float(softmax_scale),
                                                        _ptr(task_map), task_map.numel(), _ptr(workspace),
                                                        workspace.numel(), _stream(q.device)))
    return workspace


def decode_combine(batch: int, num_heads: int, num_kv_heads: int, num_workgroups: int, task_map, workspace,
                   out=None, head_dim: int = HEAD_DIM, q_len: int = 1):
    """Combine kernel only; returns bf16 [B, Hq, D] (or [B, q_len, Hq, D] for q_len > 1)."""
    if out is None:
        shape = (batch, num_heads, head_dim) if q_len == 1 else (batch, q_len, num_heads, head_dim)
        out = torch.empty(shape, dtype=torch.bfloat16, device=workspace.device)
    shape = (batch, num_heads, head_dim) if q_len == 1 else (batch, q_len, num_heads, head_dim)
    assert out.dtype == torch.bfloat16 and out.is_contiguous() and out.device == workspace.device
    assert out.numel() == batch * q_len * num_heads * head_dim, (tuple(out.shape), shape)
    _check_bytes(workspace, workspace.device, "workspace")
    _check_bytes(task_map, workspace.device, "task map")
    _check("lbsa_decode_combine", lib().lbsa_decode_combine(batch, q_len, num_heads, num_kv_heads, head_dim,
                                                            num_workgroups, _ptr(task_map), task_map.numel(),
                                                            _ptr(workspace), workspace.numel(), _ptr(out),
                                                            _stream(workspace.device)))
    return out


def decode_static(q, k_cache, v_cache, page_table, seqlens, num_splits: int, softmax_scale: float,
                  q_scale=None, k_scale=None, v_scale=None, workspace=None, out=None):
    """Static split-KV baseline (fixed split count per request)."""
    args, (B, QL, Hq, Hkv, D) = _attn_args(q, q_scale, k_cache, v_cache, k_scale, v_scale, page_table)
    assert seqlens.dtype == torch.int32 and seqlens.is_contiguous()
    if workspace is None:
        workspace = torch.empty(static_workspace_bytes(B, Hq, Hkv, num_splits, D, QL), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=q.device)
    _check_out(out, q)
    _check_bytes(workspace, q.device, "workspace")
    assert seqlens.device == q.device and seqlens.numel() == B
    a = args
    _check("lbsa_decode_static", lib().lbsa_decode_static(*a[:8], _ptr(seqlens), *a[8:], num_splits,
                                                          float(softmax_scale), _ptr(workspace),
                                                          workspace.numel(), _ptr(out), _stream(q.device)))
    return out


def prefill(q, k_cache, v_cache, page_table, seqlens, softmax_scale: float, out=None):
    """Prefill / extend attention: q bf16 [B, q_len, Hq, D] are the last q_len tokens of each
    request's seqlens[b] cached tokens (causal); returns bf16 [B, q_len, Hq, D]."""
    assert q.dtype == torch.bfloat16 and k_cache.dtype == torch.bfloat16 and v_cache.dtype == torch.bfloat16
    for t in (q, k_cache, v_cache, page_table, seqlens):
        assert t.is_contiguous()
    if q.dim() == 3:                                   # [B, Hq, D]: one new token per request
        (B, Hq, D), QL = q.shape, 1
    else:
        B, QL, Hq, D = q.shape
    num_pages, page, Hkv, D2 = k_cache.shape
    assert page == PAGE_SIZE and D2 == D and tuple(v_cache.shape) == tuple(k_cache.shape)
    assert page_table.dtype == torch.int32 and page_table.shape[0] == B
    assert seqlens.dtype == torch.int32 and seqlens.numel() == B
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=q.device)
    _check_out(out, q)
    _check("lbsa_prefill", lib().lbsa_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), KV_BF16, _ptr(page_table),
                                              _ptr(seqlens), B, QL, Hq, Hkv, D, page, int(page_table.shape[1]),
                                              int(num_pages), float(softmax_scale), _ptr(out), _stream(q.device)))
    return out


# ---------------------------------------------------------------------------
# prefill / extend / decode rows on one task map (query blocks of 24 positions)
# ---------------------------------------------------------------------------

QBLOCK = 24   # the library's query positions per block (header word 15 of a built map)


def varlen_task_map_layout(batch: int, num_kv_heads: int, P: int, total_q: int) -> dict:
    lay = _VarlenMapLayout()
    _check("lbsa_varlen_task_map_layout_get",
           lib().lbsa_varlen_task_map_layout_get(batch, num_kv_heads, P, total_q, ctypes.byref(lay)))
    return {n: int(getattr(lay, n)) for n, _ in lay._fields_}


def varlen_task_map_bytes(batch: int, num_kv_heads: int, P: int, total_q: int) -> int:
    out = ctypes.c_size_t()
    _check("lbsa_varlen_task_map_bytes",
           lib().lbsa_varlen_task_map_bytes(batch, num_kv_heads, P, total_q, ctypes.byref(out)))
    return out.value


def varlen_workspace_bytes(num_heads: int, num_kv_heads: int, P: int) -> int:
    out = ctypes.c_size_t()
    _check("lbsa_varlen_workspace_bytes",
           lib().lbsa_varlen_workspace_bytes(num_heads, num_kv_heads, HEAD_DIM, P, ctypes.byref(out)))
    return out.value


def varlen_default_workgroups(device: int = 0) -> int:
    out = ctypes.c_int32()
    _check("lbsa_varlen_default_workgroups", lib().lbsa_varlen_default_workgroups(device, ctypes.byref(out)))
    return out.value


def varlen_auto_workgroups(qlens, num_kv_heads: int, device: int = 0) -> int:
    """P for a prefill / extend map from the q counts (host values)."""
    q = np.ascontiguousarray(np.asarray(qlens, dtype=np.int32).ravel())
    out = ctypes.c_int32()
    _check("lbsa_varlen_auto_workgroups",
           lib().lbsa_varlen_auto_workgroups(int(device), q.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                            int(q.size), int(num_kv_heads), ctypes.byref(out)))
    return out.value


def plan_varlen(seqlens: torch.Tensor, qlens: torch.Tensor, num_heads: int, num_kv_heads: int, max_pages: int,
                num_workgroups: int, min_tiles_per_bin: int = 0, total_q: int | None = None,
                task_map: torch.Tensor | None = None):
    """Task map with query blocks for requests bringing qlens[b] new tokens each
    (packed q rows in request order); total_q = sum(qlens) (read from the device
    tensor when not given)."""
    B = int(seqlens.numel())
    assert qlens.numel() == B and seqlens.dtype == torch.int32 and qlens.dtype == torch.int32
    assert seqlens.is_contiguous() and qlens.is_contiguous()
    if total_q is None:
        total_q = int(qlens.sum())
    nbytes = varlen_task_map_bytes(B, num_kv_heads, num_workgroups, total_q)
    if task_map is None:
        task_map = torch.empty(nbytes, dtype=torch.uint8, device=seqlens.device)
    _check("lbsa_plan_varlen", lib().lbsa_plan_varlen(
        _ptr(seqlens), _ptr(qlens), B, num_heads, num_kv_heads, PAGE_SIZE, max_pages, total_q, num_workgroups,
        min_tiles_per_bin, _ptr(task_map), task_map.numel() * task_map.element_size(), _stream(seqlens.device)))
    return task_map


def attend_varlen(q, k_cache, v_cache, page_table, task_map, num_workgroups: int, softmax_scale: float, B: int,
                  workspace=None, out=None):
    """Attention of packed queries q bf16 [total_q, Hq, D] on a map from plan_varlen;
    returns bf16 [total_q, Hq, D]."""
    assert q.dtype == torch.bfloat16 and k_cache.dtype == torch.bfloat16 and v_cache.dtype == torch.bfloat16
    for t in (q, k_cache, v_cache, page_table, task_map):
        assert t.is_contiguous()
    total_q, Hq, D = q.shape
    num_pages, page, Hkv, D2 = k_cache.shape
    assert page == PAGE_SIZE and D2 == D and tuple(v_cache.shape) == tuple(k_cache.shape)
    assert page_table.dtype == torch.int32 and page_table.shape[0] == B
    if workspace is None:
        workspace = torch.empty(varlen_workspace_bytes(Hq, Hkv, num_workgroups), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=q.device)
    _check_out(out, q)
    _check("lbsa_attend_varlen", lib().lbsa_attend_varlen(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), B, Hq, Hkv, D, page, int(page_table.shape[1]),
        int(num_pages), total_q, num_workgroups, float(softmax_scale), _ptr(task_map),
        task_map.numel() * task_map.element_size(), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(out), _stream(q.device)))
    return out


def read_varlen_task_map(task_map: torch.Tensor, batch: int, num_kv_heads: int, P: int, total_q: int) -> dict:
    """Copy a query-block task map to the host and split it into its arrays."""
    lay = varlen_task_map_layout(batch, num_kv_heads, P, total_q)
    raw = task_map.detach().cpu().numpy()[:lay["total"]]

    def arr(off, n, shape=None):
        a = raw[off:off + 4 * n].view(np.int32).copy()
        return a if shape is None else a.reshape(shape)

    header = arr(lay["header"], 16)
    nq_max = batch + total_q // QBLOCK
    cap = num_kv_heads * nq_max + P
    NQ = int(header[14])
    S = num_kv_heads * NQ
    out = {"header": header, "bin_desc_begin": arr(lay["bin_desc_begin"], P + 1),
           "desc_all": arr(lay["desc"], 8 * cap, (cap, 8)),
           "seg_first_desc": arr(lay["seg_first_desc"], S), "seg_num_chunks": arr(lay["seg_num_chunks"], S),
           "seg_slot0": arr(lay["seg_slot0"], S), "blk_req": arr(lay["blk_req"], NQ), "blk_k": arr(lay["blk_k"], NQ),
           "qbase": arr(lay["qbase"], batch + 1), "qstart": arr(lay["qstart"], batch + 1),
           "seqlens": arr(lay["seqlens"], batch), "qlens": arr(lay["qlens"], batch)}
    for i, name in enumerate(HEADER_FIELDS):
        out[name] = int(header[i])
    out["NQ"], out["QB"] = NQ, int(header[15])
    nd = max(0, min(out["Ndesc"], cap))
    out["desc"] = out["desc_all"][:nd].copy()
    out["desc_slot"] = arr(lay["desc_slot"], cap)[:nd].copy()
    out["claim_order"] = arr(lay["claim_order"], cap)[:nd].copy()
    return out


def router_weight_shape(n: int, k: int) -> tuple:
    """Shape of one blocked weight part: [n/16][k/64][2][64][8] bf16 (per 16
    experts and 64 k, the halves b of the lanes' 16 k: lane = 16 g + n % 16
    holds k % 64 = 16 g + 8 b + e at [b][lane][e])."""
    return (n // 16, k // 64, 2, 64, 8)


def router_split_weights(w, w_high=None, w_low=None):
    """fp32 router weights [N, K] -> (w_high, w_low): truncation and the bf16
    of the residual x 256, both blocked (router_weight_shape)."""
    assert w.dtype == torch.float32 and w.dim() == 2 and w.is_contiguous()
    N, K = w.shape
    shape = router_weight_shape(N, K)
    if w_high is None:
        w_high = torch.empty(shape, dtype=torch.bfloat16, device=w.device)
    if w_low is None:
        w_low = torch.empty(shape, dtype=torch.bfloat16, device=w.device)
    assert w_high.numel() == N * K and w_low.numel() == N * K
    _check("lbsa_router_split_weights", lib().lbsa_router_split_weights(_ptr(w), N, K, _ptr(w_high), _ptr(w_low),
                                                                        _stream(w.device)))
    return w_high, w_low


def router_unpack_weights(part) -> torch.Tensor:
    """A blocked weight part -> the same values as [N, K] (a copy, for checks)."""
    nt, ks = part.shape[0], part.shape[1]
    t = part.reshape(nt, ks, 2, 4, 16, 8)                     # [n/16][k/64][b][g][r][e]
    return t.permute(0, 4, 1, 3, 2, 5).reshape(16 * nt, 64 * ks)


def router_workspace_bytes(m: int, n: int, k: int) -> int:
    out = ctypes.c_size_t()
    _check("lbsa_router_workspace_bytes", lib().lbsa_router_workspace_bytes(m, n, k, ctypes.byref(out)))
    return int(out.value)


def router_gemm(x, w_high, w_low, out=None, workspace=None):
    """fp32 scores [M, N] = x w_high^T + (x w_low^T) / 256 for bf16 x [M, K] and
    the blocked weight parts of router_split_weights."""
    assert x.dtype == torch.bfloat16 and w_high.dtype == torch.bfloat16 and w_low.dtype == torch.bfloat16
    for t in (x, w_high, w_low):
        assert t.is_contiguous()
    M, K = x.shape
    N = 16 * w_high.shape[0]
    assert tuple(w_high.shape) == router_weight_shape(N, K) and tuple(w_low.shape) == router_weight_shape(N, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    need = router_workspace_bytes(M, N, K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check("lbsa_router_gemm", lib().lbsa_router_gemm(_ptr(x), _ptr(w_high), _ptr(w_low), M, N, K, _ptr(out),
                                                      _ptr(workspace) if workspace is not None else None,
                                                      0 if workspace is None else workspace.numel(),
                                                      _stream(x.device)))
    return out


# ---------------------------------------------------------------------------
# reading results back (host side, for checks and reports)
# ---------------------------------------------------------------------------

def read_task_map(task_map: torch.Tensor, batch: int, num_kv_heads: int, P: int) -> dict:
    """Copy a task map to the host and split it into its arrays (library layout)."""
    lay = task_map_layout(batch, num_kv_heads, P)
    raw = task_map.detach().cpu().numpy()[:lay["total"]]
    S = batch * num_kv_heads
    cap = S + P

    def arr(off, n, shape=None):
        a = raw[off:off + 4 * n].view(np.int32).copy()
        return a if shape is None else a.reshape(shape)

    header = arr(lay["header"], 16)
    out = {"header": header, "bin_desc_begin": arr(lay["bin_desc_begin"], P + 1),
           "desc_all": arr(lay["desc"], 4 * cap, (cap, 4)),
           "seg_first_desc": arr(lay["seg_first_desc"], S), "seg_num_chunks": arr(lay["seg_num_chunks"], S),
           "seqlens": arr(lay["seqlens"], batch), "bin_head": arr(lay["bin_head"], 8 * P, (P, 8)),
           "desc_len_all": arr(lay["desc_len"], cap)}
    for i, name in enumerate(HEADER_FIELDS):
        out[name] = int(header[i])
    nd = max(0, min(out["Ndesc"], cap))
    out["desc"] = out["desc_all"][:nd].copy()
    out["desc_len"] = out["desc_len_all"][:nd].copy()
    max_long = cap // (LONG_SEGMENT_CHUNKS + 1)
    out["nlong"] = int(header[14])
    out["long_seg"] = arr(lay["long_seg"], 4 * max_long, (max_long, 4))[:max(0, min(out["nlong"], max_long))].copy()
    return out


def read_partials(workspace: torch.Tensor, batch: int, num_heads: int, num_kv_heads: int, P: int,
                  ndesc: int, q_len: int = 1):
    """(part_o [ndesc, q_len*8, 128], part_lse [ndesc, q_len*8]) as float32 numpy arrays
    (row 8 * query + head)."""
    lay = workspace_layout(batch, num_heads, num_kv_heads, P, q_len=q_len)
    raw = workspace.detach().cpu().numpy()
    R = GROUP * q_len
    lse = raw[lay["part_lse"]:lay["part_lse"] + 4 * R * ndesc].view(np.float32).reshape(ndesc, R)
    o = raw[lay["part_o"]:lay["part_o"] + 4 * R * HEAD_DIM * ndesc].view(np.float32)
    return o.reshape(ndesc, R, HEAD_DIM).copy(), lse.copy()


def prologue(qkv, positions, slot_mapping, q_norm_weight, k_norm_weight, num_heads: int, num_kv_heads: int,
             k_cache, v_cache, rope_theta: float = 10000.0, eps: float = 1e-6, k_scale=None, v_scale=None,
             q_out=None, q_scale_out=None):
    """Fused QK-Norm -> RoPE -> Q out (bf16, or fp8 + scale when the caches are
    fp8) and K / V written into the paged caches.  Returns (q_out, q_scale_out)."""
    T = int(qkv.shape[0])
    fp8 = k_cache.dtype == torch.float8_e4m3fn
    dev = qkv.device
    if q_out is None:
        q_out = torch.empty((T, num_heads, HEAD_DIM), dtype=torch.float8_e4m3fn if fp8 else torch.bfloat16,
                            device=dev)
    if fp8 and q_scale_out is None:
        q_scale_out = torch.empty((T, num_heads), dtype=torch.float32, device=dev)
    _check("lbsa_prologue", lib().lbsa_prologue(
        _ptr(qkv), _ptr(positions), _ptr(slot_mapping), _ptr(q_norm_weight), _ptr(k_norm_weight),
        float(rope_theta), float(eps), T, int(num_heads), int(num_kv_heads), int(qkv.shape[1]) // (
            int(num_heads) + 2 * int(num_kv_heads)), int(k_cache.shape[1]), KV_FP8_E4M3 if fp8 else KV_BF16,
        _ptr(q_out), _ptr(q_scale_out), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        int(k_cache.shape[0]), _stream(dev)))
    return q_out, q_scale_out
