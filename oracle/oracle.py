"""ctypes/numpy front end of the plain-C CPU oracle (``lbsa_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP library and never imports it.

Inputs are plain numpy arrays (or CPU torch tensors, converted here) holding the
raw bit patterns of bf16 / e4m3 values, exactly as the seeded generator made
them.  The method it follows is described in the HPC-Ops vLLM integration post,
section "The solution: a per-step, load-balanced decode scheduler" (bullets
"Assign" and "Compute and combine").
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblbsa_oracle.so")
_lib = None

HEADER_FIELDS = ("T", "K", "q", "r", "Ndesc", "P", "F", "B", "Hq", "Hkv",
                 "error", "N", "max_pages", "page_size")
TILE = 64


class _Inputs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("seqlens", ctypes.c_void_p),
        ("kv_dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("softmax_scale", ctypes.c_double),
        ("q_len", ctypes.c_int32),
        ("qlens", ctypes.c_void_p), ("qstart", ctypes.c_void_p),
    ]


def lib():
    """Load (building if needed) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or any(
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, f))
                for f in ("lbsa_oracle.c", "prologue_oracle.c")):
            from oracle import build as _b  # noqa: PLC0415
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_assign.argtypes = [P, i32, i32, i32, i32, i32, i32, P, P, P, i64, P, P]
        L.oracle_assign.restype = ctypes.c_int
        L.oracle_attention.argtypes = [ctypes.POINTER(_Inputs), P, P, ctypes.c_int]
        L.oracle_attention.restype = ctypes.c_int
        L.oracle_attention_rows.argtypes = [ctypes.POINTER(_Inputs), P, i64, P, P, ctypes.c_int]
        L.oracle_attention_rows.restype = ctypes.c_int
        L.oracle_partials.argtypes = [ctypes.POINTER(_Inputs), P, i64, P, P, ctypes.c_int]
        L.oracle_partials.restype = ctypes.c_int
        L.oracle_assign_varlen.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, P, P, P, i64, P, P, i64]
        L.oracle_assign_varlen.restype = ctypes.c_int
        L.oracle_attention_varlen.argtypes = [ctypes.POINTER(_Inputs), P, P, ctypes.c_int]
        L.oracle_attention_varlen.restype = ctypes.c_int
        L.oracle_attention_varlen_rows.argtypes = [ctypes.POINTER(_Inputs), P, i64, P, P, ctypes.c_int]
        L.oracle_attention_varlen_rows.restype = ctypes.c_int
        L.oracle_partials_varlen.argtypes = [ctypes.POINTER(_Inputs), P, i64, i32, P, P, ctypes.c_int]
        L.oracle_partials_varlen.restype = ctypes.c_int
        L.oracle_merge.argtypes = [P, P, i64, i64, P, P]
        L.oracle_merge.restype = None
        L.oracle_bf16_values.argtypes = [P, i64, P]
        L.oracle_e4m3_values.argtypes = [P, i64, P]
        L.oracle_num_threads.restype = ctypes.c_int
        d = ctypes.c_double
        L.oracle_rmsnorm.argtypes = [P, P, ctypes.c_int, d, P]
        L.oracle_rmsnorm.restype = None
        L.oracle_rope.argtypes = [P, ctypes.c_int, d, d]
        L.oracle_rope.restype = None
        L.oracle_quant_e4m3.argtypes = [P, ctypes.c_int, P, P]
        L.oracle_quant_e4m3.restype = None
        L.oracle_bf16_nearest.argtypes = [d]
        L.oracle_bf16_nearest.restype = ctypes.c_uint16
        L.oracle_prologue.argtypes = [P, i32, i32, i32, i32, P, P, P, d, d, P, P, P]
        L.oracle_prologue.restype = None
        _lib = L
    return _lib


def _np(x, dtype=None):
    """CPU, C-contiguous numpy view of a numpy array or torch tensor."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch  # noqa: PLC0415
        x = x.detach()
        if x.device.type != "cpu":
            x = x.cpu()
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16)
        elif x.dtype in (torch.float8_e4m3fn,):
            x = x.view(torch.uint8)
        x = x.contiguous().numpy()
    x = np.ascontiguousarray(x)
    if dtype is not None:
        x = x.view(dtype) if x.dtype.itemsize == np.dtype(dtype).itemsize else x.astype(dtype)
    return x


def _ptr(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_values(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns (uint16/int16 array)."""
    a = _np(bits, np.uint16).ravel()
    out = np.empty(a.size, np.float64)
    lib().oracle_bf16_values(_ptr(a), a.size, _ptr(out))
    return out.reshape(np.shape(bits))


def e4m3_values(bits) -> np.ndarray:
    """float64 values of OCP E4M3FN bit patterns (uint8 array)."""
    a = _np(bits, np.uint8).ravel()
    out = np.empty(a.size, np.float64)
    lib().oracle_e4m3_values(_ptr(a), a.size, _ptr(out))
    return out.reshape(np.shape(bits))


# ---------------------------------------------------------------------------
# assign
# ---------------------------------------------------------------------------

def assign(seqlens, num_heads: int, num_kv_heads: int, P: int, F: int, max_pages: int) -> dict:
    """Reference task map.

    Returns a dict with ``header`` int32[16], ``bin_desc_begin`` int32[P+1],
    ``desc`` int32[Ndesc, 4] (kv_head, request, tile_begin, tile_end),
    ``seg_first_desc`` / ``seg_num_chunks`` int32[Hkv*B] (index h*B + b) and the
    header fields by name.
    """
    sl = _np(seqlens, None).astype(np.int32).ravel()
    B = sl.size
    cap = num_kv_heads * B + P
    header = np.zeros(16, np.int32)
    bdb = np.zeros(P + 1, np.int32)
    desc = np.zeros((cap, 4), np.int32)
    sfd = np.zeros(num_kv_heads * B, np.int32)
    snc = np.zeros(num_kv_heads * B, np.int32)
    rc = lib().oracle_assign(_ptr(sl), B, num_heads, num_kv_heads, P, F, max_pages,
                             _ptr(header), _ptr(bdb), _ptr(desc), cap, _ptr(sfd), _ptr(snc))
    if rc != 0:
        raise ValueError("oracle_assign: invalid arguments")
    nd = int(header[4])
    out = {"header": header, "bin_desc_begin": bdb, "desc": desc[:nd].copy(),
           "seg_first_desc": sfd, "seg_num_chunks": snc}
    for i, name in enumerate(HEADER_FIELDS):
        out[name] = int(header[i])
    return out


def assign_varlen(seqlens, qlens, num_heads: int, num_kv_heads: int, P: int, F: int, max_pages: int,
                  QB: int = 16) -> dict:
    """Reference task map with query blocks (prefill / extend, reading Q1).

    ``desc`` is int32[Ndesc, 5] (kv_head, request, query_block, tile_begin,
    tile_end); ``seg_first_desc`` / ``seg_num_chunks`` are int32[Hkv * NQ], index
    h * NQ + (query blocks of earlier requests) + block; header word 14 is NQ,
    15 is QB."""
    sl = _np(seqlens, None).astype(np.int32).ravel()
    ql = _np(qlens, None).astype(np.int32).ravel()
    B = sl.size
    nq = int(sum(-(-max(int(x), 0) // QB) for x in ql))
    seg_cap = max(1, num_kv_heads * nq)
    cap = seg_cap + P
    header = np.zeros(16, np.int32)
    bdb = np.zeros(P + 1, np.int32)
    desc = np.zeros((cap, 5), np.int32)
    sfd = np.zeros(seg_cap, np.int32)
    snc = np.zeros(seg_cap, np.int32)
    rc = lib().oracle_assign_varlen(_ptr(sl), _ptr(ql), B, num_heads, num_kv_heads, P, F, max_pages, QB,
                                    _ptr(header), _ptr(bdb), _ptr(desc), cap, _ptr(sfd), _ptr(snc), seg_cap)
    if rc != 0:
        raise ValueError("oracle_assign_varlen: invalid arguments")
    nd = int(header[4])
    S = num_kv_heads * int(header[14])
    out = {"header": header, "bin_desc_begin": bdb, "desc": desc[:nd].copy(),
           "seg_first_desc": sfd[:S].copy(), "seg_num_chunks": snc[:S].copy()}
    for i, name in enumerate(HEADER_FIELDS):
        out[name] = int(header[i])
    out["NQ"], out["QB"] = int(header[14]), int(header[15])
    return out


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

class _Batch:
    """Keeps the numpy buffers alive while the C struct points at them."""

    def __init__(self, batch: dict):
        self.kv_dtype = 0 if batch["kv_dtype"] == "bf16" else 1
        if self.kv_dtype == 0:
            self.q = _np(batch["q"], np.uint16)
            self.k = _np(batch["k_cache"], np.uint16)
            self.v = _np(batch["v_cache"], np.uint16)
            self.qs = self.ks = self.vs = None
        else:
            self.q = _np(batch["q"], np.uint8)
            self.k = _np(batch["k_cache"], np.uint8)
            self.v = _np(batch["v_cache"], np.uint8)
            self.qs = _np(batch["q_scale"], np.float32)
            self.ks = _np(batch["k_scale"], np.float32)
            self.vs = _np(batch["v_scale"], np.float32)
        self.pt = _np(batch["page_table"], None).astype(np.int32)
        self.sl = _np(batch["seqlens"], None).astype(np.int32)
        self.ql = self.qs0 = None
        if batch.get("qlens") is not None:
            # Q1: q packed [sum q_b, Hq, D], request b's queries from row qstart[b]
            self.ql = _np(batch["qlens"], None).astype(np.int32).ravel()
            self.qs0 = np.concatenate([[0], np.cumsum(self.ql)]).astype(np.int32)
            B, (_, Hq, D), QL = self.sl.size, self.q.shape, 1
        # q [B, Hq, D] (one query per request) or [B, q_len, Hq, D]
        elif self.q.ndim == 3:
            (B, Hq, D), QL = self.q.shape, 1
        else:
            B, QL, Hq, D = self.q.shape
        num_pages, page, Hkv, D2 = self.k.shape
        assert page == TILE and D2 == D
        self.shape = (B, Hq, Hkv, D)
        self.q_len = QL
        self.s = _Inputs(
            _ptr(self.q), _ptr(self.qs), _ptr(self.k), _ptr(self.v), _ptr(self.ks), _ptr(self.vs),
            _ptr(self.pt), _ptr(self.sl), self.kv_dtype, B, Hq, Hkv, D,
            self.pt.shape[1], num_pages, float(batch["softmax_scale"]), QL, _ptr(self.ql), _ptr(self.qs0))


def attention(batch: dict, nthreads: int = 0):
    """fp64 attention of every (request, query head): returns (out, lse) shaped like q
    without / with its last axis: [B,Hq,D] and [B,Hq], or [B,q_len,Hq,D] and [B,q_len,Hq]."""
    bb = _Batch(batch)
    B, Hq, Hkv, D = bb.shape
    out = np.zeros(bb.q.shape, np.float64)
    lse = np.zeros(bb.q.shape[:-1], np.float64)
    if lib().oracle_attention(ctypes.byref(bb.s), _ptr(out), _ptr(lse), nthreads) != 0:
        raise ValueError("oracle_attention: page_table entry out of range")
    return out, lse


def attention_rows(batch: dict, rows, nthreads: int = 0):
    """fp64 attention for selected rows int[n, 2] = (request, j), j = query * Hq + head."""
    bb = _Batch(batch)
    D = bb.shape[3]
    rows = np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1, 2))
    out = np.zeros((rows.shape[0], D), np.float64)
    lse = np.zeros(rows.shape[0], np.float64)
    if lib().oracle_attention_rows(ctypes.byref(bb.s), _ptr(rows), rows.shape[0],
                                   _ptr(out), _ptr(lse), nthreads) != 0:
        raise ValueError("oracle_attention_rows: page_table entry out of range")
    return out, lse


def partials(batch: dict, desc, nthreads: int = 0):
    """fp64 partials of descriptors desc int[n, 4]: (part_o [n, q_len*G, D], part_lse [n, q_len*G]),
    row i*G + g for query i, head g of the group."""
    bb = _Batch(batch)
    B, Hq, Hkv, D = bb.shape
    G = Hq // Hkv * bb.q_len
    desc = np.ascontiguousarray(np.asarray(desc, np.int32).reshape(-1, 4))
    n = desc.shape[0]
    po = np.zeros((n, G, D), np.float64)
    pl = np.zeros((n, G), np.float64)
    if lib().oracle_partials(ctypes.byref(bb.s), _ptr(desc), n, _ptr(po), _ptr(pl), nthreads) != 0:
        raise ValueError("oracle_partials: page_table entry out of range")
    return po, pl


def attention_varlen(batch: dict, nthreads: int = 0):
    """fp64 attention of every packed query row (reading Q1): (out [sum q_b, Hq, D],
    lse [sum q_b, Hq])."""
    bb = _Batch(batch)
    out = np.zeros(bb.q.shape, np.float64)
    lse = np.zeros(bb.q.shape[:-1], np.float64)
    if lib().oracle_attention_varlen(ctypes.byref(bb.s), _ptr(out), _ptr(lse), nthreads) != 0:
        raise ValueError("oracle_attention_varlen: page_table entry out of range")
    return out, lse


def attention_varlen_rows(batch: dict, rows, nthreads: int = 0):
    """fp64 attention of selected packed rows int[n, 2] = (query row t, head hq)."""
    bb = _Batch(batch)
    D = bb.shape[3]
    rows = np.ascontiguousarray(np.asarray(rows, np.int32).reshape(-1, 2))
    out = np.zeros((rows.shape[0], D), np.float64)
    lse = np.zeros(rows.shape[0], np.float64)
    if lib().oracle_attention_varlen_rows(ctypes.byref(bb.s), _ptr(rows), rows.shape[0], _ptr(out), _ptr(lse),
                                          nthreads) != 0:
        raise ValueError("oracle_attention_varlen_rows: page_table entry out of range")
    return out, lse


def partials_varlen(batch: dict, desc, QB: int = 16, nthreads: int = 0):
    """fp64 partials of query-block descriptors desc int[n, 5]: (part_o [n, QB*G, D],
    part_lse [n, QB*G]), row p*G + g for query QB*k + p, head g of the group."""
    bb = _Batch(batch)
    B, Hq, Hkv, D = bb.shape
    G = Hq // Hkv
    desc = np.ascontiguousarray(np.asarray(desc, np.int32).reshape(-1, 5))
    n = desc.shape[0]
    po = np.zeros((n, QB * G, D), np.float64)
    pl = np.zeros((n, QB * G), np.float64)
    if lib().oracle_partials_varlen(ctypes.byref(bb.s), _ptr(desc), n, QB, _ptr(po), _ptr(pl), nthreads) != 0:
        raise ValueError("oracle_partials_varlen: page_table entry out of range")
    return po, pl


def merge(part_o, part_lse):
    """LSE merge of n partials of one row: part_o [n, width], part_lse [n]."""
    o = np.ascontiguousarray(np.asarray(part_o, np.float64))
    n = o.shape[0]
    o = o.reshape(n, int(np.prod(o.shape[1:])))
    l = np.ascontiguousarray(np.asarray(part_lse, np.float64).reshape(n))
    out = np.zeros(o.shape[1], np.float64)
    out_lse = np.zeros(1, np.float64)
    lib().oracle_merge(_ptr(o), _ptr(l), n, o.shape[1], _ptr(out), _ptr(out_lse))
    return out, float(out_lse[0])


# ---------------------------------------------------------------------------
# fused prologue (QK-Norm -> RoPE -> Q as bf16 or fp8 + scale; K/V to the cache)
# ---------------------------------------------------------------------------

def rmsnorm(x, w, eps: float) -> np.ndarray:
    """RMSNorm of the last axis of x (float64) with weight w."""
    x = np.ascontiguousarray(np.asarray(x, np.float64))
    w = np.ascontiguousarray(np.asarray(w, np.float64))
    n = x.shape[-1]
    flat = x.reshape(-1, n)
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        lib().oracle_rmsnorm(_ptr(flat[i]), _ptr(w), n, float(eps), _ptr(out[i]))
    return out.reshape(x.shape)


def rope(x, pos, theta: float) -> np.ndarray:
    """RoPE of the last axis of x (float64) at positions pos (one per row)."""
    x = np.array(np.asarray(x, np.float64), copy=True, order="C")
    n = x.shape[-1]
    flat = x.reshape(-1, n)
    pos = np.broadcast_to(np.asarray(pos, np.float64).ravel(), (flat.shape[0],))
    for i in range(flat.shape[0]):
        lib().oracle_rope(_ptr(flat[i]), n, float(pos[i]), float(theta))
    return flat.reshape(x.shape)


def quant_e4m3(x):
    """fp8 codes (uint8) and scale of the last axis of x (float64), per row."""
    x = np.ascontiguousarray(np.asarray(x, np.float64))
    n = x.shape[-1]
    flat = x.reshape(-1, n)
    codes = np.empty(flat.shape, np.uint8)
    scales = np.empty(flat.shape[0], np.float64)
    sc = ctypes.c_double()
    for i in range(flat.shape[0]):
        lib().oracle_quant_e4m3(_ptr(flat[i]), n, _ptr(codes[i]), ctypes.byref(sc))
        scales[i] = sc.value
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1])


def bf16_nearest(x) -> np.ndarray:
    """bf16 bit patterns (uint16) nearest to the float64 values x (ties to even)."""
    x = np.asarray(x, np.float64)
    f = lib().oracle_bf16_nearest
    return np.array([f(float(v)) for v in x.ravel()], np.uint16).reshape(x.shape)


def prologue(qkv, positions, q_weight, k_weight, num_heads: int, num_kv_heads: int, theta: float,
             eps: float):
    """float64 (q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,D]) of the prologue of T tokens;
    qkv holds bf16 bits [T, (Hq + 2 Hkv) * D]."""
    a = _np(qkv, np.uint16)
    T = a.shape[0]
    D = np.asarray(q_weight).size
    Hq, Hkv = int(num_heads), int(num_kv_heads)
    pos = _np(positions, None).astype(np.int32).ravel()
    qw = np.ascontiguousarray(np.asarray(q_weight, np.float64))
    kw = np.ascontiguousarray(np.asarray(k_weight, np.float64))
    q = np.zeros((T, Hq, D), np.float64)
    k = np.zeros((T, Hkv, D), np.float64)
    v = np.zeros((T, Hkv, D), np.float64)
    lib().oracle_prologue(_ptr(a), T, Hq, Hkv, D, _ptr(pos), _ptr(qw), _ptr(kw), float(theta), float(eps),
                          _ptr(q), _ptr(k), _ptr(v))
    return q, k, v
