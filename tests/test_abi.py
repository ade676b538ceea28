"""The C ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before anything is enqueued (no GPU needed: these calls
return before touching the device)."""
import ctypes
import os
import re

import pytest

from load_balanced_split_assign_amd import lbsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lbsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lbsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    L = lbsa.lib()
    for n in names:
        assert hasattr(L, n), n
        assert getattr(L, n) is not None


def test_version_and_status_strings():
    assert lbsa.lib().lbsa_version() == 209
    assert lbsa.status_string(0) == "ok"
    assert "invalid" in lbsa.status_string(-1)
    assert "unsupported" in lbsa.status_string(-2)


def test_task_map_layout_is_aligned_and_sized():
    for B, Hkv, P in [(4, 1, 32), (64, 8, 768), (1, 8, 2048), (8, 8, 512)]:
        lay = lbsa.task_map_layout(B, Hkv, P)
        S, cap = B * Hkv, B * Hkv + P
        assert lay["header"] == 0 and lay["bin_desc_begin"] == 64
        assert lay["desc"] % 16 == 0 and lay["desc"] >= 64 + 4 * (P + 1)
        assert lay["seg_first_desc"] == lay["desc"] + 16 * cap
        assert lay["seg_num_chunks"] == lay["seg_first_desc"] + 4 * S
        assert lay["seqlens"] == lay["seg_num_chunks"] + 4 * S
        assert lay["bin_head"] % 32 == 0 and lay["bin_head"] >= lay["seqlens"] + 4 * B
        assert lay["desc_len"] == lay["bin_head"] + 32 * P
        assert lay["long_seg"] % 16 == 0 and lay["long_seg"] >= lay["desc_len"] + 4 * cap
        assert lay["total"] >= lay["long_seg"] + 16 * (cap // 9) and lay["total"] % 256 == 0
        assert lbsa.task_map_bytes(B, Hkv, P) == lay["total"]


def test_workspace_layout():
    w = lbsa.workspace_layout(64, 64, 8, 768)
    cap = 64 * 8 + 768
    assert w["part_o"] >= 4 * 8 * cap and w["part_o"] % 256 == 0
    assert w["total"] >= w["part_o"] + 4 * 8 * 128 * cap
    assert lbsa.static_workspace_bytes(64, 64, 8, 4) >= 4 * 8 * 129 * 64 * 8 * 4
    # two query tokens per request: twice the partial rows
    w2 = lbsa.workspace_layout(64, 64, 8, 768, q_len=2)
    assert w2["part_o"] >= 4 * 16 * cap and w2["total"] >= w2["part_o"] + 4 * 16 * 128 * cap
    assert lbsa.static_workspace_bytes(64, 64, 8, 4, q_len=2) >= 4 * 16 * 129 * 64 * 8 * 4


def _plan_status(**kw):
    a = dict(seqlens=ctypes.c_void_p(16), B=4, Hq=8, Hkv=1, page=64, mp=65, P=32, F=0,
             map=ctypes.c_void_p(256), nbytes=1 << 20, stream=None)
    a.update(kw)
    return lbsa.lib().lbsa_plan(a["seqlens"], a["B"], a["Hq"], a["Hkv"], a["page"], a["mp"], a["P"], a["F"],
                                a["map"], a["nbytes"], a["stream"])


def test_plan_rejects_bad_arguments_on_host():
    assert _plan_status(seqlens=None) == lbsa.ERR_INVALID_ARGUMENT
    assert _plan_status(map=None) == lbsa.ERR_INVALID_ARGUMENT
    assert _plan_status(B=0) == lbsa.ERR_INVALID_ARGUMENT
    assert _plan_status(Hq=12, Hkv=8) == lbsa.ERR_INVALID_ARGUMENT      # Hq % Hkv != 0
    assert _plan_status(Hq=16, Hkv=1) == lbsa.ERR_UNSUPPORTED           # group 16
    assert _plan_status(page=32) == lbsa.ERR_UNSUPPORTED
    assert _plan_status(P=0) == lbsa.ERR_INVALID_ARGUMENT
    assert _plan_status(F=-1) == lbsa.ERR_INVALID_ARGUMENT
    assert _plan_status(nbytes=100) == lbsa.ERR_INVALID_ARGUMENT        # map too small
    assert _plan_status(map=ctypes.c_void_p(8)) == lbsa.ERR_INVALID_ARGUMENT   # misaligned
    assert _plan_status(B=9000, Hq=8, Hkv=1) == lbsa.ERR_UNSUPPORTED    # LDS of the assign workgroup


def _decode_status(**kw):
    a = dict(q=16, qs=None, k=256, v=512, ks=None, vs=None, dt=0, pt=1024, B=4, QL=1, Hq=8, Hkv=1, D=128,
             page=64, mp=65, npages=100, P=32, scale=0.088, map=4096, mapb=1 << 20, ws=1 << 16, wsb=1 << 30,
             out=8192)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lbsa.lib().lbsa_decode(vp(a["q"]), vp(a["qs"]), vp(a["k"]), vp(a["v"]), vp(a["ks"]), vp(a["vs"]),
                                  a["dt"], vp(a["pt"]), a["B"], a["QL"], a["Hq"], a["Hkv"], a["D"], a["page"],
                                  a["mp"], a["npages"], a["P"], a["scale"], vp(a["map"]), a["mapb"], vp(a["ws"]),
                                  a["wsb"], vp(a["out"]), None)


def test_decode_rejects_bad_arguments_on_host():
    assert _decode_status(q=None) == lbsa.ERR_INVALID_ARGUMENT
    assert _decode_status(D=64) == lbsa.ERR_UNSUPPORTED
    assert _decode_status(dt=7) == lbsa.ERR_INVALID_ARGUMENT
    assert _decode_status(dt=1) == lbsa.ERR_INVALID_ARGUMENT              # fp8 without scales
    assert _decode_status(mapb=64) == lbsa.ERR_INVALID_ARGUMENT           # map too small
    assert _decode_status(wsb=64) == lbsa.ERR_INVALID_ARGUMENT            # workspace too small
    assert _decode_status(ws=(1 << 16) + 4) == lbsa.ERR_INVALID_ARGUMENT  # misaligned workspace
    assert _decode_status(k=260) == lbsa.ERR_INVALID_ARGUMENT             # misaligned cache
    assert _decode_status(npages=0) == lbsa.ERR_INVALID_ARGUMENT
    assert _decode_status(out=None) == lbsa.ERR_INVALID_ARGUMENT
    assert _decode_status(scale=float("nan")) == lbsa.ERR_INVALID_ARGUMENT
    assert _decode_status(QL=0) == lbsa.ERR_INVALID_ARGUMENT
    assert _decode_status(QL=3) == lbsa.ERR_UNSUPPORTED                   # at most 2 query tokens
    assert _decode_status(QL=2, wsb=lbsa.workspace_bytes(4, 8, 1, 32)) == lbsa.ERR_INVALID_ARGUMENT  # sized for 1


def _prologue_status(**kw):
    a = dict(qkv=16, pos=32, slots=64, qw=128, kw=256, theta=10000.0, eps=1e-6, T=4, Hq=8, Hkv=1, D=128,
             page=64, dt=0, q=4096, qs=None, k=8192, v=16384, ks=None, vs=None, npages=10)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lbsa.lib().lbsa_prologue(vp(a["qkv"]), vp(a["pos"]), vp(a["slots"]), vp(a["qw"]), vp(a["kw"]),
                                    a["theta"], a["eps"], a["T"], a["Hq"], a["Hkv"], a["D"], a["page"], a["dt"],
                                    vp(a["q"]), vp(a["qs"]), vp(a["k"]), vp(a["v"]), vp(a["ks"]), vp(a["vs"]),
                                    a["npages"], None)


def test_prologue_rejects_bad_arguments_on_host():
    assert _prologue_status(qkv=None) == lbsa.ERR_INVALID_ARGUMENT
    assert _prologue_status(D=64) == lbsa.ERR_UNSUPPORTED
    assert _prologue_status(page=16) == lbsa.ERR_UNSUPPORTED
    assert _prologue_status(Hq=12, Hkv=8) == lbsa.ERR_INVALID_ARGUMENT
    assert _prologue_status(dt=1) == lbsa.ERR_INVALID_ARGUMENT             # fp8 without scales
    assert _prologue_status(theta=1.0) == lbsa.ERR_INVALID_ARGUMENT
    assert _prologue_status(eps=-1.0) == lbsa.ERR_INVALID_ARGUMENT
    assert _prologue_status(qw=130) == lbsa.ERR_INVALID_ARGUMENT           # misaligned weights
    assert _prologue_status(slots=68) == lbsa.ERR_INVALID_ARGUMENT         # misaligned int64
    assert _prologue_status(qkv=24) == lbsa.ERR_INVALID_ARGUMENT           # 16-byte loads
    assert _prologue_status(q=4104) == lbsa.ERR_INVALID_ARGUMENT           # 16-byte bf16 stores
    assert _prologue_status(k=8196, dt=1, qs=512, ks=1024, vs=2048) == lbsa.ERR_INVALID_ARGUMENT  # 8 B fp8
    assert _prologue_status(T=-1) == lbsa.ERR_INVALID_ARGUMENT
    assert _prologue_status(npages=0) == lbsa.ERR_INVALID_ARGUMENT
    assert _prologue_status(T=0, qkv=None) == lbsa.OK                      # nothing to do


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(lbsa, "_lib", None)
    monkeypatch.setattr(lbsa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        lbsa.lib()


def test_router_rejects_bad_arguments_on_host():
    L = lbsa.lib()
    vp = ctypes.c_void_p
    out = ctypes.c_size_t()
    assert L.lbsa_router_workspace_bytes(4, 192, 4096, ctypes.byref(out)) == lbsa.OK
    assert L.lbsa_router_workspace_bytes(4, 100, 4096, ctypes.byref(out)) == lbsa.ERR_UNSUPPORTED    # n % 16
    assert L.lbsa_router_workspace_bytes(4, 192, 4000, ctypes.byref(out)) == lbsa.ERR_UNSUPPORTED    # k % 256
    assert L.lbsa_router_workspace_bytes(4, 192, 384, ctypes.byref(out)) == lbsa.ERR_UNSUPPORTED
    assert L.lbsa_router_workspace_bytes(4, 16, 1 << 21, ctypes.byref(out)) == lbsa.ERR_UNSUPPORTED   # k > 2^20
    # a split of k: one fp32 plane of scores per part
    assert L.lbsa_router_workspace_bytes(4, 192, 4096, ctypes.byref(out)) == lbsa.OK
    assert out.value == 16 * 4 * 192 * 4
    assert L.lbsa_router_workspace_bytes(4, 192, 256, ctypes.byref(out)) == lbsa.OK and out.value == 0
    # many tokens: k in parts of at most 1024 (the X tile of a workgroup sits in LDS)
    assert L.lbsa_router_workspace_bytes(65536, 192, 1024, ctypes.byref(out)) == lbsa.OK and out.value == 0
    assert L.lbsa_router_workspace_bytes(65536, 192, 4096, ctypes.byref(out)) == lbsa.OK
    assert out.value == 4 * 65536 * 192 * 4
    assert L.lbsa_router_workspace_bytes(-1, 192, 4096, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_router_workspace_bytes(0, 192, 4096, ctypes.byref(out)) == lbsa.OK and out.value == 0
    assert L.lbsa_router_split_weights(None, 192, 4096, vp(256), vp(512), None) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_router_split_weights(vp(8), 192, 4096, vp(256), vp(512), None) == lbsa.ERR_INVALID_ARGUMENT
    # (every call below must fail validation: none may reach a launch with these fake pointers)
    assert L.lbsa_router_workspace_bytes(100, 192, 4096, ctypes.byref(out)) == lbsa.OK and out.value > 0
    assert L.lbsa_router_gemm(vp(256), vp(512), vp(1024), 100, 192, 4096, vp(2048), None, 0, None) == \
        lbsa.ERR_INVALID_ARGUMENT                                                              # workspace needed
    assert L.lbsa_router_gemm(None, vp(512), vp(1024), 4, 192, 4096, vp(2048), vp(4096), 1 << 30, None) == \
        lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_router_gemm(None, None, None, 0, 192, 4096, None, None, 0, None) == lbsa.OK       # nothing to do

def test_default_workgroups_rejects_bad_arguments_on_host():
    L = lbsa.lib()
    out = ctypes.c_int32()
    assert L.lbsa_default_workgroups(0, 0, 3, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT     # q_len 3
    assert L.lbsa_default_workgroups(0, 0, 0, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_default_workgroups(0, 7, 1, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT     # kv dtype
    assert L.lbsa_default_workgroups(0, 0, 1, None) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_auto_workgroups(0, 0, 1, 0, 1000, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT    # no KV head
    assert L.lbsa_auto_workgroups(0, 0, 1, 8, -1, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT      # tiles
    assert L.lbsa_auto_workgroups(0, 0, 3, 8, 1000, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT    # q_len
    assert L.lbsa_auto_workgroups(0, 0, 1, 8, 1000, None) == lbsa.ERR_INVALID_ARGUMENT


def test_timing_hook_arms_and_disarms_without_a_gpu():
    """The hook only stores the two handles for the next launch on this
    thread; disarming it is a host-only call."""
    L = lbsa.lib()
    assert L.lbsa_time_next_kernel(None, None) == 0
    lbsa.time_next_kernel(None, None)
    vp = ctypes.c_void_p
    arr = (vp * 9)()
    assert L.lbsa_time_next_kernels(0, None, None) == 0
    assert L.lbsa_time_next_kernels(9, arr, arr) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_time_next_kernels(-1, arr, arr) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_time_next_kernels(2, None, arr) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_time_next_kernels(2, arr, arr) == 0       # NULL events: armed, nothing stamped
    lbsa.time_next_kernels([])


def test_varlen_map_layout_and_workspace():
    """Query-block maps (24 positions per block): 32-byte descriptors for
    Hkv * (B + total_q / 24) + P slots, their partial-slot words and claim order,
    every array after them; the workspace: 8 claim and P arrival counters, then
    2 P partial slots of 24 * 8 = 192 rows."""
    for B, Hkv, P, tq in [(2, 1, 4, 21), (64, 8, 512, 8255), (1, 8, 512, 8192)]:
        lay = lbsa.varlen_task_map_layout(B, Hkv, P, tq)
        nq = B + tq // lbsa.QBLOCK
        S, cap = Hkv * nq, Hkv * nq + P
        assert lay["header"] == 0 and lay["bin_desc_begin"] == 64
        assert lay["desc"] % 32 == 0 and lay["desc"] >= 64 + 4 * (P + 1)
        assert lay["desc_slot"] == lay["desc"] + 32 * cap
        assert lay["claim_order"] == lay["desc_slot"] + 4 * cap
        assert lay["seg_first_desc"] == lay["claim_order"] + 4 * cap
        assert lay["seg_num_chunks"] == lay["seg_first_desc"] + 4 * S
        assert lay["seg_slot0"] == lay["seg_num_chunks"] + 4 * S
        assert lay["blk_req"] == lay["seg_slot0"] + 4 * S and lay["blk_k"] == lay["blk_req"] + 4 * nq
        assert lay["qbase"] == lay["blk_k"] + 4 * nq and lay["qstart"] == lay["qbase"] + 4 * (B + 1)
        assert lay["seqlens"] == lay["qstart"] + 4 * (B + 1) and lay["qlens"] == lay["seqlens"] + 4 * B
        assert lay["total"] >= lay["qlens"] + 4 * B and lay["total"] % 256 == 0
        assert lbsa.varlen_task_map_bytes(B, Hkv, P, tq) == lay["total"]
    for P in (1, 512, 1000):
        counters = -(-4 * (8 + P) // 256) * 256            # 8 claim + P arrival counters, 256-aligned
        rows = 8 * lbsa.QBLOCK
        lse = -(-2 * P * rows * 4 // 256) * 256
        assert lbsa.varlen_workspace_bytes(64, 8, P) == counters + lse + 2 * P * rows * 128 * 4


def test_varlen_host_argument_errors():
    L = lbsa.lib()
    vp, sz = ctypes.c_void_p, ctypes.c_size_t()
    assert L.lbsa_varlen_task_map_bytes(4, 1, 32, 3, ctypes.byref(sz)) == lbsa.ERR_INVALID_ARGUMENT   # total_q < B
    assert L.lbsa_varlen_task_map_bytes(1, 8, 512, 1 << 20, ctypes.byref(sz)) == lbsa.ERR_UNSUPPORTED  # LDS
    ok = dict(sl=vp(16), ql=vp(32), B=2, Hq=8, Hkv=1, page=64, mp=4, tq=21, P=4, F=0, map=vp(256), nb=1 << 20)

    def plan(**kw):
        a = dict(ok, **kw)
        return L.lbsa_plan_varlen(a["sl"], a["ql"], a["B"], a["Hq"], a["Hkv"], a["page"], a["mp"], a["tq"], a["P"],
                                  a["F"], a["map"], a["nb"], None)
    assert plan(ql=None) == lbsa.ERR_INVALID_ARGUMENT
    assert plan(nb=64) == lbsa.ERR_INVALID_ARGUMENT                 # map too small
    assert plan(page=32) == lbsa.ERR_UNSUPPORTED
    assert plan(map=vp(272)) == lbsa.ERR_INVALID_ARGUMENT           # 32-byte descriptors need 32-byte alignment

    def attend(**kw):
        a = dict(q=vp(256), k=vp(256), v=vp(256), pt=vp(256), B=2, Hq=8, Hkv=1, D=128, page=64, mp=4, np_=8, tq=21,
                 P=4, sc=0.088, map=vp(256), mb=1 << 20, ws=vp(256), wb=1 << 30, out=vp(256))
        a.update(kw)
        return L.lbsa_attend_varlen(a["q"], a["k"], a["v"], a["pt"], a["B"], a["Hq"], a["Hkv"], a["D"], a["page"],
                                    a["mp"], a["np_"], a["tq"], a["P"], a["sc"], a["map"], a["mb"], a["ws"], a["wb"],
                                    a["out"], None)
    assert attend(sc=0.0) == lbsa.ERR_INVALID_ARGUMENT
    assert attend(wb=1024) == lbsa.ERR_INVALID_ARGUMENT              # workspace too small
    assert attend(out=None) == lbsa.ERR_INVALID_ARGUMENT
    assert attend(D=64) == lbsa.ERR_UNSUPPORTED


def test_query_block_size_matches_the_header():
    """The binding's query-block size is the public header's LBSA_QBLOCK (the
    library asserts the same of its own constant at compile time)."""
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "lbsa.h")).read()
    assert int(re.search(r"#define LBSA_QBLOCK (\d+)", hdr).group(1)) == lbsa.QBLOCK


def test_varlen_auto_workgroups_argument_errors():
    """Rejected on the host before any device query."""
    L = lbsa.lib()
    i32 = ctypes.c_int32
    q = (i32 * 2)(8192, 1)
    out = i32()
    assert L.lbsa_varlen_auto_workgroups(0, None, 2, 8, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_varlen_auto_workgroups(0, q, 0, 8, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_varlen_auto_workgroups(0, q, 2, 0, ctypes.byref(out)) == lbsa.ERR_INVALID_ARGUMENT
    assert L.lbsa_varlen_auto_workgroups(0, q, 2, 8, None) == lbsa.ERR_INVALID_ARGUMENT
