"""Seeded synthetic decode batches (inputs only; none of the method's arithmetic).

The workloads are the mixed-length decode batches the HPC-Ops posts measure on:
Table 3 of the vLLM integration post ("Decode latency (ms) across KV-length
distributions") labels a batch ``A x B`` = A requests at KV length B, and the
"Attention" sections of both posts describe batches that mix short and very long
live KV lengths.  The shapes are the Hy3 per-GPU share (8 query heads, 1 KV
head) and the full Hy3 attention (64 query heads, 8 KV heads), head_dim 128,
page size 64 (serving flags quoted in the SGLang post's launch example).

Every draw comes from one ``torch.Generator`` seeded per workload, in this
order: sequence lengths -> physical page permutation -> Q -> K -> V.

* values ~ N(0, 1) in fp32, then bf16 (round to nearest even), or, for the fp8
  path, per (token, head): scale = max|x| / 448, x8 = e4m3fn(x / scale);
* the page pool holds exactly sum_b ceil(L_b / 64) pages; ``page_table[b]`` is
  request b's slice of a random permutation of the pool; unused entries are -1;
* tail slots past L_b in a request's last page hold NaN (``tail="nan"``, parity
  runs: they must never reach the output) or N(0, 1) (``tail="normal"``).

Layouts: q [B, Hq, D] (or [B, q_len, Hq, D] with q_len > 1 query tokens per
request, multi-token decode); k_cache / v_cache [pages, 64, Hkv, D] (token-major);
k_scale / v_scale [pages, Hkv, 64] fp32; q_scale [B, Hq] (or [B, q_len, Hq]) fp32; page_table
[B, max_pages] int32; seqlens [B] int32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

TILE = 64
HEAD_DIM = 128
FP8_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_heads: int
    num_kv_heads: int
    kv_dtype: str                    # "bf16" | "fp8"
    seqlens: tuple = ()              # explicit lengths, or
    batch: int = 0                   # with a random distribution:
    dist: tuple = ()                 # ("loguniform", a, b) | ("uniform_int", a, b)
    num_workgroups: int = 0          # 0 = library default (CUs x occupancy)
    head_dim: int = HEAD_DIM
    q_len: int = 1                   # query tokens per request (> 1: multi-token decode)
    note: str = ""
    extra: dict = field(default_factory=dict)


def _mix(*parts):
    out = []
    for count, length in parts:
        out += [length] * count
    return tuple(out)


WORKLOADS = {
    # parity case: the oracle finishes it in well under a second
    "tiny": Workload("tiny", 0, 8, 1, "bf16", seqlens=(37, 64, 1000, 4097), num_workgroups=32,
                     note="batch 4, 8/1 heads, bf16, 32 persistent workgroups"),
    # one GPU's share of Hy3 at TP8: 8 query heads, 1 KV head
    "tp8_share": Workload("tp8_share", 1, 8, 1, "bf16", batch=32, dist=("loguniform", 1024, 32768),
                          note="batch 32, 8/1 heads, L log-uniform in [1K, 32K], bf16"),
    # skewed tail: 63 short requests and one 128K request, full 64/8 heads
    "skewed": Workload("skewed", 2, 64, 8, "bf16", seqlens=_mix((63, 512), (1, 131072)),
                       note="63 x 512 + 1 x 131072, 64/8 heads, bf16"),
    "fp8": Workload("fp8", 3, 64, 8, "fp8", batch=64, dist=("loguniform", 1024, 65536),
                    note="batch 64, 64/8 heads, L log-uniform in [1K, 64K], e4m3fn K/V/Q"),
    "long": Workload("long", 4, 64, 8, "bf16", batch=8, dist=("uniform_int", 65536, 262144),
                     note="batch 8, 64/8 heads, L uniform in [64K, 256K], bf16"),
    "floor": Workload("floor", 5, 64, 8, "bf16", seqlens=(200,),
                      note="batch 1, 200 tokens, 64/8 heads: the minimum-work floor binds"),
}

# The six KV-length mixes of the vLLM post's Table 3 (FP8 KV), at the per-GPU
# Hy3 share of 8 query heads / 1 KV head.
TABLE3 = {
    "t3_64x0.5K": _mix((64, 512)),
    "t3_64x4K": _mix((64, 4096)),
    "t3_32x0.125K+32x4K": _mix((32, 128), (32, 4096)),
    "t3_2x32K+30x4K": _mix((2, 32768), (30, 4096)),
    "t3_1x64K+15x4K": _mix((1, 65536), (15, 4096)),
    "t3_1x128K+31x4K": _mix((1, 131072), (31, 4096)),
}
for _i, (_name, _lens) in enumerate(TABLE3.items()):
    WORKLOADS[_name] = Workload(_name, 10 + _i, 8, 1, "fp8", seqlens=_lens,
                                note="vLLM post Table 3 mix, 8/1 heads, fp8")


def draw_seqlens(w: Workload, gen: torch.Generator) -> torch.Tensor:
    """Sequence lengths of workload ``w`` (first draw of its generator)."""
    if w.seqlens:
        return torch.tensor(w.seqlens, dtype=torch.int32)
    kind, a, b = w.dist
    if kind == "loguniform":
        u = torch.rand(w.batch, dtype=torch.float64, generator=gen)
        x = torch.exp(math.log(a) + u * (math.log(b) - math.log(a)))
        return torch.floor(x).clamp(a, b).to(torch.int32)
    if kind == "uniform_int":
        return torch.randint(a, b + 1, (w.batch,), generator=gen, dtype=torch.int64).to(torch.int32)
    raise ValueError(f"unknown length distribution {kind!r}")


def _normal(shape, gen, device, chunk_rows=1 << 14):
    """N(0,1) fp32 drawn in row chunks (bounds the fp32 temporaries)."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device)
    return out


def _to_fp8(x: torch.Tensor):
    """Per-row (last dim) e4m3fn quantisation: returns (codes, scale)."""
    amax = x.abs().amax(dim=-1).clamp_min(1e-30)
    scale = (amax / FP8_MAX).to(torch.float32)
    q = (x / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q, scale


def make_batch(w: Workload | str | None = None, *, seqlens=None, num_heads=None, num_kv_heads=None,
               kv_dtype=None, seed=None, tail: str = "nan", device="cpu", max_pages=None,
               head_dim=HEAD_DIM, q_len=None, qlens=None) -> dict:
    """Build one synthetic decode batch.

    Either pass a workload (object or name) or explicit ``seqlens`` with
    ``num_heads``, ``num_kv_heads``, ``kv_dtype`` and ``seed``.  ``q_len``
    (default: the workload's, 1) query tokens per request.  ``qlens`` (one per
    request) instead gives each request its own number of new tokens, and q is
    packed [sum(qlens), Hq, D] in request order (a prefill / extend / decode
    mix).  Returns a dict of tensors on ``device`` plus scalar metadata.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w is None:
        w = Workload("custom", int(seed or 0), int(num_heads), int(num_kv_heads), kv_dtype or "bf16",
                     seqlens=tuple(int(x) for x in seqlens), head_dim=head_dim)
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    gen_cpu = gen if dev.type == "cpu" else torch.Generator().manual_seed(w.seed)

    sl = draw_seqlens(w, gen_cpu)
    B, Hq, Hkv, D = int(sl.numel()), w.num_heads, w.num_kv_heads, w.head_dim
    QL = int(q_len or w.q_len)
    n = (sl.to(torch.int64) + TILE - 1) // TILE
    n_pages = int(n.sum())
    pool = max(1, n_pages)
    perm = torch.randperm(pool, generator=gen_cpu).to(torch.int32)
    mp = int(max_pages) if max_pages is not None else max(1, int(n.max()) if B else 1)
    pt = torch.full((B, mp), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        nb = int(n[b])
        pt[b, :nb] = perm[off:off + nb]
        off += nb

    if qlens is not None:
        qlens = torch.tensor([int(x) for x in qlens], dtype=torch.int32)
        assert qlens.numel() == B
        q32 = _normal((int(qlens.sum()), Hq, D), gen, dev)
    else:
        q32 = _normal((B, Hq, D) if QL == 1 else (B, QL, Hq, D), gen, dev)
    k32 = _normal((pool, TILE, Hkv, D), gen, dev)
    k_cache, k_scale = _finish_cache(k32, w.kv_dtype)
    del k32
    v32 = _normal((pool, TILE, Hkv, D), gen, dev)
    v_cache, v_scale = _finish_cache(v32, w.kv_dtype)
    del v32
    if w.kv_dtype == "bf16":
        q, q_scale = q32.to(torch.bfloat16), None
    else:
        q, q_scale = _to_fp8(q32)
    del q32

    if tail == "nan":
        _poison_tails(sl, pt, k_cache, v_cache, k_scale, v_scale)
    elif tail != "normal":
        raise ValueError("tail must be 'nan' or 'normal'")

    return {
        "name": w.name, "seed": w.seed, "kv_dtype": w.kv_dtype,
        "q": q, "q_scale": q_scale, "k_cache": k_cache, "v_cache": v_cache,
        "k_scale": k_scale, "v_scale": v_scale,
        "page_table": pt.to(dev), "seqlens": sl.to(dev),
        "B": B, "num_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "q_len": QL,
        "max_pages": mp, "num_pages": pool,
        "softmax_scale": 1.0 / math.sqrt(D),
        "num_workgroups": w.num_workgroups,
        "qlens": None if qlens is None else qlens.to(dev),
    }


# A prefill / extend / decode mix on one map: request 0 extends an 8K-token
# context by 8K new tokens (the vLLM post's Table 4 extend rows, at q8k's
# length), 63 decode requests of log-uniform 1K-16K tokens beside it, full Hy3
# attention (64 query / 8 KV heads), bf16.
MIXED_EXTEND = dict(extend_len=16384, extend_q=8192, decode_rows=63, decode_lo=1024, decode_hi=16384, seed=90)


def mixed_extend_lengths(extend_len=16384, extend_q=8192, decode_rows=63, decode_lo=1024, decode_hi=16384,
                         seed=90):
    """(seqlens, qlens) of the mix: the extend request first, then the decode rows."""
    gen = torch.Generator().manual_seed(seed)
    u = torch.rand(decode_rows, generator=gen, dtype=torch.float64)
    dec = torch.exp(math.log(decode_lo) + u * (math.log(decode_hi) - math.log(decode_lo))).floor()
    dec = dec.clamp(decode_lo, decode_hi).to(torch.int64).tolist()
    return [int(extend_len)] + [int(x) for x in dec], [int(extend_q)] + [1] * decode_rows


def make_mixed_extend_batch(tail: str = "normal", device="cpu", **kw) -> dict:
    """Seeded batch of the mix (q packed [8192 + 63, 64, 128])."""
    cfg = dict(MIXED_EXTEND, **kw)
    sl, ql = mixed_extend_lengths(**cfg)
    return make_batch(seqlens=sl, qlens=ql, num_heads=64, num_kv_heads=8, kv_dtype="bf16", seed=cfg["seed"],
                      tail=tail, device=device)


def _finish_cache(x32: torch.Tensor, kv_dtype: str):
    """fp32 [pages, 64, Hkv, D] -> (cache, scale [pages, Hkv, 64] or None)."""
    if kv_dtype == "bf16":
        return x32.to(torch.bfloat16), None
    if kv_dtype != "fp8":
        raise ValueError("kv_dtype must be 'bf16' or 'fp8'")
    codes, scale = _to_fp8(x32)                       # scale [pages, 64, Hkv]
    return codes, scale.permute(0, 2, 1).contiguous()


def _poison_tails(sl, pt, k_cache, v_cache, k_scale, v_scale):
    """NaN in every slot past L_b of request b's last page."""
    for b in range(int(sl.numel())):
        L = int(sl[b])
        if L % TILE == 0:
            continue
        page = int(pt[b, L // TILE])
        s0 = L % TILE
        for cache in (k_cache, v_cache):
            if cache.dtype == torch.bfloat16:
                cache[page, s0:] = float("nan")
            else:
                cache.view(torch.uint8)[page, s0:] = 0x7F      # e4m3fn NaN code
        for sc in (k_scale, v_scale):
            if sc is not None:
                sc[page, :, s0:] = float("nan")


# ---------------------------------------------------------------------------
# inputs of the fused attention prologue (random draws only)
# ---------------------------------------------------------------------------

# The attention shapes of the vLLM post's Table 4 ("Attention latency (ms) vs
# FlashAttention, Triton and FlashInfer"), read as (batch, q_len new tokens per
# request, L cached tokens per request including the new ones): "q512" is a
# 512-token prefill, "q1ks2k" 1K new tokens over a 2K sequence, "8q1s1k" 8
# decode requests at 1K.  Full Hy3 attention: 64 query / 8 KV heads, bf16.
TABLE4 = {
    "q512": ("prefill", 1, 512, 512),
    "q1ks2k": ("extend", 1, 1024, 2048),
    "q2k": ("prefill", 1, 2048, 2048),
    "q4k": ("prefill", 1, 4096, 4096),
    "q8k": ("prefill", 1, 8192, 8192),
    "2q1ks4k": ("extend", 2, 1024, 4096),
    "8q1s1k": ("decode", 8, 1, 1024),
    "16q1s2k": ("decode", 16, 1, 2048),
    "32q1s1k": ("decode", 32, 1, 1024),
    "64q1s4k": ("decode", 64, 1, 4096),
}


def make_table4_batch(name: str, tail: str = "normal", device="cpu", seed: int = 80) -> dict:
    """Seeded batch of one Table 4 shape (q [B, q_len, Hq, D] for prefill / extend)."""
    kind, B, QL, L = TABLE4[name]
    return make_batch(seqlens=[L] * B, num_heads=64, num_kv_heads=8, kv_dtype="bf16", seed=seed, tail=tail,
                      device=device, q_len=None if kind == "decode" else QL)


PROLOGUE_WORKLOADS = {
    # decode step of the tp8_share batch: one new token per request
    "decode_8_1": dict(tokens=32, num_heads=8, num_kv_heads=1, kv_dtype="bf16", seed=31),
    # decode step of the full 64/8-head model, fp8 cache
    "decode_64_8_fp8": dict(tokens=64, num_heads=64, num_kv_heads=8, kv_dtype="fp8", seed=32),
    # a prefill chunk: 8192 tokens, 64/8 heads
    "prefill_64_8": dict(tokens=8192, num_heads=64, num_kv_heads=8, kv_dtype="bf16", seed=33),
    "prefill_64_8_fp8": dict(tokens=8192, num_heads=64, num_kv_heads=8, kv_dtype="fp8", seed=34),
}


def make_prologue_inputs(tokens: int, num_heads: int, num_kv_heads: int, kv_dtype: str = "bf16", seed: int = 0,
                         num_pages: int | None = None, max_position: int = 262143, padding: int = 0,
                         zero_heads: int = 0, magnitude: float = 16.0, device="cpu") -> dict:
    """Seeded inputs of the prologue.

    * qkv bf16 [T, (Hq + 2 Hkv) * 128] ~ N(0, 1) times a per-(token, head)
      magnitude log-uniform in [1/magnitude, magnitude]; ``zero_heads`` head
      vectors are zero;
    * positions int32 uniform in [0, max_position];
    * slot_mapping int64: distinct random slots of a pool of ``num_pages`` pages
      (default: just enough), the last ``padding`` tokens get -1;
    * norm weights fp32 ~ 1 + 0.2 N(0, 1);
    * caches pre-filled with random contents (bf16 N(0, 1), or fp8 codes that
      are not NaN and scales in [0.5, 2)), so a write to a wrong slot shows.
    """
    gen = torch.Generator().manual_seed(seed)
    D, NV = HEAD_DIM, num_heads + 2 * num_kv_heads
    mag = torch.exp(math.log(magnitude) * (2 * torch.rand((tokens, NV, 1), generator=gen, dtype=torch.float64) - 1))
    x = torch.randn((tokens, NV, D), generator=gen, dtype=torch.float64) * mag
    if zero_heads:
        idx = torch.randperm(tokens * NV, generator=gen)[:zero_heads]
        x.view(tokens * NV, D)[idx] = 0.0
    qkv = x.to(torch.float32).to(torch.bfloat16).reshape(tokens, NV * D)
    positions = torch.randint(0, max_position + 1, (tokens,), generator=gen, dtype=torch.int64).to(torch.int32)
    pages = num_pages or max(1, (tokens + TILE - 1) // TILE + 2)
    slots = torch.randperm(pages * TILE, generator=gen)[:tokens].to(torch.int64)
    if padding:
        slots[tokens - padding:] = -1
    qw = (1.0 + 0.2 * torch.randn(D, generator=gen, dtype=torch.float64)).to(torch.float32)
    kw = (1.0 + 0.2 * torch.randn(D, generator=gen, dtype=torch.float64)).to(torch.float32)
    shape = (pages, TILE, num_kv_heads, D)
    if kv_dtype == "bf16":
        k_cache = torch.randn(shape, generator=gen).to(torch.bfloat16)
        v_cache = torch.randn(shape, generator=gen).to(torch.bfloat16)
        k_scale = v_scale = None
    elif kv_dtype == "fp8":
        codes = torch.randint(0, 256, (2,) + shape, generator=gen, dtype=torch.int64).to(torch.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x7E                      # no NaN codes
        k_cache, v_cache = codes[0].view(torch.float8_e4m3fn), codes[1].view(torch.float8_e4m3fn)
        k_scale = 0.5 + 1.5 * torch.rand((pages, num_kv_heads, TILE), generator=gen)
        v_scale = 0.5 + 1.5 * torch.rand((pages, num_kv_heads, TILE), generator=gen)
    else:
        raise ValueError("kv_dtype must be 'bf16' or 'fp8'")
    out = {"qkv": qkv, "positions": positions, "slot_mapping": slots, "q_weight": qw, "k_weight": kw,
           "k_cache": k_cache.contiguous(), "v_cache": v_cache.contiguous(), "k_scale": k_scale,
           "v_scale": v_scale, "num_heads": num_heads, "num_kv_heads": num_kv_heads, "kv_dtype": kv_dtype,
           "tokens": tokens, "num_pages": pages, "theta": 10000.0, "eps": 1e-6}
    for k, v in list(out.items()):
        if isinstance(v, torch.Tensor):
            out[k] = v.to(device)
    return out
