"""Plain fp64 oracle of the split-bf16 router GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library.

Source: the SGLang post, section "Router GEMM: balancing routing precision and
throughput" (the router projects hidden states to expert scores; fp32 router
weights are kept for top-k fidelity).  The method splits each fp32 weight into
two bf16 parts:

* W_high: the bf16 obtained by direct truncation of the fp32 weight;
* W_low: the bf16 of the scaled residual (W - W_high) * 256,

so that W ~ W_high + W_low / 256 and the product X W^T becomes two bf16 GEMMs
whose fp32 partial results are combined with the 1/256 correction in the
epilogue; the output is fp32 router scores.

Readings taken where the page is silent (listed with reasons in the design
notes of the repository):
* G1  the weight is laid out [N][K] (one row per expert, as a linear layer
      stores it) and the scores are [M][N] = X [M][K] times W^T;
* G2  the residual's conversion to bf16 rounds to nearest, ties to even (the
      page says "truncation" only for W_high);
* G3  bf16 inputs X are used as they are (their values are exact in fp64).

Every function computes in fp64 (numpy); numbers formats come from their bit
definitions here.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their values: the upper half of an fp32."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_truncate_to_bf16(w) -> np.ndarray:
    """W_high bits: the fp32 pattern with its low 16 mantissa bits dropped
    (truncation toward zero of the magnitude)."""
    u = np.ascontiguousarray(np.asarray(w, np.float32)).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def f64_to_bf16_rne(x) -> np.ndarray:
    """bf16 bits nearest to x (finite, within bf16 range), ties to the even
    pattern.  x is first rounded to fp32 exactly when it already is an fp32
    value (the scaled residuals are: they keep at most 16 significant bits)."""
    x32 = np.asarray(x, np.float64).astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, np.float64)), "input must be fp32-exact"
    u = np.ascontiguousarray(x32).view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + round_up.astype(np.uint64)).astype(np.uint16)


def split_weights(w):
    """(W_high bits, W_low bits), both uint16 [N][K], from fp32 weights [N][K]."""
    w32 = np.asarray(w, np.float32)
    hi = f32_truncate_to_bf16(w32)
    resid = w32.astype(np.float64) - bf16_bits_to_f64(hi)       # exact: the dropped mantissa bits
    lo = f64_to_bf16_rne(resid * 256.0)                          # exact scaling by a power of two
    return hi, lo


def router_gemm(x_bits, hi, lo):
    """Scores [M][N] of the split form: X W_high^T + (X W_low^T) / 256, fp64."""
    x = bf16_bits_to_f64(x_bits)
    return x @ bf16_bits_to_f64(hi).T + (x @ bf16_bits_to_f64(lo).T) / 256.0


def router_exact(x_bits, w):
    """Scores [M][N] with the fp32 weights themselves: X W^T, fp64."""
    return bf16_bits_to_f64(x_bits) @ np.asarray(w, np.float32).astype(np.float64).T
