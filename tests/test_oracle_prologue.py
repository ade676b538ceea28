"""Pins of the prologue oracle (QK-Norm -> RoPE -> Q output / fp8 quantisation).

Each function is checked against something that is not itself: a library
routine (torch's rms_norm, its bf16 and float8_e4m3fn conversions), an
independent formulation (RoPE as multiplication by a unit complex number),
closed forms and invariants.  The pages fix the order: QK-Norm before RoPE
(vLLM post, "A fused attention prologue"; SGLang post, the attention prologue
section).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O

D = 128


def rng(seed):
    return np.random.default_rng(seed)


def test_rmsnorm_matches_torch():
    for seed, rows, eps in ((0, 5, 1e-6), (1, 3, 1e-5), (2, 1, 0.0)):
        x = rng(seed).standard_normal((rows, D)) * rng(seed + 10).uniform(0.01, 30)
        w = rng(seed + 20).standard_normal(D)
        ref = torch.nn.functional.rms_norm(torch.tensor(x), (D,), torch.tensor(w), eps).numpy()
        np.testing.assert_allclose(O.rmsnorm(x, w, eps), ref, rtol=1e-12, atol=1e-12)


def test_rmsnorm_closed_forms():
    w = rng(3).standard_normal(D)
    for c in (2.0, -0.5, 7.0):
        y = O.rmsnorm(np.full(D, c), w, 0.0)
        np.testing.assert_allclose(y, w * np.sign(c), rtol=1e-13)       # x / rms(x) = sign(c)
    x = rng(4).standard_normal(D)
    np.testing.assert_allclose(O.rmsnorm(3.7 * x, w, 0.0), O.rmsnorm(x, w, 0.0), rtol=1e-12)  # scale-free


def test_rope_is_identity_at_position_zero():
    x = rng(5).standard_normal((4, D))
    np.testing.assert_array_equal(O.rope(x, 0, 10000.0), x)


@pytest.mark.parametrize("theta", [10000.0, 1e6])
def test_rope_matches_complex_rotation(theta):
    """Rotating the pairs (d, d + D/2) is multiplying x_d + i x_{d+D/2} by e^{i a_d}."""
    x = rng(6).standard_normal((6, D))
    pos = np.array([0, 1, 7, 300, 65535, 262143], np.float64)
    z = x[:, :D // 2] + 1j * x[:, D // 2:]
    freq = theta ** (-np.arange(D // 2) * 2.0 / D)
    zr = z * np.exp(1j * pos[:, None] * freq[None, :])
    got = O.rope(x, pos, theta)
    np.testing.assert_allclose(got[:, :D // 2], zr.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(got[:, D // 2:], zr.imag, rtol=0, atol=1e-9)


def test_rope_invariants():
    q, k = rng(7).standard_normal(D), rng(8).standard_normal(D)
    th = 10000.0
    # rotation keeps every pair's length
    r = O.rope(q, 1234, th)
    np.testing.assert_allclose(r[:64] ** 2 + r[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)
    # q.k after rotation depends only on the position difference
    a = O.rope(q, 100, th) @ O.rope(k, 40, th)
    b = O.rope(q, 5060, th) @ O.rope(k, 5000, th)
    np.testing.assert_allclose(a, b, rtol=1e-9)
    # unit vector e_0 at angle pos (frequency 1 for d = 0)
    e = np.zeros(D)
    e[0] = 1.0
    y = O.rope(e, 3, th)
    assert abs(y[0] - np.cos(3)) < 1e-14 and abs(y[64] - np.sin(3)) < 1e-14


def test_quant_e4m3_matches_torch_conversion():
    for seed in range(4):
        x = rng(seed).standard_normal((8, D)) * rng(seed + 5).uniform(1e-3, 1e3, (8, 1))
        codes, scale = O.quant_e4m3(x)
        np.testing.assert_allclose(scale, np.abs(x).max(axis=1) / 448.0, rtol=1e-15)
        ref = torch.tensor(x / scale[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(codes, ref)
        # the largest |x| of a row lands exactly on +-448 (code 0x7E)
        am = np.abs(x).argmax(axis=1)
        assert ((codes[np.arange(8), am] & 0x7F) == 0x7E).all()


def test_quant_e4m3_zero_row():
    codes, scale = O.quant_e4m3(np.zeros((1, D)))
    assert scale[0] == 1.0 and (codes == 0).all()


def test_quant_e4m3_error_bound():
    x = rng(9).standard_normal((16, D))
    codes, scale = O.quant_e4m3(x)
    deq = O.e4m3_values(codes) * scale[:, None]
    # half an e4m3 step: 2^-4 relative for normals, 2^-10 of the scale below 2^-6
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale[:, None] * 2.0 ** -10)
    assert (np.abs(deq - x) <= bound * (1 + 1e-12)).all()


def test_bf16_nearest_matches_torch():
    x = np.concatenate([rng(10).standard_normal(500) * 10.0 ** rng(11).uniform(-8, 8, 500),
                        [0.0, -0.0, 1.0, -2.0, 3.0e38, 1e-40]])
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_nearest(x), ref)
    # exact ties go to the even code: 1 + 2^-8 is halfway between 0x3F80 and 0x3F81
    assert O.bf16_nearest(1.0 + 2.0 ** -8) == 0x3F80
    assert O.bf16_nearest(1.0 + 3 * 2.0 ** -8) == 0x3F82


def test_prologue_composition_and_order():
    Hq, Hkv, T = 8, 1, 5
    x = rng(12).standard_normal((T, (Hq + 2 * Hkv) * D)).astype(np.float32)
    bits = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vals = O.bf16_values(bits).reshape(T, Hq + 2 * Hkv, D)
    pos = np.array([0, 3, 64, 1000, 262143], np.int32)
    qw, kw = 1.0 + 0.3 * rng(13).standard_normal(D), 1.0 + 0.3 * rng(14).standard_normal(D)
    q, k, v = O.prologue(bits, pos, qw, kw, Hq, Hkv, 10000.0, 1e-6)
    # V passes through; Q and K are normalised, then rotated
    np.testing.assert_array_equal(v, vals[:, Hq + Hkv:])
    np.testing.assert_allclose(q, O.rope(O.rmsnorm(vals[:, :Hq], qw, 1e-6), np.repeat(pos, Hq), 10000.0),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(k, O.rope(O.rmsnorm(vals[:, Hq:Hq + Hkv], kw, 1e-6), pos, 10000.0),
                               rtol=0, atol=1e-12)
    # the order matters with a non-uniform weight: RoPE first would give something else
    other = O.rmsnorm(O.rope(vals[1:, :Hq], np.repeat(pos[1:], Hq), 10000.0), qw, 1e-6)
    assert np.abs(other - q[1:]).max() > 1e-3
    # position 0: QK-Norm only
    np.testing.assert_allclose(q[0], O.rmsnorm(vals[0, :Hq], qw, 1e-6), rtol=0, atol=1e-12)
