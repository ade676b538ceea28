"""Pins of the split-bf16 router GEMM oracle.

SGLang post, section "Router GEMM: balancing routing precision and
throughput": W_high is the bf16 truncation of the fp32 weight, W_low the bf16
of (W - W_high) * 256, and the scores are X W_high^T + X W_low^T / 256.

Pins, independent of the oracle's code:
* W_high: bf16-representable, same sign, never larger in magnitude, within one
  bf16 step of W; a weight that already is a bf16 value splits into (W, 0);
* W_low: torch's own bf16 conversion of the fp32 residual times 256;
* the reconstruction W_high + W_low / 256 is within 2^-16 |W| of W (closed
  form: the residual is below one bf16 step, its bf16 rounding loses 2^-9 of
  it), and a wrong scale (128 or 512) breaks that bound;
* the GEMM: brute-force Python sums on a tiny case, and the exact fp32-weight
  product within the bound sum_k |x_k| 2^-16 |w_k|.
"""
import numpy as np
import torch

from oracle import router_oracle as R


def rng(seed):
    return np.random.default_rng(seed)


def weights(seed, shape, scale=0.02):
    w = (rng(seed).standard_normal(shape) * scale).astype(np.float32)
    w.flat[:7] = [0.0, -0.0, 1.0, -3.5, 1e-30, 3.0e38, -2.0 ** -126]        # special values
    return w


def test_high_part_is_the_truncation():
    w = weights(0, (64, 96))
    hi, _ = R.split_weights(w)
    h = R.bf16_bits_to_f64(hi)
    wd = w.astype(np.float64)
    # bf16-representable: converting back through torch changes nothing
    assert np.array_equal(torch.tensor(h.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64), h)
    assert (np.signbit(h) == np.signbit(wd)).all()
    assert (np.abs(h) <= np.abs(wd)).all()
    # within one bf16 step (2^(e - 7) for |w| in [2^e, 2^(e+1))) of w
    step = 2.0 ** (np.floor(np.log2(np.abs(np.where(wd != 0, wd, 1.0)))) - 7)
    assert ((np.abs(wd - h) < step) | (wd == h)).all()
    assert (wd != h).any()


def test_bf16_weights_split_exactly():
    w = torch.randn(32, 64, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).float().numpy()
    hi, lo = R.split_weights(w)
    np.testing.assert_array_equal(R.bf16_bits_to_f64(hi), w.astype(np.float64))
    assert (lo & 0x7FFF == 0).all()                              # +0 (or -0)


def test_low_part_matches_torch_conversion():
    w = weights(2, (48, 128))
    hi, lo = R.split_weights(w)
    resid = (torch.tensor(w) - torch.tensor(R.bf16_bits_to_f64(hi).astype(np.float32))) * 256.0
    ref = resid.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(lo, ref)


def test_reconstruction_bound_and_scale():
    w = weights(3, (40, 200), scale=1.0)
    hi, lo = R.split_weights(w)
    wd = w.astype(np.float64)
    rec = R.bf16_bits_to_f64(hi) + R.bf16_bits_to_f64(lo) / 256.0
    assert (np.abs(rec - wd) <= np.abs(wd) * 2.0 ** -16).all()
    for wrong in (128.0, 512.0):
        bad = R.bf16_bits_to_f64(hi) + R.bf16_bits_to_f64(lo) / wrong
        assert (np.abs(bad - wd) > np.abs(wd) * 2.0 ** -16).any()
    # the split keeps far more of W than one bf16 rounding does
    one = torch.tensor(w).to(torch.bfloat16).double().numpy()
    assert np.abs(rec - wd).max() < np.abs(one - wd).max() / 64


def test_gemm_brute_force_tiny():
    x = torch.randn(3, 5, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    w = weights(5, (4, 5), scale=1.0)
    w.flat[:7] = 0.25
    hi, lo = R.split_weights(w)
    got = R.router_gemm(xb, hi, lo)
    xv = [[float(v) for v in row] for row in x.float()]
    for m in range(3):
        for n in range(4):
            s = 0.0
            for k in range(5):
                wh = float(torch.tensor(int(hi[n, k]), dtype=torch.int32).to(torch.int16).view(torch.bfloat16))
                wl = float(torch.tensor(int(lo[n, k]), dtype=torch.int32).to(torch.int16).view(torch.bfloat16))
                s += xv[m][k] * wh + xv[m][k] * wl / 256.0
            assert abs(got[m, n] - s) <= 1e-12 * max(1.0, abs(s))


def test_gemm_close_to_exact_weights():
    x = torch.randn(16, 4096, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    w = (rng(7).standard_normal((192, 4096)) * 0.02).astype(np.float32)
    hi, lo = R.split_weights(w)
    got = R.router_gemm(xb, hi, lo)
    exact = R.router_exact(xb, w)
    bound = (np.abs(R.bf16_bits_to_f64(xb)) @ np.abs(w.astype(np.float64)).T) * 2.0 ** -16
    assert (np.abs(got - exact) <= bound).all()
    assert np.abs(got - exact).max() < 1e-4
