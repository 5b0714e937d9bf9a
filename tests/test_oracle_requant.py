"""Pins of the oracle's startup requantisation of Q8_0 weights (no GPU).

The review page, section "Compute shared evidence once": the Q8_0 weights
are requantised with SmoothQuant at startup.  Q8_0 keeps blocks of 32 int8
codes with one binary16 scale; SmoothQuant multiplies weight column k by the
smoothing value s_k that divides activation channel k.  Pinned against
exact-rational brute force, a closed form, numpy's binary16 conversion, the
rounding bound, and the purpose of smoothing: with outlier activation
channels, smoothing lowers the W8A8 error against the float64 product.
"""
from fractions import Fraction

import numpy as np
import pytest

import brute
import oracle


def _q8_0(seed, N, K, d_lo=1e-3, d_hi=1e-2):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, (N, K), dtype=np.int8)
    d = rng.uniform(d_lo, d_hi, (N, K // 32)).astype(np.float16)
    return q, d.view(np.uint16), rng


def _brute_row(q_row, d_row_bits, s):
    d = np.asarray(d_row_bits, np.uint16).view(np.float16).astype(np.float64)   # exact
    wp = [brute.round_f32(brute.round_f32(Fraction(float(d[k // 32])) * int(q_row[k])) * brute.f32(s[k]))
          for k in range(len(q_row))]
    amax = max(abs(v) for v in wp)
    sw = brute.round_f32(Fraction(amax) / 127)
    codes = []
    for v in wp:
        if sw == 0:
            codes.append(0)
            continue
        t = Fraction(brute.round_f32(Fraction(v) / Fraction(sw)))
        r = brute._round_half_even_int(abs(t)) * (1 if t >= 0 else -1)
        codes.append(max(-127, min(127, r)))
    return codes, sw


def test_requantize_matches_exact_rational_bruteforce():
    q, d, rng = _q8_0(1, 6, 128)
    s = rng.uniform(0.25, 8.0, 128).astype(np.float32)
    wq, sw = oracle.requantize_q8_0(q, d, s)
    for n in range(6):
        codes, swb = _brute_row(q[n], d[n], s)
        assert sw[n] == np.float32(swb), n
        assert list(wq[n]) == codes, n


def test_unit_smoothing_and_one_power_of_two_scale_give_back_the_codes():
    q, _, _ = _q8_0(2, 5, 256)
    q[:, 7] = 127                                  # every row reaches |q| = 127
    d = np.full((5, 8), 2.0 ** -7, np.float16).view(np.uint16)
    wq, sw = oracle.requantize_q8_0(q, d, np.ones(256, np.float32))
    assert np.array_equal(wq, q)
    assert (sw == np.float32(2.0 ** -7)).all()


def test_binary16_scales_decode_exactly():
    bits = np.array([0x0001, 0x03ff, 0x0400, 0x3c00, 0x7bff, 0x8400, 0x1234, 0x5a5a], np.uint16)
    N, K = len(bits), 32
    q = np.zeros((N, K), np.int8)
    q[:, 0] = 1
    wq, sw = oracle.requantize_q8_0(q, bits.reshape(N, 1), np.ones(K, np.float32))
    d = bits.view(np.float16).astype(np.float32)
    want = np.abs(d) / np.float32(127)          # binary32 division, correctly rounded
    assert np.array_equal(sw.view(np.uint32), want.view(np.uint32))
    assert (wq[:, 0] == np.sign(d).astype(np.int8) * 127).all() and (wq[:, 1:] == 0).all()


def test_zero_rows_and_rounding_bound():
    q, d, rng = _q8_0(3, 20, 512)
    q[4] = 0
    s = rng.uniform(0.5, 4.0, 512).astype(np.float32)
    wq, sw = oracle.requantize_q8_0(q, d, s)
    assert sw[4] == 0 and (wq[4] == 0).all()
    dd = np.repeat(d.view(np.float16).astype(np.float64), 32, axis=1)
    wp = (dd * q) * s                               # within a rounding of w'
    err = np.abs(wq.astype(np.float64) * sw[:, None] - wp)
    assert (err <= sw[:, None].astype(np.float64) * (0.5 + 1e-5) + 1e-30).all()


def test_smoothing_lowers_the_w8a8_error_on_outlier_activations():
    # SmoothQuant's purpose: migrate activation outliers into the weights
    rng = np.random.default_rng(9)
    M, N, K = 64, 96, 512
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, 8, replace=False)] *= 60.0
    q, d, _ = _q8_0(4, N, K)
    w = np.repeat(d.view(np.float16).astype(np.float64), 32, axis=1) * q     # dequantised Q8_0
    ref = x.astype(np.float64) @ w.T
    err = {}
    for name, s in (("none", np.ones(K, np.float32)),
                    ("smoothquant", np.sqrt(np.abs(x).max(0) / np.abs(w).max(0)).astype(np.float32))):
        wq, sw = oracle.requantize_q8_0(q, d, s)
        xq, sx = oracle.quantize_act(x, s)
        y = oracle.gemm(xq, sx, wq, sw).astype(np.float64)
        err[name] = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert err["smoothquant"] < 0.5 * err["none"], err


def _nonfinite_rows(q, d_bits, s):
    """Rows whose smoothed weights d*q*s hold a NaN or an infinity (binary32)."""
    d = np.repeat(np.asarray(d_bits, np.uint16).view(np.float16).astype(np.float32), 32, axis=1)
    with np.errstate(invalid="ignore", over="ignore"):
        wp = (d * q.astype(np.float32)).astype(np.float32) * s
    return ~np.isfinite(wp).all(axis=1)


def test_rows_with_non_finite_smoothed_weights_have_no_scale():
    # the activations' rule for a row that cannot be quantised: sw = NaN and
    # every code 0; the other rows are untouched (exact-rational brute force)
    q, d, rng = _q8_0(11, 8, 128)
    d = d.copy()
    s = rng.uniform(0.5, 2.0, 128).astype(np.float32)
    d[0, 1] = 0x7e00                      # a NaN block scale
    d[1, 2] = 0x7c00                      # +inf with nonzero codes
    q[1, 64] = 5
    d[2, 3] = 0xfc00                      # -inf times all-zero codes: NaN
    q[2, 96:128] = 0
    d[3, 0] = 0x7bff                      # 65504 * 127 * 2^124: overflows binary32
    q[3, 5] = 127
    s[5] = np.float32(2.0 ** 124)
    wq, sw = oracle.requantize_q8_0(q, d, s)
    bad = _nonfinite_rows(q, d, s)
    assert list(bad) == [True, True, True, True, False, False, False, False]
    for n in range(8):
        if bad[n]:
            assert np.isnan(sw[n]) and not wq[n].any(), n
        else:
            codes, swb = _brute_row(q[n], d[n], s)
            assert sw[n] == np.float32(swb) and list(wq[n]) == codes, n


@pytest.mark.parametrize("v", [np.nan, np.inf, -np.inf])
def test_a_non_finite_smoothing_value_leaves_no_row_a_scale(v):
    q, d, rng = _q8_0(12, 5, 64)
    s = rng.uniform(0.5, 2.0, 64).astype(np.float32)
    s[9] = v                              # w' of column 9 is non-finite in every row
    wq, sw = oracle.requantize_q8_0(q, d, s)
    assert _nonfinite_rows(q, d, s).all()
    assert np.isnan(sw).all() and not wq.any()
