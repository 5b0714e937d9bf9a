"""Startup requantisation of Q8_0 weights on the GPU, bit-exact against the
oracle (review page, section "Compute shared evidence once": the Q8_0
weights are requantised with SmoothQuant at startup), and the requantised
weights through the whole W8A8 layer."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_bits_equal, dev, host, say

torch = pytest.importorskip("torch")
B = pytest.importorskip("deterministic_w8a8_int8_amd.binding")

pytestmark = pytest.mark.gpu


def _case(seed, N, K):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, (N, K), dtype=np.int8)
    d = rng.uniform(1e-4, 1e-2, (N, K // 32)).astype(np.float16)
    s = rng.uniform(0.25, 8.0, K).astype(np.float32)
    if N > 3:
        d[1, :] = 0                                   # a zero row
        d[2, ::3] = np.float16(6e-8)                  # subnormal binary16 scales
        q[3, :] = 0
        q[3, 5] = -127
    return q, d.view(np.uint16), s


# one shape per kernel configuration: a wave per row with 1..6 chunks a lane
# (64, 1088 with lanes past the row, 5120, 6144), a workgroup per row
# (6208: 2 chunks a lane; 17408: 5, the last block partly past the row;
# 24576: 6) and the two-pass long-row kernel (24640); row counts that are
# not multiples of the four rows a workgroup takes
@pytest.mark.parametrize("N,K", [(1, 64), (5, 64), (37, 1024), (3, 1088), (300, 5120), (6, 6144), (7, 6208),
                                 (9, 17408), (2, 24576), (3, 24640)])
def test_requantize_matches_oracle(N, K):
    say(f"requantize N={N} K={K}")
    q, d, s = _case(N + K, N, K)
    w, sw = B.w8a8_requantize_q8_0(dev(q), dev(d.view(np.int16)), dev(s))
    ow, osw = oracle.requantize_q8_0(q, d, s)
    assert_bits_equal(host(sw), osw, "sw")
    np.testing.assert_array_equal(host(w), ow)


@pytest.mark.parametrize("N,K", [(40, 2048), (6, 17408), (5, 24640)])
def test_requantize_in_place(N, K):
    q, d, s = _case(5, N, K)
    ow, osw = oracle.requantize_q8_0(q, d, s)
    qd = dev(q)
    w, sw = B.w8a8_requantize_q8_0(qd, dev(d.view(np.int16)), dev(s), w=qd)
    np.testing.assert_array_equal(host(qd), ow)
    assert_bits_equal(host(sw), osw, "sw in place")


@pytest.mark.parametrize("big", [True, False])
def test_requantize_scale_extremes(big):
    # channel scales on both sides of 2^120 and of 2^-120, where the division
    # by the row's reciprocal stops being exact and every value goes through
    # the true division instead (and, for the small ones, subnormal w')
    rng = np.random.default_rng(31 + big)
    N, K = 12, 1024
    q = rng.integers(-127, 128, (N, K), dtype=np.int8)
    q[:, 0] = 127
    u = rng.uniform(0.25, 1.0, K).astype(np.float32)
    u[0] = 1.0
    if big:    # w' = d q 2^121 u: sw = d 2^121 for the row maximum 127 d 2^121
        s = (u * np.float32(2.0 ** 121)).astype(np.float32)
        dr = np.float16([1.0, 0.5, 0.5, 0.25, 0.75, 1.0, 0.5, 0.375, 0.5, 0.999, 0.5, 0.5])
        q[2, 0] = 126      # sw just below 2^120
        q[6, 0] = -127
        q[10, 0] = 125
    else:      # w' = d q 2^-104 u: sw = d 2^-104, subnormal (and so are some w') for d = 2^-24
        s = (u * np.float32(2.0 ** -104)).astype(np.float32)
        dr = np.float16([2.0 ** -16, 2.0 ** -17, 2.0 ** -24, 2.0 ** -15, 2.0 ** -16 * 1.5, 2.0 ** -18,
                         2.0 ** -16, 2.0 ** -23, 2.0 ** -16 * 0.75, 2.0 ** -14, 2.0 ** -16, 2.0 ** -24 * 3])
        q[6, 0] = 126      # sw just below 2^-120
    d = np.repeat(dr[:, None], K // 32, axis=1).astype(np.float16)
    say(f"requantize scale extremes big={big}")
    w, sw = B.w8a8_requantize_q8_0(dev(q), dev(d.view(np.uint16).view(np.int16)), dev(s))
    ow, osw = oracle.requantize_q8_0(q, d.view(np.uint16), s)
    lim = np.float32(2.0 ** 120) if big else np.float32(2.0 ** -120)
    assert np.any(osw > lim) and np.any(osw < lim) and np.any(osw == lim), osw   # both routes and the edge
    assert np.all(np.isfinite(osw)) and np.all(osw > 0)
    assert_bits_equal(host(sw), osw, "sw")
    np.testing.assert_array_equal(host(w), ow)


def test_requantised_weights_through_the_layer():
    # activations divided by s, weights multiplied by s: the W8A8 layer on the
    # requantised weights equals the oracle's chain bit for bit
    rng = np.random.default_rng(12)
    M, N, K = 96, 160, 1024
    q, d, s = _case(7, N, K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, 10, replace=False)] *= 40.0
    w, sw = B.w8a8_requantize_q8_0(dev(q), dev(d.view(np.int16)), dev(s))
    xq, sx = B.w8a8_quantize_act(dev(x), dev(s))
    y = host(B.w8a8_gemm(xq, sx, w, sw))
    ow, osw = oracle.requantize_q8_0(q, d, s)
    oxq, osx = oracle.quantize_act(x, s)
    assert_bits_equal(y, oracle.gemm(oxq, osx, ow, osw), "layer on requantised weights")


def test_requantize_half_integer_quotients():
    # quotients w'/sw exactly on half-integers (ties to even) and a few ulps
    # either side of them: the cases where one rounding of the quotient
    # decides the code.  Column 0 holds the row maximum 127 * d with s = 1, so
    # sw = d exactly; odd codes on columns smoothed by 0.5 give q/2.
    rng = np.random.default_rng(21)
    N, K = 64, 2048
    q = rng.integers(-127, 128, (N, K), dtype=np.int8)
    q[:, 0] = 127
    q[:, 1::2] |= 1
    d = np.repeat(rng.uniform(1e-4, 1e-2, (N, 1)), K // 32, axis=1).astype(np.float16)
    s = np.ones(K, np.float32)
    s[1::2] = 0.5
    s[3::8] = np.nextafter(np.float32(0.5), np.float32(1))
    s[5::8] = np.nextafter(np.float32(0.5), np.float32(0))
    s[7::16] = np.float32(0.5) * np.float32(1 + 2.0 ** -13)
    say(f"requantize ties N={N} K={K}")
    w, sw = B.w8a8_requantize_q8_0(dev(q), dev(d.view(np.uint16).view(np.int16)), dev(s))
    ow, osw = oracle.requantize_q8_0(q, d.view(np.uint16), s)
    assert np.array_equal(osw, d[:, 0].astype(np.float32))
    ties = ow[:, s == np.float32(0.5)].astype(np.int64)
    assert ties.size and np.all(ties % 2 == 0)        # the fixture really ties
    assert_bits_equal(host(sw), osw, "sw")
    np.testing.assert_array_equal(host(w), ow)


def _assert_same_rows(w, sw, ow, osw):
    assert np.array_equal(np.isnan(sw), np.isnan(osw))
    fin = ~np.isnan(osw)
    assert_bits_equal(sw[fin], osw[fin], "sw")
    np.testing.assert_array_equal(w, ow)


@pytest.mark.parametrize("K", [1024, 17408, 24640])
def test_requantize_non_finite_rows(K):
    # rows whose w' holds a NaN or an infinity get sw = NaN and all codes 0
    # (the oracle's rule); the other rows are untouched
    q, d, s = _case(K + 3, 10, K)
    d = d.copy()
    d[0, 1] = 0x7e00                      # a NaN block scale
    d[1, 2] = 0x7c00                      # +inf with nonzero codes
    q[1, 64] = 5
    d[2, 3] = 0xfc00                      # -inf times all-zero codes: NaN
    q[2, 96:128] = 0
    d[4, K // 32 - 1] = 0x7bff            # 65504 * 127 * 2^124 overflows, in the last block
    q[4, K - 3] = 127
    s[K - 3] = np.float32(2.0 ** 124)
    say(f"requantize non-finite rows K={K}")
    w, sw = B.w8a8_requantize_q8_0(dev(q), dev(d.view(np.int16)), dev(s))
    ow, osw = oracle.requantize_q8_0(q, d, s)
    assert np.isnan(osw[[0, 1, 2, 4]]).all() and np.isfinite(osw[[3, 5, 6, 7, 8, 9]]).all()
    _assert_same_rows(host(w), host(sw), ow, osw)
    s[7] = np.nan                         # now every row
    w, sw = B.w8a8_requantize_q8_0(dev(q), dev(d.view(np.int16)), dev(s))
    ow, osw = oracle.requantize_q8_0(q, d, s)
    assert np.isnan(osw).all()
    _assert_same_rows(host(w), host(sw), ow, osw)


def _random_shapes(seed, n):
    """Seeded (N, K, in_place) cases: K a multiple of 64 up to 30000, drawn
    half from the neighbourhoods of the kernels' boundaries (one wave per row
    up to 6144 columns, a workgroup up to 24576, two passes beyond; chunks of
    1024 columns per wave load)."""
    rng = np.random.default_rng(seed)
    edges = [64, 1024, 6144, 24576]
    out = []
    for i in range(n):
        if i % 2:
            k = int(rng.choice(edges)) + 64 * int(rng.integers(-2, 3))
        else:
            k = 64 * int(rng.integers(1, 30000 // 64 + 1))
        out.append((int(rng.integers(1, 71)), max(64, k), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("N,K,in_place", _random_shapes(2027, 24))
def test_requantize_random_shapes(N, K, in_place):
    say(f"requantize random N={N} K={K} in_place={in_place}")
    q, d, s = _case(N * 7 + K, N, K)
    ow, osw = oracle.requantize_q8_0(q, d, s)
    qd = dev(q)
    w, sw = B.w8a8_requantize_q8_0(qd, dev(d.view(np.int16)), dev(s), w=qd if in_place else None)
    assert_bits_equal(host(sw), osw, "sw")
    np.testing.assert_array_equal(host(qd if in_place else w), ow)
