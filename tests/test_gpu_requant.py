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


@pytest.mark.parametrize("N,K", [(1, 64), (37, 1024), (300, 5120), (9, 17408)])
def test_requantize_matches_oracle(N, K):
    say(f"requantize N={N} K={K}")
    q, d, s = _case(N + K, N, K)
    w, sw = B.w8a8_requantize_q8_0(dev(q), dev(d.view(np.int16)), dev(s))
    ow, osw = oracle.requantize_q8_0(q, d, s)
    assert_bits_equal(host(sw), osw, "sw")
    np.testing.assert_array_equal(host(w), ow)


def test_requantize_in_place():
    q, d, s = _case(5, 40, 2048)
    ow, osw = oracle.requantize_q8_0(q, d, s)
    qd = dev(q)
    w, sw = B.w8a8_requantize_q8_0(qd, dev(d.view(np.int16)), dev(s), w=qd)
    np.testing.assert_array_equal(host(qd), ow)
    assert_bits_equal(host(sw), osw, "sw in place")


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
