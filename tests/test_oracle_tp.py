"""Pins of the oracle's row-parallel steps (no GPU).

The review page, section "Bitwise consistency is not lossless quantization",
has tensor parallelism combine integer partial sums before scaling.  A rank
of a row-parallel layer holds a K-slice; its partials can only be added as
integers if every rank quantises with one per-token scale, so the oracle
splits quantisation into the slice maximum (``row_absmax``), an exact MAX
across ranks, and quantisation with the global maximum
(``quantize_act_amax``); ``epilogue_acc`` applies the fixed epilogue to the
added integer partials.  Pinned here against exact-rational brute force,
against the already pinned ``quantize_act`` / ``gemm`` as special cases, and
against the integer-split invariants.
"""
import numpy as np
import pytest

import brute
import oracle
from deterministic_w8a8_int8_amd import synth


def _rows(seed, M, K, outlier=25.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 50), replace=False)] *= outlier
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    return x, s


def test_row_absmax_matches_exact_rational_bruteforce():
    x, s = _rows(1, 12, 96)
    got = oracle.row_absmax(x, s)
    for m in range(12):
        want = max(abs(brute.round_f32(brute.f32(a) / brute.f32(b))) for a, b in zip(x[m], s))
        assert got[m] == np.float32(want), m


def test_quantize_with_own_maximum_is_quantize_act():
    x, s = _rows(2, 64, 320)
    xq, sx = oracle.quantize_act(x, s)
    xq2, sx2 = oracle.quantize_act_amax(x, s, oracle.row_absmax(x, s))
    assert np.array_equal(xq, xq2)
    assert np.array_equal(sx.view(np.uint32), sx2.view(np.uint32))


@pytest.mark.parametrize("factor", [1.0, 1.7, 2.0, 100.0])
def test_quantize_with_larger_maximum_matches_bruteforce(factor):
    x, s = _rows(3, 8, 64)
    amax = (oracle.row_absmax(x, s) * np.float32(factor)).astype(np.float32)
    xq, sx = oracle.quantize_act_amax(x, s, amax)
    for m in range(8):
        q, sxb = brute.quantize_row_amax(x[m], s, amax[m])
        assert sx[m] == np.float32(sxb)
        assert list(xq[m]) == q, m
    # with twice the row's own maximum no code exceeds 64 in magnitude
    if factor == 2.0:
        assert np.abs(xq.astype(np.int32)).max() <= 64


def test_nonfinite_slices_and_maxima():
    # A slice with a NaN or infinite smoothed value has an infinite maximum,
    # so the global MAX is infinite and every rank's row is invalid (sx =
    # NaN, codes 0), as on one device.  A given maximum that is NaN,
    # negative or infinite is invalid too.  With a finite given maximum, a
    # NaN element quantises to 0 and an infinite one to +-127.
    rng = np.random.default_rng(9)
    K = 64
    x = rng.standard_normal((6, K)).astype(np.float32)
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    x[1, 3] = np.nan
    x[2, 4] = -np.inf
    amax = oracle.row_absmax(x, s)
    assert np.isinf(amax[1]) and np.isinf(amax[2]) and np.isfinite(amax[[0, 3, 4, 5]]).all()
    given = amax.copy()
    given[3] = np.nan
    given[4] = np.float32(-1.0)
    given[5] = np.inf
    xq, sx = oracle.quantize_act_amax(x, s, given)
    assert np.isnan(sx[1:]).all() and not xq[1:].any()
    xq_full, sx_full = oracle.quantize_act(x, s)
    assert np.isnan(sx_full[[1, 2]]).all() and not xq_full[[1, 2]].any()
    # finite given maxima over rows holding non-finite elements
    fin = np.full(6, np.float32(4.0))
    xq, sx = oracle.quantize_act_amax(x, s, fin)
    for m in range(6):
        q, sxb = brute.quantize_row_amax(x[m], s, fin[m])
        assert sx[m] == np.float32(sxb)
        assert list(xq[m]) == q, m
    assert xq[1, 3] == 0 and xq[2, 4] == -127


def test_zero_maximum_gives_zero_codes():
    x, s = _rows(4, 3, 64)
    xq, sx = oracle.quantize_act_amax(x, s, np.zeros(3, np.float32))
    assert (xq == 0).all() and (sx == 0).all()


def test_epilogue_acc_is_the_gemm_epilogue():
    d = synth.tiny_linear()
    xq, sx = oracle.quantize_act(d["x"], d["smooth"])
    acc = oracle.gemm_acc(xq, d["w"])
    y = oracle.epilogue_acc(acc, sx, d["sw"], d["r"])
    want = oracle.gemm(xq, sx, d["w"], d["sw"], d["r"])
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    for (m, n) in [(0, 0), (3, 17), (15, 255)]:
        b = brute.epilogue(int(acc[m, n]), sx[m], d["sw"][n], d["r"][m, n])
        assert y[m, n] == np.float32(b)


def test_epilogue_acc_rejects_accumulators_beyond_int32():
    acc = np.array([[2 ** 31]], dtype=np.int64)
    with pytest.raises(RuntimeError):
        oracle.epilogue_acc(acc, np.ones(1, np.float32), np.ones(1, np.float32))


@pytest.mark.parametrize("ranks", [1, 2, 4, 8])
def test_row_parallel_split_gives_the_single_device_bits(ranks):
    # a down-projection-like layer: K split into `ranks` contiguous slices
    M, N, K = 24, 80, 1024
    x, s = _rows(10 + ranks, M, K)
    rng = np.random.default_rng(5)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    xq, sx = oracle.quantize_act(x, s)
    want = oracle.gemm(xq, sx, w, sw, r)
    ks = np.array_split(np.arange(K), ranks)
    amax = np.max([oracle.row_absmax(x[:, k], s[k]) for k in ks], axis=0)   # exact MAX
    assert np.array_equal(amax, oracle.row_absmax(x, s))
    acc = np.zeros((M, N), dtype=np.int64)
    for k in ks:
        xq_k, sx_k = oracle.quantize_act_amax(x[:, k], s[k], amax)
        assert np.array_equal(xq_k, xq[:, k])
        assert np.array_equal(sx_k.view(np.uint32), sx.view(np.uint32))
        acc += oracle.gemm_acc(xq_k, np.ascontiguousarray(w[:, k]))      # exact SUM
    assert np.array_equal(acc, oracle.gemm_acc(xq, w))
    y = oracle.epilogue_acc(acc, sx, sw, r)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
