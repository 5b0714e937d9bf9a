"""Row-parallel (tensor-parallel) steps on one GPU, and the split they emulate.

The review page, section "Bitwise consistency is not lossless quantization",
combines the integer partial sums of tensor-parallel ranks before scaling,
and reports one GPU against two or four as giving consistent output.  One
GPU cannot run the collectives of several, so here every rank's share runs
in turn on the one device, and the collectives are done exactly (a MAX of
the slice maxima, an in-order SUM of the int32 partials inside
w8a8_epilogue_int32).  Checks:
* each step bit-exact against its oracle function;
* for 1, 2, 4 and 8 ranks the result is bit-identical to the single-device
  layer, at a mixed-size shape and at the real down projection
  8192 x 5120 x 17408 (slices of 8704, 4352 and 2176).
"""
import numpy as np
import pytest

import oracle
from deterministic_w8a8_int8_amd import synth
from tests.gpu_util import assert_bits_equal, dev, host, say

torch = pytest.importorskip("torch")
B = pytest.importorskip("deterministic_w8a8_int8_amd.binding")

pytestmark = pytest.mark.gpu


def _layer(seed, M, N, K, outlier=25.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= outlier
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    return x, s, w, sw, r


@pytest.mark.parametrize("M,K", [(37, 256), (130, 5120), (9, 34816)])
def test_row_absmax_and_given_maximum_quantisation_match_oracle(M, K):
    say(f"row_absmax / quantize_act_amax M={M} K={K}")
    x, s, _, _, _ = _layer(M + K, M, 8, K)
    xd, sd = dev(x), dev(s)
    amax = B.w8a8_row_absmax(xd, sd)
    want = oracle.row_absmax(x, s)
    assert np.array_equal(host(amax).view(np.uint32), want.view(np.uint32))
    for f in (1.0, 1.7, 100.0):
        a = (want * np.float32(f)).astype(np.float32)
        xq, sx = B.w8a8_quantize_act_amax(xd, sd, dev(a))
        oxq, osx = oracle.quantize_act_amax(x, s, a)
        assert np.array_equal(host(xq), oxq), f
        assert_bits_equal(host(sx), osx, f"sx factor {f}")
    # with its own maximum it is exactly w8a8_quantize_act
    xq1, sx1 = B.w8a8_quantize_act(xd, sd)
    xq2, sx2 = B.w8a8_quantize_act_amax(xd, sd, amax)
    assert torch.equal(xq1, xq2) and torch.equal(sx1.view(torch.int32), sx2.view(torch.int32))


def test_row_absmax_accumulates_over_slices_and_gathers_rows():
    x, s, _, _, _ = _layer(3, 50, 8, 1024)
    rows = np.array([49, 0, 7, 7, 31], dtype=np.int32)
    xd, sd, rd = dev(x), dev(s), dev(rows)
    amax = B.w8a8_row_absmax(xd[:, :384], sd[:384], row_idx=rd)
    B.w8a8_row_absmax(xd[:, 384:], sd[384:], row_idx=rd, amax=amax, accumulate=True)
    want = oracle.row_absmax(x, s, row_idx=rows)
    assert np.array_equal(host(amax).view(np.uint32), want.view(np.uint32))


def test_given_maximum_invalid_rows():
    x, s, _, _, _ = _layer(4, 4, 8, 128)
    a = oracle.row_absmax(x, s)
    a[1] = np.nan
    a[2] = -1.0
    a[3] = 0.0
    xq, sx = B.w8a8_quantize_act_amax(dev(x), dev(s), dev(a))
    xq, sx = host(xq), host(sx)
    assert np.isnan(sx[1]) and np.isnan(sx[2]) and sx[3] == 0.0 and np.isfinite(sx[0])
    assert (xq[1:] == 0).all()


@pytest.mark.parametrize("M,N,K", [(5, 70, 192), (64, 300, 1024), (257, 513, 1216)])
def test_gemm_int32_matches_oracle(M, N, K):
    rng = np.random.default_rng(M * N)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    acc = host(B.w8a8_gemm_int32(dev(xq), dev(w)))
    assert np.array_equal(acc.astype(np.int64), oracle.gemm_acc(xq, w))


@pytest.mark.parametrize("S", [1, 3, 8])
def test_epilogue_int32_matches_oracle(S):
    rng = np.random.default_rng(S)
    M, N = 70, 132
    parts = rng.integers(-2 ** 27, 2 ** 27, (S, M, N)).astype(np.int32)
    sx = rng.uniform(1e-4, 1e-2, M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    want = oracle.epilogue_acc(parts.astype(np.int64).sum(axis=0), sx, sw, r)
    got = host(B.w8a8_epilogue_int32(dev(parts), dev(sx), dev(sw), residual=dev(r)))
    assert_bits_equal(got, want, f"S={S}")
    # in place on the residual, and from a slice stack that is not 16-byte aligned
    big = torch.zeros(S * M * N + 1, dtype=torch.int32, device="cuda")
    big[1:] = dev(parts).reshape(-1)
    rd = dev(r)
    B.w8a8_epilogue_int32(big[1:].view(S, M, N), dev(sx), dev(sw), residual=rd, y=rd)
    assert_bits_equal(host(rd), want, f"S={S} unaligned, in place")


def _tp_emulation(x, s, w, sw, r, ranks):
    """Every rank's share in turn on this device; exact collectives."""
    M, K = x.shape
    N = w.shape[0]
    ks = K // ranks
    assert ks % 64 == 0
    amax = None
    for q in range(ranks):                       # MAX across ranks
        sl = slice(q * ks, (q + 1) * ks)
        amax = B.w8a8_row_absmax(x[:, sl], s[sl], amax=amax, accumulate=amax is not None)
    parts = torch.empty((ranks, M, N), dtype=torch.int32, device="cuda")
    sx = None
    for q in range(ranks):                       # each rank's slice
        sl = slice(q * ks, (q + 1) * ks)
        xq, sx = B.w8a8_quantize_act_amax(x[:, sl], s[sl], amax)
        B.w8a8_gemm_int32(xq, w[:, sl].contiguous(), acc=parts[q])
    return B.w8a8_epilogue_int32(parts, sx, sw, residual=r)   # SUM, then scale


@pytest.mark.parametrize("ranks", [1, 2, 4, 8])
def test_row_parallel_split_is_bit_identical(ranks):
    M, N, K = 200, 320, 2048
    x, s, w, sw, r = _layer(50 + ranks, M, N, K)
    xd, sd, wd, swd, rd = dev(x), dev(s), dev(w), dev(sw), dev(r)
    y_tp = host(_tp_emulation(xd, sd, wd, swd, rd, ranks))
    xq, sx = oracle.quantize_act(x, s)
    assert_bits_equal(y_tp, oracle.gemm(xq, sx, w, sw, r), f"{ranks} ranks vs oracle")


def test_row_parallel_split_at_down_projection_size():
    d = synth.long_prefill("down")              # 8192 x 17408 -> 5120, residual
    xd, sd, wd, swd, rd = dev(d["x"]), dev(d["smooth"]), dev(d["w"]), dev(d["sw"]), dev(d["r"])
    xq, sx = B.w8a8_quantize_act(xd, sd)
    ref = host(B.w8a8_gemm(xq, sx, wd, swd, residual=rd))
    for ranks in (2, 4, 8):
        say(f"down projection, {ranks} ranks")
        y = host(_tp_emulation(xd, sd, wd, swd, rd, ranks))
        assert_bits_equal(y, ref, f"{ranks} ranks vs one device")
    # and the single-device result against the oracle at sampled outputs
    oxq, osx = oracle.quantize_act(d["x"], d["smooth"])
    mi, ni = synth.sample_points(np.random.default_rng(11), 8192, 5120, 2000)
    want = oracle.gemm_sampled(oxq, osx, d["w"], d["sw"], mi, ni, residual=d["r"])
    assert_bits_equal(ref[mi, ni], want, "down projection samples vs oracle")
