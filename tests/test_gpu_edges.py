"""GPU edge cases: the largest K the int32 accumulators allow, the extreme
codes that drive them to their bound, empty inputs and all-zero rows, on
every kernel path (panel, tiled, skinny forced, split-K), bit for bit
against the oracle.

The int32 bound: every code and weight lies in [-127, 127], so a dot
product over K terms is at most K * 127^2, below 2^31 for K <= 133144; the
library accepts K up to 133120, the largest multiple of 64 (review page
"StartLux-Prism: Fast, exact inference for StartLux-Decision models on NVIDIA
GPUs", section "Bitwise consistency is not lossless quantization": exact
int32 accumulation).
"""
import numpy as np
import pytest

import oracle
from gpu_util import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
from deterministic_w8a8_int8_amd import binding as B  # noqa: E402

K_MAX = B.W8A8_MAX_K


def _extreme_codes(M, N, K, seed):
    """Rows and weight rows of all +127 and all -127 (the accumulator reaches
    +-K*127^2), plus random rows; scales that keep the outputs finite."""
    rng = np.random.default_rng(seed)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    xq[0] = 127
    if M > 1:
        xq[1] = -127
    w[0] = 127
    if N > 1:
        w[1] = -127
    sx = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    return xq, sx, w, sw


@pytest.mark.parametrize("M,N", [(3, 40), (70, 48), (600, 40)])
def test_gemm_at_the_int32_bound(M, N):
    K = K_MAX
    say(f"max K gemm M={M} N={N} K={K}")
    xq, sx, w, sw = _extreme_codes(M, N, K, seed=M + N)
    acc = oracle.gemm_acc(xq, w)
    assert acc[0, 0] == K * 127 * 127 and acc[0, 1] == -K * 127 * 127   # the bound is reached
    want = oracle.gemm(xq, sx, w, sw)
    d = [dev(xq), dev(sx), dev(w), dev(sw)]
    plan = B.w8a8_gemm_plan(M, N, K, 1, False)
    assert_bits_equal(host(B.w8a8_gemm(*d)), want, f"gemm max K (path {plan[0]})")
    assert_bits_equal(host(B.w8a8_gemm_splitk(*d, 5)), want, "gemm max K split-K 5")
    assert np.array_equal(host(B.w8a8_gemm_int32(d[0], d[2])), acc), "int32 accumulators at max K"
    # every kernel, whichever the router picks for this shape
    forced = [(6, "tiled 256x320"), (B.W8A8_TILE_OVERRIDE_PANEL, "panel")]
    if M <= 64:
        forced.append((B.W8A8_TILE_OVERRIDE_SKINNY, "skinny"))
    for kind, name in forced:
        B.set_tile_override(kind)
        try:
            assert_bits_equal(host(B.w8a8_gemm(*d)), want, f"{name} forced, max K")
        finally:
            B.set_tile_override(-1)


def test_gemm_rejects_k_past_the_bound():
    d = [torch.zeros(1, K_MAX + 64, dtype=torch.int8, device="cuda"), torch.ones(1, device="cuda"),
         torch.zeros(1, K_MAX + 64, dtype=torch.int8, device="cuda"), torch.ones(1, device="cuda")]
    with pytest.raises(B.W8A8Error) as e:
        B.w8a8_gemm(*d)
    assert e.value.status == B.W8A8_ERR_K_BOUND


def test_quantize_at_max_k():
    K = K_MAX
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, K), dtype=np.float32)
    x[2] = 0.0                                    # all-zero row: sx = 0, codes 0
    x[3, rng.choice(K, 7, replace=False)] *= 1e4   # a few huge outliers
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    xq, sx = B.w8a8_quantize_act(dev(x), dev(s))
    xq_o, sx_o = oracle.quantize_act(x, s)
    assert_bits_equal(host(sx), sx_o, "sx at max K")
    assert np.array_equal(host(xq), xq_o), "codes at max K"
    assert host(sx)[2] == 0.0 and not host(xq)[2].any()


@pytest.mark.parametrize("M,N,K", [(0, 64, 128), (5, 0, 128), (0, 0, 64)])
def test_empty_products(M, N, K):
    xq = torch.zeros(M, K, dtype=torch.int8, device="cuda")
    w = torch.zeros(N, K, dtype=torch.int8, device="cuda")
    sx, sw = torch.ones(M, device="cuda"), torch.ones(N, device="cuda")
    y = B.w8a8_gemm(xq, sx, w, sw)
    assert tuple(y.shape) == (M, N)
    assert tuple(B.w8a8_gemm_splitk(xq, sx, w, sw, 4).shape) == (M, N)
    xq2, sx2 = B.w8a8_quantize_act(torch.zeros(M, K, device="cuda"), torch.ones(K, device="cuda"))
    assert tuple(xq2.shape) == (M, K) and tuple(sx2.shape) == (M,)


@pytest.mark.parametrize("M,N,K", [(4, 300, 320), (200, 520, 704), (700, 300, 256)])
def test_zero_rows_give_the_residual(M, N, K):
    """A row quantised with sx = 0 (all zeros) multiplies to 0, so its outputs
    are exactly fl(0 + r) = r on every path (reading: zero rows keep sx = 0)."""
    rng = np.random.default_rng(M + N + K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[::3] = 0.0
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N), dtype=np.float32)
    xq, sx = B.w8a8_quantize_act(dev(x), dev(s))
    got = host(B.w8a8_gemm(xq, sx, dev(w), dev(sw), residual=dev(r)))
    xq_o, sx_o = oracle.quantize_act(x, s)
    assert_bits_equal(got, oracle.gemm(xq_o, sx_o, w, sw, r), "zero rows")
    assert_bits_equal(got[::3], r[::3], "zero rows equal the residual")


def test_narrowing_stream_probe_writes_each_top_byte():
    """The narrowing-stream diagnostic (the quantizer's traffic mix) does the
    work it is timed for: byte i of the output is the top byte of word i,
    over a length with a ragged last chunk."""
    n = 4 * 1000003
    src = torch.randn(n, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    assert B.w8a8_probe_stream_narrow(src, dst) == 5 * n
    want = (src.view(torch.int32) >> 24) & 255
    assert torch.equal(dst.to(torch.int32), want)
