"""GPU parity over seeded random shapes: the whole layer (quantisation, GEMM,
split-K, epilogue with and without a residual) against the CPU oracle, bit
for bit, on shapes drawn around the kernels' boundaries: the skinny, panel
and tiled kernels' row ranges (16, 64, 384, 512, 1024 and 1536 rows), ragged row and
column tails, K from one 64-byte block to several hundred, split-K from 1 to
more chunks than K-blocks.  Definitions: review page "StartLux-Prism: Fast,
exact inference for StartLux-Decision models on NVIDIA GPUs", sections
"Compute shared evidence once" (per-token quantisation) and "Bitwise
consistency is not lossless quantization" (exact int32 accumulation, integer
split-K partials, one fixed rounding sequence).
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

# row counts at and around each routing boundary, then anything up to 640
_M_EDGES = [1, 2, 15, 16, 17, 63, 64, 65, 383, 384, 385, 511, 512, 513, 1023, 1024, 1025, 1536, 1537]


def _shape(rng, i):
    M = int(_M_EDGES[i]) if i < len(_M_EDGES) else int(rng.integers(1, 641))
    N = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 1500)), int(rng.integers(1500, 3000))]))
    K = 64 * int(rng.choice([1, 2, 3, int(rng.integers(4, 17)), int(rng.integers(17, 40))]))
    S = int(rng.choice([1, 1, 2, 3, 5, int(rng.integers(6, 65))]))
    residual = bool(rng.integers(0, 2))
    return M, N, K, S, residual


def _wide(rng):
    """Wide layers (the wide panel kinds, the non-temporal weight stream, the
    tiled kernel past 384 rows) at small K, so the oracle stays quick."""
    return (int(rng.integers(1, 513)), int(rng.integers(3000, 36001)), 64 * int(rng.integers(1, 5)),
            int(rng.choice([1, 1, 4])), bool(rng.integers(0, 2)))


CASES = [_shape(np.random.default_rng(9000 + i), i) for i in range(41)] + \
        [_wide(np.random.default_rng(9100 + i)) for i in range(10)]


@pytest.mark.parametrize("M,N,K,S,residual", CASES)
def test_random_layer_matches_oracle(M, N, K, S, residual):
    say(f"random layer M={M} N={N} K={K} S={S} residual={residual} plan={B.w8a8_gemm_plan(M, N, K, S, residual)}")
    rng = np.random.default_rng(M * 7919 + N * 31 + K + S)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(30.0)
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N), dtype=np.float32) if residual else None
    xq, sx = B.w8a8_quantize_act(dev(x), dev(s))
    xq_o, sx_o = oracle.quantize_act(x, s)
    assert np.array_equal(host(xq), xq_o), "codes"
    assert_bits_equal(host(sx), sx_o, "token scales")
    want = oracle.gemm(xq_o, sx_o, w, sw, r)
    got = B.w8a8_gemm_splitk(xq, sx, dev(w), dev(sw), S, residual=dev(r)) if S > 1 else \
        B.w8a8_gemm(xq, sx, dev(w), dev(sw), residual=dev(r))
    assert_bits_equal(host(got), want, f"layer {M}x{N}x{K} S={S}")
