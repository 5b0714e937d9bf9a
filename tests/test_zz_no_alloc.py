"""The allocation-free split-K entry point against the one with a workspace.

w8a8_gemm_splitk_noalloc keeps its int32 partials in the library's own
scratch array instead of a caller workspace.  Called through the raw C ABI
(ctypes), twice in a row with the second input smaller than the first, it
must give exactly the bits of w8a8_gemm_splitk with a caller workspace and
of the oracle; sizes beyond the scratch are rejected before any launch.
"""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
from deterministic_w8a8_int8_amd import binding as B  # noqa: E402


def _case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, rng.choice(K, 3, replace=False)] *= np.float32(30.0)
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    xq, sx = oracle.quantize_act(x, s)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N), dtype=np.float32)
    return xq, sx, w, sw, r


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(xq, sx, w, sw, r, y, splitk):
    M, K = xq.shape
    N = w.shape[0]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return B._lib.w8a8_gemm_splitk_noalloc(_p(xq), _p(sx), _p(w), _p(sw), _p(r), _p(y), M, N, K,
                                           splitk, st)


def _with_workspace(xq, sx, w, sw, r, y, splitk):
    M, K = xq.shape
    N = w.shape[0]
    n = B._lib.w8a8_gemm_splitk_workspace_bytes(M, N, K, splitk)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = B._lib.w8a8_gemm_splitk(_p(xq), _p(sx), _p(w), _p(sw), _p(r), _p(y), M, N, K, splitk, _p(ws),
                                 n, st)
    torch.cuda.synchronize()
    return rc


# (first call, second smaller call): tiled kernel (M > 512), column-panel
# kernel (64 < M <= 512, which picks S <= splitk) and the skinny range (M <= 64)
CASES = [((600, 520, 1024, 4), (300, 264, 704, 3)),
         ((256, 5120, 2048, 8), (130, 1000, 1024, 2)),
         ((48, 700, 1536, 4), (5, 40, 512, 2))]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_entry_point(first, second):
    for call, (M, N, K, S) in enumerate((first, second)):
        say(f"noalloc call {call}: M={M} N={N} K={K} splitk={S}")
        xq, sx, w, sw, r = _case(M, N, K, seed=M + N + K + S)
        d = [dev(a) for a in (xq, sx, w, sw, r)]
        y_na = torch.full((M, N), float("nan"), device="cuda")
        y_ws = torch.full((M, N), float("nan"), device="cuda")
        assert _noalloc(*d, y_na, S) == B.W8A8_OK
        torch.cuda.synchronize()
        assert _with_workspace(*d, y_ws, S) == B.W8A8_OK
        got, ref = host(y_na), host(y_ws)
        assert_bits_equal(got, ref, f"call {call} noalloc vs workspace")
        assert_bits_equal(got, oracle.gemm(xq, sx, w, sw, r), f"call {call} noalloc vs oracle")
        # in place on the residual stream
        rr = dev(r)
        assert _noalloc(d[0], d[1], d[2], d[3], rr, rr, S) == B.W8A8_OK
        assert_bits_equal(host(rr), ref, f"call {call} noalloc in place")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    # 8192 x 5120 at split-K 2 needs 336 MB of partials: rejected before any
    # launch, the output untouched
    M, N, K = 8192, 5120, 128
    assert B._lib.w8a8_gemm_splitk_workspace_bytes(M, N, K, 2) > B.W8A8_NOALLOC_SCRATCH_BYTES
    xq = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    sx = torch.ones(M, device="cuda")
    w = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    sw = torch.ones(N, device="cuda")
    y = torch.full((M, N), 7.0, device="cuda")
    assert _noalloc(xq, sx, w, sw, None, y, 2) == B.W8A8_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    # split-K 1 needs no scratch at any size
    assert _noalloc(xq, sx, w, sw, None, y, 1) == B.W8A8_OK
    torch.cuda.synchronize()
    assert bool((y == 0.0).all())
