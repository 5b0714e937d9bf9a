"""GPU parity: the column-panel kernel under plans the planner would not pick.

Exact int32 accumulation makes every plan (configuration, row splits R,
column panels P, K splits S) give the same bits, so each forced plan is
checked against the oracle over the whole output.  Shapes are ragged in M, N
and K (a short last K stage), with and without a residual.  What is computed
is defined on the review page "StartLux-Prism: Fast, exact inference for
StartLux-Decision models on NVIDIA GPUs", section "Bitwise consistency is not
lossless quantization" (exact int32 accumulation, integer split-K partials,
one fixed epilogue).
"""
import numpy as np
import pytest

import oracle
from gpu_util import assert_bits_equal, dev, host, say
from panel_cases import SHAPES, sample_plans

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
from deterministic_w8a8_int8_amd import binding as B  # noqa: E402


@pytest.mark.parametrize("M,N,K,res", SHAPES)
def test_forced_panel_plans_match_oracle(M, N, K, res):
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sx = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N), dtype=np.float32) if res else None
    want = oracle.gemm(xq, sx, w, sw, r)
    d_xq, d_sx, d_w, d_sw, d_r = dev(xq), dev(sx), dev(w), dev(sw), dev(r)
    y = torch.full((M, N), float("nan"), device="cuda")
    ws = torch.full((B.w8a8_gemm_splitk_workspace_bytes(M, N, K, 5),), 0x5A, dtype=torch.uint8,
                    device="cuda")   # dirty workspace
    good, bad = sample_plans(M, N, K)
    for plan in bad:   # rejected before any launch
        with pytest.raises(B.W8A8Error) as e:
            B.w8a8_gemm_panel_forced(d_xq, d_sx, d_w, d_sw, plan, residual=d_r, y=y, workspace=ws)
        assert e.value.status == B.W8A8_ERR_INVALID_ARG, plan
    for plan, _ in good:   # each checked in bounds on the CPU (test_panel_plan.py)
        say(f"forced panel plan {plan} on {M}x{N}x{K} residual={res}")
        B.w8a8_gemm_panel_forced(d_xq, d_sx, d_w, d_sw, plan, residual=d_r, y=y, workspace=ws)
        assert_bits_equal(host(y), want, f"plan {plan}")
        y.fill_(float("nan"))
