"""GPU parity: every C-ABI entry point against the CPU oracle, bit for bit.

Sizes here let the oracle compute every output in seconds, yet they span
several tiles, ragged M/N tails, half K-stages, every tile shape, both GEMM
kernels and several split-K factors.  The workload-sized cases live in
test_gpu_configs.py.  The definitions come from the review page
"StartLux-Prism: Fast, exact inference for StartLux-Decision models on NVIDIA
GPUs", sections "Compute shared evidence once" and "Bitwise consistency is
not lossless quantization".
"""
import numpy as np
import pytest

import oracle
from deterministic_w8a8_int8_amd import synth
from gpu_util import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
from deterministic_w8a8_int8_amd import binding as B  # noqa: E402


def _quant_case(M, K, seed, n_out=3, mult=30.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if n_out:
        x[:, rng.choice(K, n_out, replace=False)] *= np.float32(mult)
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    return x, s


# ------------------------------------------------------------------ quantisation

# (1543, 5120) and (2357, 17408): more rows than workgroups resident at once
# (several rounds of workgroups), with ragged remainders; up to 64 rows with
# 2048 < K <= 6144 take the wider few-row workgroups (1024 or 512 threads)
@pytest.mark.parametrize("M,K", [(1, 64), (16, 256), (37, 1024), (300, 5120), (5, 17408), (2, 40960),
                                 (1543, 5120), (2357, 17408), (1, 2112), (64, 4096), (3, 5120), (40, 6144),
                                 (65, 6144)])
def test_quantize_matches_oracle(M, K):
    say(f"quantize M={M} K={K}")
    x, s = _quant_case(M, K, seed=M * 7 + K)
    x[0, :] = 0.0                         # sx = 0 row
    if M > 1:
        x[1, :] = 0.0
        x[1, 3] = np.float32(1e-44)       # amax/127 underflows
    xq, sx = B.w8a8_quantize_act(dev(x), dev(s))
    xq_o, sx_o = oracle.quantize_act(x, s)
    assert_bits_equal(host(sx), sx_o, "sx")
    np.testing.assert_array_equal(host(xq), xq_o)


def test_quantize_ties_and_strides():
    # rows whose quotients land exactly on .5 (s = 1, amax 127 or 254)
    K = 128
    x = np.zeros((4, 256), np.float32)
    x[0, :8] = [127, 0.5, 1.5, 2.5, -2.5, -0.5, 126.5, 125.5]
    x[1, :8] = [-254, 1, 3, 5, 7, -3, 253, 0]
    x[2, :K] = np.arange(K, dtype=np.float32) - 63.5
    x[3, :K] = 1e-30
    s = np.ones(K, np.float32)
    xd = dev(x)[:, 64:64 + K]             # row stride 256 > K
    xq, sx = B.w8a8_quantize_act(xd, dev(s))
    xq_o, sx_o = oracle.quantize_act(x[:, 64:64 + K], s)
    assert_bits_equal(host(sx), sx_o, "sx")
    np.testing.assert_array_equal(host(xq), xq_o)
    xq, sx = B.w8a8_quantize_act(dev(x[:, :K]), dev(s))
    np.testing.assert_array_equal(host(xq)[0, :8], [127, 0, 2, 2, -2, 0, 126, 126])
    np.testing.assert_array_equal(host(xq)[1, :8], [-127, 0, 2, 2, 4, -2, 126, 0])


def _extreme_rows(K, seed):
    """Rows that leave the fast path's error bounds: smoothing values outside
    [2^-120, 2^120] (subnormal ones included), subnormal activations, rows
    whose maximum is tiny, and rows with many equal maxima."""
    rng = np.random.default_rng(seed)
    g = lambda: rng.standard_normal(K)
    rows, smooths = [], []
    # 1: tiny smoothing values (some subnormal), small activations
    s = np.exp2(rng.uniform(-140, -110, K))
    rows.append(g() * 2.0 ** -20); smooths.append(s)
    # 2: huge smoothing values: smoothed values near 2^-110 (tiny row maximum)
    s = np.exp2(rng.uniform(100, 126, K))
    rows.append(g()); smooths.append(s)
    # 3: huge smoothing values with large activations
    rows.append(g() * 2.0 ** 100); smooths.append(s)
    # 4: mixed columns: normal, just below 2^-120 and just above 2^120
    s = np.where(rng.random(K) < 0.5, rng.uniform(0.5, 4.0, K),
                 np.where(rng.random(K) < 0.5, np.exp2(rng.uniform(-126, -121, K)),
                          np.exp2(rng.uniform(121, 126, K))))
    rows.append(g() * s); smooths.append(s)
    # 5: subnormal activations with ordinary smoothing
    s = rng.uniform(0.5, 4.0, K)
    rows.append(g() * 1e-40); smooths.append(s)
    # 6: many equal maxima and exact halves
    x = np.round(g() * 4) / 2
    x[rng.choice(K, 9, replace=False)] = 63.5
    rows.append(x); smooths.append(np.ones(K))
    return [np.asarray(r, np.float32) for r in rows], [np.asarray(v, np.float32) for v in smooths]


# tall=True repeats each case over 1100 rows, more workgroups than a round of
# CUs holds, so the rare exact paths also run while other rows stream in
@pytest.mark.parametrize("K,tall", [(1024, False), (5120, False), (17408, False), (40960, False),
                                    (5120, True), (17408, True)])
def test_quantize_extreme_values_match_oracle(K, tall):
    say(f"quantize extremes K={K} tall={tall}")
    rows, smooths = _extreme_rows(K, seed=K)
    for i, (x, s) in enumerate(zip(rows, smooths)):
        # the row alone and with ordinary rows around it (same smoothing)
        rng = np.random.default_rng(i)
        typical = np.float64(np.median(np.abs(x.astype(np.float64) / s)))
        other = (np.clip(rng.standard_normal(K), -3, 3) * typical * s).astype(np.float32)
        block = np.stack([x, other, x])
        if tall:
            block = np.tile(block, (367, 1))[:1100]
        with np.errstate(all="ignore"):
            assert np.isfinite(block).all() and np.isfinite(block / s).all(), "inputs must be finite"
        xq, sx = B.w8a8_quantize_act(dev(block), dev(s))
        xq_o, sx_o = oracle.quantize_act(block, s)
        assert_bits_equal(host(sx), sx_o, f"K={K} case {i + 1} sx")
        np.testing.assert_array_equal(host(xq), xq_o, err_msg=f"K={K} case {i + 1}")


def _nonfinite_block(K, seed, tall):
    """Ordinary rows mixed with rows holding a NaN, +Inf or -Inf input, a
    finite input whose smoothed value overflows (3e38 / 0.25), and a finite
    row just inside the range (3e38 / 1)."""
    x, s = _quant_case(8, K, seed)
    s[5] = np.float32(0.25)
    s[6] = np.float32(1.0)
    x[1, 9] = np.nan
    x[2, K - 1] = np.inf
    x[3, 0] = -np.inf
    x[4, 5] = np.float32(3e38)
    x[5, 6] = np.float32(3e38)
    x[6, K // 2] = np.nan
    x[6, K // 2 + 1] = np.inf
    if tall:
        x = np.tile(x, (140, 1))[:1100]
    return x, s


# Rows with a non-finite smoothed value get sx = NaN and all codes 0 on both
# sides; their GEMM outputs are NaN, every other output is bit-exact.  K =
# 40960 runs the two-pass kernel; tall repeats the rows over 1100 workgroups.
@pytest.mark.parametrize("K,tall", [(1024, False), (5120, False), (17408, True), (40960, False)])
def test_quantize_nonfinite_rows_match_oracle(K, tall):
    say(f"quantize non-finite rows K={K} tall={tall}")
    x, s = _nonfinite_block(K, seed=K + 3, tall=tall)
    xq, sx = B.w8a8_quantize_act(dev(x), dev(s))
    with np.errstate(all="ignore"):
        xq_o, sx_o = oracle.quantize_act(x, s)
    assert_bits_equal(host(sx), sx_o, f"K={K} sx")
    np.testing.assert_array_equal(host(xq), xq_o)
    assert np.isnan(sx_o[[1, 2, 3, 4, 6]]).all() and np.isfinite(sx_o[[0, 5, 7]]).all()
    # the row-parallel steps: the slice maximum is +Inf on those rows, and the
    # global-maximum quantisation gives the same bits as one device
    amax = B.w8a8_row_absmax(dev(x), dev(s))
    with np.errstate(all="ignore"):
        amax_o = oracle.row_absmax(x, s)
    assert_bits_equal(host(amax), amax_o, f"K={K} amax")
    xq2, sx2 = B.w8a8_quantize_act_amax(dev(x), dev(s), amax)
    assert_bits_equal(host(sx2), sx_o, f"K={K} sx (given maximum)")
    np.testing.assert_array_equal(host(xq2), xq_o)
    # GEMM over those rows
    rng = np.random.default_rng(K)
    N = 96
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((x.shape[0], N), dtype=np.float32)
    got = host(B.w8a8_gemm(xq, sx, dev(w), dev(sw), residual=dev(r)))
    with np.errstate(all="ignore"):
        want = oracle.gemm(xq_o, sx_o, w, sw, r)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert_bits_equal(got[fin], want[fin], f"K={K} gemm")


def test_quantize_given_maximum_nonfinite_elements():
    # A finite given maximum over rows holding NaN / +-Inf elements: NaN -> 0,
    # +-Inf -> +-127 on both sides; NaN, negative and infinite maxima give an
    # invalid row.
    K = 256
    x, s = _quant_case(6, K, seed=21)
    x[1, 3], x[2, 4], x[3, 5] = np.nan, np.inf, -np.inf
    amax = np.array([4.0, 4.0, 4.0, 4.0, np.nan, np.inf], np.float32)
    amax[0] = -1.0
    xq, sx = B.w8a8_quantize_act_amax(dev(x), dev(s), dev(amax))
    with np.errstate(all="ignore"):
        xq_o, sx_o = oracle.quantize_act_amax(x, s, amax)
    assert_bits_equal(host(sx), sx_o, "sx")
    np.testing.assert_array_equal(host(xq), xq_o)
    assert xq_o[1, 3] == 0 and xq_o[2, 4] == 127 and xq_o[3, 5] == -127


def test_quantize_row_gather_and_bad_index():
    x, s = _quant_case(40, 512, seed=5)
    idx = np.array([39, 0, 17, 17, 5, -1, 40, 2], np.int32)
    xq, sx = B.w8a8_quantize_act(dev(x), dev(s), row_idx=dev(idx))
    xq_h, sx_h = host(xq), host(sx)
    ok = (idx >= 0) & (idx < 40)
    xq_o, sx_o = oracle.quantize_act(x, s, row_idx=np.where(ok, idx, 0))
    assert_bits_equal(sx_h[ok], sx_o[ok], "sx")
    np.testing.assert_array_equal(xq_h[ok], xq_o[ok])
    assert np.isnan(sx_h[~ok]).all() and not xq_h[~ok].any()


# --------------------------------------------------------------------------- GEMM

def _gemm_case(M, N, K, seed, residual):
    rng = np.random.default_rng(seed)
    x, s = _quant_case(M, K, seed + 1)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N), dtype=np.float32) if residual else None
    xq, sx = oracle.quantize_act(x, s)
    return xq, sx, w, sw, r


SHAPES = [
    (1, 7, 64), (3, 256, 320), (16, 256, 256), (64, 130, 192),      # M <= 64 (panel kernel by default)
    (3, 300, 2048), (40, 500, 2560), (5, 40, 4096), (16, 1000, 5120),  # (skinny: K split over waves)
    (3, 20, 1024),   # two column tiles: half of the workgroup has no columns (LDS staging regression)
    (65, 100, 64), (200, 257, 192), (300, 520, 1024), (513, 264, 320), (256, 256, 256),
    (1100, 300, 256), (1537, 70, 448),      # past 1024 rows: the tiled kernel by default (here)
    (48, 20000, 512), (130, 17000, 320),    # narrow-kind panels over many columns
    (40, 34816, 256), (160, 34816, 256),    # wide kinds with the non-temporal weight stream
]
SMALL_M = [s for s in SHAPES if s[0] <= 64]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("residual", [False, True])
def test_gemm_matches_oracle(M, N, K, residual):
    say(f"gemm M={M} N={N} K={K} residual={residual}")
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=M + N + K, residual=residual)
    want = oracle.gemm(xq, sx, w, sw, r)
    got = host(B.w8a8_gemm(dev(xq), dev(sx), dev(w), dev(sw), residual=dev(r)))
    assert_bits_equal(got, want, f"gemm {M}x{N}x{K}")


# Between 385 and 1024 rows the two GEMM kernels' time models pick the
# kernel: a wide layer of 448 rows runs on the tiled kernel (its panels would
# need two rounds of workgroups), a long-K narrow layer of 1024 rows on the
# panel kernel.  Both sides of the crossover, sampled in every 16 x 16 output
# block (and in two whole rows) against the oracle, with the route checked.
@pytest.mark.parametrize("M,N,K,path", [(448, 34816, 5120, 1), (384, 34816, 5120, 2), (512, 15360, 1024, 2),
                                        (1024, 5120, 17408, 2), (896, 15360, 5120, 1)])
def test_routing_crossover_matches_oracle(M, N, K, path):
    say(f"crossover gemm M={M} N={N} K={K}")
    assert B.w8a8_gemm_plan(M, N, K, 1, True)[0] == path
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=M + N, residual=True)
    got = host(B.w8a8_gemm(dev(xq), dev(sx), dev(w), dev(sw), residual=dev(r)))
    rng = np.random.default_rng(M)
    bi, bj = synth.block_points(rng, M, N, 16, 16)
    rows = np.array([0, M - 1])
    mi = np.concatenate([bi, np.repeat(rows, N)])
    ni = np.concatenate([bj, np.tile(np.arange(N), rows.size)])
    want = oracle.gemm_sampled(xq, sx, w, sw, mi, ni, residual=r)
    assert_bits_equal(got[mi, ni], want, f"gemm {M}x{N}x{K} (path {path})")


# The skinny kernel forced for M <= 64 (by default most of those shapes run
# on the column-panel kernel, which is faster there; the skinny kernel keeps
# the full-vocabulary read-out and narrow long-K layers of a few rows): its
# register-streamed weights, the K-parallel mode and ragged tiles, bit for
# bit, and the panel kernel forced on the same shapes.
@pytest.mark.parametrize("M,N,K", SMALL_M)
@pytest.mark.parametrize("residual", [False, True])
def test_skinny_kernel_forced_matches_oracle(M, N, K, residual):
    say(f"skinny forced M={M} N={N} K={K} residual={residual}")
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=M + N + K, residual=residual)
    want = oracle.gemm(xq, sx, w, sw, r)
    for kind, path, name in ((B.W8A8_TILE_OVERRIDE_SKINNY, 0, "skinny"), (B.W8A8_TILE_OVERRIDE_PANEL, 2, "panel")):
        B.set_tile_override(kind)
        try:
            assert B.w8a8_gemm_plan(M, N, K, 1, residual)[0] == path
            got = host(B.w8a8_gemm(dev(xq), dev(sx), dev(w), dev(sw), residual=dev(r)))
        finally:
            B.set_tile_override(-1)
        assert_bits_equal(got, want, f"{name} forced {M}x{N}x{K}")


# At least 1024 column tiles and activation rows that fit in LDS: the weight
# rows are copied into LDS in 256-byte K-stages (ragged N, K-steps past the
# last whole stage, M from 1 to 16).
@pytest.mark.parametrize("M,N,K", [(1, 16400, 256), (3, 16421, 320), (16, 20000, 640), (5, 17003, 1344)])
@pytest.mark.parametrize("residual", [False, True])
def test_skinny_weight_stream_through_lds(M, N, K, residual):
    say(f"skinny lds stream M={M} N={N} K={K} residual={residual}")
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=5 * M + N + K, residual=residual)
    want = oracle.gemm(xq, sx, w, sw, r)
    got = host(B.w8a8_gemm(dev(xq), dev(sx), dev(w), dev(sw), residual=dev(r)))
    assert_bits_equal(got, want, f"skinny {M}x{N}x{K}")
    if residual:   # the output may alias the residual
        rd = dev(r)
        B.w8a8_gemm(dev(xq), dev(sx), dev(w), dev(sw), residual=rd, y=rd)
        assert_bits_equal(host(rd), want, f"skinny {M}x{N}x{K} in place")


@pytest.mark.parametrize("kind", list(range(B.W8A8_TILE_OVERRIDE_PANEL + 1)))
def test_every_tile_shape_gives_identical_bits(kind):
    M, N, K = 300, 520, 704
    say(f"tile kind {kind}")
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=11, residual=True)
    want = oracle.gemm(xq, sx, w, sw, r)
    B.set_tile_override(kind)
    try:
        got = host(B.w8a8_gemm(dev(xq), dev(sx), dev(w), dev(sw), residual=dev(r)))
        got_s = host(B.w8a8_gemm_splitk(dev(xq), dev(sx), dev(w), dev(sw), 3, residual=dev(r)))
    finally:
        B.set_tile_override(-1)
    assert_bits_equal(got, want, f"kind {kind}")
    assert_bits_equal(got_s, want, f"kind {kind} split 3")


@pytest.mark.parametrize("M,N,K", [(8, 100, 640), (130, 300, 1024), (257, 513, 1216)])
@pytest.mark.parametrize("splitk", [2, 3, 4, 8, 13])
def test_splitk_matches_oracle(M, N, K, splitk):
    say(f"splitk M={M} N={N} K={K} S={splitk}")
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=3 * M + N, residual=True)
    want = oracle.gemm(xq, sx, w, sw, r)
    ws = B.splitk_workspace(M, N, K, splitk)
    ws.fill_(0xA5)  # whatever the workspace holds on entry is overwritten
    xq_d, sx_d, w_d, sw_d, r_d = dev(xq), dev(sx), dev(w), dev(sw), dev(r)
    for rep in range(2):  # and it serves the next call as it is left
        got = host(B.w8a8_gemm_splitk(xq_d, sx_d, w_d, sw_d, splitk, residual=r_d, workspace=ws))
        assert_bits_equal(got, want, f"split {splitk} rep {rep}")


# Column-panel kernel (64 < M <= 512 by default; forced here on ragged shapes):
# N not a multiple of 4 (scalar epilogue), K not a multiple of 256 (short
# last LDS stage), fewer row blocks than waves, panels of unequal width.
PANEL_SHAPES = [(65, 100, 64), (80, 17, 128), (96, 1001, 448), (130, 300, 1024), (200, 257, 192),
                (257, 513, 1216), (300, 2100, 704), (333, 555, 1088), (512, 260, 320),
                (17, 333, 256), (1, 50, 320)]


@pytest.mark.parametrize("M,N,K", PANEL_SHAPES)
def test_panel_kernel_matches_oracle(M, N, K):
    say(f"panel M={M} N={N} K={K}")
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=2 * M + 3 * N + K, residual=True)
    want_r = oracle.gemm(xq, sx, w, sw, r)
    want = oracle.gemm(xq, sx, w, sw)
    d = [dev(xq), dev(sx), dev(w), dev(sw)]
    B.set_tile_override(B.W8A8_TILE_OVERRIDE_PANEL)
    try:
        got = host(B.w8a8_gemm(*d))
        got_r = host(B.w8a8_gemm(*d, residual=dev(r)))
        got_s3 = host(B.w8a8_gemm_splitk(*d, 3, residual=dev(r)))
        got_s5 = host(B.w8a8_gemm_splitk(*d, 5))
        acc = host(B.w8a8_gemm_int32(d[0], d[2]))
        plans = [B.w8a8_gemm_plan(M, N, K, s, res) for s, res in ((1, 0), (3, 1), (5, 0))]
    finally:
        B.set_tile_override(-1)
    say(f"  plans {plans}")
    assert_bits_equal(got, want, "panel")
    assert_bits_equal(got_r, want_r, "panel + residual")
    assert_bits_equal(got_s3, want_r, "panel split<=3 + residual")
    assert_bits_equal(got_s5, want, "panel split<=5")
    np.testing.assert_array_equal(acc, oracle.gemm_acc(xq, w))


def test_splitk_more_chunks_than_kblocks():
    M, N, K = 70, 90, 192                  # 3 k-blocks, 8 chunks: several are empty
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=77, residual=False)
    got = host(B.w8a8_gemm_splitk(dev(xq), dev(sx), dev(w), dev(sw), 8))
    assert_bits_equal(got, oracle.gemm(xq, sx, w, sw), "empty chunks")


def test_residual_in_place():
    M, N, K = 100, 200, 256
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=9, residual=True)
    want = oracle.gemm(xq, sx, w, sw, r)
    rd = dev(r)
    B.w8a8_gemm(dev(xq), dev(sx), dev(w), dev(sw), residual=rd, y=rd)
    assert_bits_equal(host(rd), want, "in place")
    rd = dev(r)
    B.w8a8_gemm_splitk(dev(xq), dev(sx), dev(w), dev(sw), 2, residual=rd, y=rd)
    assert_bits_equal(host(rd), want, "in place, split 2")


# Interior tiles of the 256x256 and 256x320 configurations with a residual
# copy it into LDS one pass ahead of its use; ragged tiles take the checked
# sweep.  Both, separate and in place (y aliasing the residual).
@pytest.mark.parametrize("kind", [4, 6])
@pytest.mark.parametrize("M,N,K", [(600, 640, 320), (1030, 960, 576)])
def test_tiled_residual_epilogue(kind, M, N, K):
    say(f"tiled residual kind={kind} M={M} N={N} K={K}")
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=M + 7 * kind, residual=True)
    want = oracle.gemm(xq, sx, w, sw, r)
    d = dev(xq), dev(sx), dev(w), dev(sw)
    B.set_tile_override(kind)
    try:
        got = host(B.w8a8_gemm(*d, residual=dev(r)))
        rd = dev(r)
        B.w8a8_gemm(*d, residual=rd, y=rd)
        got_in_place = host(rd)
    finally:
        B.set_tile_override(-1)
    assert_bits_equal(got, want, f"kind {kind}")
    assert_bits_equal(got_in_place, want, f"kind {kind} in place")


def test_rows_identical_across_kernels_and_batches():
    # the same 3 rows alone (skinny kernel), inside a 70-row batch (tiled
    # kernel), at the end of a 300-row batch, and split 4 ways
    K, N = 512, 384
    rng = np.random.default_rng(21)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    x, s = _quant_case(300, K, seed=22)
    wd, swd, sd = dev(w), dev(sw), dev(s)
    rows = [297, 298, 299]
    outs = []
    for sub in (x[rows], x[230:], x):
        xq, sx = B.w8a8_quantize_act(dev(sub), sd)
        outs.append(host(B.w8a8_gemm(xq, sx, wd, swd))[-3:])
        outs.append(host(B.w8a8_gemm_splitk(xq, sx, wd, swd, 4))[-3:])
    for o in outs[1:]:
        assert_bits_equal(o, outs[0], "row invariance")
    xq_o, sx_o = oracle.quantize_act(x[rows], s)
    assert_bits_equal(outs[0], oracle.gemm(xq_o, sx_o, w, sw), "vs oracle")


def test_repeat_runs_identical():
    M, N, K = 333, 555, 1088
    xq, sx, w, sw, r = _gemm_case(M, N, K, seed=5, residual=True)
    args = (dev(xq), dev(sx), dev(w), dev(sw))
    first = host(B.w8a8_gemm(*args, residual=dev(r)))
    for _ in range(5):
        assert_bits_equal(host(B.w8a8_gemm(*args, residual=dev(r))), first, "repeat")


# ------------------------------------------------------------------------ read-out

def test_readout_equals_full_columns_and_oracle():
    V, K, M, C = 5000, 512, 3, 4
    head = synth.lm_head(V=V, K=K, base=55, layer=0)
    rng = np.random.default_rng(56)
    h = rng.standard_normal((40, K), dtype=np.float32)
    answer = np.array([10, 25, 39], np.int32)
    cand = np.stack([rng.choice(V, C, replace=False) for _ in range(M)]).astype(np.int32)
    xq, sx = B.w8a8_quantize_act(dev(h), dev(head["smooth"]), row_idx=dev(answer))
    wd, swd = dev(head["w"]), dev(head["sw"])
    full = host(B.w8a8_gemm(xq, sx, wd, swd))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = host(B.w8a8_readout_candidates(xq, sx, wd, swd, dev(cand), err_flag=flag))
    assert host(flag)[0] == 0
    assert_bits_equal(logits, np.take_along_axis(full, cand.astype(np.int64), 1), "cand vs full")
    xq_o, sx_o = oracle.quantize_act(h, head["smooth"], row_idx=answer)
    want, f = oracle.readout_candidates(xq_o, sx_o, head["w"], head["sw"], cand)
    assert f == 0
    assert_bits_equal(logits, want, "cand vs oracle")


# K <= 18432 runs one workgroup per row (256 threads up to K = 2048, 512
# above), larger K the skinny kernel's gather mode: both, and each launch
# shape's edges
@pytest.mark.parametrize("M,C,K", [(1, 1, 256), (5, 64, 256), (70, 3, 256), (130, 17, 256), (3, 4, 1024),
                                   (2, 5, 2048), (4, 7, 2112), (3, 4, 5120), (6, 33, 18432), (3, 4, 18496),
                                   (5, 64, 20480), (70, 3, 40960)])
def test_readout_shapes(M, C, K):
    V = 3000
    head = synth.lm_head(V=V, K=K, base=57, layer=0)
    rng = np.random.default_rng(M * C)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    sx = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    cand = rng.integers(0, V, (M, C), dtype=np.int32)
    got = host(B.w8a8_readout_candidates(dev(xq), dev(sx), dev(head["w"]), dev(head["sw"]), dev(cand)))
    want, _ = oracle.readout_candidates(xq, sx, head["w"], head["sw"], cand)
    assert_bits_equal(got, want, f"readout M={M} C={C}")


@pytest.mark.parametrize("K", [128, 5120, 20480])
def test_readout_bad_ids_flagged(K):
    V = 1000
    head = synth.lm_head(V=V, K=K, base=58, layer=0)
    rng = np.random.default_rng(1)
    xq = rng.integers(-127, 128, (2, K), dtype=np.int8)
    sx = np.ones(2, np.float32)
    cand = np.array([[1, V, 3], [-5, 7, 999]], np.int32)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = host(B.w8a8_readout_candidates(dev(xq), dev(sx), dev(head["w"]), dev(head["sw"]), dev(cand),
                                         err_flag=flag))
    assert host(flag)[0] == 1
    assert np.isnan(got[0, 1]) and np.isnan(got[1, 0])
    want, f = oracle.readout_candidates(xq, sx, head["w"], head["sw"], cand)
    ok = ~np.isnan(want)
    assert_bits_equal(got[ok], want[ok], "good ids")


def test_readout_rejects_too_many_candidates():
    xq = torch.zeros((1, 64), dtype=torch.int8, device="cuda")
    sx = torch.ones(1, device="cuda")
    w = torch.zeros((100, 64), dtype=torch.int8, device="cuda")
    sw = torch.ones(100, device="cuda")
    cand = torch.zeros((1, 65), dtype=torch.int32, device="cuda")
    with pytest.raises(B.W8A8Error) as e:
        B.w8a8_readout_candidates(xq, sx, w, sw, cand)
    assert e.value.status == B.W8A8_ERR_TOO_MANY_CANDIDATES


def test_host_side_errors_leave_outputs_untouched():
    xq = torch.zeros((4, 96), dtype=torch.int8, device="cuda")       # K = 96: not a multiple of 64
    sx = torch.ones(4, device="cuda")
    w = torch.zeros((8, 96), dtype=torch.int8, device="cuda")
    sw = torch.ones(8, device="cuda")
    y = torch.full((4, 8), 7.0, device="cuda")
    with pytest.raises(B.W8A8Error) as e:
        B.w8a8_gemm(xq, sx, w, sw, y=y)
    assert e.value.status == B.W8A8_ERR_SHAPE
    assert (host(y) == 7.0).all()
