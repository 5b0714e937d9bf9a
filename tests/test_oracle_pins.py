"""Pins for the CPU oracle, checked against things other than the oracle.

The sources are:
* hand-derived golden fixtures (tests/golden);
* exact rational brute force (tests/brute.py) that rounds each binary32
  step from the IEEE definition;
* Python-int dot products;
* closed forms (all-127 rows, alternating signs, identity weights,
  power-of-two scales);
* invariants (split-K, batch composition, column order, row gather);
* the candidate softmax identity on the dsiab.com post, section "方案".

The layer is defined on the review page "StartLux-Prism: Fast, exact
inference for StartLux-Decision models on NVIDIA GPUs".  Section "Compute
shared evidence once" covers SmoothQuant and per-token W8A8.  Section
"Bitwise consistency is not lossless quantization" covers exact int32
accumulation, integer split-K and fixed-order scaling.
"""
import math

import numpy as np
import pytest

import oracle
import brute
from conftest import read_golden
from deterministic_w8a8_int8_amd import synth


def bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ----------------------------------------------------------- brute-force self-check

def test_round_f32_agrees_with_ieee_hardware_on_simple_quotients():
    # Independent implementations must agree: integer-only rounding vs the
    # host's IEEE binary32 division of small integers (both exact inputs).
    rng = np.random.default_rng(7)
    for _ in range(2000):
        p, q = int(rng.integers(-10**6, 10**6)), int(rng.integers(1, 10**6))
        want = np.float32(p) / np.float32(q)
        assert brute.round_f32(brute.Fraction(p, q)) == float(want)


def test_round_f32_edges():
    F = brute.Fraction
    assert brute.round_f32(F(2 ** 24 + 1)) == 2.0 ** 24           # tie -> even
    assert brute.round_f32(F(2 ** 24 + 3)) == 2.0 ** 24 + 4
    assert brute.round_f32(F(1, 2 ** 150)) == 0.0                  # half of min subnormal -> 0 (even)
    assert brute.round_f32(F(3, 2 ** 151)) == 2.0 ** -149          # 0.75 ulp -> 1 ulp
    assert brute.round_f32(F(3, 2 ** 150)) == 2.0 ** -148          # 1.5 ulp -> 2 (even)


# ------------------------------------------------------------------- quantisation

def _golden_rows(name):
    g = read_golden(name)
    xs = [np.array(v, dtype=np.float32) for v in g["x"]]
    qs = [np.array(v, dtype=np.int64) for v in g["q"]]
    return list(zip(xs, qs))


def test_quantize_round_half_even_golden():
    for x, q_want in _golden_rows("rne_ties.txt"):
        K = 64
        row = np.zeros((1, K), dtype=np.float32)
        row[0, :x.size] = x
        xq, sx = oracle.quantize_act(row, np.ones(K, np.float32))
        assert sx[0] in (1.0, 2.0)
        np.testing.assert_array_equal(xq[0, :x.size].astype(np.int64), q_want)
        assert not xq[0, x.size:].any()


def test_quantize_integer_rows_are_identity():
    # s = 1, integer x in [-127,127] with |x| = 127 present: sx = 1, q = x.
    rng = np.random.default_rng(11)
    x = rng.integers(-127, 128, size=(9, 320)).astype(np.float32)
    x[np.arange(9), rng.integers(0, 320, 9)] = rng.choice([-127.0, 127.0], 9)
    xq, sx = oracle.quantize_act(x, np.ones(320, np.float32))
    np.testing.assert_array_equal(sx, np.ones(9, np.float32))
    np.testing.assert_array_equal(xq.astype(np.float32), x)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantize_matches_exact_rational_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    M, K = 6, 64
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, [3, 17]] *= np.float32(30.0)                    # outlier channels
    x[2] = 0.0                                           # all-zero row: sx = 0, q = 0
    x[3] = 0.0
    x[3, 5] = np.float32(1e-44)                          # amax/127 underflows to 0
    x[4] = 0.0
    x[4, 9] = np.float32(-2.5e-40)                       # subnormal max, sx subnormal
    x[4, 10] = np.float32(1.1e-40)
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    xq, sx = oracle.quantize_act(x, s)
    for m in range(M):
        q_want, sx_want = brute.quantize_row(x[m], s)
        assert brute.f32_bits(sx_want) == int(bits(sx[m])), m
        np.testing.assert_array_equal(xq[m].astype(np.int64), np.array(q_want), err_msg=f"row {m}")
    assert sx[2] == 0 and not xq[2].any()
    assert sx[3] == 0 and not xq[3].any()
    assert sx[4] > 0 and xq[4, 9] == -127


def test_quantize_scale_and_quotient_bruteforce_many_rows():
    # Thousands of rows whose maxima span many binades: sx = fl(amax/127) and
    # q = rne(fl(x'/sx)) against exact rational rounding, element by element
    # for a sample of rows.  (x'/sx and the scale are where a reciprocal
    # multiply would silently differ from a true division.)
    rng = np.random.default_rng(41)
    M, K = 3000, 64
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-20, 20, (M, 1)))).astype(np.float32)
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    xq, sx = oracle.quantize_act(x, s)
    F = brute.Fraction
    xs = [[brute.round_f32(brute.f32(x[m, k]) / brute.f32(s[k])) for k in range(K)] for m in range(M)]
    for m in range(M):
        amax = max(abs(v) for v in xs[m])
        assert brute.f32_bits(brute.round_f32(F(amax) / 127)) == int(bits(sx[m])), m
    for m in range(0, M, 25):
        q_want, _ = brute.quantize_row(x[m], s)
        np.testing.assert_array_equal(xq[m].astype(np.int64), np.array(q_want), err_msg=f"row {m}")


def _nonfinite_rows():
    """Rows of every non-finite kind next to ordinary ones: NaN, +Inf, -Inf
    inputs, a finite input whose smoothed value overflows (3e38 / 0.25), and
    a finite one just inside the range (3e38 / 1)."""
    rng = np.random.default_rng(77)
    K = 64
    x = rng.standard_normal((8, K)).astype(np.float32)
    s = rng.uniform(0.5, 4.0, K).astype(np.float32)
    s[5] = np.float32(0.25)
    s[6] = np.float32(1.0)
    x[1, 9] = np.nan
    x[2, 0] = np.inf
    x[3, 63] = -np.inf
    x[4, 5] = np.float32(3e38)     # / 0.25 overflows
    x[5, 6] = np.float32(3e38)     # / 1 stays finite: an ordinary (huge) row
    x[6, 9] = np.nan
    x[6, 10] = np.inf
    return x, s


def test_quantize_nonfinite_rows_bruteforce():
    # A row with a non-finite smoothed value has no scale (the reading: like
    # a row that cannot be read): sx = NaN, all codes 0.  Every row, finite
    # or not, against the exact-rational reference; the other rows do not
    # change.
    x, s = _nonfinite_rows()
    xq, sx = oracle.quantize_act(x, s)
    for m in range(x.shape[0]):
        q_want, sx_want = brute.quantize_row(x[m], s)
        if math.isnan(sx_want):
            assert np.isnan(sx[m]), m
        else:
            assert brute.f32_bits(sx_want) == int(bits(sx[m])), m
        np.testing.assert_array_equal(xq[m].astype(np.int64), np.array(q_want), err_msg=f"row {m}")
    assert [m for m in range(8) if np.isnan(sx[m])] == [1, 2, 3, 4, 6]
    assert sx[5] > 0 and xq[5, 6] == 127
    ok = [0, 5, 7]
    xq_ok, sx_ok = oracle.quantize_act(x[ok], s)
    np.testing.assert_array_equal(xq[ok], xq_ok)
    np.testing.assert_array_equal(bits(sx[ok]), bits(sx_ok))


def test_quantize_column_order_invariance():
    d = synth.tiny_linear()
    x, s = d["x"], d["smooth"]
    perm = np.random.default_rng(3).permutation(x.shape[1])
    xq, sx = oracle.quantize_act(x, s)
    xq_p, sx_p = oracle.quantize_act(np.ascontiguousarray(x[:, perm]), s[perm])
    np.testing.assert_array_equal(bits(sx), bits(sx_p))
    np.testing.assert_array_equal(xq[:, perm], xq_p)


def test_quantize_row_gather_equals_gather_after():
    d = synth.tiny_linear()
    idx = np.array([15, 0, 7, 7, 3], dtype=np.int32)
    xq, sx = oracle.quantize_act(d["x"], d["smooth"])
    xq_g, sx_g = oracle.quantize_act(d["x"], d["smooth"], row_idx=idx)
    np.testing.assert_array_equal(xq[idx], xq_g)
    np.testing.assert_array_equal(bits(sx[idx]), bits(sx_g))


def test_quantize_strided_rows():
    d = synth.tiny_linear()
    wide = np.zeros((16, 320), dtype=np.float32)
    wide[:, 32:288] = d["x"]
    xq, sx = oracle.quantize_act(d["x"], d["smooth"])
    xq2, sx2 = oracle.quantize_act(wide[:, 32:288], d["smooth"])
    np.testing.assert_array_equal(xq, xq2)
    np.testing.assert_array_equal(bits(sx), bits(sx2))


# --------------------------------------------------------------------- integer GEMM

def test_gemm_acc_matches_python_int():
    rng = np.random.default_rng(5)
    M, N, K = 5, 7, 192
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    acc = oracle.gemm_acc(xq, w)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == brute.dot(xq[m].tolist(), w[n].tolist())


def test_gemm_acc_closed_forms():
    K = 17408
    ones = np.full((1, K), 127, np.int8)
    assert oracle.gemm_acc(ones, ones)[0, 0] == K * 127 * 127 == 280773632
    alt = np.tile(np.array([127, -127], np.int8), K // 2)[None, :]
    assert oracle.gemm_acc(alt, ones)[0, 0] == 0
    rng = np.random.default_rng(9)
    q = rng.integers(-127, 128, (3, 256), dtype=np.int8)
    eye = (127 * np.eye(256)).astype(np.int8)
    np.testing.assert_array_equal(oracle.gemm_acc(q, eye), 127 * q.astype(np.int64))


def test_int32_bound_is_enforced():
    # K * 127^2 < 2^31 holds up to K = 133144.
    ok = np.full((1, 133144), 127, np.int8)
    assert oracle.gemm_acc(ok, ok)[0, 0] == 133144 * 16129 <= 2 ** 31 - 1
    bad = np.full((1, 133145), 127, np.int8)
    with pytest.raises(RuntimeError):
        oracle.gemm_acc(bad, bad)


@pytest.mark.parametrize("K", [64, 256, 704, 5120])
def test_split_k_gives_identical_bits(K):
    rng = np.random.default_rng(K)
    M, N = 4, 33
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sx = rng.uniform(1e-3, 1, M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    y1 = oracle.gemm(xq, sx, w, sw, r, splitk=1)
    for s in (2, 3, 4, 8, 16):
        np.testing.assert_array_equal(bits(y1), bits(oracle.gemm(xq, sx, w, sw, r, splitk=s)))
    ref = np.array([[brute.dot(xq[m].tolist(), w[n].tolist()) for n in range(N)] for m in range(M)])
    np.testing.assert_array_equal(oracle.gemm_acc(xq, w, splitk=8), ref)


# ------------------------------------------------------------------------ epilogue

def test_epilogue_matches_exact_rational_bruteforce():
    rng = np.random.default_rng(21)
    M, N, K = 6, 9, 128
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sx = rng.uniform(1e-3, 0.5, M).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    for res in (r, None):
        y = oracle.gemm(xq, sx, w, sw, res)
        for m in range(M):
            for n in range(N):
                acc = brute.dot(xq[m].tolist(), w[n].tolist())
                want = brute.epilogue(acc, sx[m], sw[n], None if res is None else res[m, n])
                assert brute.f32_bits(want) == int(bits(y[m, n])), (m, n)


def _row_pair_for(acc, K):
    """int8 rows q, w of length K whose exact dot product is ``acc``."""
    sgn = -1 if acc < 0 else 1
    a = abs(acc)
    full, rem = divmod(a, 127 * 127)
    assert full + 2 <= K
    q = np.zeros(K, np.int8)
    w = np.zeros(K, np.int8)
    q[:full + 2] = 127
    w[:full] = 127 * sgn
    q[full + 1] = 1
    w[full] = sgn * (rem // 127)
    w[full + 1] = sgn * (rem % 127)
    assert brute.dot(q.tolist(), w.tolist()) == acc
    return q, w


def test_epilogue_int32_to_f32_golden():
    g = read_golden("int32_to_f32.txt")
    accs = [int(v) for v in g["acc"][0]]
    ys = [float(v) for v in g["y"][0]]
    K = 133184
    for acc, y_want in zip(accs, ys):
        q, w = _row_pair_for(acc, K)
        y = oracle.gemm(q[None], np.ones(1, np.float32), w[None], np.ones(1, np.float32))
        assert float(y[0, 0]) == y_want, acc


def test_epilogue_power_of_two_scales_closed_form():
    # sx = 2^-7, sw = 2^-9: both products are exact, so y = fl(acc * 2^-16 + r).
    rng = np.random.default_rng(23)
    M, N, K = 4, 16, 256
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    r = rng.standard_normal((M, N)).astype(np.float32)
    y = oracle.gemm(xq, np.full(M, 2.0 ** -7, np.float32), w, np.full(N, 2.0 ** -9, np.float32), r)
    acc = xq.astype(np.int64) @ w.astype(np.int64).T
    for m in range(M):
        for n in range(N):
            exact = brute.Fraction(int(acc[m, n]), 2 ** 16) + brute.f32(r[m, n])
            assert float(y[m, n]) == brute.round_f32(exact)


def test_golden_tiny_layer():
    g = read_golden("tiny_layer.txt")
    K = int(g["K"][0][0])
    s = np.ones(K, np.float32)
    s[0] = float(g["smooth0"][0][0])
    x = np.zeros((2, K), np.float32)
    for i, key in enumerate(("x0", "x1")):
        v = np.array(g[key][0], np.float32)
        x[i, :v.size] = v
    w = np.zeros((2, K), np.int8)
    for i, key in enumerate(("w0", "w1")):
        v = np.array(g[key][0], np.int64)
        w[i, :v.size] = v
    sw = np.array(g["sw"][0], np.float32)
    r = np.array([g["r0"][0], g["r1"][0]], np.float32)
    xq, sx = oracle.quantize_act(x, s)
    for i, key in enumerate(("q0", "q1")):
        v = np.array(g[key][0], np.int64)
        np.testing.assert_array_equal(xq[i, :v.size], v)
        assert not xq[i, v.size:].any()
    np.testing.assert_array_equal(sx, np.array(g["sx"][0], np.float32))
    np.testing.assert_array_equal(oracle.gemm_acc(xq, w).ravel(), np.array(g["acc"][0], np.int64))
    y = oracle.gemm(xq, sx, w, sw, r)
    np.testing.assert_array_equal(y.ravel(), np.array(g["y"][0], np.float32))


# ----------------------------------------------------------------- batch invariance

def test_rows_do_not_depend_on_batch_composition():
    reqs, layer = synth.invariance_requests(n_req=5, lo=3, hi=9, K=256, N=48)
    s, w, sw = layer["smooth"], layer["w"], layer["sw"]
    alone = []
    for x in reqs:
        xq, sx = oracle.quantize_act(x, s)
        alone.append(oracle.gemm(xq, sx, w, sw))
    for k in range(3):
        xa, starts = synth.arrangement(reqs, k, align=16)
        xq, sx = oracle.quantize_act(xa, s)
        y = oracle.gemm(xq, sx, w, sw, splitk=1 + k)
        for i, x in enumerate(reqs):
            np.testing.assert_array_equal(bits(y[starts[i]:starts[i] + x.shape[0]]), bits(alone[i]))


def test_sampled_equals_full():
    d = synth.tiny_linear()
    xq, sx = oracle.quantize_act(d["x"], d["smooth"])
    y = oracle.gemm(xq, sx, d["w"], d["sw"], d["r"])
    mi, ni = synth.sample_points(np.random.default_rng(1), 16, 256, 50)
    ys = oracle.gemm_sampled(xq, sx, d["w"], d["sw"], mi, ni, residual=d["r"], splitk=4)
    np.testing.assert_array_equal(bits(ys), bits(y[mi, ni]))


# ------------------------------------------------------------------------ read-out

def test_readout_equals_gemm_columns_and_flags_bad_ids():
    head = synth.lm_head(V=3000, K=256)
    rng = np.random.default_rng(4)
    h = rng.standard_normal((5, 256)).astype(np.float32)
    xq, sx = oracle.quantize_act(h, head["smooth"])
    cand = np.stack([rng.choice(3000, 4, replace=False) for _ in range(5)]).astype(np.int32)
    y = oracle.gemm(xq, sx, head["w"], head["sw"])
    logits, flag = oracle.readout_candidates(xq, sx, head["w"], head["sw"], cand)
    assert flag == 0
    np.testing.assert_array_equal(bits(logits), bits(np.take_along_axis(y, cand.astype(np.int64), 1)))
    cand[1, 2] = 3000
    cand[3, 0] = -1
    logits, flag = oracle.readout_candidates(xq, sx, head["w"], head["sw"], cand)
    assert flag == 1 and np.isnan(logits[1, 2]) and np.isnan(logits[3, 0])
    assert np.isfinite(np.delete(logits.ravel(), [1 * 4 + 2, 3 * 4 + 0])).all()


def test_candidate_softmax_closed_forms():
    p = oracle.candidate_softmax(np.full((1, 4), 3.25))
    np.testing.assert_allclose(p, 0.25, rtol=0, atol=1e-16)
    a, b = 1.5, -0.75
    p = oracle.candidate_softmax(np.array([[a, b]]))
    assert abs(p[0, 0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-15


def test_candidate_softmax_identity_small_vocab_bruteforce():
    rng = np.random.default_rng(31)
    V, C = 50, 4
    y = rng.standard_normal((3, V)) * 4
    cand = np.stack([rng.choice(V, C, replace=False) for _ in range(3)])
    p_full, picked = oracle.full_softmax_renormalised(y, cand)
    p_sub = oracle.candidate_softmax(np.take_along_axis(y, cand, 1))
    for m in range(3):
        z = [math.exp(v) for v in y[m]]
        tot = math.fsum(z)
        pick = [z[c] / tot for c in cand[m]]
        ref = [v / math.fsum(pick) for v in pick]
        assert max(abs(a - b) for a, b in zip(ref, p_full[m])) < 1e-14
        assert max(abs(a - b) for a, b in zip(ref, p_sub[m])) < 1e-14
    assert np.abs(p_full - p_sub).max() <= 1e-5


def test_candidate_softmax_identity_on_quantised_logits():
    head = synth.lm_head(V=20000, K=512)
    rng = np.random.default_rng(8)
    h = rng.standard_normal((3, 512)).astype(np.float32)
    xq, sx = oracle.quantize_act(h, head["smooth"])
    y = oracle.gemm(xq, sx, head["w"], head["sw"])
    cand = np.stack([rng.choice(20000, 4, replace=False) for _ in range(3)]).astype(np.int32)
    logits, _ = oracle.readout_candidates(xq, sx, head["w"], head["sw"], cand)
    p_sub = oracle.candidate_softmax(logits)
    p_full, picked = oracle.full_softmax_renormalised(y, cand)
    p_lse = oracle.full_softmax_renormalised_lse(y, cand)
    assert np.abs(p_lse - p_sub).max() <= 1e-5
    ok = (picked > np.finfo(np.float64).tiny).all(axis=1)
    assert np.abs(p_full[ok] - p_sub[ok]).max(initial=0.0) <= 1e-5


# ------------------------------------------------------------- float64 yardstick

def test_reference_fp64_exact_when_quantisation_is_exact():
    # s = 1, integer x with 127 present: q = x and sx = 1 exactly, so the int8
    # path differs from float64 only by the binary32 epilogue roundings.
    rng = np.random.default_rng(12)
    M, K, N = 8, 256, 40
    x = rng.integers(-127, 128, (M, K)).astype(np.float32)
    x[:, 0] = 127
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    r = rng.standard_normal((M, N)).astype(np.float32)
    xq, sx = oracle.quantize_act(x, np.ones(K, np.float32))
    y = oracle.gemm(xq, sx, w, sw, r)
    y64 = oracle.reference_fp64(x, np.ones(K), w, sw, r)
    assert oracle.rel_frobenius(y, y64) < 1e-6
    # the yardstick itself: a transposed or unscaled weight would be far off
    assert oracle.rel_frobenius(y, oracle.reference_fp64(x, np.ones(K), w, np.ones(N), r)) > 0.5


def test_relative_error_on_tiny_layer():
    d = synth.tiny_linear()
    xq, sx = oracle.quantize_act(d["x"], d["smooth"])
    y = oracle.gemm(xq, sx, d["w"], d["sw"], d["r"])
    rel = oracle.rel_frobenius(y, oracle.reference_fp64(d["x"], d["smooth"], d["w"], d["sw"], d["r"]))
    assert rel <= 0.15
    # outlier-free companion input with s = 1 meets the 2e-2 screen
    c = synth.linear(1000, 0, 16, 256, 256, n_out=0, mult=1.0, residual=True, smooth=False)
    xq, sx = oracle.quantize_act(c["x"], c["smooth"])
    y = oracle.gemm(xq, sx, c["w"], c["sw"], c["r"])
    assert oracle.rel_frobenius(y, oracle.reference_fp64(c["x"], c["smooth"], c["w"], c["sw"], c["r"])) <= 2e-2
