"""The candidate softmax and the end-to-end answer head on the GPU.

The probabilities follow the dsiab.com post, section "方案" (scores of the
candidate tokens only, normalised within the candidate set), in one fixed
sequence of binary64 operations.  Checks:
* every probability within (C + 6) binary64 units in the last place of a
  40-digit decimal softmax (tests/brute.py), the bound include/w8a8.h states;
* within 2^-44 relative of the oracle's numpy softmax;
* exact where binary64 makes the value unique (one candidate, equal logits);
* NaN rows for a non-finite logit, exact zeros on underflow;
* the same bits on every run and whatever rows share the launch;
* w8a8_answer_head equals quantize + candidate read-out + softmax called in
  turn, bit for bit, and the oracle's logits bit for bit.
"""
import math

import numpy as np
import pytest

import oracle
from deterministic_w8a8_int8_amd import synth
from tests.brute import softmax_decimal
from tests.gpu_util import assert_bits_equal, dev, host, say

torch = pytest.importorskip("torch")
B = pytest.importorskip("deterministic_w8a8_int8_amd.binding")

pytestmark = pytest.mark.gpu

ULP64 = 2.0 ** -52


def _logit_rows(seed, M, C, scale):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, C)) * scale).astype(np.float32)


def _check_vs_decimal(logits, probs):
    worst = 0.0
    for m in range(logits.shape[0]):
        ref = softmax_decimal(logits[m])
        C = logits.shape[1]
        for c in range(C):
            r, g = ref[c], probs[m, c]
            if r < 1e-290:
                # underflowed or subnormal: the relative bound does not apply
                assert abs(g - r) <= 1e-300, (m, c, g, r)
                continue
            err = abs(g - r) / r / ULP64
            worst = max(worst, err)
            assert err <= C + 6, f"row {m} cand {c}: {err:.1f} ulp (bound {C + 6})"
    return worst


@pytest.mark.parametrize("C,scale", [(2, 1.0), (4, 3.0), (4, 40.0), (17, 8.0), (64, 5.0), (64, 300.0)])
def test_softmax_within_stated_ulp_bound(C, scale):
    M = 24
    lg = _logit_rows(100 + C, M, C, scale)
    p = host(B.w8a8_candidate_softmax(dev(lg)))
    worst = _check_vs_decimal(lg, p)
    np.testing.assert_allclose(p, oracle.candidate_softmax(lg), rtol=2.0 ** -44, atol=1e-300)
    say(f"softmax C={C} scale={scale}: worst {worst:.2f} ulp against the 40-digit reference")


def test_softmax_exact_cases():
    one = np.array([[0.5], [-3.0], [1e30]], dtype=np.float32)
    p = host(B.w8a8_candidate_softmax(dev(one)))
    assert (p == 1.0).all()
    for C in (2, 3, 4, 7, 64):
        eq = np.full((3, C), 2.75, dtype=np.float32)
        p = host(B.w8a8_candidate_softmax(dev(eq)))
        assert (p == 1.0 / C).all(), C          # exp(0) = 1 exactly, S = C exactly
    # a spread beyond the binary64 range: the small ones are exactly zero
    lg = np.array([[0.0, -800.0, -1e4, -5.0]], dtype=np.float32)
    p = host(B.w8a8_candidate_softmax(dev(lg)))
    assert p[0, 1] == 0.0 and p[0, 2] == 0.0 and p[0, 0] > 0.99
    ref = softmax_decimal(lg[0])
    assert abs(p[0, 3] - ref[3]) <= 6 * ULP64 * ref[3]


def test_softmax_non_finite_rows_are_nan():
    lg = _logit_rows(7, 5, 4, 2.0)
    lg[1, 2] = np.nan
    lg[3, 0] = np.inf
    p = host(B.w8a8_candidate_softmax(dev(lg)))
    assert np.isnan(p[1]).all() and np.isnan(p[3]).all()
    good = [0, 2, 4]
    assert np.isfinite(p[good]).all()
    np.testing.assert_allclose(p[good].sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_softmax_bits_do_not_depend_on_batch_or_run():
    lg = _logit_rows(9, 50, 6, 4.0)
    full = host(B.w8a8_candidate_softmax(dev(lg)))
    again = host(B.w8a8_candidate_softmax(dev(lg)))
    assert np.array_equal(full.view(np.uint64), again.view(np.uint64))
    for m in (0, 17, 49):
        alone = host(B.w8a8_candidate_softmax(dev(lg[m:m + 1])))
        assert np.array_equal(alone.view(np.uint64), full[m:m + 1].view(np.uint64)), m


def test_softmax_host_errors():
    lg = torch.zeros((2, 65), dtype=torch.float32, device="cuda")
    with pytest.raises(B.W8A8Error):
        B.w8a8_candidate_softmax(lg)
    e = torch.zeros((0, 4), dtype=torch.float32, device="cuda")
    assert B.w8a8_candidate_softmax(e).shape == (0, 4)


def _answer_head_case():
    head = synth.lm_head(V=30000, K=1024)
    rng = np.random.default_rng(77)
    h = rng.standard_normal((40, 1024)).astype(np.float32)
    h[:, ::53] *= 25.0
    rows = np.array([39, 5, 17], dtype=np.int32)
    cand = np.stack([rng.choice(30000, 5, replace=False) for _ in range(3)]).astype(np.int32)
    return head, h, rows, cand


def test_answer_head_matches_separate_calls_and_oracle():
    head, h, rows, cand = _answer_head_case()
    hd, rd, sd = dev(h), dev(rows), dev(head["smooth"])
    wd, swd, cd = dev(head["w"]), dev(head["sw"]), dev(cand)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits, probs = B.w8a8_answer_head(hd, rd, sd, wd, swd, cd, err_flag=err)
    xq, sx = B.w8a8_quantize_act(hd, sd, row_idx=rd)
    lg2 = B.w8a8_readout_candidates(xq, sx, wd, swd, cd)
    pr2 = B.w8a8_candidate_softmax(lg2)
    assert_bits_equal(host(logits), host(lg2), "answer head logits vs separate calls")
    assert np.array_equal(host(probs).view(np.uint64), host(pr2).view(np.uint64))
    assert int(host(err)[0]) == 0
    # against the oracle: gather, quantise, read out (bits), softmax (bound)
    oxq, osx = oracle.quantize_act(h[rows], head["smooth"])
    olg, flag = oracle.readout_candidates(oxq, osx, head["w"], head["sw"], cand)
    assert flag == 0
    assert_bits_equal(host(logits), olg, "answer head logits vs oracle")
    _check_vs_decimal(olg, host(probs))
    np.testing.assert_allclose(host(probs), oracle.candidate_softmax(olg), rtol=2.0 ** -44, atol=0)


def test_answer_head_bad_candidate_marks_row():
    head, h, rows, cand = _answer_head_case()
    cand = cand.copy()
    cand[1, 3] = 30000          # outside the vocabulary
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits, probs = B.w8a8_answer_head(dev(h), dev(rows), dev(head["smooth"]), dev(head["w"]),
                                       dev(head["sw"]), dev(cand), err_flag=err)
    lg, p = host(logits), host(probs)
    assert int(host(err)[0]) & 1
    assert np.isnan(lg[1, 3]) and np.isnan(p[1]).all()
    assert np.isfinite(p[[0, 2]]).all()


def _same_or_both_nan(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return bool(np.all((a.view(np.uint8).reshape(a.shape + (-1,)) == b.view(np.uint8).reshape(b.shape + (-1,))).all(-1)
                       | (np.isnan(a) & np.isnan(b))))


# The answer head runs as one kernel for K <= 18432 (256 threads up to K =
# 2048, 512 above) and as three launches beyond.  Every output (quantised
# rows, token scales, logits, probabilities) must equal the separate calls
# bit for bit, with bad row indices and bad candidate ids, several candidate
# groups (C up to 64) and many answer rows; valid rows' logits must equal the
# oracle's.
@pytest.mark.parametrize("K,C,M", [(256, 1, 1), (1024, 4, 3), (2112, 2, 2), (3072, 3, 4), (5120, 4, 1), (5120, 7, 70), (6144, 64, 5),
                                   (8192, 5, 9), (17408, 4, 3), (40960, 4, 2)])
def test_answer_head_fused_matches_separate_calls(K, C, M):
    say(f"answer head K={K} C={C} M={M}")
    V = 3000
    rng = np.random.default_rng(K + C + M)
    h = rng.standard_normal((M + 7, K)).astype(np.float32)
    h[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(30.0)
    smooth = rng.uniform(0.5, 4.0, K).astype(np.float32)
    w = rng.integers(-127, 128, (V, K), dtype=np.int8)
    sw = rng.uniform(1e-3, 1e-2, V).astype(np.float32)
    rows = rng.integers(0, M + 7, M).astype(np.int32)
    cand = np.stack([rng.choice(V, C, replace=False) for _ in range(M)]).astype(np.int32)
    if M > 1:
        rows[1] = -1                    # a row that cannot be read: sx NaN, codes 0, NaN logits
        cand[0, C - 1] = V + 5          # a candidate outside the vocabulary
    d = {k: dev(v) for k, v in dict(h=h, rows=rows, smooth=smooth, w=w, sw=sw, cand=cand).items()}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    logits, probs = B.w8a8_answer_head(d["h"], d["rows"], d["smooth"], d["w"], d["sw"], d["cand"], xq=xq, sx=sx,
                                       err_flag=err)
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    xq2, sx2 = B.w8a8_quantize_act(d["h"], d["smooth"], row_idx=d["rows"])
    lg2 = B.w8a8_readout_candidates(xq2, sx2, d["w"], d["sw"], d["cand"], err_flag=err2)
    pr2 = B.w8a8_candidate_softmax(lg2)
    assert np.array_equal(host(xq), host(xq2))
    assert _same_or_both_nan(host(sx), host(sx2))
    assert _same_or_both_nan(host(logits), host(lg2))
    assert _same_or_both_nan(host(probs), host(pr2))
    assert int(host(err)[0]) == int(host(err2)[0]) == (1 if M > 1 else 0)
    ok = rows >= 0
    oxq, osx = oracle.quantize_act(h[rows[ok]], smooth)
    assert np.array_equal(host(xq)[ok], oxq)
    good = cand.copy()
    good[good >= V] = 0
    olg, _ = oracle.readout_candidates(oxq, osx, w, sw, good[ok])
    lg = host(logits)[ok]
    valid_c = (cand[ok] < V)
    assert_bits_equal(lg[valid_c], olg[valid_c], "fused answer head logits vs oracle")
    rows_ok = valid_c.all(1)
    if rows_ok.any():
        np.testing.assert_allclose(host(probs)[ok][rows_ok], oracle.candidate_softmax(olg[rows_ok]),
                                   rtol=2.0 ** -44, atol=0)
