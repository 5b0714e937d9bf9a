"""GPU parity at the workload sizes of the decision-model layer.

Each case runs the C-ABI path at full size.  The oracle cannot afford every
output of these shapes, so the checks are:
* every quantised activation and token scale, bit for bit;
* whole output rows, several thousand random outputs and one output in
  every 16 x 16 or 32 x 32 output block (so every tile and every wave's
  sub-tile), bit for bit against the oracle, computed one by one;
* properties that hold at any size: split-K, batch arrangement, padding and
  forest branches, each bitwise equal to the reference run, and candidate
  logits bitwise equal to the full-vocabulary columns;
* the candidate softmax identity in float64 (dsiab.com post, section
  "方案"), and the relative Frobenius error against the unquantised float64
  layer on sampled rows.

The layer is defined on the review page "StartLux-Prism: Fast, exact
inference for StartLux-Decision models on NVIDIA GPUs".  Section "Compute
shared evidence once" covers SmoothQuant and per-token W8A8.  Section
"Bitwise consistency is not lossless quantization" covers exact int32,
integer split-K and the fixed rounding sequence.
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

N_SAMPLES = 3000


def check_layer(d, *, splits=(1,), rows_full=2, seed=0, label=""):
    """Quantise + GEMM a layer on the GPU and check it against the oracle.
    Returns the device output of the split-K 1 run."""
    M, K, N = d["M"], d["K"], d["N"]
    say(f"{label}: M={M} K={K} N={N} splits={splits}")
    x_d, s_d = dev(d["x"]), dev(d["smooth"])
    w_d, sw_d, r_d = dev(d["w"]), dev(d["sw"]), dev(d["r"])
    xq, sx = B.w8a8_quantize_act(x_d, s_d)
    xq_o, sx_o = oracle.quantize_act(d["x"], d["smooth"])
    assert_bits_equal(host(sx), sx_o, f"{label} sx")
    assert np.array_equal(host(xq), xq_o), f"{label} xq differs"
    y1 = B.w8a8_gemm(xq, sx, w_d, sw_d, residual=r_d)
    for s in splits:
        if s == 1:
            continue
        ys = B.w8a8_gemm_splitk(xq, sx, w_d, sw_d, s, residual=r_d)
        assert torch.equal(ys.view(torch.int32), y1.view(torch.int32)), f"{label} split {s} differs"
        del ys
    rng = np.random.default_rng(seed)
    mi, ni = synth.sample_points(rng, M, N, N_SAMPLES)
    # plus one output in every 16 x 16 block (the skinny and panel kernels'
    # row groups and 16-column wave strips) or 32 x 32 block (the tiled
    # kernel's per-wave MFMA tiles), so every tile is touched
    blk = 32 if B.w8a8_gemm_plan(M, N, K, 1, d["r"] is not None)[0] == 1 else 16
    bi, bj = synth.block_points(rng, M, N, blk, blk)
    mi, ni = np.concatenate([mi, bi]), np.concatenate([ni, bj])
    say(f"{label}: {mi.size} sampled outputs")
    got = host(y1[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()])
    want = oracle.gemm_sampled(xq_o, sx_o, d["w"], d["sw"], mi, ni, residual=d["r"])
    assert_bits_equal(got, want, f"{label} sampled")
    rows = rng.choice(M, rows_full, replace=False)
    for m in rows:
        want_row = oracle.gemm(xq_o[m:m + 1], sx_o[m:m + 1], d["w"], d["sw"],
                               None if d["r"] is None else d["r"][m:m + 1])
        assert_bits_equal(host(y1[int(m)]), want_row[0], f"{label} row {m}")
    return y1, rows


def rel_error_rows(d, y_rows, rows):
    """Relative Frobenius error of the given output rows vs the unquantised
    float64 layer."""
    y64 = oracle.reference_fp64(d["x"][rows], d["smooth"], d["w"], d["sw"],
                                None if d["r"] is None else d["r"][rows])
    return oracle.rel_frobenius(y_rows, y64)


def companion(d, base, layer):
    """The same shapes and seeds without outlier channels and with s = 1."""
    return synth.linear(base, layer, d["M"], d["K"], d["N"], n_out=0, mult=1.0,
                        residual=d["r"] is not None, smooth=False)


# ----------------------------------------------------------------------- tiny

def test_tiny_linear_full():
    d = synth.tiny_linear()
    xq, sx = B.w8a8_quantize_act(dev(d["x"]), dev(d["smooth"]))
    y = host(B.w8a8_gemm(xq, sx, dev(d["w"]), dev(d["sw"]), residual=dev(d["r"])))
    xq_o, sx_o = oracle.quantize_act(d["x"], d["smooth"])
    assert_bits_equal(y, oracle.gemm(xq_o, sx_o, d["w"], d["sw"], d["r"]), "tiny")
    rel = oracle.rel_frobenius(y, oracle.reference_fp64(d["x"], d["smooth"], d["w"], d["sw"], d["r"]))
    say(f"tiny relF vs fp64 (literal inputs) = {rel:.4f}")
    assert rel <= 0.15


# --------------------------------------------------------------- short request

@pytest.mark.parametrize("layer", ["gate_up", "down"])
def test_short_request(layer):
    d = synth.short_request(layer)
    y, rows = check_layer(d, splits=(1, 2, 4, 8), seed=11, label=f"short {layer}")
    rel = rel_error_rows(d, host(y[torch.from_numpy(rows).cuda()]), rows)
    say(f"short {layer} relF (literal, sampled rows) = {rel:.4f}")
    assert rel <= 0.15
    c = companion(d, 1001, 0 if layer == "gate_up" else 1)
    xq, sx = B.w8a8_quantize_act(dev(c["x"][:8]), dev(c["smooth"]))
    yc = host(B.w8a8_gemm(xq, sx, dev(c["w"]), dev(c["sw"]),
                          residual=None if c["r"] is None else dev(c["r"][:8])))
    relc = rel_error_rows(c, yc, np.arange(8))
    say(f"short {layer} relF (outlier-free companion, s=1) = {relc:.4f}")
    assert relc <= 2e-2


# ------------------------------------------------------------- forest + read-out

def test_forest_projections_and_branch_invariance():
    M, answers = synth.forest_rows()
    for layer in ("qkv", "gate_up"):
        d = synth.forest_batch(layer)
        y, _ = check_layer(d, seed=21, label=f"forest {layer}")
        # each question branch alone with its trunk (a request of its own)
        s_d, w_d, sw_d = dev(d["smooth"]), dev(d["w"]), dev(d["sw"])
        start = synth.FOREST_TRUNK
        for b in synth.FOREST_BRANCHES:
            rows = np.r_[0:synth.FOREST_TRUNK, start:start + b]
            xq, sx = B.w8a8_quantize_act(dev(d["x"][rows]), s_d)
            alone = B.w8a8_gemm(xq, sx, w_d, sw_d)
            idx = torch.from_numpy(rows).cuda()
            assert torch.equal(alone.view(torch.int32), y[idx].view(torch.int32)), f"branch at {start}"
            start += b
        del y


@pytest.fixture(scope="module")
def lm_head():
    say("generating the 248000 x 5120 lm_head")
    return synth.lm_head()


def test_readout_candidates_full_vocab(lm_head):
    rd = synth.readout_inputs()
    head = lm_head
    wd, swd = dev(head["w"]), dev(head["sw"])
    h_d = dev(rd["h"])
    ans = rd["answer_rows"]
    # gather-then-quantise equals quantise-then-gather
    xq, sx = B.w8a8_quantize_act(h_d, dev(head["smooth"]), row_idx=dev(ans))
    xq_all, sx_all = B.w8a8_quantize_act(h_d, dev(head["smooth"]))
    idx = torch.from_numpy(ans.astype(np.int64)).cuda()
    assert torch.equal(xq, xq_all[idx]) and torch.equal(sx.view(torch.int32), sx_all[idx].view(torch.int32))
    say("full-vocabulary skinny GEMM 3 x 248000 x 5120")
    y_full = B.w8a8_gemm(xq, sx, wd, swd)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    cand = rd["cand"]
    logits = B.w8a8_readout_candidates(xq, sx, wd, swd, dev(cand), err_flag=flag)
    assert host(flag)[0] == 0
    cidx = torch.from_numpy(cand.astype(np.int64)).cuda()
    assert torch.equal(logits.view(torch.int32), torch.gather(y_full, 1, cidx).view(torch.int32))
    xq_o, sx_o = oracle.quantize_act(rd["h"], head["smooth"], row_idx=ans)
    want, f = oracle.readout_candidates(xq_o, sx_o, head["w"], head["sw"], cand)
    assert f == 0
    assert_bits_equal(host(logits), want, "candidate logits")
    rng = np.random.default_rng(31)
    mi, ni = synth.sample_points(rng, 3, head["N"], N_SAMPLES)
    got = host(y_full[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()])
    assert_bits_equal(got, oracle.gemm_sampled(xq_o, sx_o, head["w"], head["sw"], mi, ni),
                      "full-vocabulary sampled")
    # candidate softmax == full softmax renormalised over the candidates
    yf = host(y_full).astype(np.float64)
    p_sub = oracle.candidate_softmax(host(logits))
    p_full, picked = oracle.full_softmax_renormalised(yf, cand)
    p_lse = oracle.full_softmax_renormalised_lse(yf, cand)
    ok = (picked > np.finfo(np.float64).tiny).all(axis=1)
    say(f"softmax identity: literal form usable on {ok.sum()} of 3 rows; "
        f"max diff {np.abs(p_lse - p_sub).max():.2e}")
    assert np.abs(p_lse - p_sub).max() <= 1e-5
    if ok.any():
        assert np.abs(p_full[ok] - p_sub[ok]).max() <= 1e-5


# ---------------------------------------------------------- long-evidence prefill

def test_long_prefill_gate_up():
    d = synth.long_prefill("gate_up")
    y, rows = check_layer(d, seed=41, label="prefill gate_up")
    rel = rel_error_rows(d, host(y[torch.from_numpy(rows).cuda()]), rows)
    say(f"prefill gate_up relF (literal, sampled rows) = {rel:.4f}")
    assert rel <= 0.15
    del y


def test_long_prefill_down_splitk():
    d = synth.long_prefill("down")
    y, rows = check_layer(d, splits=(1, 2, 4, 8), seed=43, label="prefill down")
    rel = rel_error_rows(d, host(y[torch.from_numpy(rows).cuda()]), rows)
    say(f"prefill down relF (literal, sampled rows) = {rel:.4f}")
    assert rel <= 0.15
    del y


# --------------------------------------------------------- batch-invariance stress

def test_batch_invariance_stress():
    reqs, layer = synth.invariance_requests()
    K, N = layer["K"], layer["N"]
    s_d, w_d, sw_d = dev(layer["smooth"]), dev(layer["w"]), dev(layer["sw"])
    ref = None
    for k in range(5):
        xa, starts = synth.arrangement(reqs, k)
        say(f"arrangement {k}: M={xa.shape[0]}")
        xq, sx = B.w8a8_quantize_act(dev(xa), s_d)
        for s in (1, 4):
            y = B.w8a8_gemm(xq, sx, w_d, sw_d) if s == 1 else B.w8a8_gemm_splitk(xq, sx, w_d, sw_d, s)
            outs = [y[int(starts[i]):int(starts[i]) + reqs[i].shape[0]] for i in range(len(reqs))]
            if ref is None:
                ref = [o.clone() for o in outs]
                canon_xq, canon_sx, canon_starts = host(xq), host(sx), starts
                canon_x, canon_y = xa, y.clone()
            else:
                for i, o in enumerate(outs):
                    assert torch.equal(o.view(torch.int32), ref[i].view(torch.int32)), \
                        f"request {i} differs in arrangement {k} split {s}"
            del y, outs
    # the canonical run against the oracle on sampled rows of every request
    rng = np.random.default_rng(51)
    mi, ni = [], []
    for i, r in enumerate(reqs):
        m = rng.integers(0, r.shape[0], 8)
        mi.append(canon_starts[i] + m)
        ni.append(rng.integers(0, N, 8))
    mi, ni = np.concatenate(mi), np.concatenate(ni)
    xq_rows = canon_xq[mi]
    want = oracle.gemm_sampled(xq_rows, canon_sx[mi], layer["w"], layer["sw"],
                               np.arange(mi.size), ni)
    req_of = np.repeat(np.arange(len(reqs)), 8)
    got = np.array([host(ref[q][int(m - canon_starts[q]), int(n)]) for q, m, n in zip(req_of, mi, ni)],
                   dtype=np.float32)
    assert_bits_equal(got, want, "stress sampled")
    # the whole canonical batch (pad rows included): one output in every
    # 32 x 32 block of the tiled kernel's output, and every quantised row
    M = canon_y.shape[0]
    bi, bj = synth.block_points(np.random.default_rng(52), M, N, 32, 32)
    say(f"stress: {bi.size} block samples over {M}x{N}")
    got = host(canon_y[torch.from_numpy(bi).cuda(), torch.from_numpy(bj).cuda()])
    want = oracle.gemm_sampled(canon_xq, canon_sx, layer["w"], layer["sw"], bi, bj)
    assert_bits_equal(got, want, "stress block samples")
    xq_o, sx_o = oracle.quantize_act(canon_x, layer["smooth"])
    assert_bits_equal(canon_sx, sx_o, "stress sx")
    assert np.array_equal(canon_xq, xq_o), "stress quantised rows differ"
