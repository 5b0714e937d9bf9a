"""The hot path replayed from a captured HIP graph.

Every entry point launches only on the caller's stream and allocates,
synchronises and clears nothing, so a whole step can be captured once per
token bucket and replayed.  The per-request tables (answer rows, candidate
ids) live in device memory and are rewritten between replays without a new
capture.  A graph is replayed several times with eager work and
synchronisations between the replays, and every replay is checked bit for
bit against the eager result of the same inputs.
"""
import numpy as np
import pytest

from deterministic_w8a8_int8_amd import synth
from tests.gpu_util import dev, say

torch = pytest.importorskip("torch")
B = pytest.importorskip("deterministic_w8a8_int8_amd.binding")

pytestmark = pytest.mark.gpu


class ShortRequestStep:
    """One 256-token request through gate+up, down (split-K 4) and the answer
    head, with every buffer allocated up front."""

    def __init__(self):
        gu, dn = synth.short_request("gate_up"), synth.short_request("down")
        head = synth.lm_head(V=50000)
        M, K1, N1, K2, N2 = 256, gu["K"], gu["N"], dn["K"], dn["N"]
        self.x1, self.s1, self.w1, self.sw1 = dev(gu["x"]), dev(gu["smooth"]), dev(gu["w"]), dev(gu["sw"])
        # the down layer's input is the request's own intermediate activations
        self.x2, self.s2, self.w2, self.sw2 = dev(dn["x"]), dev(dn["smooth"]), dev(dn["w"]), dev(dn["sw"])
        self.r2 = dev(dn["r"])
        self.wh, self.swh, self.sh = dev(head["w"]), dev(head["sw"]), dev(head["smooth"])
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
        self.xq1, self.sx1 = e((M, K1), torch.int8), e((M,), torch.float32)
        self.y1 = e((M, N1), torch.float32)
        self.xq2, self.sx2 = e((M, K2), torch.int8), e((M,), torch.float32)
        self.y2 = e((M, N2), torch.float32)
        self.ws = B.splitk_workspace(M, N2, K2, 4)
        self.rows = torch.tensor([M - 1, 100], dtype=torch.int32, device="cuda")
        self.cand = torch.tensor([[3, 17, 4000, 49999], [5, 6, 7, 8]], dtype=torch.int32, device="cuda")
        self.xq3, self.sx3 = e((2, N2), torch.int8), e((2,), torch.float32)
        self.logits, self.probs = e((2, 4), torch.float32), e((2, 4), torch.float64)

    def __call__(self):
        B.w8a8_quantize_act(self.x1, self.s1, xq=self.xq1, sx=self.sx1)
        B.w8a8_gemm(self.xq1, self.sx1, self.w1, self.sw1, y=self.y1)
        B.w8a8_quantize_act(self.x2, self.s2, xq=self.xq2, sx=self.sx2)
        B.w8a8_gemm_splitk(self.xq2, self.sx2, self.w2, self.sw2, 4, residual=self.r2, y=self.y2,
                           workspace=self.ws)
        B.w8a8_answer_head(self.y2, self.rows, self.sh, self.wh, self.swh, self.cand, xq=self.xq3,
                           sx=self.sx3, logits=self.logits, probs=self.probs)

    def outputs(self):
        torch.cuda.synchronize()
        return [t.clone() for t in (self.y1, self.y2, self.logits, self.probs)]


def _same(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


def test_captured_step_replays_bit_identical_with_changing_tables():
    step = ShortRequestStep()
    step()
    eager = step.outputs()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for t in (step.y1, step.y2, step.logits, step.probs):
            t.fill_(float("nan"))                # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        assert _same(step.outputs(), eager), f"replay {rep}"
    # new device tables, same graph: the replay equals an eager step on them
    step.rows.copy_(torch.tensor([0, 255], dtype=torch.int32))
    step.cand.copy_(torch.tensor([[10, 20, 30, 40], [49998, 1, 2, 3]], dtype=torch.int32))
    step()
    eager2 = step.outputs()
    assert not _same(eager2[2:], eager[2:])
    for rep in range(3):
        step.logits.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        assert _same(step.outputs(), eager2), f"replay {rep} with new tables"
    say("graph: 7 replays bit-identical to eager, tables rewritten between them")


def test_token_bucket_graph_serves_requests_of_any_length_against_the_oracle():
    """One capture of a 256-row token bucket serves requests of 100, 200 and
    256 tokens.  Before each replay the request's rows are written into the
    bucket's input buffers (the rows past its length hold random padding) and
    the device tables get the answer row (the request's last token) and its
    candidate ids.  Every replay is checked against the oracle, computed from
    the request's own inputs alone: sampled outputs of its rows of both
    layers, its answer row's whole output rows bit for bit, the candidate
    logits bit for bit and the probabilities within 2^-44 (the review page,
    section "Compute shared evidence once": per-request structure in device
    tables, read-out only at the answer positions)."""
    import oracle
    step = ShortRequestStep()
    gu, dn, head = synth.short_request("gate_up"), synth.short_request("down"), synth.lm_head(V=50000)
    rng = np.random.default_rng(2024)
    cap = 256
    step.rows.copy_(torch.tensor([cap - 1, cap - 1], dtype=torch.int32))
    step()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for L in (100, 200, 256):
        say(f"bucket replay: {L} live rows of {cap}")
        x1 = rng.standard_normal((cap, gu["K"])).astype(np.float32) * np.float32(8.0)   # padding
        x2 = rng.standard_normal((cap, dn["K"])).astype(np.float32) * np.float32(8.0)
        x1[:L], x2[:L] = gu["x"][:L], dn["x"][:L]
        cand = np.stack([rng.choice(50000, 4, replace=False) for _ in range(2)]).astype(np.int32)
        step.x1.copy_(torch.from_numpy(x1))
        step.x2.copy_(torch.from_numpy(x2))
        step.rows.copy_(torch.tensor([L - 1, L // 2], dtype=torch.int32))
        step.cand.copy_(torch.from_numpy(cand))
        for t in (step.y1, step.y2, step.logits, step.probs):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        y1, y2, logits, probs = [t.cpu().numpy() for t in step.outputs()]
        # layer 1: sampled outputs of the live rows and the whole answer row
        mi, ni = synth.sample_points(rng, L, gu["N"], 400, must_rows=(L - 1,))
        xq1, sx1 = oracle.quantize_act(gu["x"][:L], gu["smooth"])
        want = oracle.gemm_sampled(xq1, sx1, gu["w"], gu["sw"], mi, ni)
        assert np.array_equal(y1[mi, ni].view(np.uint32), want.view(np.uint32)), f"L={L} y1 sampled"
        # layer 2 (split-K 4, residual): sampled outputs and the two answer rows
        xq2, sx2 = oracle.quantize_act(dn["x"][:L], dn["smooth"])
        mi, ni = synth.sample_points(rng, L, dn["N"], 400)
        want = oracle.gemm_sampled(xq2, sx2, dn["w"], dn["sw"], mi, ni, residual=dn["r"][:L])
        assert np.array_equal(y2[mi, ni].view(np.uint32), want.view(np.uint32)), f"L={L} y2 sampled"
        ans = np.array([L - 1, L // 2])
        y2_ans = oracle.gemm(xq2[ans], sx2[ans], dn["w"], dn["sw"], dn["r"][ans])
        assert np.array_equal(y2[ans].view(np.uint32), y2_ans.view(np.uint32)), f"L={L} y2 answer rows"
        # answer head on the oracle's own answer rows
        xq3, sx3 = oracle.quantize_act(y2_ans, head["smooth"])
        olg, flag = oracle.readout_candidates(xq3, sx3, head["w"], head["sw"], cand)
        assert flag == 0
        assert np.array_equal(logits.view(np.uint32), olg.view(np.uint32)), f"L={L} logits"
        np.testing.assert_allclose(probs, oracle.candidate_softmax(olg), rtol=2.0 ** -44, atol=0)
