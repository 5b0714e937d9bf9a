"""Seeded synthetic inputs with the shapes of a decision-model W8A8 layer.

This module draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Tests, the benchmark and the CPU oracle all take their
inputs from here, so the GPU path and the oracle see the same bytes.

The shapes follow the decision-model workload the StartLux-Prism pages
describe (a 27B model, per-token W8A8 projections, an lm_head over about 248k
vocabulary rows, shared evidence with branching questions): hidden size 5120,
gate+up 34816, down 17408 -> 5120, an attention-like projection 15360, and a
248000-row lm_head.  Every stream comes from
``numpy.random.SeedSequence([base, layer]).spawn(8)``, one child per role in
the fixed order ``ROLES``; a role not used by a layer is simply skipped, so
adding a role never shifts another role's numbers.

Value recipe (all float32 unless stated):
  x        N(0,1); ``n_out`` fixed outlier columns multiplied by ``mult``
  smooth   U(0.5, 4) per input channel
  w        int8 uniform on [-127, 127]
  sw       U(1e-3, 1e-2) per output channel
  r        N(0,1) residual, when the layer writes back into the residual stream
"""
from __future__ import annotations

import numpy as np

ROLES = ("x", "outlier_idx", "smooth", "w", "sw", "r", "cand_len", "perm_pad")

HIDDEN = 5120
GATE_UP = 34816
INTER = 17408
QKV = 15360
VOCAB = 248000


def streams(base: int, layer: int = 0) -> dict:
    kids = np.random.SeedSequence([int(base), int(layer)]).spawn(len(ROLES))
    return {role: np.random.default_rng(k) for role, k in zip(ROLES, kids)}


def outlier_count(K: int, frac: float) -> int:
    return int(round(frac * K))


def activations(rng_x, rng_idx, M: int, K: int, n_out: int, mult: float):
    """x [M,K] float32 N(0,1) with ``n_out`` outlier columns scaled by ``mult``."""
    x = rng_x.standard_normal((M, K), dtype=np.float32)
    idx = np.sort(rng_idx.choice(K, size=n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    if n_out:
        x[:, idx] *= np.float32(mult)
    return x, idx


def linear(base: int, layer: int, M: int, K: int, N: int, *, n_out: int, mult: float,
           residual: bool, smooth: bool = True, x: bool = True) -> dict:
    """One W8A8 linear layer's inputs.

    ``smooth=False`` gives s = 1 (the outlier-free companion inputs use it);
    ``x=False`` skips drawing activations (e.g. the lm_head).
    """
    g = streams(base, layer)
    out = {"M": M, "K": K, "N": N}
    if x:
        out["x"], out["outlier_idx"] = activations(g["x"], g["outlier_idx"], M, K, n_out, mult)
    if smooth:
        out["smooth"] = g["smooth"].uniform(0.5, 4.0, K).astype(np.float32)
    else:
        out["smooth"] = np.ones(K, dtype=np.float32)
    out["w"] = g["w"].integers(-127, 128, size=(N, K), dtype=np.int8)
    out["sw"] = g["sw"].uniform(1e-3, 1e-2, N).astype(np.float32)
    out["r"] = g["r"].standard_normal((M, N), dtype=np.float32) if residual else None
    return out


# ------------------------------------------------------------------ workloads

def tiny_linear() -> dict:
    """16 x 256 -> 256 with 4 outlier channels x20, residual, split-K 1."""
    return linear(1000, 0, 16, 256, 256, n_out=4, mult=20.0, residual=True)


def short_request(layer: str) -> dict:
    """A 256-token request: fused gate+up 5120 -> 34816 (no residual) or down
    17408 -> 5120 (residual); 1% outlier channels x30."""
    if layer == "gate_up":
        return linear(1001, 0, 256, HIDDEN, GATE_UP, n_out=outlier_count(HIDDEN, 0.01),
                      mult=30.0, residual=False)
    if layer == "down":
        return linear(1001, 1, 256, INTER, HIDDEN, n_out=outlier_count(INTER, 0.01),
                      mult=30.0, residual=True)
    raise ValueError(layer)


FOREST_TRUNK = 256
FOREST_BRANCHES = (24, 24, 24)


def forest_rows():
    """Row layout of one evidence trunk followed by its question branches;
    returns (M, answer_rows) where each answer row is the last token of a
    branch."""
    M = FOREST_TRUNK + sum(FOREST_BRANCHES)
    ends, pos = [], FOREST_TRUNK
    for b in FOREST_BRANCHES:
        pos += b
        ends.append(pos - 1)
    return M, np.asarray(ends, dtype=np.int32)


def forest_batch(layer: str) -> dict:
    """Shared-evidence batch (256 trunk + 3 x 24 question rows = 328)."""
    M, _ = forest_rows()
    if layer == "qkv":
        return linear(1002, 0, M, HIDDEN, QKV, n_out=outlier_count(HIDDEN, 0.01), mult=30.0,
                      residual=False)
    if layer == "gate_up":
        return linear(1002, 1, M, HIDDEN, GATE_UP, n_out=outlier_count(HIDDEN, 0.01), mult=30.0,
                      residual=False)
    raise ValueError(layer)


def lm_head(V: int = VOCAB, K: int = HIDDEN, base: int = 1002, layer: int = 2) -> dict:
    """int8 lm_head [V,K], its per-row scale and its smoothing vector."""
    return linear(base, layer, 0, K, V, n_out=0, mult=1.0, residual=False, x=False)


def readout_inputs(n_cand: int = 4, V: int = VOCAB, K: int = HIDDEN) -> dict:
    """Hidden rows of the forest batch and C distinct candidate ids per answer
    row, uniform over [0, V)."""
    M, answer_rows = forest_rows()
    g = streams(1002, 3)
    h, idx = activations(g["x"], g["outlier_idx"], M, K, outlier_count(K, 0.01), 30.0)
    cand = np.stack([g["cand_len"].choice(V, size=n_cand, replace=False)
                     for _ in range(len(answer_rows))]).astype(np.int32)
    return {"h": h, "answer_rows": answer_rows, "cand": cand}


def long_prefill(layer: str, M: int = 8192) -> dict:
    """Long evidence prefill: gate+up 5120 -> 34816 and down 17408 -> 5120
    (residual) at M tokens; 1% outlier channels x30."""
    if layer == "gate_up":
        return linear(1003, 0, M, HIDDEN, GATE_UP, n_out=outlier_count(HIDDEN, 0.01), mult=30.0,
                      residual=False)
    if layer == "down":
        return linear(1003, 1, M, INTER, HIDDEN, n_out=outlier_count(INTER, 0.01), mult=30.0,
                      residual=True)
    raise ValueError(layer)


def invariance_requests(n_req: int = 64, lo: int = 32, hi: int = 512, K: int = HIDDEN,
                        N: int = QKV, base: int = 1004):
    """Requests of lengths U{lo..hi} with shared outlier columns, and the
    weight of a K -> N layer.  Returns (requests, layer) where requests is a
    list of float32 [len_i, K] arrays."""
    g = streams(base, 0)
    lens = g["cand_len"].integers(lo, hi + 1, size=n_req)
    x, idx = activations(g["x"], g["outlier_idx"], int(lens.sum()), K, outlier_count(K, 0.01), 30.0)
    offs = np.concatenate([[0], np.cumsum(lens)])
    reqs = [x[offs[i]:offs[i + 1]] for i in range(n_req)]
    layer = linear(base, 1, 0, K, N, n_out=0, mult=1.0, residual=False, x=False)
    return reqs, layer


def arrangement(reqs, k: int, base: int = 1004, max_pad: int = 15, align: int = 256):
    """The k-th arrangement of the requests: a random order, 0..max_pad
    random-valued pad rows after each request, and random pad rows at the end
    up to a multiple of ``align``.  Returns (x [M,K], starts) where starts[i]
    is the first row of request i in x."""
    g = streams(base, 100 + k)
    rng = g["perm_pad"]
    n = len(reqs)
    K = reqs[0].shape[1]
    order = rng.permutation(n)
    pads = rng.integers(0, max_pad + 1, size=n)
    blocks, starts, pos = [], np.zeros(n, dtype=np.int64), 0
    for j, i in enumerate(order):
        starts[i] = pos
        blocks.append(reqs[i])
        pos += reqs[i].shape[0]
        if pads[j]:
            blocks.append(rng.standard_normal((int(pads[j]), K), dtype=np.float32) * np.float32(8.0))
            pos += int(pads[j])
    tail = (-pos) % align
    if tail:
        blocks.append(rng.standard_normal((tail, K), dtype=np.float32) * np.float32(8.0))
        pos += tail
    return np.concatenate(blocks, axis=0), starts


def block_points(rng, M: int, N: int, bm: int, bn: int):
    """One random output coordinate inside every bm x bn block of an M x N
    output (the ragged edge blocks included), so that a sampled check touches
    every tile and every per-wave sub-tile of a blocked kernel."""
    rb, cb = -(-M // bm), -(-N // bn)
    r0 = np.repeat(np.arange(rb, dtype=np.int64) * bm, cb)
    c0 = np.tile(np.arange(cb, dtype=np.int64) * bn, rb)
    hr = np.minimum(bm, M - r0)
    hc = np.minimum(bn, N - c0)
    mi = r0 + (rng.random(r0.size) * hr).astype(np.int64)
    ni = c0 + (rng.random(c0.size) * hc).astype(np.int64)
    return mi, ni


def sample_points(rng, M: int, N: int, count: int, must_rows=(), must_cols=()):
    """Sampled output coordinates: random ones plus the corners and the given
    rows/columns' first entries, for checking huge outputs one by one."""
    mi = list(rng.integers(0, M, size=count))
    ni = list(rng.integers(0, N, size=count))
    for m in (0, M - 1, *must_rows):
        for n in (0, N - 1, *must_cols):
            mi.append(m)
            ni.append(n)
    return np.asarray(mi, dtype=np.int64), np.asarray(ni, dtype=np.int64)
