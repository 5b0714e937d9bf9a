"""CPU oracle for the deterministic W8A8 int8 linear layer and candidate read-out.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU product
path (``deterministic_w8a8_int8_amd``) never imports it and shares no code,
header, table or helper with it.

The integer and binary32 stages live in ``w8a8_oracle.c`` (scalar loops,
int64 accumulation, built without floating-point contraction); this module
loads that library with ctypes and adds the float64 stages that the pages
state in float64:

* ``candidate_softmax`` / ``full_softmax_renormalised`` -- the identity on the
  dsiab.com post (section "方案" and its equivalence check under "实现要点"):
  a softmax over the candidate logits equals the full-vocabulary softmax
  restricted to the candidates and renormalised.
* ``reference_fp64`` -- the unquantised layer ``(x/s) @ (w*sw)^T + r`` in
  float64, the yardstick for the relative Frobenius error of the quantised
  path (the review page, section "Bitwise consistency is not lossless
  quantization", stresses that the int8 path is exact, not lossless).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w8a8_oracle.c")
_LIB = os.path.join(_HERE, "libw8a8_oracle.so")

# gcc flags: every binary32 operation stays a separate, correctly rounded op.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-Wall", "-Wextra"]

# Split-K chunks are rounded up to this many K elements (one K-step of 64).
KTILE = 64


def build(force: bool = True) -> str:
    """Compile the oracle library with gcc (the checker, not the product)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def load(path: str) -> ctypes.CDLL:
    """Load an oracle library build and declare its C signatures."""
    L = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.oracle_quantize_act.argtypes = [p, i64, p, p, i64, i64, p, p]
    L.oracle_gemm.argtypes = [p, p, p, p, p, p, i64, i64, i64, i32, i64]
    L.oracle_gemm_sampled.argtypes = [p, p, p, p, p, i64, i64, i64, i32, i64, p, p, i64, p]
    L.oracle_gemm_acc.argtypes = [p, p, i64, i64, i64, i32, i64, p]
    L.oracle_readout_candidates.argtypes = [p, p, i64, i64, p, p, i64, p, i64, p, p]
    L.oracle_row_absmax.argtypes = [p, i64, p, p, i64, i64, p]
    L.oracle_quantize_act_amax.argtypes = [p, i64, p, p, p, i64, i64, p, p]
    L.oracle_epilogue_acc.argtypes = [p, p, p, p, p, i64, i64]
    L.oracle_requantize_q8_0.argtypes = [p, p, p, i64, i64, p, p]
    L.oracle_set_num_threads.argtypes = [i32]
    L.oracle_set_num_threads.restype = None
    for f in ("oracle_quantize_act", "oracle_gemm", "oracle_gemm_sampled", "oracle_gemm_acc",
              "oracle_readout_candidates", "oracle_num_threads", "oracle_row_absmax",
              "oracle_quantize_act_amax", "oracle_epilogue_acc", "oracle_requantize_q8_0"):
        getattr(L, f).restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load(_LIB)
    return _lib


def swap_library(L):
    """Route this module's functions to another build (the mutation tests use
    it to run the pins against deliberately broken copies).  Returns the
    previous library."""
    global _lib
    prev = lib()
    _lib = L
    return prev


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of later calls (each output is computed by one thread
    in a fixed order, so this never changes a bit)."""
    lib().oracle_set_num_threads(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _rows(x):
    """Row-strided binary32 view and its row pitch in elements (numpy may
    report any stride for a dimension of size 1; one row's pitch is K)."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.strides[1] != 4:
        x = np.ascontiguousarray(x)
    return x, (x.strides[0] // 4 if x.shape[0] > 1 else x.shape[1])


def quantize_act(x, smooth, row_idx=None):
    """Per-token int8 quantisation after the SmoothQuant per-channel divide.

    Returns ``(xq int8 [M,K], sx float32 [M])``; with ``row_idx`` the output row
    m is input row ``row_idx[m]``.
    """
    x, ldx = _rows(x)
    K = x.shape[1]
    smooth = _c(smooth, np.float32)
    ri = None if row_idx is None else _c(row_idx, np.int32)
    M = x.shape[0] if ri is None else ri.shape[0]
    xq = np.empty((M, K), dtype=np.int8)
    sx = np.empty((M,), dtype=np.float32)
    _check(lib().oracle_quantize_act(_ptr(x), ldx, _ptr(ri), _ptr(smooth), M, K, _ptr(xq), _ptr(sx)),
           "quantize_act")
    return xq, sx


def row_absmax(x, smooth, row_idx=None):
    """max_k |fl(x[m,k] / smooth[k])| per row (the first two quantisation
    steps on their own, as a rank of a row-parallel layer computes them on
    its K-slice before the exact MAX across ranks)."""
    x, ldx = _rows(x)
    smooth = _c(smooth, np.float32)
    ri = None if row_idx is None else _c(row_idx, np.int32)
    M = x.shape[0] if ri is None else ri.shape[0]
    amax = np.empty((M,), dtype=np.float32)
    _check(lib().oracle_row_absmax(_ptr(x), ldx, _ptr(ri), _ptr(smooth), M, x.shape[1], _ptr(amax)),
           "row_absmax")
    return amax


def quantize_act_amax(x, smooth, amax, row_idx=None):
    """The last two quantisation steps with a given per-token maximum (the
    global one of a row-parallel layer): returns ``(xq, sx)``."""
    x, ldx = _rows(x)
    smooth = _c(smooth, np.float32)
    amax = _c(amax, np.float32)
    ri = None if row_idx is None else _c(row_idx, np.int32)
    M = x.shape[0] if ri is None else ri.shape[0]
    K = x.shape[1]
    xq = np.empty((M, K), dtype=np.int8)
    sx = np.empty((M,), dtype=np.float32)
    _check(lib().oracle_quantize_act_amax(_ptr(x), ldx, _ptr(ri), _ptr(smooth), _ptr(amax), M, K,
                                          _ptr(xq), _ptr(sx)), "quantize_act_amax")
    return xq, sx


def epilogue_acc(acc, sx, sw, residual=None):
    """The fixed binary32 epilogue of given exact accumulators [M,N]."""
    acc = _c(acc, np.int64)
    sx, sw = _c(sx, np.float32), _c(sw, np.float32)
    M, N = acc.shape
    r = None if residual is None else _c(residual, np.float32)
    y = np.empty((M, N), dtype=np.float32)
    _check(lib().oracle_epilogue_acc(_ptr(acc), _ptr(sx), _ptr(sw), _ptr(r), _ptr(y), M, N),
           "epilogue_acc")
    return y


def requantize_q8_0(q, d_bits, smooth):
    """Q8_0 weights (int8 codes q [N,K], binary16 block scales d_bits [N,K/32]
    as uint16 bit patterns) smoothed by ``smooth`` [K] and requantised per
    output channel: returns ``(wq int8 [N,K], sw float32 [N])``."""
    q = _c(q, np.int8)
    d_bits = _c(d_bits, np.uint16)
    smooth = _c(smooth, np.float32)
    N, K = q.shape
    assert d_bits.shape == (N, K // 32) and smooth.shape == (K,)
    wq = np.empty((N, K), dtype=np.int8)
    sw = np.empty((N,), dtype=np.float32)
    _check(lib().oracle_requantize_q8_0(_ptr(q), _ptr(d_bits), _ptr(smooth), N, K, _ptr(wq), _ptr(sw)),
           "requantize_q8_0")
    return wq, sw


def gemm(xq, sx, w, sw, residual=None, splitk=1):
    """Exact int64 accumulation + fixed binary32 epilogue over all outputs."""
    xq, w = _c(xq, np.int8), _c(w, np.int8)
    sx, sw = _c(sx, np.float32), _c(sw, np.float32)
    M, K = xq.shape
    N = w.shape[0]
    assert w.shape[1] == K
    r = None if residual is None else _c(residual, np.float32)
    if r is not None:
        assert r.shape == (M, N)
    y = np.empty((M, N), dtype=np.float32)
    _check(lib().oracle_gemm(_ptr(xq), _ptr(sx), _ptr(w), _ptr(sw), _ptr(r), _ptr(y), M, N, K,
                             int(splitk), KTILE), "gemm")
    return y


def gemm_sampled(xq, sx, w, sw, mi, ni, residual=None, splitk=1):
    """The same definition at sampled outputs: returns y[mi[p], ni[p]]."""
    xq, w = _c(xq, np.int8), _c(w, np.int8)
    sx, sw = _c(sx, np.float32), _c(sw, np.float32)
    M, K = xq.shape
    N = w.shape[0]
    mi, ni = _c(mi, np.int64), _c(ni, np.int64)
    r = None if residual is None else _c(residual, np.float32)
    out = np.empty(mi.shape, dtype=np.float32)
    _check(lib().oracle_gemm_sampled(_ptr(xq), _ptr(sx), _ptr(w), _ptr(sw), _ptr(r), M, N, K,
                                     int(splitk), KTILE, _ptr(mi), _ptr(ni), mi.size, _ptr(out)),
           "gemm_sampled")
    return out


def gemm_acc(xq, w, splitk=1):
    """The exact integer accumulators (int64 container), before the epilogue."""
    xq, w = _c(xq, np.int8), _c(w, np.int8)
    M, K = xq.shape
    N = w.shape[0]
    acc = np.empty((M, N), dtype=np.int64)
    _check(lib().oracle_gemm_acc(_ptr(xq), _ptr(w), M, N, K, int(splitk), KTILE, _ptr(acc)),
           "gemm_acc")
    return acc


def readout_candidates(xq, sx, w_vocab, sw_vocab, cand):
    """Candidate-only logits [M,C]; returns ``(logits, err_flag)``."""
    xq, w_vocab = _c(xq, np.int8), _c(w_vocab, np.int8)
    sx, sw_vocab = _c(sx, np.float32), _c(sw_vocab, np.float32)
    cand = _c(cand, np.int32)
    M, K = xq.shape
    V = w_vocab.shape[0]
    C = cand.shape[1]
    logits = np.empty((M, C), dtype=np.float32)
    flag = np.zeros((1,), dtype=np.int32)
    _check(lib().oracle_readout_candidates(_ptr(xq), _ptr(sx), M, K, _ptr(w_vocab), _ptr(sw_vocab),
                                           V, _ptr(cand), C, _ptr(logits), _ptr(flag)),
           "readout_candidates")
    return logits, int(flag[0])


# ---------------------------------------------------------------- float64 stages

def _softmax64(z):
    """Row softmax in float64 with the row maximum subtracted first."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def candidate_softmax(logits):
    """Softmax over the candidate logits only (the specialised path)."""
    return _softmax64(logits)


def full_softmax_renormalised(y_full, cand):
    """Full-vocabulary softmax, restricted to ``cand`` and renormalised (the
    general path).  Returns ``(p, picked)`` where ``picked`` are the
    full-softmax probabilities at the candidates before renormalising, so the
    caller can check that none of them underflowed."""
    p = _softmax64(y_full)
    cand = np.asarray(cand)
    picked = np.take_along_axis(p, cand.astype(np.int64), axis=-1)
    return picked / picked.sum(axis=-1, keepdims=True), picked


def full_softmax_renormalised_lse(y_full, cand):
    """The same quantity through log-sum-exp, for rows whose candidate
    probabilities underflow float64 in the literal form."""
    y = np.asarray(y_full, dtype=np.float64)
    mx = y.max(axis=-1, keepdims=True)
    lse = mx + np.log(np.exp(y - mx).sum(axis=-1, keepdims=True))
    logp = np.take_along_axis(y, np.asarray(cand).astype(np.int64), axis=-1) - lse
    return _softmax64(logp)


def reference_fp64(x, smooth, w, sw, residual=None):
    """Unquantised float64 layer: (x/s) @ (w*sw)^T (+ r)."""
    xs = np.asarray(x, dtype=np.float64) / np.asarray(smooth, dtype=np.float64)[None, :]
    ws = np.asarray(w, dtype=np.float64) * np.asarray(sw, dtype=np.float64)[:, None]
    y = xs @ ws.T
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)
    return y


def rel_frobenius(y, y64):
    y = np.asarray(y, dtype=np.float64)
    return float(np.linalg.norm(y - y64) / np.linalg.norm(y64))
