"""Thin ctypes binding of libw8a8.so: the same entry points as include/w8a8.h.

Argument marshalling only.  These functions take torch tensors on the GPU,
allocate outputs the caller did not pass, and hand ``data_ptr()``s and the
current HIP stream to the C ABI.  Every step of the computation runs in the
library's gfx950 kernels.  There is no fallback: if the library is missing
or cannot be loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw8a8.so")

W8A8_OK = 0
W8A8_ERR_INVALID_ARG = -1
W8A8_ERR_SHAPE = -2
W8A8_ERR_ALIGN = -3
W8A8_ERR_WORKSPACE = -4
W8A8_ERR_K_BOUND = -5
W8A8_ERR_TOO_MANY_CANDIDATES = -6
W8A8_ERR_HIP = -7
W8A8_MAX_K = 133120
W8A8_MAX_CANDIDATES = 64
W8A8_MAX_SPLITK = 64
W8A8_MAX_ROWS = 4194303
W8A8_TILE_OVERRIDE_PANEL = 7
W8A8_TILE_OVERRIDE_SKINNY = 8
W8A8_NOALLOC_SCRATCH_BYTES = 67108864

# Every symbol the headers in include/ declare (w8a8.h, w8a8_diag.h), with its
# ctypes signature.
_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "w8a8_status_string": (ctypes.c_char_p, [_I32]),
    "w8a8_abi_version": (_I32, []),
    "w8a8_set_tile_override": (_I32, [_I32]),
    "w8a8_gemm_plan": (_I32, [_I64, _I64, _I64, _I32, _I32, _P]),
    "w8a8_gemm_panel_forced": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "w8a8_probe_mfma_ceiling": (_I32, [_I32, _I64, _I64, _P, _P, _P]),
    "w8a8_probe_stream_read": (_I32, [_P, _I64, _P, _P]),
    "w8a8_probe_stream_narrow": (_I32, [_P, _I64, _P, _P]),
    "w8a8_quantize_act": (_I32, [_P, _I64, _I64, _P, _P, _I64, _I64, _P, _P, _P]),
    "w8a8_gemm": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "w8a8_gemm_splitk_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I32]),
    "w8a8_gemm_splitk": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _SZ, _P]),
    "w8a8_gemm_splitk_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P]),
    "w8a8_readout_candidates": (_I32, [_P, _P, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _P, _P]),
    "w8a8_candidate_softmax": (_I32, [_P, _I64, _I64, _P, _P]),
    "w8a8_requantize_q8_0": (_I32, [_P, _P, _P, _I64, _I64, _P, _P, _P]),
    "w8a8_row_absmax": (_I32, [_P, _I64, _I64, _P, _P, _I64, _I64, _I32, _P, _P]),
    "w8a8_quantize_act_amax": (_I32, [_P, _I64, _I64, _P, _P, _P, _I64, _I64, _P, _P, _P]),
    "w8a8_gemm_int32": (_I32, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "w8a8_epilogue_int32": (_I32, [_P, _I32, _P, _P, _P, _P, _I64, _I64, _P]),
    "w8a8_answer_head": (_I32, [_P, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, _P, _P,
                                _P, _P, _P, _P]),
}


class W8A8Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__; __graft_entry__.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load()


def status_string(status: int) -> str:
    return _lib.w8a8_status_string(int(status)).decode()


def abi_version() -> int:
    return int(_lib.w8a8_abi_version())


def set_tile_override(kind: int) -> None:
    _check(_lib.w8a8_set_tile_override(int(kind)), "w8a8_set_tile_override")


def w8a8_gemm_plan(M, N, K, splitk=1, residual=False) -> list:
    """The kernel choice for a shape (host only): ten ints, see the header."""
    out = (ctypes.c_int32 * 10)()
    _check(_lib.w8a8_gemm_plan(int(M), int(N), int(K), int(splitk), int(bool(residual)),
                               ctypes.cast(out, ctypes.c_void_p)), "w8a8_gemm_plan")
    return list(out)


def w8a8_probe_mfma_ceiling(operand_kind, blocks, iters, sink, stream=None) -> int:
    """Launch the MFMA-only diagnostic kernel; returns the int8 ops launched."""
    ops = ctypes.c_int64(0)
    _check(_lib.w8a8_probe_mfma_ceiling(int(operand_kind), int(blocks), int(iters), _ptr(sink),
                                        ctypes.byref(ops), _stream(stream)), "w8a8_probe_mfma_ceiling")
    return ops.value


def w8a8_probe_stream_narrow(src, dst, stream=None) -> int:
    """Launch the narrowing-stream diagnostic: src (float32 device tensor, n
    elements) -> dst (n bytes); returns the bytes moved (5 per element)."""
    n = src.numel()
    if src.dtype != torch.float32 or dst.numel() * dst.element_size() < n:
        raise ValueError("src must be float32 and dst hold one byte per element")
    _check(_lib.w8a8_probe_stream_narrow(_ptr(src), n, _ptr(dst), _stream(stream)), "w8a8_probe_stream_narrow")
    return 5 * n


def w8a8_probe_stream_read(buf, sink, stream=None) -> int:
    """Launch the streaming-read diagnostic over all of `buf` (a device
    tensor); returns the bytes read."""
    n = buf.numel() * buf.element_size()
    n -= n % 16
    _check(_lib.w8a8_probe_stream_read(_ptr(buf), n, _ptr(sink), _stream(stream)),
           "w8a8_probe_stream_read")
    return n


def _check(rc: int, what: str) -> None:
    if rc != W8A8_OK:
        raise W8A8Error(rc, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _want(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")


def _need(t, dtype, numel, name):
    """A caller-supplied buffer: right dtype, on the GPU, contiguous and
    exactly `numel` elements.  The C ABI receives bare pointers, so a short
    buffer would otherwise be read or written past its end."""
    _want(t, dtype, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    return t


def _new(shape, dtype, device, stream):
    """An output or workspace the caller did not pass, allocated on the
    stream the call runs on, so that torch's caching allocator does not hand
    the block to other work before that stream is done with it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _out(t, shape, dtype, device, stream, name):
    n = 1
    for d in shape:
        n *= d
    return _new(shape, dtype, device, stream) if t is None else _need(t, dtype, n, name)


def w8a8_quantize_act(x, smooth, row_idx=None, xq=None, sx=None, stream=None):
    """Per-token int8 quantisation of x [rows, K] (row stride may exceed K).
    Returns (xq int8 [M,K], sx float32 [M]); M = len(row_idx) or rows."""
    _want(x, torch.float32, "x")
    _want(smooth, torch.float32, "smooth")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, K = x.shape
    _need(smooth, torch.float32, K, "smooth")
    if row_idx is not None:
        _need(row_idx, torch.int32, row_idx.numel(), "row_idx")
        M = row_idx.numel()
    else:
        M = rows
    xq = _out(xq, (M, K), torch.int8, x.device, stream, "xq")
    sx = _out(sx, (M,), torch.float32, x.device, stream, "sx")
    _check(_lib.w8a8_quantize_act(_ptr(x), x.stride(0), rows, _ptr(row_idx), _ptr(smooth), M, K,
                                  _ptr(xq), _ptr(sx), _stream(stream)), "w8a8_quantize_act")
    return xq, sx


def _gemm_shapes(xq, sx, w, sw, residual):
    for t, dt, n in ((xq, torch.int8, "xq"), (sx, torch.float32, "sx"), (w, torch.int8, "w"),
                     (sw, torch.float32, "sw")):
        _want(t, dt, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    M, K = xq.shape
    N = w.shape[0]
    if w.shape[1] != K or sx.numel() != M or sw.numel() != N:
        raise ValueError("shape mismatch")
    if residual is not None:
        _want(residual, torch.float32, "residual")
        if tuple(residual.shape) != (M, N) or not residual.is_contiguous():
            raise ValueError("residual must be a contiguous [M, N] float32 tensor")
    return M, N, K


def w8a8_gemm(xq, sx, w, sw, residual=None, y=None, stream=None):
    """y = fixed epilogue of the exact int32 product xq @ w^T (+ residual)."""
    M, N, K = _gemm_shapes(xq, sx, w, sw, residual)
    y = _out(y, (M, N), torch.float32, xq.device, stream, "y")
    _check(_lib.w8a8_gemm(_ptr(xq), _ptr(sx), _ptr(w), _ptr(sw), _ptr(residual), _ptr(y), M, N, K,
                          _stream(stream)), "w8a8_gemm")
    return y


def w8a8_gemm_splitk_workspace_bytes(M, N, K, splitk) -> int:
    n = int(_lib.w8a8_gemm_splitk_workspace_bytes(int(M), int(N), int(K), int(splitk)))
    if n == ctypes.c_size_t(-1).value:
        raise W8A8Error(W8A8_ERR_INVALID_ARG, "w8a8_gemm_splitk_workspace_bytes")
    return n


def splitk_workspace(M, N, K, splitk, device="cuda", stream=None):
    """A workspace of the size w8a8_gemm_splitk needs (contents irrelevant)."""
    n = w8a8_gemm_splitk_workspace_bytes(M, N, K, splitk)
    return _new((max(n, 1),), torch.uint8, device, stream)


def w8a8_gemm_splitk(xq, sx, w, sw, splitk, residual=None, y=None, workspace=None, stream=None):
    """Same result as w8a8_gemm, K split into `splitk` integer partials."""
    M, N, K = _gemm_shapes(xq, sx, w, sw, residual)
    y = _out(y, (M, N), torch.float32, xq.device, stream, "y")
    if workspace is None:
        workspace = splitk_workspace(M, N, K, splitk, xq.device, stream)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    _check(_lib.w8a8_gemm_splitk(_ptr(xq), _ptr(sx), _ptr(w), _ptr(sw), _ptr(residual), _ptr(y),
                                 M, N, K, int(splitk), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "w8a8_gemm_splitk")
    return y


def w8a8_gemm_panel_forced(xq, sx, w, sw, plan, residual=None, y=None, workspace=None, stream=None):
    """Tuning hook: w8a8_gemm's product on the column-panel kernel with the
    given plan (configuration, R, P, S); same result bits as w8a8_gemm."""
    M, N, K = _gemm_shapes(xq, sx, w, sw, residual)
    kind, R, P, S = (int(v) for v in plan)
    y = _out(y, (M, N), torch.float32, xq.device, stream, "y")
    need = w8a8_gemm_splitk_workspace_bytes(M, N, K, S) if S > 1 else 0
    if workspace is None:
        workspace = _new((max(need, 1),), torch.uint8, xq.device, stream)
    elif not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    p = (ctypes.c_int32 * 4)(kind, R, P, S)
    _check(_lib.w8a8_gemm_panel_forced(_ptr(xq), _ptr(sx), _ptr(w), _ptr(sw), _ptr(residual), _ptr(y),
                                       M, N, K, ctypes.cast(p, ctypes.c_void_p),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)),
           "w8a8_gemm_panel_forced")
    return y


def w8a8_gemm_splitk_noalloc(xq, sx, w, sw, splitk, residual=None, y=None, stream=None):
    """w8a8_gemm_splitk with the library's own split-K scratch: the library
    allocates nothing (y is allocated here only when the caller passes none)."""
    M, N, K = _gemm_shapes(xq, sx, w, sw, residual)
    y = _out(y, (M, N), torch.float32, xq.device, stream, "y")
    _check(_lib.w8a8_gemm_splitk_noalloc(_ptr(xq), _ptr(sx), _ptr(w), _ptr(sw), _ptr(residual), _ptr(y),
                                         M, N, K, int(splitk), _stream(stream)),
           "w8a8_gemm_splitk_noalloc")
    return y


def w8a8_readout_candidates(xq, sx, w_vocab, sw_vocab, cand, logits=None, err_flag=None,
                            stream=None):
    """Candidate-only logits [M, C] for vocabulary ids cand [M, C]."""
    _want(xq, torch.int8, "xq")
    _want(sx, torch.float32, "sx")
    _want(w_vocab, torch.int8, "w_vocab")
    _want(sw_vocab, torch.float32, "sw_vocab")
    _want(cand, torch.int32, "cand")
    for t, n in ((xq, "xq"), (w_vocab, "w_vocab"), (cand, "cand")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    M, K = xq.shape
    V = w_vocab.shape[0]
    if cand.dim() != 2 or cand.shape[0] != M:
        raise ValueError("cand must be [M, C]")
    C = cand.shape[1]
    if w_vocab.dim() != 2 or w_vocab.shape[1] != K:
        raise ValueError("w_vocab must be [V, K]")
    _need(sx, torch.float32, M, "sx")
    _need(sw_vocab, torch.float32, V, "sw_vocab")
    if err_flag is not None:
        _want(err_flag, torch.int32, "err_flag")
        if err_flag.numel() < 1:
            raise ValueError("err_flag must hold at least one int32")
    logits = _out(logits, (M, C), torch.float32, xq.device, stream, "logits")
    _check(_lib.w8a8_readout_candidates(_ptr(xq), _ptr(sx), M, K, _ptr(w_vocab), _ptr(sw_vocab), V,
                                        _ptr(cand), C, _ptr(logits), _ptr(err_flag), _stream(stream)),
           "w8a8_readout_candidates")
    return logits


def w8a8_requantize_q8_0(q, d_bits, smooth, w=None, sw=None, stream=None):
    """Q8_0 codes q [N, K] (int8) with binary16 block scales d_bits
    [N, K/32] (int16/uint16 bit patterns, or float16) smoothed by ``smooth``
    [K] and requantised per output channel; returns (w int8 [N, K], sw fp32 [N])."""
    _want(q, torch.int8, "q")
    _want(smooth, torch.float32, "smooth")
    if d_bits.dtype == torch.float16:
        d_bits = d_bits.view(torch.int16)
    if d_bits.dtype not in (torch.int16, torch.uint16):
        raise TypeError("d_bits must hold binary16 bit patterns (int16/uint16/float16)")
    for t, n in ((q, "q"), (d_bits, "d_bits")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    N, K = q.shape
    if d_bits.shape != (N, K // 32):
        raise ValueError("d_bits must be [N, K/32]")
    _need(smooth, torch.float32, K, "smooth")
    w = _out(w, (N, K), torch.int8, q.device, stream, "w")
    sw = _out(sw, (N,), torch.float32, q.device, stream, "sw")
    _check(_lib.w8a8_requantize_q8_0(_ptr(q), _ptr(d_bits), _ptr(smooth), N, K, _ptr(w), _ptr(sw),
                                     _stream(stream)), "w8a8_requantize_q8_0")
    return w, sw


def w8a8_row_absmax(x, smooth, row_idx=None, amax=None, accumulate=False, stream=None):
    """Exact per-row maximum of the smoothed slice x [rows, K]; with
    ``accumulate`` it is max-combined into ``amax``."""
    _want(x, torch.float32, "x")
    _want(smooth, torch.float32, "smooth")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, K = x.shape
    _need(smooth, torch.float32, K, "smooth")
    if row_idx is not None:
        _need(row_idx, torch.int32, row_idx.numel(), "row_idx")
    M = row_idx.numel() if row_idx is not None else rows
    if amax is None and accumulate:
        raise ValueError("accumulate needs an existing amax")
    amax = _out(amax, (M,), torch.float32, x.device, stream, "amax")
    _check(_lib.w8a8_row_absmax(_ptr(x), x.stride(0), rows, _ptr(row_idx), _ptr(smooth), M, K,
                                1 if accumulate else 0, _ptr(amax), _stream(stream)), "w8a8_row_absmax")
    return amax


def w8a8_quantize_act_amax(x, smooth, amax, row_idx=None, xq=None, sx=None, stream=None):
    """Per-token quantisation with the given per-token maxima amax [M]."""
    _want(x, torch.float32, "x")
    _want(smooth, torch.float32, "smooth")
    _want(amax, torch.float32, "amax")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows, K = x.shape
    _need(smooth, torch.float32, K, "smooth")
    if row_idx is not None:
        _need(row_idx, torch.int32, row_idx.numel(), "row_idx")
    M = row_idx.numel() if row_idx is not None else rows
    _need(amax, torch.float32, M, "amax")
    xq = _out(xq, (M, K), torch.int8, x.device, stream, "xq")
    sx = _out(sx, (M,), torch.float32, x.device, stream, "sx")
    _check(_lib.w8a8_quantize_act_amax(_ptr(x), x.stride(0), rows, _ptr(row_idx), _ptr(smooth),
                                       _ptr(amax), M, K, _ptr(xq), _ptr(sx), _stream(stream)),
           "w8a8_quantize_act_amax")
    return xq, sx


def w8a8_gemm_int32(xq, w, acc=None, stream=None):
    """Exact int32 accumulators [M, N] of xq [M, K] and w [N, K]."""
    for t, n in ((xq, "xq"), (w, "w")):
        _want(t, torch.int8, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    M, K = xq.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K]")
    acc = _out(acc, (M, N), torch.int32, xq.device, stream, "acc")
    _check(_lib.w8a8_gemm_int32(_ptr(xq), _ptr(w), M, N, K, _ptr(acc), _stream(stream)), "w8a8_gemm_int32")
    return acc


def w8a8_epilogue_int32(parts, sx, sw, residual=None, y=None, stream=None):
    """y = epilogue(sum over the S slices of parts [S, M, N] int32, in order)."""
    _want(parts, torch.int32, "parts")
    if parts.dim() == 2:
        parts = parts.unsqueeze(0)
    if parts.dim() != 3 or not parts.is_contiguous():
        raise ValueError("parts must be a contiguous [S, M, N] tensor")
    S, M, N = parts.shape
    _need(sx, torch.float32, M, "sx")
    _need(sw, torch.float32, N, "sw")
    if residual is not None:
        _need(residual, torch.float32, M * N, "residual")
    y = _out(y, (M, N), torch.float32, parts.device, stream, "y")
    _check(_lib.w8a8_epilogue_int32(_ptr(parts), S, _ptr(sx), _ptr(sw), _ptr(residual), _ptr(y), M, N,
                                    _stream(stream)), "w8a8_epilogue_int32")
    return y


def w8a8_candidate_softmax(logits, probs=None, stream=None):
    """Binary64 probabilities [M, C] over each row's candidates."""
    _want(logits, torch.float32, "logits")
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [M, C] tensor")
    M, C = logits.shape
    probs = _out(probs, (M, C), torch.float64, logits.device, stream, "probs")
    _check(_lib.w8a8_candidate_softmax(_ptr(logits), M, C, _ptr(probs), _stream(stream)),
           "w8a8_candidate_softmax")
    return probs


def w8a8_answer_head(h, answer_rows, smooth, w_vocab, sw_vocab, cand, xq=None, sx=None,
                     logits=None, probs=None, err_flag=None, stream=None):
    """Gather, quantise, candidate logits and candidate softmax of the
    answer rows of h [rows, K].  Returns (logits fp32 [M, C], probs fp64 [M, C])."""
    _want(h, torch.float32, "h")
    _want(answer_rows, torch.int32, "answer_rows")
    _want(smooth, torch.float32, "smooth")
    _want(w_vocab, torch.int8, "w_vocab")
    _want(sw_vocab, torch.float32, "sw_vocab")
    _want(cand, torch.int32, "cand")
    if h.dim() != 2 or h.stride(1) != 1:
        raise ValueError("h must be 2-D with unit column stride")
    rows, K = h.shape
    M = answer_rows.numel()
    if cand.dim() != 2 or cand.shape[0] != M or not cand.is_contiguous() or not w_vocab.is_contiguous():
        raise ValueError("cand must be a contiguous [M, C] tensor and w_vocab contiguous")
    C = cand.shape[1]
    if w_vocab.dim() != 2 or w_vocab.shape[1] != K:
        raise ValueError("w_vocab must be [V, K]")
    _need(answer_rows, torch.int32, M, "answer_rows")
    _need(smooth, torch.float32, K, "smooth")
    _need(sw_vocab, torch.float32, w_vocab.shape[0], "sw_vocab")
    if err_flag is not None:
        _want(err_flag, torch.int32, "err_flag")
        if err_flag.numel() < 1:
            raise ValueError("err_flag must hold at least one int32")
    dev = h.device
    xq = _out(xq, (M, K), torch.int8, dev, stream, "xq")
    sx = _out(sx, (M,), torch.float32, dev, stream, "sx")
    logits = _out(logits, (M, C), torch.float32, dev, stream, "logits")
    probs = _out(probs, (M, C), torch.float64, dev, stream, "probs")
    _check(_lib.w8a8_answer_head(_ptr(h), h.stride(0), rows, _ptr(answer_rows), M, _ptr(smooth), K,
                                 _ptr(w_vocab), _ptr(sw_vocab), w_vocab.shape[0], _ptr(cand), C,
                                 _ptr(xq), _ptr(sx), _ptr(logits), _ptr(probs), _ptr(err_flag),
                                 _stream(stream)), "w8a8_answer_head")
    return logits, probs
