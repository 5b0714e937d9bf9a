"""The C-ABI library without a GPU.

These checks cover: it loads; it exports every function the headers in
include/ declare; and the host-side argument checks reject bad calls before
any HIP call.  No call here reaches a kernel.  Every rejected call below fails
validation before the library touches the device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADER = os.path.join(INCLUDE, "w8a8.h")
LIB = os.path.join(ROOT, "deterministic_w8a8_int8_amd", "libw8a8.so")


def declared_functions(path=None):
    """Functions declared in one header, or in every header of include/."""
    paths = [path] if path else [os.path.join(INCLUDE, f) for f in sorted(os.listdir(INCLUDE))
                                 if f.endswith(".h")]
    names = set()
    for p in paths:
        text = re.sub(r"/\*.*?\*/", "", open(p).read(), flags=re.S)
        names |= set(re.findall(r"\b(w8a8_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from deterministic_w8a8_int8_amd import build
        build.build()
    from deterministic_w8a8_int8_amd import binding
    return binding._lib


def test_header_declares_the_four_entry_points():
    names = declared_functions(HEADER)
    for n in ("w8a8_quantize_act", "w8a8_gemm", "w8a8_gemm_splitk", "w8a8_readout_candidates",
              "w8a8_gemm_splitk_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from deterministic_w8a8_int8_amd import binding
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.SIGNATURES), "binding and header disagree"


def test_status_strings_and_version(lib):
    from deterministic_w8a8_int8_amd import binding as B
    for s in range(-7, 1):
        assert B.status_string(s) and B.status_string(s) != "unknown status"
    assert B.status_string(-99) == "unknown status"
    assert B.abi_version() == 10000


def test_workspace_query(lib):
    from deterministic_w8a8_int8_amd import binding as B
    assert B.w8a8_gemm_splitk_workspace_bytes(8192, 5120, 17408, 1) == 0
    n2 = B.w8a8_gemm_splitk_workspace_bytes(8192, 5120, 17408, 2)
    n8 = B.w8a8_gemm_splitk_workspace_bytes(8192, 5120, 17408, 8)
    # at least S int32 partials of the output plus counters
    assert n2 >= 2 * 8192 * 5120 * 4 and n8 >= 8 * 8192 * 5120 * 4 and n8 > n2
    with pytest.raises(B.W8A8Error):
        B.w8a8_gemm_splitk_workspace_bytes(16, 16, 100, 2)       # K not a multiple of 64
    with pytest.raises(B.W8A8Error):
        B.w8a8_gemm_splitk_workspace_bytes(16, 16, 64, 0)
    with pytest.raises(B.W8A8Error):
        B.w8a8_gemm_splitk_workspace_bytes(16, 16, 64, 65)


def _fake(n=1 << 20, align=256):
    """A host buffer used only as a non-null, aligned pointer: every call that
    receives it is rejected before any device access."""
    buf = ctypes.create_string_buffer(n + align)
    p = (ctypes.addressof(buf) + align - 1) // align * align
    return buf, ctypes.c_void_p(p)


def test_argument_checks_reject_before_launch(lib):
    from deterministic_w8a8_int8_amd import binding as B
    keep, p = _fake()
    odd = ctypes.c_void_p(p.value + 1)
    nul = None
    S = None
    # quantize: K not multiple of 64, K too large, ldx < K, M > x_rows, null, misaligned
    assert lib.w8a8_quantize_act(p, 96, 4, nul, p, 4, 96, p, p, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_quantize_act(p, 133184, 1, nul, p, 1, 133184, p, p, S) == B.W8A8_ERR_K_BOUND
    assert lib.w8a8_quantize_act(p, 60, 4, nul, p, 4, 64, p, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_quantize_act(p, 64, 3, nul, p, 4, 64, p, p, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_quantize_act(nul, 64, 4, nul, p, 4, 64, p, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_quantize_act(odd, 64, 4, nul, p, 4, 64, p, p, S) == B.W8A8_ERR_ALIGN
    assert lib.w8a8_quantize_act(p, 64, 4, nul, p, 0, 64, p, p, S) == B.W8A8_OK       # M = 0 no-op
    # gemm
    assert lib.w8a8_gemm(p, p, p, p, nul, p, 4, 4, 100, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_gemm(p, p, p, p, nul, p, -1, 4, 64, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_gemm(p, p, odd, p, nul, p, 4, 4, 64, S) == B.W8A8_ERR_ALIGN
    assert lib.w8a8_gemm(p, p, p, p, nul, nul, 4, 4, 64, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_gemm(p, p, p, p, nul, p, 0, 4, 64, S) == B.W8A8_OK                # empty
    # residual overlapping y without being y
    r = ctypes.c_void_p(p.value + 4)
    assert lib.w8a8_gemm(p, p, p, p, r, p, 4, 4, 64, S) == B.W8A8_ERR_INVALID_ARG
    # split-K workspace checks
    assert lib.w8a8_gemm_splitk(p, p, p, p, nul, p, 300, 300, 256, 2, nul, 0, S) == B.W8A8_ERR_WORKSPACE
    assert lib.w8a8_gemm_splitk(p, p, p, p, nul, p, 300, 300, 256, 2, p, 16, S) == B.W8A8_ERR_WORKSPACE
    assert lib.w8a8_gemm_splitk(p, p, p, p, nul, p, 300, 300, 256, 2, odd, 1 << 20, S) == B.W8A8_ERR_WORKSPACE
    assert lib.w8a8_gemm_splitk(p, p, p, p, nul, p, 300, 300, 256, 0, p, 1 << 20, S) == B.W8A8_ERR_INVALID_ARG
    # read-out
    assert lib.w8a8_readout_candidates(p, p, 3, 64, p, p, 10, p, 65, p, nul, S) == B.W8A8_ERR_TOO_MANY_CANDIDATES
    assert lib.w8a8_readout_candidates(p, p, 3, 64, p, p, 0, p, 4, p, nul, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_readout_candidates(p, p, 3, 64, p, p, 10, p, 0, p, nul, S) == B.W8A8_OK
    # Q8_0 requantisation
    assert lib.w8a8_requantize_q8_0(p, p, p, 4, 96, p, p, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_requantize_q8_0(p, p, p, -1, 64, p, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_requantize_q8_0(odd, p, p, 4, 64, p, p, S) == B.W8A8_ERR_ALIGN
    assert lib.w8a8_requantize_q8_0(p, odd, p, 4, 64, p, p, S) == B.W8A8_ERR_ALIGN
    assert lib.w8a8_requantize_q8_0(p, p, nul, 4, 64, p, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_requantize_q8_0(p, p, p, 4, 64, ctypes.c_void_p(p.value + 64), p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_requantize_q8_0(p, p, p, 0, 64, p, p, S) == B.W8A8_OK
    # candidate softmax
    assert lib.w8a8_candidate_softmax(p, 3, 65, p, S) == B.W8A8_ERR_TOO_MANY_CANDIDATES
    assert lib.w8a8_candidate_softmax(p, -1, 4, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_candidate_softmax(nul, 3, 4, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_candidate_softmax(p, 3, 4, ctypes.c_void_p(p.value + 4), S) == B.W8A8_ERR_ALIGN
    assert lib.w8a8_candidate_softmax(p, 3, 4, ctypes.c_void_p(p.value + 8), S) == B.W8A8_ERR_INVALID_ARG  # overlap
    assert lib.w8a8_candidate_softmax(p, 0, 4, p, S) == B.W8A8_OK
    # answer head: every stage's checks run before the first launch
    q = ctypes.c_void_p(p.value + 4096)
    assert lib.w8a8_answer_head(p, 64, 8, nul, 3, p, 64, p, p, 10, p, 4, p, p, p, q, nul, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_answer_head(p, 64, 8, p, 3, p, 96, p, p, 10, p, 4, p, p, p, q, nul, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_answer_head(p, 64, 8, p, 3, p, 64, p, p, 10, p, 65, p, p, p, q, nul, S) == B.W8A8_ERR_TOO_MANY_CANDIDATES
    assert lib.w8a8_answer_head(p, 64, 8, p, 3, p, 64, odd, p, 10, p, 4, p, p, p, q, nul, S) == B.W8A8_ERR_ALIGN
    assert lib.w8a8_answer_head(p, 64, 8, p, 3, p, 64, p, p, 10, p, 4, p, p, p, odd, nul, S) == B.W8A8_ERR_ALIGN
    assert lib.w8a8_answer_head(p, 64, 8, p, 0, p, 64, p, p, 10, p, 4, p, p, p, q, nul, S) == B.W8A8_OK
    # the per-row entry points: at most W8A8_MAX_ROWS rows (one workgroup each)
    R = B.W8A8_MAX_ROWS
    assert lib.w8a8_quantize_act(p, 64, R + 1, nul, p, R + 1, 64, p, p, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_quantize_act(nul, 64, R, nul, p, R, 64, p, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_row_absmax(p, 64, R + 1, nul, p, R + 1, 64, 0, p, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_readout_candidates(p, p, R + 1, 64, p, p, 10, p, 4, p, nul, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_readout_candidates(nul, p, R, 64, p, p, 10, p, 4, p, nul, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_candidate_softmax(p, R + 1, 4, ctypes.c_void_p(p.value + (1 << 30)), S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_requantize_q8_0(p, p, p, R + 1, 64, p, p, S) == B.W8A8_ERR_SHAPE
    assert lib.w8a8_requantize_q8_0(p, p, nul, R, 64, p, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_answer_head(p, 64, R + 1, p, R + 1, p, 64, p, p, 10, p, 4, p, p, p, q, nul, S) == \
        B.W8A8_ERR_SHAPE
    # forced panel plans: the plan is checked before any launch
    def plan(*v):
        return ctypes.cast((ctypes.c_int32 * 4)(*v), ctypes.c_void_p)
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 64, 64, 256, nul, nul, 0, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 64, 64, 256, plan(99, 1, 1, 1), nul, 0, S) == \
        B.W8A8_ERR_INVALID_ARG                                     # no such configuration
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 64, 64, 256, plan(0, 1, 4, 0), nul, 0, S) == \
        B.W8A8_ERR_INVALID_ARG                                     # S = 0
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 64, 64, 256, plan(0, 1, 4, 65), nul, 0, S) == \
        B.W8A8_ERR_INVALID_ARG                                     # S past W8A8_MAX_SPLITK
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 512, 64, 256, plan(0, 1, 4, 1), nul, 0, S) == \
        B.W8A8_ERR_INVALID_ARG                                     # 32 row blocks > 4 waves x 1
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 64, 4096, 256, plan(0, 1, 2, 1), nul, 0, S) == \
        B.W8A8_ERR_INVALID_ARG                                     # 128 column blocks > 2 panels x 8
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 64, 64, 256, plan(0, 1, 4, 2), nul, 0, S) == \
        B.W8A8_ERR_WORKSPACE                                       # S = 2 without a workspace
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 64, 64, 256, plan(0, 1, 4, 2), p, 1024, S) == \
        B.W8A8_ERR_WORKSPACE                                       # 2 x 64 x 64 int32 do not fit 1 KiB
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 0, 64, 256, plan(0, 1, 4, 1), nul, 0, S) == B.W8A8_OK
    assert lib.w8a8_gemm_panel_forced(p, p, p, p, nul, p, 64, 64, 100, plan(0, 1, 4, 1), nul, 0, S) == \
        B.W8A8_ERR_SHAPE
    assert lib.w8a8_set_tile_override(99) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_set_tile_override(-2) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_probe_mfma_ceiling(4, 1, 1, p, None, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_probe_mfma_ceiling(-1, 1, 1, p, None, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_probe_mfma_ceiling(0, 0, 1, p, None, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_probe_stream_read(odd, 1024, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_probe_stream_read(p, 1000, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_probe_stream_read(p, 0, p, S) == B.W8A8_ERR_INVALID_ARG
    assert lib.w8a8_probe_stream_read(p, 1024, nul, S) == B.W8A8_ERR_INVALID_ARG
    del keep


def test_binding_constants_match_the_header():
    """Every integer #define and status code of the header has the same value in the binding."""
    from deterministic_w8a8_int8_amd import binding
    text = "".join(open(os.path.join(INCLUDE, f)).read() for f in sorted(os.listdir(INCLUDE))
                   if f.endswith(".h"))
    pairs = re.findall(r"#define\s+(W8A8_[A-Z0-9_]+)\s+(-?\d+)", text)
    pairs += re.findall(r"\b(W8A8_(?:OK|ERR_[A-Z_]+))\s*=\s*(-?\d+)", text)
    assert len(pairs) >= 12
    for name, value in pairs:
        assert getattr(binding, name) == int(value), name
