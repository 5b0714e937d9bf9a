"""Planted mistakes: every plausible slip in the oracle must fail some pin.

Each case copies the oracle's C source and changes one thing with a text
edit.  It builds the copy with
gcc into a temporary directory and points the oracle module at it.  It then
runs the pins of test_oracle_pins.py.  The case passes only if at least one
pin fails.  Everything runs on the CPU; the real oracle is never modified.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "w8a8_oracle.c")

PINS = [
    pins.test_quantize_round_half_even_golden,
    pins.test_quantize_integer_rows_are_identity,
    lambda: pins.test_quantize_matches_exact_rational_bruteforce(0),
    pins.test_quantize_row_gather_equals_gather_after,
    pins.test_gemm_acc_matches_python_int,
    pins.test_gemm_acc_closed_forms,
    lambda: pins.test_split_k_gives_identical_bits(704),
    pins.test_epilogue_matches_exact_rational_bruteforce,
    pins.test_epilogue_int32_to_f32_golden,
    pins.test_epilogue_power_of_two_scales_closed_form,
    pins.test_golden_tiny_layer,
    pins.test_readout_equals_gemm_columns_and_flags_bad_ids,
    pins.test_quantize_scale_and_quotient_bruteforce_many_rows,
    pins.test_quantize_nonfinite_rows_bruteforce,
]

# (name, [(old, new), ...], extra gcc flags)
MUTANTS = [
    ("no smoothing divide", [("float xs = xr[k] / smooth[k];", "float xs = xr[k];")], []),
    ("reciprocal instead of divide",
     [("float xs = xr[k] / smooth[k];", "float xs = xr[k] * (1.0f / smooth[k]);")], []),
    ("scale by multiply with 1/127", [("amax / 127.0f", "amax * (1.0f / 127.0f)")], []),
    ("signed max instead of abs max", [("float ab = oracle_abs_for_max(xs);", "float ab = xs;")], []),
    ("NaN dropped from the row maximum", [("if (a != a) return INFINITY;", "")], []),
    ("infinite maximum used as a scale", [("if (!oracle_usable_max(amax)) {", "if (amax != amax) {")], []),
    ("quotient by multiply with 1/sx", [("float t = xs / s;", "float t = xs * (1.0f / s);")], []),
    ("ties away from zero",
     [("return (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;", "return (f >= 0.0f) ? f + 1.0f : f;")], []),
    ("truncate instead of round", [("float r = oracle_round_half_even(t);", "float r = truncf(t);")], []),
    ("row gather ignored", [("row_idx ? (int64_t)row_idx[m] : m", "m")], []),
    ("split-K chunk dropped", [("acc += part;", "acc = part;")], []),
    ("split-K chunk overlap", [("int64_t a = (int64_t)c * kc, b = a + kc;",
                                "int64_t a = (int64_t)c * kc, b = a + kc + 1;")], []),
    ("scales folded first", [("float t1 = t0 * sxm;\n    float t2 = t1 * swn;",
                              "float t1 = sxm * swn;\n    float t2 = t0 * t1;")], []),
    ("weight scale index reversed", [("sw[n], residual ?", "sw[N - 1 - n], residual ?")], []),
    ("residual dropped", [("float y = t2 + *r;", "float y = t2;")], []),
    ("activation scale dropped", [("float t1 = t0 * sxm;", "float t1 = t0;")], []),
    ("read-out reads the wrong scale", [("sw_vocab[id], 0)", "sw_vocab[c], 0)")], []),
    ("fused multiply-add in the epilogue", [("float y = t2 + *r;", "float y = fmaf(t1, swn, *r);")], []),
]


def _build_mutant(tmp, edits, flags):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    path = os.path.join(tmp, "mutant.c")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(tmp, "libmutant.so")
    cflags = [c for c in oracle.CFLAGS if not (flags and c in ("-ffp-contract=off", "-O2"))]
    subprocess.check_call(["gcc", *cflags, *flags, path, "-o", lib, "-lm"])
    return oracle.load(lib)


@pytest.mark.parametrize("name,edits,flags", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, edits, flags):
    with tempfile.TemporaryDirectory() as tmp:
        mutant = _build_mutant(tmp, edits, flags)
        prev = oracle.swap_library(mutant)
        caught = []
        try:
            for pin in PINS:
                try:
                    pin()
                except (AssertionError, RuntimeError) as e:
                    caught.append((getattr(pin, "__name__", "pin"), type(e).__name__))
                    break
        finally:
            oracle.swap_library(prev)
    assert caught, f"no pin caught the planted mistake '{name}'"


def test_unmutated_copy_passes_every_pin():
    with tempfile.TemporaryDirectory() as tmp:
        clean = _build_mutant(tmp, [], [])
        prev = oracle.swap_library(clean)
        try:
            for pin in PINS:
                pin()
        finally:
            oracle.swap_library(prev)
