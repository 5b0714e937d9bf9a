"""The C ABI used from plain C (tests/c_abi_demo.c): a program that includes
only include/w8a8.h and the HIP runtime header.  On any host it must compile
and link against the library; on a GPU it requantises Q8_0 weights in place,
runs quantisation, the GEMM with a residual, split-K and the candidate
read-out on them, and checks each output against the oracle bit for bit (the
definitions of the review page "StartLux-Prism: Fast, exact inference for
StartLux-Decision models on NVIDIA GPUs", sections "Compute shared evidence
once" and "Bitwise consistency is not lossless quantization")."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "deterministic_w8a8_int8_amd")
ROCM = "/opt/rocm"


def _build(tmp_path):
    if shutil.which("gcc") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("gcc or the HIP headers are missing")
    if not os.path.exists(os.path.join(PKG, "libw8a8.so")):
        pytest.skip("the library is not built")
    exe = str(tmp_path / "c_abi_demo")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi_demo.c"), os.path.join(ROOT, "oracle", "w8a8_oracle.c"),
           "-L", PKG, "-lw8a8", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{PKG}:{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "warning" not in r.stderr, r.stderr
    return exe


def test_c_program_builds_against_the_abi(tmp_path):
    _build(tmp_path)


@pytest.mark.gpu
def test_c_program_matches_the_oracle(tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _build(tmp_path)
    print("running the C program", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bit-exact against the oracle" in r.stdout
