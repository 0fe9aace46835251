"""The kernels' division by the shard block size (a multiply-shift whose
constants the host builds) agrees with exact integer division: compiled for
the host with g++ and run over edge and random divisors and numerators."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_divu32_matches_exact_division(tmp_path):
    exe = tmp_path / "divu32_check"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-I",
                           os.path.join(ROOT, "jagged_embedding_sparse_amd", "csrc"),
                           os.path.join(ROOT, "tests", "cpp", "divu32_check.cpp"),
                           "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")
