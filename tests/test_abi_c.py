"""The C ABI from plain C: compile tests/abi_check.c with gcc against
include/qlinear.h, link libqlinear.so, run the host-only validation checks."""
import os
import subprocess

import int8_gemm_linear_amd as q

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_c_consumer(tmp_path):
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(q.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                           os.path.join(HERE, "abi_check.c"), "-o", exe, "-L", libdir, "-lqlinear",
                           f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL OK" in r.stdout
