"""The library's host code and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; no GPU and no HIP runtime are involved).

tests/native/host_check.cpp links the real C entry points (api.hip, compiled as plain C++ with
g++) against recording stubs of the kernel launchers and of the few HIP runtime calls they
make, and the oracle (mlp_oracle.c, compiled with gcc). It drives the argument checks, the
order of launches, the host arrays of partial pointers, the HIP error handling and the oracle
on small cases; any out-of-bounds access, leak or undefined behaviour aborts it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_host_code_and_oracle_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "tensor_mlp_block_amd", "csrc"), "-I", ROCM_INCLUDE,
           "-D__HIP_PLATFORM_AMD__"]
    api = str(tmp_path / "api.o")
    orc = str(tmp_path / "oracle.o")
    exe = str(tmp_path / "host_check")
    # host code only: the HIP headers declare the runtime API; nothing is built for the GPU
    _run(["g++", "-std=c++17", *SAN, *inc, "-x", "c++", "-c",
          os.path.join(ROOT, "tensor_mlp_block_amd", "csrc", "api.hip"), "-o", api])
    _run(["gcc", "-std=c11", *SAN, "-c", os.path.join(ROOT, "oracle", "mlp_oracle.c"), "-o", orc])
    _run(["g++", "-std=c++17", *SAN, *inc, os.path.join(ROOT, "tests", "native", "host_check.cpp"),
          api, orc, "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = _run([exe], env=env, timeout=120)
    assert "all checks passed" in res.stdout
