"""The native CMake build of libsprms (CMakeLists.txt) configures on the CPU:
HIP language for gfx950, the library, the oracle and both C clients as
targets.  Building it takes as long as the Python build step and is left to
the user (cmake --build); configuring catches a broken build file."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_CXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(shutil.which("cmake") is None or not os.path.exists(HIP_CXX), reason="cmake or ROCm clang missing")
def test_cmake_configures(tmp_path):
    env = dict(os.environ, PATH="/opt/rocm/bin:" + os.environ.get("PATH", ""))
    r = subprocess.run(["cmake", "-S", ROOT, "-B", str(tmp_path), f"-DCMAKE_HIP_COMPILER={HIP_CXX}",
                        "-DCMAKE_PREFIX_PATH=/opt/rocm"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    targets = subprocess.run(["cmake", "--build", str(tmp_path), "--target", "help"], capture_output=True,
                             text=True, env=env, timeout=120).stdout
    for t in ("sprms", "oracle_sprms", "c_abi_check", "c_gpu_client"):
        assert t in targets, t
