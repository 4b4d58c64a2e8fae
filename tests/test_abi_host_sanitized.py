"""The C ABI's host code (argument checks, split planning, workspace layout)
built with the address and undefined-behaviour sanitizers and exercised
without a GPU.

``tests/host/abi_host_check.cpp`` links ``api.cpp`` against launcher
stand-ins that record their arguments and launch nothing, then checks:
rejected arguments; that a sliding-window call accepts exactly the workspace
``kvattn_gqa_workspace_bytes`` reports (the query takes no window) and that
its splits cover the window; that every MLA workspace region lies inside the
queried size and bounds the device plan's pieces; and 20,000 random (also
extreme) argument sets for overflow and size agreement.  Only host code is
compiled (g++, no kernel sources).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
ROCM = "/opt/rocm"


def test_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("needs g++ and the ROCm runtime library")
    exe = str(tmp_path / "abi_host_check")
    sources = [os.path.join(ROOT, "decode_attention_kv_03_amd", "csrc", "api.cpp"),
               os.path.join(HOST, "stub_launch.cpp"), os.path.join(HOST, "abi_host_check.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-w", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *sources, f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout[-4000:], res.stderr[-4000:])
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "0 failed" in res.stdout
