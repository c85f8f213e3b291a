"""The host side of the C ABI (validation, the fill-state machine, split
planning, layouts) built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven on the CPU: kvq_api.cpp is compiled with g++ (host code only)
against launch stand-ins that check every launch's ranges instead of running
kernels (tests/sanitize/kvq_launch_stubs.cpp), and a C driver
(tests/sanitize/drive_abi.c) runs prefills, appends through flushes,
decodes under several workgroup targets, ragged, paged, FP8, FP16,
multi-layer and allocation-free calls and the error paths. No GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs the host C/C++ compilers")
def test_abi_host_code_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src, cc, std in (
            (os.path.join(ROOT, "kv_cache_quantization_quant_amd", "csrc", "kvq_api.cpp"), "g++",
             "-std=c++17"),
            (os.path.join(ROOT, "tests", "sanitize", "kvq_launch_stubs.cpp"), "g++", "-std=c++17"),
            (os.path.join(ROOT, "tests", "sanitize", "drive_abi.c"), "gcc", "-std=c11")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([cc, std, *SAN, "-fPIC", *inc, "-c", src, "-o", obj], check=True,
                       capture_output=True, text=True)
        objs.append(obj)
    exe = str(tmp_path / "drive_abi")
    subprocess.run(["g++", *SAN, *objs, "-o", exe], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "launches:" in r.stderr
