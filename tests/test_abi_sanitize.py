"""The C ABI's host code (argument validation, dispatch, the ATTN_LOG tile
counts) built for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer
and driven through every entry point (tests/abi_host_check.cpp), with the
kernel launchers replaced by stubs: no GPU is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
@pytest.mark.parametrize("log", [False, True])
def test_api_host_code_under_sanitizers(tmp_path, log):
    exe = tmp_path / "abi_host_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           os.path.join(ROOT, "tiled_attention_05_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "abi_host_check.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    if log:
        env["ATTN_LOG"] = "1"   # also runs the host-side tile counting of every launched forward
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout, r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    if log:
        assert "tiles per query head" in r.stderr
