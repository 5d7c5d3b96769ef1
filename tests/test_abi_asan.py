"""The C ABI's host code under AddressSanitizer, LeakSanitizer and UBSan, on the CPU.

abi.cpp is compiled host-only with the sanitizers and linked with a stand-in for
the HIP runtime and the kernel launchers (tests/asan/fake_hip.cpp: device memory
is host memory, launches do nothing); tests/asan/abi_host_main.cpp then drives
every entry point: handles built, queried, used and destroyed, every class of
rejected argument, and the BSATTN_DEBUG=2 paths (call and launch log, stream
check, the workspace canary catching a forward that writes past its bytes).  Any
sanitizer report or unexpected return code fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_abi_host_code_under_sanitizers(tmp_path):
    flags = ["-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include")]
    srcs = [os.path.join(ROOT, "block_sparse_long_bsattn_amd", "csrc", "abi.cpp"),
            os.path.join(ROOT, "tests", "asan", "fake_hip.cpp"),
            os.path.join(ROOT, "tests", "asan", "abi_host_main.cpp")]
    objs = []
    for s in srcs:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        r = subprocess.run([CLANG] + flags + ["-c", s, "-o", o], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(o)
    exe = str(tmp_path / "abi_host_asan")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", "-o", exe] + objs + ["-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), out[-4000:]
    # the level-2 debug log names the calls and launches it checked
    assert "[bsattn] call fwd" in r.stderr and "[bsattn] launch fake_fwd" in r.stderr
    assert "written past" in r.stderr
