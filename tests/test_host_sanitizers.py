"""libtq's host sources built with AddressSanitizer and UndefinedBehaviorSanitizer
into a host-only harness (tests/sanitize/harness.cpp) and run on the CPU.

The host compiler is the ROCm clang++ (the one HIP uses for host code); the
sanitizers instrument host code only, and no GPU code is compiled here."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_decode_attention_tq_amd", "csrc")
HOST_SOURCES = ["api.cpp", "host_state.cpp", "host_codebook.cpp", "profile.cpp"]
CXX = "/opt/rocm/llvm/bin/clang++"
ROCM_INC, ROCM_LIB = "/opt/rocm/include", "/opt/rocm/lib"


@pytest.mark.skipif(not os.path.exists(CXX), reason="ROCm clang++ not installed")
def test_host_code_under_asan_ubsan(tmp_path):
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC,
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-w"]
    objs = []
    for src in HOST_SOURCES + ["harness"]:
        path = os.path.join(ROOT, "tests", "sanitize", "harness.cpp") if src == "harness" else os.path.join(CSRC, src)
        obj = str(tmp_path / (os.path.basename(path) + ".o"))
        r = subprocess.run([CXX] + flags + ["-c", path, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(tmp_path / "harness")
    r = subprocess.run([CXX, "-fsanitize=address,undefined"] + objs +
                       ["-L", ROCM_LIB, "-lamdhip64", "-Wl,-rpath," + ROCM_LIB, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: the sanitizer runtime need not be the first library
    # of the process if the environment preloads another one
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "host harness: 0 unexpected results" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
