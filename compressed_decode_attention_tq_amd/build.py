"""Ahead-of-time build of libtq.so for gfx950 (every kernel variant compiled in).

Usage: python -m compressed_decode_attention_tq_amd.build
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-I", SRC,
          "--offload-arch=gfx950"]
# Packed fp32 VALU forms are kept out of the generated code.  Matrix-core
# accumulators are kept in ordinary VGPRs (gfx950 MFMAs read and write them
# directly), so loop-carried accumulators are not copied to and from AGPRs.
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=fast",
          "-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCES = ["api.cpp", "host_state.cpp", "host_codebook.cpp", "profile.cpp", "compress.hip", "compress_mfma.hip", "decode.hip", "decode_mainloop.hip",
           "decode_bypass.hip", "decompress.hip"]


def _compile(src):
    out = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC] + COMMON + (DEVICE if src.endswith(".hip") else []) + ["-c", os.path.join(SRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return out


def build(verbose=True):
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
