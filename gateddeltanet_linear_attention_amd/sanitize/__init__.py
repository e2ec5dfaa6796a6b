"""Host-only AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI.

gdn_api.cpp (argument validation, the transaction planner, the offset and size
arithmetic) is compiled with g++ and linked with launch stubs that refuse as the real
launchers do without a GPU, into a libgdn.so that is loaded in place of the real one
through the GDN_LIBRARY environment variable.  Nothing here runs device code.

    python -m gateddeltanet_linear_attention_amd.sanitize [out_dir]
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(_HERE)
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")

SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def runtime_preload() -> str:
    """The ASan runtime, which must be loaded first into an uninstrumented python."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build(out_dir: str = OUT_DIR) -> str:
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libgdn.so")
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", *SANITIZE, "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC,
           os.path.join(CSRC, "gdn_api.cpp"), os.path.join(_HERE, "host_stubs.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitizer build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return lib

