"""Build the gfx950 shared library ``libmoe_mi355x.so`` in the package directory.

Every source under ``csrc/`` is compiled with hipcc for gfx950 only.  Packed
fp32 VALU forms are disabled for device code (``-packed-fp32-ops``); hipcc's
host pass warns that it does not know that feature, which is harmless.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
BUILD_DIR = os.path.join(REPO_DIR, "_build")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["moe_api.cpp", "route.hip", "permute.hip", "experts.hip", "pack.hip", "probe.hip", "experts_mx.hip", "redequant.hip", "dense.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
    "-Wno-unused-command-line-argument",
]


def _compile(src, extra):
    out = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", out]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    return src, out, proc


def build(verbose=False, extra_flags=()):
    """Compile all sources and link the library; raises on any compiler error."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    errors = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        for src, out, proc in ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES):
            if proc.returncode != 0:
                errors.append(f"--- {src} ---\n{proc.stderr}")
            elif verbose and proc.stderr.strip():
                filtered = "\n".join(l for l in proc.stderr.splitlines()
                                     if "packed-fp32-ops" not in l)
                if filtered.strip():
                    print(f"--- {src} ---\n{filtered}", file=sys.stderr)
            objs.append(out)
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("link failed:\n" + proc.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
