"""Build libmoe_rocm.so (HIP for gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_rocm.so")
SOURCES = ["api.cpp", "router.hip", "permute.hip", "grouped_gemm.hip", "combine.hip", "backward.hip", "generic.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-FP32 instructions: the compiler is told the target lacks them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (libmoe_rocm_san.so): the argument
# checks, sizing and launch code in api.cpp and the launchers are instrumented; device code is not
# (every flag is given to the host compilation only). Loaded instead of libmoe_rocm.so when
# MOE_SANITIZE_LIB=1, with clang's shared ASan runtime preloaded (tests/sanitizers.py does both).
SAN_LIB = os.path.join(PKG, "libmoe_rocm_san.so")
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_HOST = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
            "-g", "-shared-libsan"]


def _host_only(flags):
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(_host_only(SAN_HOST) if sanitize else [])]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link libmoe_rocm.so (libmoe_rocm_san.so with sanitize)."""
    out = SAN_LIB if sanitize else LIB
    os.makedirs(SAN_BUILD if sanitize else BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *(_host_only(SAN_HOST) if sanitize else []),
           "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
