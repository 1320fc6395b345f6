"""Compile the HIP library (kernels + C ABI) for gfx950, in-tree.

Produces paged_mla_decode_03_amd/libmla_decode.so from csrc/mla_decode.hip.
Every HIP translation unit is compiled with packed-fp32 instruction selection
disabled (the v_pk_*_f32 forms are avoided on this hardware).  Also links the
plain C++ test caller tests/c_caller/mla_c_caller against the library (host
code only: the C header and HIP runtime calls).
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "mla_decode.hip")
OUT = os.path.join(PKG, "libmla_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False):
    tmp = OUT + ".tmp"
    cmd = [HIPCC] + FLAGS + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, OUT)
    build_c_caller(verbose)
    return OUT


C_CALLER = os.path.join(ROOT, "tests", "c_caller", "mla_c_caller")


def build_c_caller(verbose=False):
    """Link the test caller of the C ABI (a plain host program) against the library."""
    src = C_CALLER + ".cpp"
    if not os.path.exists(src):
        return None
    cmd = [HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), src, "-L", PKG, "-lmla_decode",
           "-Wl,-rpath,$ORIGIN/../../paged_mla_decode_03_amd", "-o", C_CALLER + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on the C caller ({res.returncode}):\n{res.stderr}")
    os.replace(C_CALLER + ".tmp", C_CALLER)
    return C_CALLER


if __name__ == "__main__":
    print(build(verbose=True))
