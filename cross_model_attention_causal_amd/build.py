"""Compile the HIP sources into the in-tree shared library ``libcma.so`` (gfx950 only)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcma.so")
SOURCES = ["capi.hip", "attn_maps.hip", "cosine.hip", "compress.hip", "mapped_av.hip"]


def hipcc_command(out=LIB, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [
        hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU ops are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", SRC,
        *extra,
        *[os.path.join(SRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building libcma.so")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
