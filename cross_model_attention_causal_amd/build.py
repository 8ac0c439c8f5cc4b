"""Compile the HIP sources into the in-tree shared library ``libcma.so`` (gfx950 only).

Each source is compiled to an object of its own (in parallel, under ``_build/``
at the repository root) and the objects are linked into the library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcma.so")
OBJ = os.path.join(ROOT, "_build")
SOURCES = ["capi.hip", "attn_maps.hip", "cosine.hip", "compress.hip", "mapped_av.hip", "prefix_index.hip", "probes.hip"]


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def compile_flags(extra=()):
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", SRC,
        *extra,
    ]


def hipcc_command(out=LIB, extra=()):
    """One-shot command (all sources, one hipcc call); kept for reference builds."""
    return [_hipcc(), *compile_flags(extra), "-shared", *[os.path.join(SRC, s) for s in SOURCES], "-o", out]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, msgs


def build(verbose=False, extra=()):
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in SOURCES:
        src = os.path.join(SRC, s)
        obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        lang = [] if s.endswith(".hip") else ["-x", "hip"]
        jobs.append((s, [_hipcc(), *compile_flags(extra), *lang, "-c", src, "-o", obj], obj))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    failed = False
    for (name, _, _), (rc, msgs) in zip(jobs, results):
        if rc != 0:
            failed = True
            sys.stderr.write(f"--- {name}\n" + "\n".join(msgs) + "\n")
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("hipcc failed building libcma.so")
    tmp = LIB + ".tmp"
    rc, msgs = _run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[j[2] for j in jobs], "-o", tmp])
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("linking libcma.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
