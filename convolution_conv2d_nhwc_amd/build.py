"""Build ``libconv_nhwc.so`` (the HIP library) in-tree for gfx950.

Usage:  python -m convolution_conv2d_nhwc_amd.build [-v] [--incremental]

Each source under ``csrc/`` is compiled with hipcc in parallel, then linked
into ``convolution_conv2d_nhwc_amd/libconv_nhwc.so``. The flags disable the
packed-fp32 instructions (v_pk_*_f32) for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libconv_nhwc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-x", "hip", "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _deps(path: str, seen=None) -> set:
    """The file and every quoted #include it pulls in, recursively."""
    seen = set() if seen is None else seen
    if path in seen or not os.path.exists(path):
        return seen
    seen.add(path)
    for line in open(path, errors="replace"):
        line = line.strip()
        if line.startswith("#include \""):
            inc = line.split('"')[1]
            _deps(os.path.normpath(os.path.join(os.path.dirname(path), inc)), seen)
    return seen


def _compile(src: str, verbose: bool, incremental: bool = False) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        newest = max(os.path.getmtime(d) for d in _deps(src))
        if os.path.getmtime(obj) >= newest:
            return obj
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False, jobs: int = 8, incremental: bool = False) -> str:
    """Compile every source and link the shared library. Rebuilds every
    object unless `incremental`, which recompiles only objects older than
    their source or a header it includes."""
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    # the longest compiles first
    srcs.sort(key=lambda p: -os.path.getsize(p))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    t = build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv)
    print(t)
