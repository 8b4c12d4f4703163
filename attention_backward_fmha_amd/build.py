"""Build libfmha_bwd.so (gfx950) in-tree with hipcc.

    python -m attention_backward_fmha_amd.build          # or build() from Python

Every HIP source is compiled with packed-fp32 instruction selection turned off
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does not know the
feature, which is harmless.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfmha_bwd.so")
SOURCES = ["kernels.hip", "kernels_wide.hip", "api.cpp", "plan.cpp", "noalloc.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    return res.returncode, msgs


def build(verbose=False, sources=None, out=None):
    """Compile every source to an object (in parallel), then link the shared library.
    ``sources`` maps a source name to another file (used to build variants); ``out`` is the
    library path (default: the package's)."""
    out = out or LIB
    objdir = os.path.join(os.path.dirname(out), "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = [(sources or {}).get(s, os.path.join(CSRC, s)) for s in SOURCES]
    objs = [os.path.join(objdir, os.path.basename(s) + ".%d.o" % os.getpid()) for s in srcs]
    cmds = [[hipcc()] + _flags() + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    msgs = [m for _, ms in results for m in ms]
    tmp = out + ".tmp%d" % os.getpid()
    try:
        if any(rc != 0 for rc, _ in results):
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        rc, lmsgs = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(lmsgs))
        if verbose and msgs:
            print("\n".join(msgs))
        os.replace(tmp, out)
    finally:
        for o in objs + [tmp]:
            if os.path.exists(o):
                os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
