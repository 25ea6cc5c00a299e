"""Build libfftconv.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m fft_long_convolution_amd.build   (always recompiles)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libfftconv.so")
SOURCES = [os.path.join(HERE, "csrc", "fftconv_host.cpp"),
           os.path.join(HERE, "csrc", "fftconv_kernels.hip"),
           os.path.join(HERE, "csrc", "fftconv_row.hip"),
           os.path.join(HERE, "csrc", "fftconv_wide.hip"),
           os.path.join(HERE, "csrc", "fftconv_mp.hip"),
           os.path.join(HERE, "csrc", "fftconv_inner.hip"),
           os.path.join(HERE, "csrc", "fftconv_kgrad.hip"),
           os.path.join(HERE, "csrc", "fftconv_scratch.hip")]
# per-source extra flags: the inner multi-pass kernel schedules best with the
# max-ILP strategy (measured; the other kernels are slower with it)
EXTRA = {"fftconv_inner.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("FFTCONV_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=" + ARCH,
    # keep hipcc from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel, each with its own
    flags), then link the shared library."""
    import tempfile
    tmpdir = tempfile.mkdtemp(prefix="fftconv_build_")
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        cmd = ([HIPCC] + [f for f in FLAGS if f != "-shared"] +
               EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    errs = []
    for src, pr in procs:
        _, err = pr.communicate()
        err = "\n".join(l for l in (err or "").splitlines()
                        if "packed-fp32-ops" not in l and "hip-link" not in l)
        if pr.returncode != 0:
            errs.append(src + ":\n" + err)
        elif verbose and err.strip():
            print(err)
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + (r.stderr or ""))
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    os.rmdir(tmpdir)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
    sys.exit(0)
