"""Compile libaqd.so (all HIP sources under csrc/) for gfx950, in the package directory.

Each source is compiled to an object in parallel (the small-batch kernels have
many instantiations), then the objects are linked into one shared library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libaqd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # kernel-argument preloading: the leading scalar arguments of a kernel arrive in SGPRs at launch,
    # so its first loads need not wait for an argument load
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]
_NOISE = ("packed-fp32-ops' is not a recognized feature",)


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if not any(n in ln for n in _NOISE)]
    return r.returncode, msgs


def build(out: str = LIB, extra=(), quiet: bool = True) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    tmpdir = tempfile.mkdtemp(prefix="aqd_build_")
    try:
        srcs = sources()
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        jobs = [[HIPCC, *FLAGS, *extra, *inc, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 4)))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(_run, jobs))
        msgs = [m for _, ms in results for m in ms]
        failed = [s for s, (rc, _) in zip(srcs, results) if rc != 0]
        if failed:
            raise RuntimeError("hipcc failed on " + ", ".join(os.path.basename(f) for f in failed) + ":\n" +
                               "\n".join(msgs))
        tmp = out + ".tmp"
        rc, lmsgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
        if rc != 0:
            raise RuntimeError("link failed:\n" + "\n".join(lmsgs))
        if (msgs or lmsgs) and not quiet:
            print("\n".join(msgs + lmsgs), file=sys.stderr)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
