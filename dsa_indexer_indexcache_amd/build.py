"""Builds the HIP library (gfx950) in-tree: dsa_indexer_indexcache_amd/libdsa_mi355x.so.

Every source is compiled to an object of its own in parallel (each translation unit
carries its own device code; none calls device code of another), then the objects
are linked into the shared library.  Every call compiles from scratch."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libdsa_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 4)))
    with tempfile.TemporaryDirectory(prefix="dsa_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[HIPCC, *FLAGS, *extra, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, text), s in zip(results, srcs):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s (%d):\n%s" % (s, rc, text))
            if verbose and text.strip():
                print(text)
        tmp = out + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, text = _run(link)
        if rc != 0:
            raise RuntimeError("link failed (%d):\n%s" % (rc, text))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
