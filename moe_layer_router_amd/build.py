"""Build the HIP library ``libmoe.so`` in-tree for gfx950.

Run as ``python -m moe_layer_router_amd.build`` (or through
``__graft_entry__.build()``).  Every ``csrc/*.hip`` is compiled to an object
file (in parallel, one hipcc process per source) and the objects are linked
into ``moe_layer_router_amd/libmoe.so``.  No source calls device code of
another, so the objects need no relocatable device code.
"""

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: the compiler must not form v_pk_* fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 4
    return max(1, min(n, 16))


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    inc = ["-I", os.path.join(HERE, "..", "include")]
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc()] + FLAGS + inc + ["-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, cmd, r

        with ThreadPoolExecutor(max_workers=_jobs()) as ex:
            results = list(ex.map(compile_one, srcs))
        failed = False
        for src, _, cmd, r in results:
            if verbose:
                print(" ".join(cmd), flush=True)
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                failed = True
            elif verbose and r.stderr.strip():
                # hipcc's host pass reports the packed-fp32 feature as unknown once per source
                lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
                if lines:
                    sys.stderr.write("\n".join(lines) + "\n")
        if failed:
            raise RuntimeError("hipcc failed building libmoe.so")
        tmp = LIB + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + [o for _, o, _, _ in results] + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("linking libmoe.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
