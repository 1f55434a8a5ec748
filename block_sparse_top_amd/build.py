"""Build libmsa.so (the MSA C-ABI library) for gfx950 with hipcc, in-tree.

Each source is compiled to its own object in parallel (every .hip file
carries its own device code object; no relocatable device code), then the
objects are linked into one shared library."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmsa.so")
SOURCES = ["api.cpp", "proxy_maxscore.hip", "topk_select.hip", "sparse_prefill.hip", "sparse_decode.hip",
           "proxy_kl.hip", "dense_attn.hip", "diag.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False) -> str:
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    with tempfile.TemporaryDirectory(prefix="msa_build_") as tmpd:
        jobs = []
        for s in SOURCES:
            obj = os.path.join(tmpd, os.path.splitext(s)[0] + ".o")
            jobs.append((s, obj, [HIPCC, *FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", obj]))
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(lambda j: (j[0], *_run(j[2])), jobs))
        for src, rc, out in results:
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{out}")
            if verbose and out.strip():
                print(out)
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[j[1] for j in jobs], "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, out = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
