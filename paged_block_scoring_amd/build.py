"""Build ``libqsa.so`` in-tree with hipcc for gfx950.

Each HIP translation unit is compiled to an object in parallel, then linked
into one shared library next to this file.  Packed fp32 VALU instructions are
disabled for all device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqsa.so")

SOURCES = ["qsa_api.hip", "score.hip", "score_group.hip", "stream_select.hip", "topk.hip", "fused.hip", "attend.hip",
           "compress.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE,
]


def build(verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path."""
    tmpdir = tempfile.mkdtemp(prefix="qsa_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # the host pass does not know the device-only feature; that note is expected
            text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
            if p.returncode != 0:
                failed.append((src, text))
            elif verbose and text.strip():
                print(text)
        if failed:
            msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
            raise RuntimeError(f"hipcc failed:\n{msg}")
        tmp_lib = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib] + objs
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
