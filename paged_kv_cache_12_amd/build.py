"""Compile libpa.so for gfx950 with hipcc (in-tree, no JIT cache).

Run as `python -m paged_kv_cache_12_amd.build` or through `__graft_entry__.build()`.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libpa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("PA_ARCH", "gfx950")

SOURCES = ["pa_pool.cpp", "pa_prefix.cpp", "pa_movement.hip", "pa_decode.hip", "pa_step.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-result",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, obj: str, extra: list[str]) -> subprocess.Popen:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile every source and link libpa.so (or `out`); returns its path."""
    extra = list(extra or [])
    out = out or LIB
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = tempfile.mkdtemp(prefix="pa_build_")
    try:
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            procs.append((src, obj, _compile(src, obj, extra)))
        objs = []
        for src, obj, pr in procs:
            outp, _ = pr.communicate()
            noise = [ln for ln in outp.splitlines()
                     if "packed-fp32-ops" not in ln or "not a recognized feature" not in ln]
            if pr.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
            if verbose and noise:
                print("\n".join(noise), file=sys.stderr)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libpa.so")
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        shutil.move(tmp_lib, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
