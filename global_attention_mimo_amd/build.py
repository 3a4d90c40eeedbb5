"""Builds libmimo_attn.so (HIP, gfx950 only) in-tree with hipcc.

    python -m global_attention_mimo_amd.build

Every source is compiled for gfx950 with packed-fp32 instruction selection
disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libmimo_attn.so")
SOURCES = ["prefill.hip", "decode.hip", "append.hip", "backward.hip", "rope.hip", "check.hip", "api.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Inputs are finite by contract: max/min need no NaN canonicalisation.
    "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


def _quiet(stderr: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is harmless.
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    """Compiles every source (always) and links LIBRARY; returns its path."""
    with tempfile.TemporaryDirectory(prefix="mimo_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        failed = []
        for src, p in procs:
            out, err = p.communicate()
            msg = _quiet(err).strip()
            if p.returncode != 0:
                failed.append(f"{src}:\n{msg}")
            elif verbose and msg:
                print(msg, file=sys.stderr)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        tmp_lib = f"{LIBRARY}.{os.getpid()}.tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + _quiet(r.stderr))
        os.replace(tmp_lib, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
