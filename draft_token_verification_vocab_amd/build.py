"""Build the HIP library in-tree with hipcc for gfx950.

    python -m draft_token_verification_vocab_amd.build

produces draft_token_verification_vocab_amd/libspecverify.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [os.path.join(HERE, "csrc", "specverify.hip"),
           os.path.join(HERE, "csrc", "specverify_noalloc.hip")]
ARCH = os.environ.get("SPECVERIFY_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def compile_command(out: str) -> list[str]:
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wextra", "-Wno-unused-function",
            # no packed-fp32 instructions (see the design notes)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
            "-o", out] + SOURCES


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB_NAME)
    errs = [l for l in res.stderr.splitlines()
            if "packed-fp32-ops" not in l and l.strip()]
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
