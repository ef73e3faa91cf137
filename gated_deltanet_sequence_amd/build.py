"""Build libgdn.so (the gfx950 HIP library behind include/gdn.h) in-tree with hipcc.

Usage: ``python -m gated_deltanet_sequence_amd.build`` (also run by
``__graft_entry__.build()``).  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["api.hip", "decode.hip", "chunk_local.hip", "chunk_local2.hip", "chunk_local2_f32.hip", "state_scan.hip", "epilogue.hip", "prologue.hip", "bwd2.hip"]
ARCH = "gfx950"


BUILD_DIR = os.path.join(PKG, "_build")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from emitting packed float32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core accumulators in ordinary VGPRs (no AGPR <-> VGPR copies)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wall", "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_cmd(out: str = LIB):
    """The single-command form of the build (all sources, one hipcc)."""
    return [_hipcc(), *_flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    return r.returncode, msgs


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object (in parallel), then link libgdn.so.  Always
    recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[_hipcc(), *_flags(), "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for (rc, msgs), src in zip(results, SOURCES):
        if rc != 0:
            failed = True
            sys.stderr.write(f"--- {src}\n" + "\n".join(msgs) + "\n")
        elif verbose and msgs:
            sys.stderr.write("\n".join(msgs) + "\n")
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    link = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, msgs = _run(link)
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc link failed with exit code {rc}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
