"""Compile libattn.so for gfx950 with hipcc, in-tree.

Each HIP source is compiled to an object under ``_build/`` (in parallel), then
linked into ``libattn.so`` next to this file.  Packed fp32 VALU instructions
are turned off for device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ("attn_api.hip", "attn_fwd.hip", "attn_fwd_pipe.hip", "attn_bwd.hip", "attn_bwd_pipe.hip",
           "attn_bob.hip", "attn_bob_pipe.hip")
# The pipelined kernels keep long-lived operands in AGPRs (pinned in the
# source) and want every MFMA result and accumulator in VGPRs, where the VALU
# can read them without copies.
PER_SOURCE_FLAGS = {"attn_bwd_pipe.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
                    "attn_fwd_pipe.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
                    "attn_bob_pipe.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return r.returncode, r.stdout


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source and link libattn.so; return its path.  Raises on error."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [HIPCC, *COMMON_FLAGS, *PER_SOURCE_FLAGS.get(src, []), *extra_flags, "-c",
               os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, obj, cmd))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: (j, _run(j[2])), jobs))
    for (src, _, cmd), (rc, out) in results:
        if verbose or rc != 0:
            sys.stderr.write(f"[build] {' '.join(cmd)}\n{out}")
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[j[1] for j in jobs], "-o", tmp]
    rc, out = _run(cmd)
    if verbose or rc != 0:
        sys.stderr.write(f"[build] {' '.join(cmd)}\n{out}")
    if rc != 0:
        raise RuntimeError("link of libattn.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
