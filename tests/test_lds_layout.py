"""LDS layout of the bf16 tiles: bank-conflict freedom and copy placement (CPU only).

Builds ``lds_layout_check.hip`` as a host program against the kernels' own
header and runs it.  It enumerates the per-lane LDS addresses of every
operand read of the pipelined backward kernels (128-bit row reads and
64-bit transposing reads, head dims 64 and 128; and 256, whose tiles the
generic kernels read at the same addresses) and asserts that each group
of lanes that may be served in one 256-byte LDS cycle touches 64 distinct
banks; it also checks that the asynchronous tile copy stores every logical
16-byte chunk exactly once, at the slot the reads address.
"""

import os
import shutil
import subprocess

import pytest

from exact_softmax_attention_attn_amd import build_lib

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which(build_lib.HIPCC) is None and not os.path.exists(build_lib.HIPCC),
                    reason="hipcc not available")
def test_tile_reads_are_conflict_free_and_copies_land_where_read(tmp_path):
    exe = tmp_path / "lds_layout_check"
    cmd = [build_lib.HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", build_lib.CSRC,
           os.path.join(HERE, "lds_layout_check.hip"), "-o", str(exe)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    out = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout[-3000:]
