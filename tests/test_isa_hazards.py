"""Static check of the pipelined backward kernels' device assembly (CPU only).

The pipelined kernels accumulate dK, dV and dQ with matrix instructions
written in inline assembly, so the compiler does not know their latency.  If
it ever moves or copies one of those accumulator registers (for instance at
the join of two control paths that allocated them differently) before the
product has been written back, the copy reads a stale value and the gradient
is silently wrong.  The kernels drain the pipeline (three long s_nop) before
reading accumulators; this test compiles the source to gfx950 assembly with
the library's own flags and asserts that no instruction outside inline
assembly touches an accumulator register between an inline product and the
next drain.
"""

import os
import re
import shutil
import subprocess

import pytest

from exact_softmax_attention_attn_amd import build_lib

pytestmark = pytest.mark.slow


def _agprs(tok):
    m = re.match(r"a\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"a(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def hazards(asm: str):
    """Per kernel: (line, instruction) pairs touching in-flight inline-product registers."""
    out = {}
    for name in re.findall(r"^(_Z\S+):", asm, re.M):
        st = asm.index(name + ":")
        en = asm.index(".Lfunc_end", st)
        inasm, flight, bad = False, set(), []
        for i, line in enumerate(asm[st:en].splitlines()):
            if ";;#ASMSTART" in line:
                inasm = True
                continue
            if ";;#ASMEND" in line:
                inasm = False
                continue
            t = line.split(";")[0].strip()
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            if inasm:
                if t.startswith("v_mfma"):
                    flight |= _agprs(t.split()[1].rstrip(","))
                elif t.startswith("s_nop 15"):
                    flight = set()
                continue
            used = set()
            for tok in t.split()[1:]:
                used |= _agprs(tok.rstrip(","))
            if used & flight:
                bad.append((i, t))
        out[name] = bad
    return out


def test_checker_flags_a_copy_after_an_inline_product():
    asm = "\n".join([
        "_Zk:", ";;#ASMSTART", "s_nop 2", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
        ";;#ASMEND", "v_accvgpr_mov_b32 a16, a3", ".Lfunc_end0:"])
    assert hazards(asm)["_Zk"] == [(5, "v_accvgpr_mov_b32 a16, a3")]
    drained = asm.replace("v_accvgpr_mov", ";;#ASMSTART\ns_nop 15\n;;#ASMEND\nv_accvgpr_mov")
    assert hazards(drained)["_Zk"] == []


@pytest.mark.skipif(shutil.which(build_lib.HIPCC) is None and not os.path.exists(build_lib.HIPCC),
                    reason="hipcc not available")
def test_pipelined_kernels_never_touch_in_flight_accumulators(tmp_path):
    src = "attn_bwd_pipe.hip"
    out = tmp_path / "pipe.s"
    flags = [f for f in build_lib.COMMON_FLAGS if f != "-fPIC"]
    cmd = [build_lib.HIPCC, *flags, *build_lib.PER_SOURCE_FLAGS.get(src, []), "--cuda-device-only",
           "-S", os.path.join(build_lib.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    found = hazards(out.read_text())
    assert found, "no kernels found in the assembly"
    assert any("dkdv" in k for k in found) and any("dq" in k for k in found)
    bad = {k: v[:3] for k, v in found.items() if v}
    assert not bad, bad
