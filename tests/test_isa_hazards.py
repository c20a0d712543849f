"""Static check of the pipelined kernels' device assembly (CPU only).

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

For the same reason the compiler cannot give an inline product the two wait
states it needs after a VALU instruction writes one of its A/B operand
registers; the second check asserts that on every path into an inline
product at least two wait states separate it from such a write.
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


def _blocks(lines):
    """Split a kernel body into basic blocks: (label, [(line index, text, in inline asm)])."""
    blocks, cur, inasm = [], ["<entry>", []], False
    for i, line in enumerate(lines):
        if ";;#ASMSTART" in line:
            inasm = True
            continue
        if ";;#ASMEND" in line:
            inasm = False
            continue
        t = line.split(";")[0].strip()
        if t.endswith(":") and not t.startswith("."):
            continue
        if re.match(r"^\.LBB\w+:$", t):
            blocks.append(cur)
            cur = [t[:-1], []]
            continue
        if not t or t.startswith("."):
            continue
        cur[1].append((i, t, inasm))
        if not inasm and re.match(r"s_(c?branch|endpgm|setpc)", t):
            blocks.append(cur)               # a branch ends the block
            cur = [None, []]
    blocks.append(cur)
    return [b for b in blocks if b[0] is not None or b[1]]


def _successors(blocks, k):
    label, ins = blocks[k]
    last = ins[-1][1] if ins else ""
    out = []
    m = re.match(r"s_c?branch\S*\s+(\.LBB\w+)", last)
    if m:
        out.append(m.group(1))
    unconditional = re.match(r"s_(branch|endpgm|setpc)", last)
    if not unconditional and k + 1 < len(blocks):
        out.append(k + 1)
    return out


def _transfer(ins, flight, bad=None):
    flight = set(flight)
    for i, t, inasm in ins:
        if inasm:
            if t.startswith("v_mfma"):
                flight |= _agprs(t.split()[1].rstrip(","))
            elif t.startswith("s_nop 15"):
                flight = set()
            continue
        used = set()
        for tok in t.split()[1:]:
            used |= _agprs(tok.rstrip(","))
        if used & flight and bad is not None:
            bad.append((i, t))
    return flight


def hazards(asm: str):
    """Per kernel: (line, instruction) pairs touching in-flight inline-product registers.

    The in-flight set of each basic block's entry is the union over its
    predecessors (branch targets and fall-through), iterated to a fixed point.
    """
    out = {}
    for name in re.findall(r"^(_Z\S+):", asm, re.M):
        st = asm.index(name + ":")
        en = asm.index(".Lfunc_end", st)
        blocks = _blocks(asm[st:en].splitlines())
        index = {b[0]: k for k, b in enumerate(blocks) if b[0] is not None}
        entry = [set() for _ in blocks]
        work = list(range(len(blocks)))
        while work:
            k = work.pop(0)
            fl = _transfer(blocks[k][1], entry[k])
            for s in _successors(blocks, k):
                j = index[s] if isinstance(s, str) else s
                if not fl <= entry[j]:
                    entry[j] |= fl
                    if j not in work:
                        work.append(j)
        bad = []
        for k, b in enumerate(blocks):
            _transfer(b[1], entry[k], bad)
        out[name] = sorted(bad)
    return out


def _vgprs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _wait_states(t):
    m = re.match(r"s_nop\s+(\d+)", t)
    return int(m.group(1)) + 1 if m else 1


def _valu_writes(t):
    op = t.split()[0]
    if not op.startswith("v_") or op.startswith(("v_mfma", "v_accvgpr_write", "v_cmp", "v_readfirstlane",
                                                 "v_readlane")):
        return set()
    parts = t.split()
    return _vgprs(parts[1].rstrip(",")) if len(parts) > 1 else set()


NEEDED_WAIT_STATES = 2


def operand_hazards(asm: str):
    """Per kernel: inline products reading a VGPR that a VALU instruction wrote
    fewer than two wait states earlier, on some path."""
    out = {}
    for name in re.findall(r"^(_Z\S+):", asm, re.M):
        st = asm.index(name + ":")
        en = asm.index(".Lfunc_end", st)
        blocks = _blocks(asm[st:en].splitlines())
        index = {b[0]: k for k, b in enumerate(blocks) if b[0] is not None}
        preds = [[] for _ in blocks]
        for k in range(len(blocks)):
            for s_ in _successors(blocks, k):
                preds[index[s_] if isinstance(s_, str) else s_].append(k)

        def back(k, j, regs, ws, seen):
            # walk back from instruction j (exclusive) of block k
            ins = blocks[k][1]
            for i in range(j - 1, -1, -1):
                if ws >= NEEDED_WAIT_STATES:
                    return []
                t = ins[i][1]
                if _valu_writes(t) & regs:
                    return [ins[i]]
                ws += _wait_states(t)
            if ws >= NEEDED_WAIT_STATES:
                return []
            bad = []
            for p_ in preds[k]:
                if (p_, ws) not in seen:
                    seen.add((p_, ws))
                    bad += back(p_, len(blocks[p_][1]), regs, ws, seen)
            return bad

        bad = []
        for k, b in enumerate(blocks):
            for j, (i, t, inasm) in enumerate(b[1]):
                if inasm and t.startswith("v_mfma"):
                    toks = [x.rstrip(",") for x in t.split()]
                    regs = _vgprs(toks[2]) | _vgprs(toks[3])
                    for w in back(k, j, regs, 0, set()):
                        bad.append((i, t, w[1]))
        out[name] = bad
    return out


def test_operand_checker_counts_wait_states_along_paths():
    prod = [";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]", ";;#ASMEND"]
    close = "\n".join(["_Za:", "v_cvt_pk_bf16_f32 v9, v1, v2", "s_nop 0", *prod, "s_endpgm",
                       ".Lfunc_end0:"])
    assert len(operand_hazards(close)["_Za"]) == 1
    guarded = close.replace("s_nop 0", "s_nop 1")
    assert operand_hazards(guarded)["_Za"] == []
    other = close.replace("v9,", "v12,")
    assert operand_hazards(other)["_Za"] == []
    # the write sits in a predecessor block that branches straight to the product
    pred = "\n".join(["_Zb:", "s_cbranch_scc0 .LBB0_2", "v_cvt_pk_bf16_f32 v5, v1, v2",
                      ".LBB0_2:", *prod, "s_endpgm", ".Lfunc_end0:"])
    assert [w for _, _, w in operand_hazards(pred)["_Zb"]] == ["v_cvt_pk_bf16_f32 v5, v1, v2"]


def test_checker_flags_a_copy_after_an_inline_product():
    asm = "\n".join([
        "_Zk:", ";;#ASMSTART", "s_nop 2", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
        ";;#ASMEND", "v_accvgpr_mov_b32 a16, a3", ".Lfunc_end0:"])
    assert hazards(asm)["_Zk"] == [(5, "v_accvgpr_mov_b32 a16, a3")]
    drained = asm.replace("v_accvgpr_mov", ";;#ASMSTART\ns_nop 15\n;;#ASMEND\nv_accvgpr_mov")
    assert hazards(drained)["_Zk"] == []


def test_checker_follows_branches_not_text_order():
    product = [";;#ASMSTART", "s_nop 2", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
               ";;#ASMEND"]
    drain = [";;#ASMSTART", "s_nop 15", ";;#ASMEND"]
    # a product at the end of a loop laid out last, branching back: the block
    # after it in the text is not reached from it
    tail = "\n".join(["_Zt:", "s_branch .LBB0_2", ".LBB0_1:", *drain, "v_accvgpr_read_b32 v0, a3",
                      "s_endpgm", ".LBB0_2:", *product, "s_cbranch_scc0 .LBB0_2", "s_branch .LBB0_1",
                      ".LBB0_3:", "v_accvgpr_read_b32 v1, a4", "s_endpgm", ".Lfunc_end0:"])
    assert hazards(tail)["_Zt"] == []
    # a product before a forward branch reaches the target block undrained
    fwd = "\n".join(["_Zf:", *product, "s_cbranch_scc0 .LBB0_1", *drain, "s_endpgm", ".LBB0_1:",
                     "v_accvgpr_read_b32 v1, a4", "s_endpgm", ".Lfunc_end0:"])
    assert [t for _, t in hazards(fwd)["_Zf"]] == ["v_accvgpr_read_b32 v1, a4"]


@pytest.mark.skipif(shutil.which(build_lib.HIPCC) is None and not os.path.exists(build_lib.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src,kinds", [("attn_bwd_pipe.hip", ("dkdv", "dq")),
                                       ("attn_fwd_pipe.hip", ("fwd",)),
                                       ("attn_bob_pipe.hip", ("bob_q2",))])
def test_pipelined_kernels_never_touch_in_flight_accumulators(tmp_path, src, kinds):
    out = tmp_path / "pipe.s"
    flags = [f for f in build_lib.COMMON_FLAGS if f != "-fPIC"]
    cmd = [build_lib.HIPCC, *flags, *build_lib.PER_SOURCE_FLAGS.get(src, []), "--cuda-device-only",
           "-S", os.path.join(build_lib.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    found = hazards(out.read_text())
    assert found, "no kernels found in the assembly"
    assert all(any(kind in k for k in found) for kind in kinds)
    bad = {k: v[:3] for k, v in found.items() if v}
    assert not bad, bad
    close = {k: v[:3] for k, v in operand_hazards(out.read_text()).items() if v}
    assert not close, close
