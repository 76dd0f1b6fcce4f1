"""Hazard check of the hand-written MFMAs in the compiled dK / dV kernel.

The pipelined dK / dV kernel issues its S and dP MFMAs as inline asm with
results in ordinary VGPRs.  The compiler's hazard recognizer does not see
inline asm as an MFMA, so the wait states it would insert around one are the
kernel's own responsibility.  This test compiles the kernel source for gfx950
to AMD assembly (no GPU needed) and checks every MFMA whose destination is a
VGPR tuple, following both sides of every branch:

* before it: no VALU op writes one of its source registers within the two
  wait states a VALU-to-MFMA operand dependency needs;
* after it: nothing reads or writes its destination registers within sixteen
  wait states (more than the 8-pass XDL-write to VALU-access distance),
  except the next MFMA of the same accumulation chain, which reads them as
  source C in exactly the same registers.

The distances are the MFMA dependency rules of the CDNA3 / CDNA4 ISA
reference guides.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_shared_tree_attn_amd", "csrc")
KERNELS = [
    "_ZN9tree_attn26tree_attn_dkdv_pipe_kernelILi128ELb0EEEvNS_7BwdArgsE",
    "_ZN9tree_attn26tree_attn_dkdv_pipe_kernelILi64ELb0EEEvNS_7BwdArgsE",
    "_ZN9tree_attn26tree_attn_dkdv_pipe_kernelILi128ELb1EEEvNS_7BwdArgsE",
    "_ZN9tree_attn26tree_attn_dkdv_pipe_kernelILi64ELb1EEEvNS_7BwdArgsE",
]
BEFORE, AFTER = 2, 16


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "bwd.s")
    # the library's own flags (prefix_shared_tree_attn_amd/build.py), so that
    # the checked code is the code that ships
    from prefix_shared_tree_attn_amd import build as libbuild
    cmd = [hipcc, *libbuild.COMMON, "-x", "hip", *libbuild.DEVICE, "--cuda-device-only", "-S",
           os.path.join(CSRC, "bwd.hip"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return open(out).read()


def _function(text, name):
    i = re.search("^" + re.escape(name) + ":", text, re.M).end()
    j = text.index(".Lfunc_end", i)
    lines = []
    for raw in text[i:j].split("\n")[1:]:
        s = raw.split(";")[0].strip()
        if s and not (s.startswith(".") and not s.endswith(":")):
            lines.append(s)
    return lines


def _regs(tok):
    """VGPR numbers named by one operand token (v7, v[4:7])."""
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _operands(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return []
    return [t.strip() for t in parts[1].split(",")]


def _wait_states(line):
    op = line.split()[0]
    if op == "s_nop":
        return int(line.split()[1], 0) + 1
    return 1


def _check(lines):
    labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}

    def successors(i):
        op = lines[i].split()[0]
        if op == "s_endpgm":
            return []
        if op == "s_branch":
            return [labels[lines[i].split()[1]]]
        if op.startswith("s_cbranch"):
            return [i + 1, labels[lines[i].split()[1]]]
        return [i + 1] if i + 1 < len(lines) else []

    preds = {i: [] for i in range(len(lines))}
    for i in range(len(lines)):
        for s in successors(i):
            preds[s].append(i)

    problems, checked = [], 0
    for i, line in enumerate(lines):
        if not line.startswith("v_mfma"):
            continue
        ops = _operands(line)
        dst = _regs(ops[0])
        if not dst:
            continue  # accumulation-register destination: compiler-managed
        checked += 1
        srcs = set().union(*(_regs(t) for t in ops[1:]))
        # backward: VALU writes of a source register too close before
        stack, seen = [(p, 0) for p in preds[i]], set()
        while stack:
            j, ws = stack.pop()
            if (j, ws) in seen or lines[j].endswith(":") and not preds[j]:
                continue
            seen.add((j, ws))
            lj = lines[j]
            if lj.endswith(":"):
                stack += [(p, ws) for p in preds[j]]
                continue
            if lj.startswith("v_") and not lj.startswith("v_mfma"):
                w = _operands(lj)
                if w and _regs(w[0]) & srcs:
                    problems.append(f"{i}: {line} <- VALU write {j}: {lj}")
            ws += _wait_states(lj)
            if ws < BEFORE:
                stack += [(p, ws) for p in preds[j]]
        # forward: any access of the destination too close after
        stack, seen = [(s, 0) for s in successors(i)], set()
        while stack:
            j, ws = stack.pop()
            if j >= len(lines) or (j, ws) in seen:
                continue
            seen.add((j, ws))
            lj = lines[j]
            if lj.endswith(":"):
                stack += [(s, ws) for s in successors(j)]
                continue
            touched = set().union(set(), *(_regs(t) for t in _operands(lj)))
            if touched & dst:
                o = _operands(lj)
                chained = (lj.startswith("v_mfma") and _regs(o[0]) == dst
                           and _regs(o[-1]) == dst)
                if not chained:
                    problems.append(f"{i}: {line} -> {j} after {ws} wait states: {lj}")
                continue  # a chained MFMA takes over the registers
            ws += _wait_states(lj)
            if ws < AFTER:
                stack += [(s, ws) for s in successors(j)]
    return checked, problems


@pytest.mark.parametrize("kernel", KERNELS)
def test_vgpr_mfma_hazards(asm, kernel):
    checked, problems = _check(_function(asm, kernel))
    assert checked > 0, "no VGPR-destination MFMA found"
    assert not problems, "\n".join(problems[:20])


MFMA = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], {c}"


@pytest.mark.parametrize("lines,bad", [
    # result read by a VALU op right away
    ([MFMA.format(c="0"), "v_add_f32_e32 v30, v3, v31", "s_endpgm"], True),
    # the same read sixteen wait states later
    ([MFMA.format(c="0"), "s_nop 7", "s_nop 7", "v_add_f32_e32 v30, v3, v31", "s_endpgm"], False),
    # fifteen wait states are not enough
    ([MFMA.format(c="0"), "s_nop 7", "s_nop 6", "v_add_f32_e32 v30, v3, v31", "s_endpgm"], True),
    # a chained MFMA may take the result as source C at once
    ([MFMA.format(c="0"), MFMA.format(c="v[0:15]"), "s_nop 7", "s_nop 7",
      "v_add_f32_e32 v30, v3, v31", "s_endpgm"], False),
    # an MFMA reading the result as an A operand is not a chain
    ([MFMA.format(c="0"), "v_mfma_f32_32x32x16_bf16 v[40:55], v[0:3], v[20:23], 0",
      "s_nop 7", "s_nop 7", "s_endpgm"], True),
    # a VALU op writing an operand just before
    (["v_mov_b32_e32 v21, 0", MFMA.format(c="0"), "s_nop 7", "s_nop 7", "s_endpgm"], True),
    (["v_mov_b32_e32 v21, 0", "s_nop 1", MFMA.format(c="0"), "s_nop 7", "s_nop 7",
      "s_endpgm"], False),
    # a read on the taken side of a branch counts too
    ([MFMA.format(c="0"), "s_cbranch_scc1 .LBB0_1", "s_nop 7", "s_nop 7", "s_endpgm",
      ".LBB0_1:", "v_add_f32_e32 v30, v3, v31", "s_endpgm"], True),
])
def test_checker_finds_planted_hazards(lines, bad):
    checked, problems = _check(lines)
    assert checked >= 1
    assert bool(problems) == bad, problems
