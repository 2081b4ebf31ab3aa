"""Wait states around the hand-written AGPR MFMAs.

The kernels that keep a long-lived accumulator in the AGPRs issue its
32x32x16 bf16 MFMAs as inline assembly, which the compiler's hazard tracking
does not see.  Two rules then fall to the source, and this test checks them
on the gfx950 assembly the build's own flags produce:

* no instruction reads or writes an MFMA's destination AGPRs fewer than 19
  wait states after it (along any control-flow path), other than a later MFMA
  accumulating into exactly the same registers -- the matrix core writes its
  results back over that many cycles, and an early read (a compiler copy at a
  branch join, say) sees the old values;
* no VALU result is read by such an MFMA as its A or B operand in the next
  2 wait states.

Compiles the sources to assembly (hipcc, a few tens of seconds); skipped
where hipcc is missing.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from causal_attention_fa_amd import build as B

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_bwd_pipe.hip"]
RESULT_WS = 19   # wait states before an MFMA's result may be touched
OPERAND_WS = 2   # wait states between a VALU write and an MFMA reading it


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _assembly(src, out):
    cmd = [_hipcc(), "-x", "hip", *B.flags_for(src), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


def _parse(text):
    """(instructions, labels): instructions are (line, text, in_asm, kernel)."""
    insts, labels = [], {}
    in_asm, kern = False, None
    for n, raw in enumerate(text.split("\n"), 1):
        s = raw.strip()
        if re.match(r"^_Z\S+:", s):
            kern = s.split(":")[0]
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^(\.LBB\d+_\d+):", s)
        if m:
            labels[m.group(1)] = len(insts)
            continue
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        insts.append((n, s.split(";")[0].strip(), in_asm, kern))
    return insts, labels


def _regs(tok, kind):
    m = re.match(kind + r"\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(kind + r"(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _ops(s):
    p = s.split(None, 1)
    return p[0], ([o.strip() for o in p[1].split(",")] if len(p) > 1 else [])


def _cost(s):
    m = re.match(r"s_nop\s+(\d+)", s)
    return int(m.group(1)) + 1 if m else 1


def result_hazards(insts, labels):
    found = []
    for k, (ln, s, in_asm, kern) in enumerate(insts):
        if not (in_asm and s.startswith("v_mfma")):
            continue
        dst = _regs(_ops(s)[1][0], "a")
        if not dst:
            continue
        seen, stack = set(), [(k + 1, 0)]
        while stack:
            j, ws = stack.pop()
            if j >= len(insts) or ws >= RESULT_WS or (j, ws) in seen:
                continue
            seen.add((j, ws))
            ln2, s2, _, kern2 = insts[j]
            if kern2 != kern:
                continue
            op, o = _ops(s2)
            if op.startswith("v_mfma") and _regs(o[0], "a") == dst and _regs(o[3], "a") == dst:
                continue   # the next product of the same accumulation chain
            if set().union(set(), *[_regs(x, "a") for x in o]) & dst:
                found.append(f"{kern}: line {ln2} '{s2}' {ws} wait states after line {ln} '{s}'")
                continue
            if op == "s_endpgm":
                continue
            nxt = ws + _cost(s2)
            if op == "s_branch":
                stack.append((labels[o[0]], nxt))
                continue
            if op.startswith("s_cbranch"):
                stack.append((labels[o[0]], nxt))
            stack.append((j + 1, nxt))
    return found


def operand_hazards(insts):
    found = []
    for k, (ln, s, in_asm, kern) in enumerate(insts):
        if not (in_asm and s.startswith("v_mfma")):
            continue
        o = _ops(s)[1]
        srcs = _regs(o[1], "v") | _regs(o[2], "v")
        ws, j = 0, k - 1
        while j >= 0 and ws < OPERAND_WS:
            _, ps, _, pk = insts[j]
            if pk != kern:
                break
            op, po = _ops(ps)
            if not op.startswith(("v_mfma", "s_", "ds_write", "ds_store", "buffer_",
                                  "global_store", "scratch_store")) and po:
                if _regs(po[0], "v") & srcs:
                    found.append(f"{kern}: line {ln} '{s}' reads '{ps}' after {ws} wait states")
            ws += _cost(ps)
            j -= 1
    return found


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_agpr_mfma_wait_states(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _assembly(s, str(tmp_path / (s + ".s"))), SOURCES))
    n_mfma, problems = 0, []
    for src, text in zip(SOURCES, texts):
        insts, labels = _parse(text)
        n_mfma += sum(1 for i in insts if i[2] and i[1].startswith("v_mfma"))
        problems += [f"{src}: {p}" for p in result_hazards(insts, labels) + operand_hazards(insts)]
    assert n_mfma > 0, "no inline-assembly MFMAs found (the checker no longer matches the sources)"
    assert not problems, "\n".join(problems[:20])


def _snippet(body):
    return "_Zk:\n" + "\n".join(
        (";;#ASMSTART\n" + l[1:] + "\n;;#ASMEND") if l.startswith("!") else l
        for l in body.strip().split("\n"))


def test_checker_finds_planted_hazards():
    """The checker itself, on hand-written code: '!' marks inline assembly."""
    mfma = "!v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"
    read = "v_accvgpr_read_b32 v8, a3"
    cases = [
        # (code, result hazards, operand hazards)
        ([mfma, read], 1, 0),
        ([mfma, "s_nop 7", "s_nop 7", "s_nop 7", read], 0, 0),
        ([mfma, "s_nop 7", "s_nop 7", read], 1, 0),                 # 16 < 19
        ([mfma, mfma, "s_nop 7", "s_nop 7", "s_nop 7", read], 0, 0),  # same chain
        ([mfma, "v_accvgpr_mov_b32 a40, a15"], 1, 0),               # a join copy
        ([mfma, "v_accvgpr_write_b32 a2, v9"], 1, 0),               # write after write
        # the read reached through a taken branch, the fall-through waits
        ([mfma, "s_cbranch_scc1 .LBB0_1", "s_nop 7", "s_nop 7", "s_nop 7", "s_endpgm",
          ".LBB0_1:", read], 1, 0),
        (["v_cvt_pk_bf16_f32 v5, v1, v2", mfma], 0, 1),
        (["v_cvt_pk_bf16_f32 v5, v1, v2", "s_nop 1", mfma], 0, 0),
        (["v_cvt_pk_bf16_f32 v9, v1, v2", mfma], 0, 0),             # not an operand
    ]
    for code, n_res, n_op in cases:
        insts, labels = _parse(_snippet("\n".join(code)))
        assert len(result_hazards(insts, labels)) == n_res, code
        assert len(operand_hazards(insts)) == n_op, code
