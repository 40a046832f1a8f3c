"""Scan of gfx950 assembly for matrix-core hazards the compiler cannot see.

The forward kernels issue their MFMA instructions as inline assembly, so the
compiler inserts no wait states around them. Two read-after-write hazards
must then be covered by the code itself:

* an MFMA writes registers (scores, or output accumulators) that vector code
  or v_accvgpr_read / mov then reads: at least ``need`` wait states (s_nop n
  counts n + 1, every other instruction 1) must separate them;
* vector code writes registers that an MFMA then reads as its A or B operand:
  at least two instructions must separate them.

The scan walks straight-line code only (it stops at labels and branches), which
is where the kernels place a product next to the code that consumes it.
"""
import re

_RANGE = re.compile(r"([va])\[(\d+):(\d+)\]")
_ONE = re.compile(r"([va])(\d+)$")


def _regs(tok):
    tok = tok.strip().lstrip("-|").rstrip("|")
    m = _RANGE.match(tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok} if _ONE.match(tok) else set()


def _instructions(lines):
    out = []
    for ln, raw in enumerate(lines, 1):
        s = raw.split(";")[0].strip()
        if not s or s.startswith("."):
            continue
        if s.endswith(":") or s.startswith("s_cbranch") or s.startswith("s_branch"):
            out.append((ln, None))   # block boundary
            continue
        out.append((ln, s))
    return out


def kernels(asm_text):
    """{mangled kernel name: list of its lines} for every kernel in the file."""
    lines = asm_text.split("\n")
    res, cur, body = {}, None, []
    for line in lines:
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is not None:
            body.append(line)
            if "s_endpgm" in line:
                res[cur] = body
                cur = None
    return res


def scan(body_lines, need=19, valu_gap=2):
    """Returns a list of (kind, line, mfma, other) hazards in one kernel."""
    ins = _instructions(body_lines)
    found = []
    for k, (ln, s) in enumerate(ins):
        if s is None or not s.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        dst, srcs = _regs(ops[0]), _regs(ops[1]) | _regs(ops[2])
        # MFMA result read too early by non-MFMA code
        ws = 0
        for ln2, s2 in ins[k + 1:]:
            if s2 is None or ws >= need:
                break
            if s2.startswith("s_nop"):
                ws += int(s2.split()[1]) + 1
                continue
            ws += 1
            if s2.startswith("v_mfma") or s2.startswith("s_") or " " not in s2:
                continue
            o2 = s2.split(None, 1)[1].split(",")
            touched = set().union(*(_regs(o) for o in o2))
            if touched & dst:
                found.append(("mfma->read", ln2, s, s2))
        # operand written by vector code just before the product
        back = 0
        for ln2, s2 in reversed(ins[:k]):
            if s2 is None or back >= valu_gap:
                break
            if s2.startswith("s_nop"):
                back += int(s2.split()[1]) + 1
                continue
            back += 1
            if s2.startswith("v_") and not s2.startswith("v_mfma") and " " in s2:
                if _regs(s2.split(None, 1)[1].split(",")[0]) & srcs:
                    found.append(("write->mfma", ln, s, s2))
    return found
