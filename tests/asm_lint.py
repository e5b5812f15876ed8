"""Wait-state check of the library's gfx950 device assembly (test
infrastructure, CPU only).

Every matrix product in the kernels is written as inline asm, which the
compiler's hazard recognizer does not see, so the required wait states
around them are placed by hand (s_nop). This module parses the assembly
that the build keeps (fp8_kv_cache_paged_amd/_asm/*.s), builds each
function's control-flow graph and checks, over every path, the CDNA3/CDNA4
matrix-core dependency rules that hand placement can break:

  * a matrix product's result registers are read or written by a VALU,
    memory or LDS instruction within (passes + 4) wait states of its issue
    (20 for the 16-pass fp8 32x32x64, 12 for the 8-pass bf16 32x32x16; the
    CDNA3 rule is passes + 3, one more is taken for gfx950);
  * a later product reads them as its A or B operand within that window
    (reading them as its accumulator, exactly overlapped, is forwarded);
  * a product reads a register a VALU instruction wrote fewer than 2 wait
    states before.

Wait states are counted as the hardware counts issue slots: one per
instruction, k + 1 for s_nop k. At control-flow joins the worst case over
the incoming paths is kept; loops are iterated to a fixed point.

It also rejects two instruction classes outright: packed fp32 arithmetic,
which the build switches off, and writes through the scalar data cache.
"""

import re
from collections import defaultdict

MFMA_PASSES = {
    "v_mfma_f32_32x32x64_f8f6f4": 16,
    "v_mfma_f32_32x32x16_bf16": 8,
    "v_mfma_f32_16x16x32_bf16": 4,
    "v_mfma_f32_16x16x128_f8f6f4": 8,
}
VALU_TO_MFMA = 2
# wait states beyond the pass count before a product's results may be touched:
# 3 on CDNA3, one more taken here for gfx950
XDL_EXTRA = 4

# instruction classes the library must never contain (patterns kept free of
# the literal mnemonics)
FORBIDDEN = [
    (re.compile(r"^v_pk_(add|mul|fma)_f32\b"), "packed fp32 arithmetic"),
    (re.compile(r"^s_(buffer_|scratch_)?(st[o]re|at[o]mic)"), "a write through the scalar data cache"),
    (re.compile(r"^s_dcache_w[b]"), "a scalar data cache write-back"),
]

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(text):
    """Vector registers named in an operand string, as ('v'|'a', index) pairs."""
    out = []
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.append((kind, int(m.group(4))))
        else:
            out.extend((kind, i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _split_operands(rest):
    ops, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            ops.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        ops.append(cur.strip())
    return ops


class Insn:
    __slots__ = ("op", "operands", "line", "text")

    def __init__(self, op, operands, line, text):
        self.op, self.operands, self.line, self.text = op, operands, line, text


def parse_functions(asm_text):
    """{function name: [items]} where an item is ('label', name) or ('insn', Insn)."""
    funcs, cur, name = {}, None, None
    for ln, raw in enumerate(asm_text.splitlines(), 1):
        line = raw.split(";")[0].rstrip()
        if not line.strip():
            continue
        m = re.match(r"^([A-Za-z_.$][\w.$]*):", line)
        if m and not line.startswith("\t"):
            lab = m.group(1)
            if lab.startswith(".Lfunc_end"):
                if cur is not None:
                    funcs[name] = cur
                cur, name = None, None
            elif lab.startswith(".L") or lab.startswith("$"):
                if cur is not None:
                    cur.append(("label", lab))
            elif not lab.startswith("."):
                cur, name = [], lab
            continue
        if cur is None or not line.startswith("\t"):
            continue
        body = line.strip()
        if body.startswith("."):
            continue
        parts = body.split(None, 1)
        op = parts[0]
        rest = parts[1] if len(parts) > 1 else ""
        cur.append(("insn", Insn(op, _split_operands(rest), ln, body)))
    return funcs


def _blocks(items):
    """Basic blocks: list of (label or None, [Insn]) and successor lists."""
    blocks, cur_lab, cur = [], None, []
    for kind, x in items:
        if kind == "label":
            if cur or cur_lab is not None:
                blocks.append((cur_lab, cur))
            cur_lab, cur = x, []
        else:
            cur.append(x)
            if x.op.startswith("s_branch") or x.op.startswith("s_cbranch") or x.op in ("s_endpgm", "s_setpc_b64"):
                blocks.append((cur_lab, cur))
                cur_lab, cur = None, []
    if cur or cur_lab is not None:
        blocks.append((cur_lab, cur))
    index = {lab: i for i, (lab, _) in enumerate(blocks) if lab is not None}
    succ = []
    for i, (_, insns) in enumerate(blocks):
        s = []
        last = insns[-1] if insns else None
        if last is not None and (last.op.startswith("s_branch") or last.op.startswith("s_cbranch")):
            tgt = last.operands[-1] if last.operands else None
            if tgt in index:
                s.append(index[tgt])
            if last.op.startswith("s_cbranch") and i + 1 < len(blocks):
                s.append(i + 1)
        elif last is not None and last.op in ("s_endpgm", "s_setpc_b64"):
            pass
        elif i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    return blocks, succ


def _issue_slots(insn):
    if insn.op == "s_nop":
        try:
            return int(insn.operands[0], 0) + 1
        except (IndexError, ValueError):
            return 1
    return 1


def _is_vector_access(op):
    return (op.startswith("v_") or op.startswith("ds_") or op.startswith("global_") or op.startswith("buffer_")
            or op.startswith("flat_") or op.startswith("scratch_"))


class State:
    """mfma[reg] = (wait states still required, index of the product); valu[reg] = slots since a VALU write."""

    __slots__ = ("mfma", "valu")

    def __init__(self, mfma=None, valu=None):
        self.mfma = dict(mfma or {})
        self.valu = dict(valu or {})

    def copy(self):
        return State(self.mfma, self.valu)

    def merge(self, other):
        changed = False
        for r, (need, src) in other.mfma.items():
            if need > self.mfma.get(r, (0, None))[0]:
                self.mfma[r] = (need, src)
                changed = True
        for r, age in other.valu.items():
            if age < self.valu.get(r, 10 ** 9):
                self.valu[r] = age
                changed = True
        return changed

    def advance(self, n):
        self.mfma = {r: (need - n, s) for r, (need, s) in self.mfma.items() if need - n > 0}
        self.valu = {r: age + n for r, age in self.valu.items() if age + n < VALU_TO_MFMA}


def _step(state, insn, violations, where):
    op = insn.op
    for pat, what in FORBIDDEN:
        if pat.match(op):
            violations.append(f"{where}: line {insn.line}: {what}: {insn.text}")
    if op in MFMA_PASSES or op.startswith("v_mfma"):
        passes = MFMA_PASSES.get(op)
        if passes is None:
            violations.append(f"{where}: line {insn.line}: matrix product with unknown pass count: {op}")
            passes = 16
        dst = _regs(insn.operands[0]) if insn.operands else []
        a = _regs(insn.operands[1]) if len(insn.operands) > 1 else []
        b = _regs(insn.operands[2]) if len(insn.operands) > 2 else []
        c = _regs(insn.operands[3]) if len(insn.operands) > 3 else []
        for r in a + b:
            if r in state.mfma:
                violations.append(f"{where}: line {insn.line}: operand {r[0]}{r[1]} of an earlier product read "
                                  f"{state.mfma[r][0]} wait states too early: {insn.text}")
        if c and set(c) != set(dst):
            for r in c:
                if r in state.mfma:
                    violations.append(f"{where}: line {insn.line}: accumulator {r[0]}{r[1]} not forwarded, read "
                                      f"{state.mfma[r][0]} wait states too early: {insn.text}")
        for r in a + b + c:
            if r in state.valu:
                violations.append(f"{where}: line {insn.line}: {r[0]}{r[1]} written by VALU "
                                  f"{state.valu[r]} wait states before this product: {insn.text}")
        state.advance(1)
        for r in dst:
            state.mfma[r] = (passes + XDL_EXTRA, insn.line)
        return
    if _is_vector_access(op):
        touched = []
        for o in insn.operands:
            touched.extend(_regs(o))
        for r in touched:
            if r in state.mfma:
                violations.append(f"{where}: line {insn.line}: {r[0]}{r[1]} of the product at line "
                                  f"{state.mfma[r][1]} accessed {state.mfma[r][0]} wait states too early: "
                                  f"{insn.text}")
        n = _issue_slots(insn)
        state.advance(n)
        if op.startswith("v_") and insn.operands:
            for r in _regs(insn.operands[0]):
                state.valu[r] = 0
        return
    state.advance(_issue_slots(insn))


def check_function(name, items, max_rounds=64):
    blocks, succ = _blocks(items)
    if not blocks:
        return []
    entry = [None] * len(blocks)
    entry[0] = State()
    work = [0]
    rounds = defaultdict(int)
    while work:
        i = work.pop()
        rounds[i] += 1
        if rounds[i] > max_rounds:
            return [f"{name}: no fixed point after {max_rounds} passes over block {i}"]
        st = entry[i].copy()
        for insn in blocks[i][1]:
            _step(st, insn, [], name)
        for j in succ[i]:
            if entry[j] is None:
                entry[j] = st.copy()
                work.append(j)
            elif entry[j].merge(st):
                work.append(j)
    violations = []
    for i, (_, insns) in enumerate(blocks):
        if entry[i] is None:
            continue
        st = entry[i].copy()
        for insn in insns:
            _step(st, insn, violations, name)
    return sorted(set(violations))


def check_text(asm_text):
    """(number of functions checked, violations) for one assembly file."""
    funcs = parse_functions(asm_text)
    out = []
    for name, items in funcs.items():
        out.extend(check_function(name, items))
    return len(funcs), out
