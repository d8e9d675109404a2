"""Wait-state check of the direct global -> LDS loads in compiled gfx950 code.

The GEMM engine issues `global_load_lds_dwordx4` from an asm statement.  On
gfx9 a vector-memory instruction that reads a scalar register written by a
vector ALU instruction (`v_readfirstlane_b32` and the like) must come at
least 5 wait states after that write; the compiler pads its own memory
instructions with `s_nop` for this (the probe in tests/test_isa_hazards.py shows it), but
it does not look inside an asm statement.  A load issued too early reads the
register's previous contents as its address.

`scan(asm_text)` finds, for every `global_load_lds*` in the assembly, each
scalar register it reads (the base pair, and m0) that a vector instruction wrote
fewer than 5 wait states before it, along every path into the load (straight
line, branches and loop back edges).  One instruction counts one wait state,
`s_nop N` counts N + 1.
"""
import re
from dataclasses import dataclass

VMEM_SGPR_AFTER_VALU = 5      # wait states
_LOAD = re.compile(r"global_load_lds")
_BRANCH = re.compile(r"s_(?:c)?branch\w*\s+(\S+)$")
_FUNC = re.compile(r"^([_A-Za-z][\w.$]*):")
# scalar instructions whose first operand is not a destination
_SALU_NO_DEST = re.compile(r"s_(?:cmp|cmpk|bitcmp|waitcnt|nop|barrier|branch|cbranch|sleep|setprio|"
                           r"sendmsg|trap|dcache|icache|endpgm|setreg|set_gpr_idx|setpc|ttrace|"
                           r"incperflevel|decperflevel|wakeup|denorm_mode|round_mode)")


@dataclass
class Hazard:
    function: str
    load: str
    writer: str
    wait_states: int


def _sregs(tok: str) -> set:
    tok = tok.strip()
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {tok} if re.fullmatch(r"s\d+|vcc|vcc_lo|vcc_hi|m0", tok) else set()


def _operands(ins: str) -> list:
    parts = ins.split(None, 1)
    return [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []


def _valu_sgpr_defs(ins: str) -> set:
    """Scalar registers a vector ALU instruction writes (its scalar dests)."""
    op = ins.split(None, 1)[0]
    if not op.startswith("v_"):
        return set()
    ops = _operands(ins)
    out = _sregs(ops[0]) if ops else set()
    # second destination: carry-out or the scale flag
    if ("_co_" in op or op.startswith(("v_div_scale", "v_mad_u64_u32", "v_mad_i64_i32"))) and len(ops) > 1:
        out |= _sregs(ops[1])
    return out


def _wait_states(ins: str) -> int:
    m = re.match(r"s_nop\s+(\S+)", ins)
    return int(m.group(1), 0) + 1 if m else 1


def functions(asm_text: str) -> dict:
    """Instruction lists per kernel symbol (labels kept as 'NAME:')."""
    funcs, cur = {}, None
    for raw in asm_text.splitlines():
        line = raw.split(";")[0].strip()
        if not line:
            continue
        m = _FUNC.match(line)
        if m and not line.startswith("."):
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None:
            continue
        if line.startswith(".") and not re.match(r"\.LBB\w*:", line):
            if line.startswith(".Lfunc_end"):
                cur = None
            continue
        funcs[cur].append(line)
    return funcs


def _scan_function(name: str, body: list) -> list:
    branches_to = {}
    for k, ins in enumerate(body):
        m = _BRANCH.match(ins)
        if m:
            branches_to.setdefault(m.group(1), []).append(k)
    found = []

    def walk(j, need, ws, load, seen):
        while j >= 0 and ws < VMEM_SGPR_AFTER_VALU and need:
            ins = body[j]
            if ins.endswith(":"):
                for k in branches_to.get(ins[:-1], []):
                    if (k, ws) not in seen:
                        seen.add((k, ws))
                        walk(k - 1, need, ws + 1, load, seen)   # the branch itself
                j -= 1
                continue
            if ins.startswith("s_branch") or ins.startswith("s_endpgm"):
                return                                   # no fall-through into what follows
            hit = _valu_sgpr_defs(ins) & need
            if hit:
                found.append(Hazard(name, load, ins, ws))
                need = need - hit
            elif _SALU_NO_DEST.match(ins) is None and ins.startswith("s_"):
                # a scalar write ends the search for that register on this path
                ops = _operands(ins)
                if ops:
                    need = need - _sregs(ops[0])
            ws += _wait_states(ins)
            j -= 1

    for i, ins in enumerate(body):
        if not _LOAD.search(ins.split(None, 1)[0]):
            continue
        need = {"m0"}                                    # the LDS address, read implicitly
        for t in _operands(ins)[1:]:
            need |= _sregs(t)
        walk(i - 1, need, 0, ins, set())
    return found


def scan(asm_text: str) -> list:
    out = []
    for name, body in functions(asm_text).items():
        out += _scan_function(name, body)
    return out


def count_loads(asm_text: str) -> int:
    return sum(1 for body in functions(asm_text).values() for ins in body
               if _LOAD.search(ins.split(None, 1)[0]))
