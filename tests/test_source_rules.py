"""Source rules the kernels rely on, checked on the host.

* No inline-assembly statement in the HIP sources loads into a register
  operand: the compiler treats an asm output as written when the statement
  issues, so a load still in flight could overwrite a register it has already
  given to something else. Loads use the builtins (whose waits the compiler
  places), or the global -> LDS copy helper, whose statement has no outputs.
* Device code is built without packed-FP32 instructions.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sequence_doc_amd", "csrc")

_LOAD = re.compile(r"\b(ds_read\w*|global_load\w*|buffer_load\w*|flat_load\w*|scratch_load\w*)\b")


def _asm_statements(text):
    """(line, statement) of every asm statement, from `asm` to its closing ')'."""
    out = []
    for m in re.finditer(r"\basm\s+(?:volatile\s*)?\(", text):
        depth, i = 1, m.end()
        while depth and i < len(text):
            depth += {"(": 1, ")": -1}.get(text[i], 0)
            i += 1
        out.append((text.count("\n", 0, m.start()) + 1, text[m.start():i]))
    return out


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))


def test_asm_statements_are_found():
    """The scanner sees the statements it is meant to check (the copy helper)."""
    found = [s for f in _sources() for _, s in _asm_statements(open(os.path.join(CSRC, f)).read())]
    assert any("global_load_lds_dwordx4" in s for s in found)


def _sections(stmt):
    """Template, outputs, inputs, ... of an asm statement: its argument list cut at
    the colons that are outside string literals and nested parentheses."""
    body = stmt[stmt.index("(") + 1:-1]
    parts, cur, depth, quoted, i = [], [], 0, False, 0
    while i < len(body):
        ch = body[i]
        if quoted:
            cur.append(ch)
            if ch == "\\":
                cur.append(body[i + 1])
                i += 1
            elif ch == '"':
                quoted = False
        elif ch == '"':
            quoted = True
            cur.append(ch)
        elif ch in "([":
            depth += 1
            cur.append(ch)
        elif ch in ")]":
            depth -= 1
            cur.append(ch)
        elif ch == ":" and depth == 0:
            parts.append("".join(cur))
            cur = []
        else:
            cur.append(ch)
        i += 1
    parts.append("".join(cur))
    return parts


def _loads_into_registers(text):
    """Lines of asm statements whose template names a load and that have output operands."""
    bad = []
    for line, stmt in _asm_statements(text):
        sec = _sections(stmt)
        if not _LOAD.search(sec[0]):
            continue
        outputs = sec[1] if len(sec) > 1 else ""
        if '"=' in outputs or '"+' in outputs:
            bad.append(line)
    return bad


def test_rule_flags_a_load_with_outputs():
    """The check catches the pattern it exists for, and passes the copy helper's form."""
    bad = 'x;\n  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "n"(8));\n'
    good = 'asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(base));'
    assert _loads_into_registers(bad) == [2]
    assert _loads_into_registers(good) == []


@pytest.mark.parametrize("name", _sources())
def test_no_asm_load_writes_a_register(name):
    bad = _loads_into_registers(open(os.path.join(CSRC, name)).read())
    assert not bad, f"{name}: inline-assembly loads with register outputs at lines {bad}"


def test_device_code_built_without_packed_fp32():
    src = open(os.path.join(ROOT, "long_context_sequence_doc_amd", "build.py")).read()
    assert '"-packed-fp32-ops"' in src
