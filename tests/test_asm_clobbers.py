"""Inline assembly in the HIP sources declares the scalar condition code it
writes.  Most scalar ALU instructions (compares, min/max, add/sub, the bit
operations) set SCC; a statement that issues one without listing "scc" among
its clobbers lets the compiler keep a comparison's result in SCC across it,
and the branch or select after it then reads the wrong value."""
import pathlib
import re

import pytest

CSRC = pathlib.Path(__file__).resolve().parents[1] / "state_space_model_mamba_amd" / "csrc"

# scalar ALU opcodes that write SCC (gfx9 family): compares, bit tests,
# arithmetic with carry or overflow, min/max, the logical and shift operations
_SCC_WRITERS = re.compile(
    r"\bs_(cmp|bitcmp|add|sub|addc|subb|min|max|and|or|xor|andn2|orn2|nand|nor|xnor|"
    r"lshl|lshr|ashr|bfe|abs|not|absdiff|bcnt|quadmask|wqm)\w*\b")


def _asm_statements(text):
    """(line, template, clobbers) of every asm statement with a non-empty template."""
    out = []
    for m in re.finditer(r"\basm\s*(?:volatile\s*)?\(", text):
        depth, i = 1, m.end()
        while depth and i < len(text):
            depth += {"(": 1, ")": -1}.get(text[i], 0)
            i += 1
        body = text[m.end():i - 1]
        strings = re.findall(r'"((?:[^"\\]|\\.)*)"', body.split(":")[0])
        parts = body.split(":")
        clobbers = parts[3] if len(parts) > 3 else ""
        out.append((text.count("\n", 0, m.start()) + 1, "".join(strings), clobbers))
    return out


def _sources():
    return sorted(p for p in CSRC.iterdir() if p.suffix in (".hip", ".h", ".cpp"))


def test_sources_found():
    assert any(p.suffix == ".hip" for p in _sources())


@pytest.mark.parametrize("path", _sources(), ids=lambda p: p.name)
def test_scalar_asm_declares_scc(path):
    for line, template, clobbers in _asm_statements(path.read_text()):
        if _SCC_WRITERS.search(template):
            assert '"scc"' in clobbers, f"{path.name}:{line}: asm writes SCC without declaring it"


def test_checker_sees_an_undeclared_write():
    bad = 'asm("s_max_i32 %0, %1, 0" : "=s"(r) : "s"(x));'
    good = 'asm("s_max_i32 %0, %1, 0" : "=s"(r) : "s"(x) : "scc");'
    (_, t_bad, c_bad), = _asm_statements(bad)
    (_, t_good, c_good), = _asm_statements(good)
    assert _SCC_WRITERS.search(t_bad) and '"scc"' not in c_bad
    assert _SCC_WRITERS.search(t_good) and '"scc"' in c_good
    # s_mov and s_waitcnt write no SCC
    assert not _SCC_WRITERS.search("s_mov_b32 m0, %0\\n\\tbuffer_load_dword %1, %2, 0 offen lds")
    assert not _SCC_WRITERS.search("s_waitcnt lgkmcnt(0)\\n\\ts_barrier")
