"""Source rules of the HIP kernels (CPU only).

Inline asm that holds instructions is invisible to the compiler's hazard
pass: a matrix-core instruction reading a register that an asm block wrote
one instruction earlier got no wait states and read a stale operand under
some schedules.  The kernels keep only empty asm templates (compiler memory
barriers and register pass-throughs) and a wait for outstanding vector
memory operations (s_waitcnt vmcnt(0)), which writes no register."""
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "quantized_kv_cache_token_amd",
                    "csrc")


def _asm_templates(text):
    # asm ( ... ) or asm volatile ( ... ): the first string literal is the template
    for m in re.finditer(r"\basm\s*(?:volatile\s*)?\(\s*((?:\"(?:[^\"\\]|\\.)*\"\s*)+)", text):
        yield "".join(re.findall(r"\"((?:[^\"\\]|\\.)*)\"", m.group(1)))


WAITS = {"s_waitcnt vmcnt(0)"}


def test_kernel_sources_hold_no_asm_instructions():
    found = []
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".h", ".cpp")):
            continue
        text = open(os.path.join(CSRC, name)).read()
        text = re.sub(r"//[^\n]*", "", text)  # comments may mention asm
        for tpl in _asm_templates(text):
            if tpl.strip() and tpl.strip() not in WAITS:
                found.append((name, tpl))
    assert not found, f"inline asm with instructions: {found}"


def test_the_rule_sees_an_instruction_template():
    text = 'x = 1; asm volatile("" ::: "memory"); asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(y) : "v"(a));'
    assert [t for t in _asm_templates(text) if t.strip()] == ["v_and_or_b32 %0, %1, %2, %3"]


def test_the_rule_allows_only_the_memory_wait():
    text = 'asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); asm volatile("s_waitcnt lgkmcnt(0)");'
    assert [t for t in _asm_templates(text) if t.strip() and t.strip() not in WAITS] == ["s_waitcnt lgkmcnt(0)"]
