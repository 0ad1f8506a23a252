"""Source checks of the HIP kernels (no GPU, no build).

Inline asm: a block of several instructions whose output operand is not
early-clobber ("=&") lets the compiler give that output the register of an
input; the first instruction then overwrites an input the later ones still
read. A popcount of a 64-bit wave mask written as two v_bcnt_u32_b32 in one
block with "=v" is that case: the compiler puts the output in the register
that holds the high half, and the result becomes
popcount(lo) + popcount(popcount(lo)). Every multi-instruction block here must
either have no outputs or mark them early-clobber.
"""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "top_routing_grouped_gemm_amd", "csrc")


def asm_blocks(text):
    """(template, outputs) of every asm statement; outputs is the text between the first and second ':'."""
    out = []
    for m in re.finditer(r"\basm\s+(?:volatile\s*)?\(", text):
        depth, i = 1, m.end()
        while depth and i < len(text):
            depth += {"(": 1, ")": -1}.get(text[i], 0)
            i += 1
        body = text[m.end():i - 1]
        parts = body.split(":")
        template = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', parts[0]))
        outputs = parts[1] if len(parts) > 1 else ""
        out.append((template, outputs))
    return out


def instructions(template):
    return [s for s in re.split(r"\\n|;", template) if s.strip() and not s.strip().startswith("//")]


def test_parser_sees_the_hazard():
    bad = 'asm volatile("v_bcnt_u32_b32 %0, %1, 0\\n\\tv_bcnt_u32_b32 %0, %2, %0" : "=v"(c) : "v"(lo), "v"(hi));'
    ok = 'asm volatile("v_bcnt_u32_b32 %0, %1, 0\\n\\tv_bcnt_u32_b32 %0, %2, %0" : "=&v"(c) : "v"(lo), "v"(hi));'
    (tb, ob), = asm_blocks(bad)
    (tk, okk), = asm_blocks(ok)
    assert len(instructions(tb)) == 2 and re.search(r'"=[^&]', ob)
    assert not re.search(r'"=[^&]', okk)


def test_multi_instruction_asm_outputs_are_early_clobber():
    files = glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
    assert files
    seen = 0
    for f in files:
        for template, outputs in asm_blocks(open(f).read()):
            if len(instructions(template)) < 2:
                continue
            seen += 1
            bad = re.findall(r'"=[^&"]*"', outputs)
            assert not bad, f"{os.path.basename(f)}: multi-instruction asm with non-early-clobber output {bad}"
    assert seen >= 1  # the direct-to-LDS loads (s_mov m0 + load) are such blocks
