"""The compiler-hazard rules the MFMA kernels depend on, checked in the sources,
the build flags and the compiled gfx950 assembly (CPU only).

1. Inline assembly that issues instructions stays in the solver's helpers
   (the DPP pivots and the cross-row swaps), and the solver issues no MFMA:
   the compiler's hazard tracking does not see inside inline assembly, so an
   instruction there must not run in a wave with matrix products in flight.
2. The bf16 pairs (-1, 0) and (0, -1) of the remainder dot products come from
   scalar registers (sgpr_pair), never from literals the compiler could
   encode as the inline constant -1.0 (whose bit pattern is the pair swapped).
3. A 16x16x16 product never accumulates onto the result of a just-issued
   16x16x32 product (a stale read was observed for that pattern).
4. The build keeps matrix results in ordinary VGPRs and packed fp32 off.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "linear_attention_recurrence_10_amd", "csrc")


def source(name):
    with open(os.path.join(CSRC, name)) as f:
        return f.read()


def function_body(text, name):
    """The brace-balanced body of the first definition of `name(`."""
    m = re.search(r"\b%s\s*\([^;{]*\)\s*\{" % re.escape(name), text)
    assert m, name
    i, depth = m.end(), 1
    while depth:
        depth += {"{": 1, "}": -1}.get(text[i], 0)
        i += 1
    return text[m.end():i - 1]


def asm_statements(text):
    """(position, instruction text) of every asm statement with a non-empty template."""
    out = []
    for m in re.finditer(r"\basm\s*(?:volatile\s*)?\(\s*\"((?:[^\"\\]|\\.)*)\"", text):
        if m.group(1).strip():
            out.append((m.start(), m.group(1)))
    return out


def _blank_comments(text):
    """`text` with comments and string literals replaced by spaces (offsets kept)."""
    def blank(m):
        return re.sub(r"[^\n]", " ", m.group(0))
    return re.sub(r'//[^\n]*|/\*.*?\*/|"(?:[^"\\\n]|\\.)*"', blank, text, flags=re.S)


def top_level_functions(text):
    """(name, body start, body end) of every function defined at namespace scope."""
    code, out, stack, start = _blank_comments(text), [], [], None
    for i, ch in enumerate(code):
        if ch == "{":
            before = code[max(0, i - 2000):i]
            if re.search(r"\bnamespace\s*\w*\s*$", before):
                stack.append("ns")
                continue
            if "fn" not in stack:
                head = re.search(r"(\w+)\s*\((?:[^()]|\([^()]*\))*\)[^;{}()]*$", before)
                start = (head.group(1) if head else None, i)
            stack.append("fn")
        elif ch == "}":
            kind = stack.pop()
            if kind == "fn" and "fn" not in stack and start:
                out.append((start[0], start[1], i))
    return out


def enclosing_function(text, pos):
    """Name of the namespace-scope function whose body contains `pos`."""
    for name, a, b in top_level_functions(text):
        if a < pos < b:
            return name
    return None


def test_instruction_asm_only_in_solver_helpers():
    text = source("kda_prefill_mfma.h")
    stmts = asm_statements(text)
    assert stmts, "expected the pivot and swap helpers"
    allowed = {"tri_pivots": ("v_fmac_f32_dpp",), "row_group_sum": ("v_permlane16_swap_b32", "v_permlane32_swap_b32")}
    for pos, body in stmts:
        fn = enclosing_function(text, pos)
        assert fn in allowed, (fn, body)
        assert any(op in body for op in allowed[fn]), (fn, body)
        assert body.lstrip().startswith("s_nop"), "each carries the wait states its operands need: " + body
    # the helpers are used by the solver only, and the solver issues no matrix product
    for helper in allowed:
        sites = [enclosing_function(text, m.start())
                 for m in re.finditer(r"\b%s\s*[<(]" % helper, _blank_comments(text))]
        assert sites.count(None) == 1, (helper, sites)  # the definition itself
        callers = set(sites) - {None, helper}             # the template recursion calls itself
        assert callers == {"solve"}, (helper, callers)
    body = function_body(text, "solve")
    assert not re.search(r"\b(mfma16|mfma32|mm16|mm32|__builtin_amdgcn_mfma\w*)\s*\(", body)
    # the other kernels issue no instruction from inline assembly
    for name in ("kda_bwd.hip", "kda_f32mfma.h", "kda_prefill_f32.hip", "kda_decode.hip", "kda_kcp.hip",
                 "kda_prefill_valu.hip"):
        assert not asm_statements(source(name)), name


def test_bf16_pair_constants_come_from_scalar_registers():
    text = source("kda_prefill_mfma.h")
    calls = re.findall(r"__builtin_amdgcn_fdot2_f32_bf16\(([^;]*?)\)\s*;", text)
    assert calls
    for args in calls:
        second = [a.strip() for a in args.split(",")][1]
        assert second in ("m0", "m1") or second.startswith("sgpr_pair("), args
    for m in re.finditer(r"const bf16x2 (m0|m1) = ([^;]*);", text):
        assert m.group(2).strip().startswith("sgpr_pair("), m.group(0)
    assert 'asm("" : "+s"(bits))' in function_body(text, "sgpr_pair")


def test_build_keeps_vgpr_mfma_form_and_no_packed_fp32():
    from linear_attention_recurrence_10_amd import build

    flags = " ".join(build.HIPCC_FLAGS)
    assert "-amdgpu-mfma-vgpr-form=1" in flags
    assert "-target-feature -Xclang -packed-fp32-ops" in flags


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc",):
        if os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


_REG = r"v\[(\d+):(\d+)\]"
_WINDOW = 16  # instructions: far more than the two seen between the pair that read a stale value


def fresh_k32_reads(listing):
    """Count the 16x16x16 products with a register accumulator in `listing`
    (gfx950 assembly), and list those whose accumulator is the result of a
    16x16x32 product issued fewer than _WINDOW instructions earlier."""
    recent, n16, bad, idx = [], 0, [], 0
    for line in listing.splitlines():
        l = line.strip()
        if not l or l.startswith((";", ".", "//")) or l.endswith(":"):
            continue
        idx += 1
        if l.startswith("s_endpgm") or l.startswith("s_setpc"):
            recent = []
        elif l.startswith("v_mfma_f32_16x16x32_bf16"):
            recent.append((idx, int(re.findall(_REG, l)[0][0])))
        elif l.startswith("v_mfma_f32_16x16x16_bf16"):
            regs = re.findall(_REG, l)
            if len(regs) == 4:
                n16 += 1
                if any(idx - j < _WINDOW and r == int(regs[3][0]) for j, r in recent):
                    bad.append(l)
        recent = [(j, r) for j, r in recent if idx - j < _WINDOW]
    return n16, bad


def test_fresh_k32_reads_finds_the_pattern():
    ok = "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n" + "v_add_f32 v20, v21, v22\n" * 16 + \
         "v_mfma_f32_16x16x16_bf16 v[0:3], v[4:5], v[8:9], v[0:3]\n"
    bad = "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n  v_add_f32 v20, v21, v22\n" \
          "  v_mfma_f32_16x16x16_bf16 v[12:15], v[4:5], v[8:9], v[0:3]\n"
    assert fresh_k32_reads(ok) == (1, [])
    n, found = fresh_k32_reads(bad)
    assert n == 1 and len(found) == 1


@pytest.mark.parametrize("unit", ["kda_prefill_mfma.hip", "kda_prefill_mfma_gate.hip"])
def test_no_k16_product_accumulates_onto_a_fresh_k32_result(unit, tmp_path):
    from linear_attention_recurrence_10_amd import build

    out = tmp_path / "kernel.s"
    cmd = [_hipcc()] + build.HIPCC_FLAGS + build.SOURCE_FLAGS.get(unit, []) + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "--cuda-device-only", "-S",
        os.path.join(CSRC, unit), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    n16, bad = fresh_k32_reads(out.read_text())
    assert n16 > 100
    assert not bad, bad[:4]
