"""Every DPP read in the gfx950 build follows the last VALU write of its source register by
at least two wait states.

The kernels read DPP operands inside inline-asm blocks (row broadcasts of table
coefficients, wave maxima), where the compiler's hazard recognizer cannot see them, so
the required wait states are written by hand (s_nop).  This test compiles every kernel
source to assembly (no GPU needed) and scans each DPP instruction backwards: a VALU
instruction writing its first source operand (the one DPP swizzles) must be at least two
wait states earlier (s_nop N counts N + 1, any other instruction one).

A second check covers the other way an inline-asm instruction escapes the compiler's
hazard model: an instruction whose result a following VALU instruction must not read too
soon (measured on gfx950: a VALU copy of a v_dot2c_f32_f16 result read within two wait
states gets the old value, at four the new one).  The compiler spaces such reads after the
dot, matrix and transcendental instructions it emits itself, but not after ones written
inside an asm statement, so none of those may appear in inline asm."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_decode_kvq_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _vregs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def dpp_hazards(asm_lines):
    """(number of DPP instructions, list of (writer, reader, wait states)) of a listing."""
    ins = [l.split(";")[0].strip() for l in asm_lines]
    ins = [l for l in ins if l and not l.startswith((".", "//")) and not l.endswith(":")]
    found, total = [], 0
    for k, line in enumerate(ins):
        if "_dpp" not in line.split()[0]:
            continue
        total += 1
        src0 = _vregs(line.split(None, 1)[1].split(",")[1])
        ws, j = 0, k - 1
        while j >= 0 and ws < 2:
            op = ins[j].split()[0]
            if op == "s_nop":
                ws += int(ins[j].split()[1], 0) + 1
            elif op.startswith("v_"):
                if _vregs(ins[j].split(None, 1)[1].split(",")[0]) & src0:
                    found.append((ins[j], line, ws))
                    break
                ws += 1
            else:
                ws += 1
            j -= 1
    return total, found


def test_scanner_flags_planted_hazards():
    planted = ["v_mov_b32_e32 v1, v2", "v_add_f32_dpp v3, v1, v4 row_newbcast:1 row_mask:0xf bank_mask:0xf",
               "v_mov_b32_e32 v5, v2", "s_nop 1", "v_add_f32_dpp v3, v5, v4 row_newbcast:1 row_mask:0xf bank_mask:0xf",
               "v_mov_b32_e32 v[6:7], v[2:3]", "s_nop 0",
               "v_add_f32_dpp v3, v7, v4 row_newbcast:1 row_mask:0xf bank_mask:0xf"]
    total, found = dpp_hazards(planted)
    assert total == 3 and [w for _, _, w in found] == [0, 1]


@pytest.mark.parametrize("src", SOURCES)
def test_dpp_reads_wait_two_states(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
           "--offload-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    total, found = dpp_hazards(open(out).read().splitlines())
    assert not found, f"{src}: {len(found)} DPP reads too soon after a VALU write of their source: {found[:3]}"


# instruction families whose results need wait states before a VALU read, handled by the
# compiler for its own instructions only
_SLOW_RESULT = re.compile(r"\bv_(dot\d|mfma|smfmac|exp|log|rcp|rsq|sqrt|sin|cos)\w*")
_ASM_STRING = re.compile(r"\basm\s*(?:volatile\s*)?\(((?:\s*\"(?:[^\"\\]|\\.)*\")+)")


def slow_result_asm(text):
    """Mnemonics of dot, matrix or transcendental instructions written in inline asm."""
    found = []
    for m in _ASM_STRING.finditer(text):
        found += _SLOW_RESULT.findall(m.group(1))
    return found


def test_slow_result_scanner_flags_planted_asm():
    planted = 'asm("v_dot2c_f32_f16_dpp %0, %1, %2 row_newbcast:3" : "+v"(a) : "v"(w), "v"(e));\n' \
              'asm volatile("s_nop 4\\n\\t"\n "v_exp_f32 %0, %1" : "=v"(x) : "v"(y));\n' \
              'asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:1" : "=v"(p) : "v"(a), "v"(b));\n' \
              'x = __builtin_amdgcn_fdot2(a, b, c, false);'
    assert slow_result_asm(planted) == ["dot2", "exp"]


@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp"))))
def test_no_slow_result_instruction_in_inline_asm(src):
    found = slow_result_asm(open(os.path.join(CSRC, src)).read())
    assert not found, f"{src}: dot/matrix/transcendental instructions in inline asm: {found}"
