"""Wait states of the hand-written MFMA statements, checked on the compiled gfx950 code.

The matrix-core kernels issue their MFMAs through inline asm, which the compiler's hazard
pass does not look into.  A VALU instruction that writes an MFMA's A or B operand needs
independent instructions (wait states) before the MFMA reads it -- two on gfx950, as many
as the compiler's own hazard pass places before its MFMAs; the same holds for a write of
the accumulator registers (`v_accvgpr_write`).  The asm statements carry three where a
weight operand has just been formed (the first output MFMA of each k-step) and none
elsewhere in the latent kernel's tile loop, whose other operands are LDS reads, query
registers loaded before the loop and weights formed at least one output MFMA earlier.
This test compiles the kernels to assembly (device code only, on the CPU) and checks that
no MFMA has a VALU write of its A, B or AGPR accumulator registers within the two
instructions before it, counting `s_nop N` as N + 1.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                "decode_attention_paged_kv_amd"))
import build as B  # noqa: E402

NEEDED = 2


def _regs(tok: str, file: str = "v") -> set:
    m = re.match(file + r"\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(file + r"(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _vregs(tok: str) -> set:
    return _regs(tok, "v")


def hazards(asm: str, needed: int = NEEDED):
    """(VALU instruction, MFMA, wait states between) for every too-close operand write."""
    ins = [l.strip() for l in asm.split("\n") if re.match(r"^\t[a-z]", l)]
    found = []
    for i, text in enumerate(ins):
        if not text.startswith("v_mfma"):
            continue
        ops = [t.strip() for t in text.split(None, 1)[1].split(",")]
        src = _vregs(ops[1]) | _vregs(ops[2])
        src_c = _regs(ops[3], "a") if len(ops) > 3 else set()   # accumulator in AGPRs
        ws, j = 0, i - 1
        while j >= 0 and ws < needed:
            prev = ins[j]
            op = prev.split()[0]
            if op == "s_nop":
                ws += int(prev.split()[1], 0) + 1
            else:
                if op.startswith("v_") and not op.startswith("v_mfma"):
                    dst = prev.split(None, 1)[1].split(",")[0].strip()
                    if _vregs(dst) & src or _regs(dst, "a") & src_c:
                        found.append((prev, text, ws))
                ws += 1
            j -= 1
    return found


def test_checker_catches_a_close_write():
    asm = "\tv_cvt_pk_bf16_f32 v161, v0, v1\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[158:161], a[0:15]\n"
    assert len(hazards(asm)) == 1
    asm_ok = "\tv_cvt_pk_bf16_f32 v161, v0, v1\n\ts_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[158:161], a[0:15]\n"
    assert hazards(asm_ok) == []
    acc = "\tv_accvgpr_write_b32 a7, v0\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[158:161], a[0:15]\n"
    assert len(hazards(acc)) == 1


@pytest.mark.parametrize("src", ["decode_mla.hip", "decode_gqa.hip"])
def test_no_valu_write_close_before_an_mfma(src):
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    flags = [f for f in B.HIPFLAGS if f != "-fPIC"]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        p = subprocess.run([hipcc, "-x", "hip", "-S", "--cuda-device-only", os.path.join(B.CSRC, src),
                            "-o", out, *flags], capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-2000:]
        asm = open(out).read()
    n_mfma = len(re.findall(r"^\tv_mfma", asm, flags=re.M))
    assert n_mfma > 0
    bad = hazards(asm)
    assert not bad, "\n".join(f"{w} wait states: {a}  ->  {m}" for a, m, w in bad[:10])
