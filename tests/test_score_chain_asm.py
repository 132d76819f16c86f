"""CPU check of the attention kernel's generated gfx950 assembly: the score chain's
accumulator is touched by nothing but the chain's own MFMAs until the wait states that
follow its last MFMA.

The chain (bf16: 32x32x16; E4M3: scaled 32x32x64) is written in inline assembly (its
accumulator lives in VGPRs), so the
compiler does not know when an MFMA's result is written and inserts no wait for it.  A
register copy that the compiler places between two chain MFMAs, or right after the last
one, would read a result that is still being computed, and the output would depend on
timing.  The sources keep the accumulator in place; this test checks that the compiler's
register allocation did so too.
"""
import os
import re
import subprocess
import tempfile

import pytest

from mla_latent_kv_03_amd import build

SRC = os.path.join(build.CSRC, "mla_attn_h128.hip")


def _regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def chain_violations(asm_lines):
    """(chains, violations): chains opened, and instructions that touch an open chain's
    accumulator.  A chain opens at an MFMA with a VGPR accumulator that starts from 0 (or,
    in a loop laid out with its head inside the chain, at the first in-place one), stays
    open through in-place MFMAs on the same registers, and closes after three
    `s_nop 7` (the wait before the result is read) or at an unconditional branch."""
    mfma = re.compile(r"v_mfma_(?:f32_32x32x16_bf16|scale_f32_32x32x64_f8f6f4) v\[(\d+):(\d+)\], \S+, \S+, ([^,\s]+)")
    chains, bad, acc, nops = 0, [], None, 0
    for ln, line in enumerate(asm_lines, 1):
        t = line.split(";")[0].strip()
        if not t:
            continue
        m = mfma.match(t)
        if m:
            regs = set(range(int(m.group(1)), int(m.group(2)) + 1))
            dst = f"v[{m.group(1)}:{m.group(2)}]"
            if m.group(3) == "0":
                acc, chains = regs, chains + 1
            elif m.group(3) == dst:
                if acc is None:
                    acc = regs
                elif acc != regs:
                    bad.append((ln, t))
            elif acc is not None and _regs(m.group(3)) & acc:
                bad.append((ln, t))
            nops = 0
            continue
        if t == "s_nop 7":
            nops += 1
            if nops == 3:
                acc = None
            continue
        if t.startswith(("s_branch", "s_setpc", "s_endpgm")):
            acc = None
            continue
        if acc is not None and _regs(t) & acc:
            bad.append((ln, t))
    return chains, bad


@pytest.fixture(scope="module")
def asm():
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("no ROCm toolchain (hipcc) to compile the kernel")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "h128.s")
        cmd = [build.hipcc(), *build.compile_flags(), "-x", "hip", "-c", SRC, "--cuda-device-only", "-S", "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return open(out).read().split("\n")


def test_score_chain_accumulator_untouched_until_its_wait(asm):
    chains, bad = chain_violations(asm)
    # two kernels (bf16 32x32x16, E4M3 scaled 32x32x64), each with the first pass and the
    # exact re-run
    assert chains >= 4, f"expected the score chains of both kernels, found {chains}"
    assert not bad, "instructions touch an open score chain's accumulator:\n" + "\n".join(f"{ln}: {t}" for ln, t in bad[:10])


def test_checker_catches_an_early_copy():
    """The check itself: a copy of the accumulator between two chain MFMAs is reported."""
    good = ["v_mfma_f32_32x32x16_bf16 v[18:33], v[2:5], v[40:43], 0",
            "ds_read_b128 v[2:5], v100",
            "v_mfma_f32_32x32x16_bf16 v[18:33], v[6:9], v[44:47], v[18:33]",
            "s_nop 7", "s_nop 7", "s_nop 7",
            "v_mov_b32_e32 v50, v18"]
    assert chain_violations(good) == (1, [])
    early = good[:3] + ["v_mov_b64_e32 v[2:3], v[18:19]"] + good[3:]
    chains, bad = chain_violations(early)
    assert chains == 1 and len(bad) == 1 and "v_mov_b64" in bad[0][1]
