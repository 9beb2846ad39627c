"""Static checks on the gfx950 assembly of the library's own kernels (CPU).

* Every DPP instruction reads its first source from another lane; the
  hardware needs two wait states after a VALU write of that register.  The
  kernels pass only LDS-loaded registers as DPP sources; this test checks the
  compiled code: no VALU instruction writes the DPP source register within the
  two preceding instructions.
* No packed fp32 VALU instructions (v_pk_add/mul/fma_f32) are emitted.
* No kernel uses scratch memory (register spills or stack arrays).
"""
import os
import re
import subprocess

import pytest

from selective_state_space_55_amd import build as hipbuild

ASM_SRCS = ["scan_fwd.hip", "scan_fwd_varlen.hip", "scan_step.hip", "scan_bwd.hip", "conv1d.hip", "ssd_fwd.hip"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in ASM_SRCS:
        path = str(d / (src + ".s"))
        flags = [f for f in hipbuild.flags() if f not in ("-shared", "-fPIC")]
        subprocess.run([hipbuild.hipcc()] + flags + ["--cuda-device-only", "-S", "-o", path,
                                                     os.path.join(hipbuild.CSRC, src)],
                       check=True, capture_output=True)
        out[src] = open(path).read()
    return out


def _regs(tok):
    """Register numbers named by an operand like v7 or v[4:7]."""
    m = re.fullmatch(r"-?\|?v(\d+)\|?", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _instructions(text):
    """(mnemonic, operand list) per instruction, in program order, per function."""
    funcs, cur = [], None
    for line in text.splitlines():
        if re.match(r"^[A-Za-z_.$][\w.$]*:", line) and not line.startswith(".L"):
            cur = []
            funcs.append(cur)
            continue
        s = line.strip()
        if cur is None or not s or s.startswith((";", ".", "//")) or s.endswith(":"):
            continue
        parts = s.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        cur.append((parts[0], ops))
    return funcs


def test_dpp_sources_not_recently_written_by_valu(asm):
    checked = 0
    for src, text in asm.items():
        for insts in _instructions(text):
            for i, (mn, ops) in enumerate(insts):
                if "_dpp" not in mn or len(ops) < 2:
                    continue
                srcregs = _regs(ops[1].split()[0])
                assert srcregs, (mn, ops)
                checked += 1
                waits = 0
                j = i - 1
                while j >= 0 and waits < 2:
                    pmn, pops = insts[j]
                    if pmn == "s_nop":
                        waits += int(pops[0], 0) + 1
                    else:
                        if pmn.startswith("v_") and pops and (_regs(pops[0].split()[0]) & srcregs):
                            raise AssertionError(f"{src}: {pmn} {pops} writes the DPP source of {mn} {ops} "
                                                 f"within {waits} wait states")
                        waits += 1
                    j -= 1
    assert checked > 0


def test_no_packed_fp32_valu(asm):
    for src, text in asm.items():
        bad = re.findall(r"\bv_pk_(add|mul|fma)_f32\b", text)
        assert not bad, (src, bad[:5])


def test_no_scratch(asm):
    for src, text in asm.items():
        sizes = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)]
        assert sizes and max(sizes) == 0, (src, sizes)
