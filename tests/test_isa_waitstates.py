"""Compiled-code check (CPU only): every LDS-direct buffer load in the gfx950 kernels has at least
5 wait states after the last VALU instruction that wrote a scalar register the load reads.

The copies into LDS are written as inline assembly (tiles.hpp, copy16_to_lds), which the compiler
does not inspect for hazards; their scalar offset comes from v_readfirstlane, a VALU write of an
SGPR, and the gfx9 family (gfx950 included) requires 5 wait states between such a write and a
vector-memory instruction that reads the SGPR.  The kernels are compiled to assembly here (device
code only) and every `buffer_load ... lds` is walked backwards: s_nop N counts N + 1 wait states,
any other instruction 1.
"""
import concurrent.futures
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_gqa_flashattention_ne_amd", "csrc")
SOURCES = ["fwd_bf16.hip", "bwd_bf16.hip", "decode.hip", "proj.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def sgprs(text):
    out = set()
    for m in re.finditer(r"\bs\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bs(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def short_waits(asm_lines, need=5):
    """(line, load, writer, wait states) for every LDS-direct load that reads an SGPR written by a
    VALU instruction fewer than `need` wait states before it."""
    found = []
    for i, line in enumerate(asm_lines):
        if not (line.startswith("buffer_load") and re.search(r"\blds\b", line)):
            continue
        operands = line.split(None, 1)[1]
        used = sgprs(operands.split(",", 1)[1])           # everything after the vector destination
        ws, j = 0, i - 1
        while j >= 0 and ws < need:
            x = asm_lines[j]
            j -= 1
            if not x or x.startswith((";", ".", "//")) or x.endswith(":"):
                continue
            m = re.match(r"s_nop\s+(\d+)", x)
            if m:
                ws += int(m.group(1)) + 1
                continue
            if x.startswith("v_") and " " in x:
                dst = sgprs(x.split(None, 1)[1].split(",")[0])
                if dst & used:
                    found.append((i + 1, line, x, ws))
                    break
            ws += 1
    return found


def compile_asm(src, outdir):
    out = os.path.join(outdir, src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "--offload-device-only",
           "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return [l.strip() for l in f]


def test_checker_flags_a_short_wait():
    asm = ["v_readfirstlane_b32 s46, v66", "s_mov_b32 m0, s45", "s_nop 0",
           "buffer_load_dwordx4 v171, s[60:63], s46 offen lds"]
    assert len(short_waits(asm)) == 1
    asm[2] = "s_nop 4"
    assert short_waits(asm) == []


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_lds_direct_loads_have_five_wait_states():
    with tempfile.TemporaryDirectory() as d:
        with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
            listings = dict(zip(SOURCES, ex.map(lambda s: compile_asm(s, d), SOURCES)))
    total = 0
    bad = []
    for src, lines in listings.items():
        total += sum(1 for l in lines if l.startswith("buffer_load") and re.search(r"\blds\b", l))
        bad += [(src,) + f for f in short_waits(lines)]
    assert total > 0
    assert not bad, "LDS-direct loads with fewer than 5 wait states: %s" % bad[:5]
