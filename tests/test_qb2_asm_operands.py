"""Host checks of the generated tile loop of the 64-rows-per-wave kernel.

The loop is one inline-asm statement that uses v0..v212 and s88..s97 as fixed
scratch registers (declared clobbered) and takes its per-lane and per-wave
scalars as compiler-placed operands. If the compiler ever placed one of those
operands inside the fixed scratch ranges, the loop would overwrite its own
addresses and fault. These tests compile the kernel file to gfx950 assembly,
line the emitted loop up against the generator's template and check every
substituted operand register; they also check that the committed include is
what the generator emits.
"""
from __future__ import annotations

import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_scaled_dot_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _gen():
    spec = importlib.util.spec_from_file_location("gen_qb2_tile", os.path.join(CSRC, "gen_qb2_tile.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_include_matches_generator():
    g = _gen()
    with open(os.path.join(CSRC, "attn_qb2_tile.inc"), encoding="utf-8") as f:
        assert f.read() == g.render(), "attn_qb2_tile.inc is stale: rerun gen_qb2_tile.py"


def _template_regex(line):
    names = []

    def sub(m):
        names.append(m.group(1))
        return r"([vsa](?:\d+|\[\d+:\d+\]))"

    parts = re.split(r"(%\[\w+\]|%=)", line)
    out = []
    for p in parts:
        if p == "%=":
            out.append(r"\d+")
        elif p.startswith("%["):
            out.append(sub(re.match(r"%\[(\w+)\]", p)))
        else:
            out.append(re.escape(p))
    return re.compile("^" + "".join(out) + "$"), names


def _first_index(reg):
    m = re.match(r"([vsa])(?:(\d+)|\[(\d+):(\d+)\])$", reg)
    assert m, reg
    kind = m.group(1)
    lo = int(m.group(2) or m.group(3))
    hi = int(m.group(2) or m.group(4))
    return kind, lo, hi


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = str(tmp_path_factory.mktemp("asm") / "attn_fwd_bf16.s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", "-I", CSRC, os.path.join(CSRC, "attn_fwd_bf16.hip"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out, encoding="utf-8") as f:
        return f.read()


def test_loop_operands_outside_fixed_registers(device_asm):
    g = _gen()
    tmpl = [ln for ln in g.loop_body()]
    pats = [_template_regex(ln) for ln in tmpl]
    fixed_v = set(g.LOOP_CLOB_V)
    fixed_s = set(range(g.SREG, g.SREG + 10))
    blocks = re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", device_asm, flags=re.S)
    loops = []
    for b in blocks:
        lines = [ln.strip() for ln in b.strip("\n").split("\n") if ln.strip()]
        if lines and pats[0][0].match(lines[0]) and len(lines) == len(tmpl):
            loops.append(lines)
    # one loop per instantiation of the kernel (three masks x two output types x two layouts at most)
    assert loops, "no instance of the tile loop found in the device assembly"
    checked = 0
    for lines in loops:
        seen = {}
        for ln, (rx, names) in zip(lines, pats):
            m = rx.match(ln)
            assert m, "emitted line does not follow the template: %r" % ln
            for name, reg in zip(names, m.groups()):
                kind, lo, hi = _first_index(reg)
                assert seen.setdefault(name, reg) == reg, "operand %s placed in two registers" % name
                if name.startswith(("o", "q")) and kind == "a":
                    continue  # accumulators bound to fixed AGPRs by the constraints themselves
                regs = set(range(lo, hi + 1))
                if kind == "v":
                    assert not regs & fixed_v, "operand %s in fixed VGPR range: %s" % (name, ln)
                elif kind == "s":
                    assert not regs & fixed_s, "operand %s in fixed SGPR range: %s" % (name, ln)
                else:
                    pytest.fail("operand %s in unexpected register %s" % (name, reg))
                checked += 1
    assert checked > 1000
