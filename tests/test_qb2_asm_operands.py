"""Host checks of the generated tile loop of the 64-rows-per-wave kernel.

The loop is one inline-asm statement that uses v0..v212 and s88..s97 as fixed
scratch registers (declared clobbered) and takes its per-lane and per-wave
scalars as compiler-placed operands. If the compiler ever placed one of those
operands inside the fixed scratch ranges, the loop would overwrite its own
addresses and fault. These tests compile the kernel file to gfx950 assembly,
line the emitted loop up against the generator's template and check every
substituted operand register; they also check that the committed include is
what the generator emits, the LDS slots each step reads and fetches into, and
(on a model of the slots) that every read finds the tile it expects across
the items a workgroup runs back to back.
"""
from __future__ import annotations

import importlib.util
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_scaled_dot_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _gen(d=128):
    spec = importlib.util.spec_from_file_location("gen_qb2_tile", os.path.join(CSRC, "gen_qb2_tile.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.configure(d)
    return mod


HEAD_DIMS = (128, 64)


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_include_matches_generator(d):
    g = _gen(d)
    name = g.OUTPUTS[d]
    with open(os.path.join(CSRC, name), encoding="utf-8") as f:
        assert f.read() == g.render(), "%s is stale: rerun gen_qb2_tile.py" % name


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


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_loop_operands_outside_fixed_registers(device_asm, d):
    g = _gen(d)
    tmpl = [ln for ln in g.loop_body()]
    pats = [_template_regex(ln) for ln in tmpl]
    fixed_v = set(g.LOOP_CLOB_V)
    fixed_s = set(g.LOOP_CLOB_S)
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


# --------------------------------------------------------------------------------------------------
# LDS slot protocol of the generated loop: which slot each step reads and which one its fetches write,
# and (as a model) which tile sits in each slot when it is read, across the items a workgroup runs.

def _slots(ins, TB=64 * 128 * 2):
    kr, vr, kw, vw = set(), set(), set(), set()
    for t in ins:
        m = re.match(r"ds_read_b128 v\[\d+:\d+\], %\[ka\d\] offset:(\d+)", t)
        if m:
            kr.add(int(m.group(1)) // TB)
        m = re.match(r"ds_read_b64_tr_b16 v\[\d+:\d+\], %\[va\d_\d\] offset:(\d+)", t)
        if m:
            vr.add(int(m.group(1)) // TB - 2)
        m = re.match(r"s_add_u32 m0, %\[lbw\], (\d+)", t)
        if m:
            sl = int(m.group(1)) // TB
            (kw if sl < 2 else vw).add(sl % 2)
    return kr, vr, kw, vw


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_step_slots(d):
    g = _gen(d)
    _slots_d = lambda ins: _slots(ins, g.TILE_B)
    for P in (0, 1):
        o, ool = g.iteration(P)
        common = o[o.index("s_cbranch_scc0 L_slow_p%d_%%=" % P):]
        general = ool[ool.index("L_slow_p%d_%%=:" % P):ool.index("L_mask_p%d_%%=:" % P)]
        last = ool[ool.index("L_last_p%d_%%=:" % P):ool.index("L_nocomp_p%d_%%=:" % P)]
        noc = ool[ool.index("L_nocomp_p%d_%%=:" % P):]
        for part in (common, general, last, noc):
            kr, vr, kw, vw = _slots_d(part)
            assert kw == {P} and vw == {1 - P}   # K(t+2) -> K slot P, V(t+1) -> V slot 1-P
            assert not (kr & kw) and not (vr & vw)
        for part in (common, general):
            kr, vr, _, _ = _slots_d(part)
            assert kr == {1 - P} and vr == {P}   # S(t+1) reads K(t+1), P.V reads V(t)
        kr, vr, _, _ = _slots_d(last)
        assert kr == set() and vr == {P}
    for off in (0, 1):
        for turn in (False, True):
            kr, vr, kw, vw = _slots_d(g.first_tile(off, turn))
            assert kr == {off} and not vr and not kw and not vw
    # step 0 fetches K(2) into the slot S(0) reads K(0) from: a barrier must separate them
    body = g.loop_body()
    assert "s_barrier" in body[body.index("L_first_done_%=:"):body.index("L_top_%=:")]
    o, _ = g.iteration(0)
    assert o[-2:] == ["s_waitcnt vmcnt(0)", "s_barrier"] or "s_barrier" in o[-3:]


def _run_items(items):
    """Tiles in the K/V slots as a workgroup runs items with the given tile counts: step t of an item
    fetches tiles t+2 (K) and t+1 (V) of the stream that continues into the next item; items of fewer
    than two tiles leave the next item's first tiles to a separate fetch."""
    K, V = [None, None], [None, None]

    def fetch_first(i, off):
        if items[i] > 0:
            K[off] = (i, 0)
            if items[i] > 1:
                K[1 - off] = (i, 1)
            V[off] = (i, 0)

    off = 0
    fetch_first(0, off)
    for i, nt in enumerate(items):
        nxt = i + 1 if i + 1 < len(items) else None

        def stream(x):
            if x < nt:
                return (i, x)
            return (nxt, x - nt) if nxt is not None else None

        if nt > 0:
            assert K[off] == (i, 0) and V[off] == (i, 0)
        for t in range(nt):
            P = (t + off) % 2
            if t + 1 < nt:
                assert K[1 - P] == (i, t + 1)
            assert V[P] == (i, t)
            K[P] = stream(t + 2)
            V[1 - P] = stream(t + 1)
        off_next = (off + nt) % 2
        if nxt is not None and nt < 2:
            fetch_first(nxt, off_next)
        off = off_next


def test_item_stream_model():
    rng = np.random.default_rng(7)
    for _ in range(5000):
        _run_items([int(x) for x in rng.choice([0, 1, 2, 3, 4, 5, 8], size=int(rng.integers(1, 7)))])


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_diagonal_step_slots_and_mask(d):
    """The step that masks the wave's causal diagonal tile inside its block uses the same slots as the
    plain step, and its mask hides exactly the keys past each row: with the tile starting at the wave's
    first row, lane (l32, hf) of query block qb holds row qb*32 + l32 and, in score register r of key
    block jb, key jb*32 + (r//4)*8 + hf*4 + r%4."""
    g = _gen(d)
    for P in (0, 1):
        _, ool = g.iteration(P)
        diag = ool[ool.index("L_diag_p%d_%%=:" % P):ool.index("L_last_p%d_%%=:" % P)]
        kr, vr, kw, vw = _slots(diag, g.TILE_B)
        assert kr == {1 - P} and vr == {P} and kw == {P} and vw == {1 - P}
    for buf in (0, 1):
        for qb in range(2):
            ins = g.diag_mask(buf, qb)
            movs = {int(re.match(r"v_mov_b32 v(\d+), v%d" % g.NINF_V, t).group(1)) for t in ins
                    if t.startswith("v_mov_b32")}
            cmps = {}
            for a, b in zip(ins, ins[1:]):
                m = re.match(r"v_cmp_gt_i32_e64 s\[\d+:\d+\], (\d+), v\d+", a)
                if m:
                    cmps[int(re.match(r"v_cndmask_b32_e64 v(\d+),", b).group(1))] = int(m.group(1))
            for jb in range(2):
                for r in range(16):
                    reg = g.s_reg(buf, qb, jb, r)
                    for l32 in range(32):
                        for hf in range(2):
                            key, row = jb * 32 + (r // 4) * 8 + hf * 4 + r % 4, qb * 32 + l32
                            if reg in movs:
                                masked = True
                            elif reg in cmps:
                                masked = cmps[reg] > row - hf * 4   # off > lim - tile start
                            else:
                                masked = False
                            assert masked == (key > row), (buf, qb, jb, r, l32, hf)


# --------------------------------------------------------------------------------------------------
# Scalar control of the generated loop, executed on a model: the scalar instructions run as written
# (vector, LDS and matrix instructions are skipped), each buffer load records the descriptor and LDS
# address it is issued with, and each step records the path it took.

M32 = (1 << 32) - 1


def _s32(x):
    x &= M32
    return x - (1 << 32) if x >> 31 else x


class _ScalarModel:
    def __init__(self, body, ops, rng):
        self.body, self.ops, self.rng = body, dict(ops), rng
        self.labels = {ln[:-1]: i for i, ln in enumerate(body) if ln.endswith(":")}
        self.s, self.scc, self.vcc, self.m0 = {}, None, None, None
        self.steps, self.loads, self.paths = [], [], []

    def val(self, x):
        x = x.strip()
        if x.startswith("%["):
            return self.ops[x[2:-1]] & M32
        if re.fullmatch(r"s\d+", x):
            return self.s[int(x[1:])]
        return int(x, 0) & M32

    def put(self, d, v):
        d = d.strip()
        if d == "m0":
            self.m0 = v & M32
        elif d.startswith("%["):
            self.ops[d[2:-1]] = _s32(v)
        else:
            self.s[int(d[1:])] = v & M32

    def run(self, limit=200000):
        pc, n = 0, 0
        while pc < len(self.body):
            n += 1
            assert n < limit, "loop did not end"
            ln = self.body[pc]
            pc += 1
            if ln.endswith(":"):
                lab = ln[:-1]
                if lab == "L_end_%=":
                    return
                m = re.match(r"L_(slow|mask|move|diag|last|nocomp)_p\d_%=$", lab)
                if m and self.paths:
                    self.paths[-1].add(m.group(1))
                continue
            op, _, args = ln.partition(" ")
            a = [x.strip() for x in args.split(",")] if args else []
            if not op.startswith(("s_", "buffer_load")):
                continue
            if op in ("s_waitcnt", "s_nop"):
                continue
            if op == "s_barrier":
                self.steps.append(self.loads)
                self.loads = []
                self.paths.append(set())
                continue
            if op == "buffer_load_dwordx4":
                r = int(re.match(r"s\[(\d+):\d+\]", a[1]).group(1))
                base = self.s[r] | (self.s[r + 1] << 32)
                self.loads.append((r, base, _s32(self.s[r + 2]), self.s[r + 3], self.m0))
                continue
            if op == "s_mov_b32":
                self.put(a[0], self.val(a[1]))
            elif op == "s_add_u32":
                v = self.val(a[1]) + self.val(a[2])
                self.put(a[0], v)
                self.scc = v >> 32
            elif op == "s_addc_u32":
                assert self.scc is not None, ln
                v = self.val(a[1]) + self.val(a[2]) + self.scc
                self.put(a[0], v)
                self.scc = v >> 32
            elif op in ("s_add_i32", "s_sub_i32", "s_max_i32", "s_min_i32"):
                x, y = _s32(self.val(a[1])), _s32(self.val(a[2]))
                v = {"s_add_i32": x + y, "s_sub_i32": x - y, "s_max_i32": max(x, y), "s_min_i32": min(x, y)}[op]
                assert -(1 << 31) <= v < (1 << 31), "signed overflow: %s" % ln
                self.put(a[0], v)
                self.scc = None
            elif op == "s_mul_i32":
                self.put(a[0], _s32(self.val(a[1])) * _s32(self.val(a[2])))
                self.scc = None
            elif op == "s_lshl_b32":
                self.put(a[0], self.val(a[1]) << self.val(a[2]))
                self.scc = None
            elif op.startswith("s_cmp_"):
                cmp, ty = op[6:8], op[9:]
                x, y = self.val(a[0]), self.val(a[1])
                if ty == "i32":
                    x, y = _s32(x), _s32(y)
                self.scc = int({"eq": x == y, "lg": x != y, "ge": x >= y, "gt": x > y, "lt": x < y,
                                "le": x <= y}[cmp])
            elif op == "s_cselect_b32":
                assert self.scc is not None, ln
                self.put(a[0], self.val(a[1]) if self.scc else self.val(a[2]))
            elif op == "s_or_b64":
                assert a[0] == "vcc"
                self.vcc = int(self.rng.random() < 0.3)   # a row's reference moves
            elif op in ("s_cbranch_scc0", "s_cbranch_scc1"):
                assert self.scc is not None, ln
                if self.scc == int(op[-1]):
                    pc = self.labels[a[0]]
            elif op in ("s_cbranch_vccnz", "s_cbranch_vccz"):
                assert self.vcc is not None, ln
                if bool(self.vcc) == (op == "s_cbranch_vccnz"):
                    pc = self.labels[a[0]]
            elif op == "s_branch":
                pc = self.labels[a[0]]
            else:
                pytest.fail("scalar instruction without a model: %s" % ln)
        pytest.fail("fell off the end of the loop")


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_loop_scalar_control_model(d):
    """For items of every tile count, wave extent, masked tile and diagonal tile, with and without the turn
    from a previous item: step t issues the four loads of K(t+2) into K slot (t+off)%2 and of V(t+1) into
    the other V slot, each with the descriptor of that tile of the stream (this item's tiles, then the next
    item's; its size the bytes below that item's kv_end, never negative), and takes the path its tile calls
    for; the next item's Q rows are fetched into the Q slots, block qw through a descriptor of the rows below
    N_q (min(64, max(0, nqr - 64 qw)) rows; nothing when nqr = 0), right after the barrier behind S(0) in
    items of fewer than five tiles, else at step nt - 5 + qw."""
    g = _gen(d)
    TB, RB, CH = g.TILE_B, g.ROWB, g.CH
    body = g.loop_body()
    rng = np.random.default_rng(11)
    TILE, BIG = TB, 0x7FFFFFFF
    for case in range(3000):
        kve = int(rng.integers(0, 64 * 7))
        nt = (kve + 63) // 64
        ntw = int(rng.integers(0, nt + 1))
        tm = int(rng.choice([BIG, int(rng.integers(0, nt + 2))]))
        dg = int(rng.choice([BIG, int(rng.integers(0, nt + 2))]))
        off = int(rng.integers(0, 2))
        nkve = int(rng.choice([0, int(rng.integers(1, 64 * 5))]))
        # bases with low words near a 4 GiB boundary, so that the carries into the high word happen
        bases = {k: int(rng.integers(1, 1 << 16)) << 32 | (M32 + 1 - TILE * int(rng.integers(1, 6)))
                 for k in ("kh", "vh", "nkh", "nvh")}
        nqr = int(rng.choice([0, int(rng.integers(1, 300))]))
        nq = int(rng.integers(1, 1 << 16)) << 32 | (M32 + 1 - TILE * int(rng.integers(1, 6)))
        tn = int(rng.integers(0, 2))
        ops = {"t": 0, "nt": nt, "ntw": ntw, "tm": tm, "dg": dg, "off": off, "kve": kve, "nkve": nkve, "lbw": 0,
               "tn": tn, "qsb": 4 * TB, "ostr": RB,
               "obl": int(rng.integers(0, M32)), "obh": int(rng.integers(0, 1 << 16)),
               "onb": int(rng.integers(0, 1 << 20)), "nql": nq & M32, "nqh": nq >> 32, "nqr": nqr}
        for k, b in bases.items():
            ops[k + "l"], ops[k + "h"] = b & M32, b >> 32
        m = _ScalarModel(body, ops, rng)
        m.run()
        assert m.ops["t"] == nt
        assert not m.steps[0]                      # the barrier after S(0): nothing fetched before it
        steps, paths = m.steps[1:], m.paths[:-1]
        assert len(steps) == nt, (case, ops)
        # the next item's Q rows into the Q slots: items of fewer than five tiles fetch them right after
        # that barrier (with step 0's loads), longer ones block qw at step nt - 5 + qw
        qload = lambda x: x[4] >= g.QSLOT
        got = [(t, x) for t, st in enumerate(steps) for x in st if qload(x)] + [(nt, x) for x in m.loads if qload(x)]
        want_q = [(0 if nt < 5 else nt - 5 + qw,
                   (g.SREG if nt >= 5 else g.KRES, nq + qw * TB, min(64, max(0, nqr - 64 * qw)) * RB, 0x20000,
                    g.QSLOT + qw * TB + j * 4096)) for qw in range(4) for j in range(CH)] if nqr > 0 else []
        assert got == want_q, (case, ops)
        steps = [[x for x in st if not qload(x)] for st in steps]
        def desc(h, x):
            if x < nt:
                return bases[h] + x * TILE, max(0, kve * RB - x * TILE)
            return bases["n" + h] + (x - nt) * TILE, max(0, nkve * RB - (x - nt) * TILE)

        for t in range(nt):
            P = (t + off) % 2
            want = [(g.KRES,) + desc("kh", t + 2) + (0x20000, P * TB + j * 4096) for j in range(CH)]
            want += [(g.VRES,) + desc("vh", t + 1) + (0x20000, 2 * TB + (1 - P) * TB + j * 4096) for j in range(CH)]
            assert sorted(steps[t]) == sorted(want), (case, ops, t)
            p = paths[t] - {"move"}
            if t >= ntw:
                exp = {"slow", "nocomp"}
            elif t + 1 >= ntw:
                exp = {"slow", "last"}
            elif t + 1 == dg:
                exp = {"slow", "diag"}
            elif t + 1 >= tm:
                exp = {"slow", "mask"}
            elif t + 2 >= nt:
                exp = {"slow"}
            else:
                exp = set() if t + 1 < min(ntw, dg, tm) else {"slow"}
            assert p == exp, (case, ops, t, paths[t])


def _ones_pattern_model(lane):
    """Executes the generated instructions that build the row-sum A operand, for one lane."""
    g = _gen()
    v, vcc = {}, None
    for t in g.ones_pattern():
        op, _, args = t.partition(" ")
        a = [x.strip() for x in args.split(",")]
        val = lambda x: v[int(x[1:])] if x.startswith("v") else int(x, 0) & 0xFFFFFFFF
        if op == "v_mbcnt_lo_u32_b32":
            v[int(a[0][1:])] = min(lane, 32) + val(a[2])
        elif op == "v_mbcnt_hi_u32_b32":
            v[int(a[0][1:])] = max(lane - 32, 0) + val(a[2])
        elif op == "v_lshrrev_b32":
            v[int(a[0][1:])] = val(a[2]) >> val(a[1])
        elif op == "v_xor_b32":
            v[int(a[0][1:])] = val(a[1]) ^ val(a[2])
        elif op == "v_and_b32":
            v[int(a[0][1:])] = val(a[1]) & val(a[2])
        elif op == "v_cmp_eq_u32":
            vcc = val(a[1]) == val(a[2])
        elif op == "v_mov_b32":
            v[int(a[0][1:])] = val(a[1])
        elif op == "v_cndmask_b32":
            v[int(a[0][1:])] = val(a[2]) if vcc else val(a[1])
        else:
            pytest.fail("no model for %s" % t)
    return v[0]


def test_row_sum_product_gives_each_lane_its_query_sum():
    """The row sums come from a 16 x 16 x 32 product whose B operand is the P^T register of the 32 x 32 x 16
    P.V product (lane l: query l % 32, keys 8 (l / 32) .. + 7 of 16) and whose A operand is the generated
    0/1 pattern. With the 16 x 16 layouts (A: lane l gives row l % 16, B: column l % 16, both at k-group
    l / 16; D: lane l holds column l % 16, rows 4 (l / 16) .. + 3), every D value a lane holds must be the
    sum of its own query's 16 weights, whatever order the k-group's eight elements take."""
    rng = np.random.default_rng(3)
    P = rng.random((32, 16))                      # P[query][key]
    Bl = np.array([P[l % 32, 8 * (l // 32):8 * (l // 32) + 8] for l in range(64)])   # lane -> 8 values
    ones = {0x3F803F80: 1.0, 0: 0.0}
    Al = np.array([[ones[_ones_pattern_model(l)]] * 8 for l in range(64)])
    for perm in (np.arange(8), rng.permutation(8)):
        A = np.zeros((16, 32))
        B = np.zeros((32, 16))
        for l in range(64):
            for j in range(8):
                k = 8 * (l // 16) + perm[j]
                A[l % 16, k] = Al[l, j]
                B[k, l % 16] = Bl[l, j]
        Dm = A @ B
        for l in range(64):
            for i in range(4):
                np.testing.assert_allclose(Dm[4 * (l // 16) + i, l % 16], P[l % 32].sum(), rtol=1e-12)


# --------------------------------------------------------------------------------------------------
# The turn between two items, executed per lane on a model: the finished item's O (fp32, in the AGPR
# layout of the 32 x 32 products) must reach global memory as bf16(O / l) at row (wave row), column d,
# through the staging area of the wave and nothing else, for both output layouts and partial row blocks.

def _bf16_bits(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)


def _run_vector(prog, O, inv, ops, lds, out, touched, v, acc, sreg):
    """Executes the vector, LDS and store instructions of a turn program for 64 lanes (scalar
    instructions: the few that compute addresses). O[k][r]: lane values of AGPR O_A + 16 k + r."""
    g = _gen()
    lanes = np.arange(64, dtype=np.int64)
    cleared = set()

    def reg(x):
        x = x.strip()
        if x.startswith("%["):
            val = ops[x[2:-1]]
            return np.broadcast_to(np.asarray(val, dtype=np.int64) & M32, (64,)).copy()
        if re.fullmatch(r"v\d+", x):
            return v[int(x[1:])].copy()
        if re.fullmatch(r"s\d+", x):
            return np.full(64, sreg[int(x[1:])], dtype=np.int64)
        return np.full(64, int(x, 0) & M32, dtype=np.int64)

    def sval(x):
        x = x.strip()
        if x.startswith("%["):
            return ops[x[2:-1]] & M32
        if re.fullmatch(r"s\d+", x):
            return sreg[int(x[1:])]
        return int(x, 0) & M32

    def vrange(x):
        m = re.fullmatch(r"[va]\[(\d+):(\d+)\]", x.strip())
        return range(int(m.group(1)), int(m.group(2)) + 1)

    for t in prog:
        op, _, args = t.partition(" ")
        a = [x.strip() for x in args.split(",")] if args else []
        if op in ("s_waitcnt", "s_nop"):
            continue
        if op.startswith("s_"):
            if a[0] in ("s80", "s81", "s82", "s83", "s88", "s89", "s90", "s91") and op == "s_mov_b32":
                continue                              # buffer descriptors: the model checks offsets against onb
            x = {"s_mov_b32": lambda: sval(a[1]), "s_lshl_b32": lambda: sval(a[1]) << sval(a[2]),
                 "s_add_u32": lambda: sval(a[1]) + sval(a[2]),
                 "s_mul_i32": lambda: sval(a[1]) * sval(a[2])}[op]()
            sreg[int(a[0][1:])] = x & M32
            continue
        if op == "v_mfma_f32_32x32x16_bf16":
            # O cleared by a product of zero operands: only after every read of that block
            m = re.fullmatch(r"a\[(\d+):(\d+)\]", a[0])
            k = (int(m.group(1)) - g.O_A) // 16
            assert a[1] == a[2] == "v[%d:%d]" % (g.TURN_ZERO_V, g.TURN_ZERO_V + 3) and a[3] == "0", t
            assert k not in cleared
            cleared.add(k)
            O[k][:] = np.nan                          # any later read of the block would show in the output
            continue
        d = int(a[0][1:]) if re.fullmatch(r"v\d+", a[0]) else None
        if op == "v_add_u32":
            v[d] = (reg(a[1]) + reg(a[2])) & M32
        elif op == "v_mov_b32":
            v[d] = reg(a[1])
        elif op == "v_mbcnt_lo_u32_b32":
            v[d] = np.minimum(lanes, 32) + reg(a[2])
        elif op == "v_mbcnt_hi_u32_b32":
            v[d] = np.maximum(lanes - 32, 0) + reg(a[2])
        elif op == "v_and_b32":
            v[d] = reg(a[1]) & reg(a[2])
        elif op == "v_xor_b32":
            v[d] = reg(a[1]) ^ reg(a[2])
        elif op == "v_lshrrev_b32":
            v[d] = reg(a[2]) >> reg(a[1])
        elif op == "v_lshlrev_b32":
            v[d] = (reg(a[2]) << reg(a[1])) & M32
        elif op == "v_lshl_add_u32":
            v[d] = ((reg(a[1]) << reg(a[2])) + reg(a[3])) & M32
        elif op == "v_mul_u32_u24":
            v[d] = ((reg(a[1]) & 0xFFFFFF) * (reg(a[2]) & 0xFFFFFF)) & M32
        elif op == "v_mad_u32_u24":
            v[d] = ((reg(a[1]) & 0xFFFFFF) * (reg(a[2]) & 0xFFFFFF) + reg(a[3])) & M32
        elif op == "v_accvgpr_read_b32":
            k, r = divmod(int(a[1][1:]) - g.O_A, 16)
            v[d] = O[k][r].astype(np.float32).view(np.uint32).astype(np.int64)
        elif op == "v_mul_f32":
            qb = int(re.match(r"%\[inv(\d)\]", a[2]).group(1))
            x = reg(a[1]).astype(np.uint32).view(np.float32) * np.float32(inv[qb])
            v[d] = x.astype(np.float32).view(np.uint32).astype(np.int64)
        elif op == "v_cvt_pk_bf16_f32":
            lo = _bf16_bits(reg(a[1]).astype(np.uint32).view(np.float32))
            hi = _bf16_bits(reg(a[2]).astype(np.uint32).view(np.float32))
            v[d] = (lo | (hi << 16)).astype(np.int64)
        elif op == "ds_write_b64":
            m = re.search(r"offset:(\d+)", t)
            addr = reg(a[0]) + (int(m.group(1)) if m else 0)
            src = list(vrange(a[1].split()[0]))
            for ln in range(64):
                for i, rr in enumerate(src):
                    lds[addr[ln] + 4 * i:addr[ln] + 4 * i + 4] = np.frombuffer(
                        np.uint32(v[rr][ln]).tobytes(), dtype=np.uint8)
            touched[0], touched[1] = min(touched[0], int(addr.min())), max(touched[1], int(addr.max()) + 8)
        elif op == "ds_read_b128":
            dst = list(vrange(a[0]))
            m = re.search(r"offset:(\d+)", t)
            addr = reg(a[1].split()[0]) + (int(m.group(1)) if m else 0)
            vals = [np.array([int(np.frombuffer(lds[addr[ln] + 4 * i:addr[ln] + 4 * i + 4].tobytes(),
                                                dtype=np.uint32)[0]) for ln in range(64)], dtype=np.int64)
                    for i in range(4)]
            for i, rr in enumerate(dst):
                (v if a[0].startswith("v") else acc)[rr] = vals[i]
            if a[0].startswith("v"):                  # the Q rows' reads are not the output's
                touched[0], touched[1] = min(touched[0], int(addr.min())), max(touched[1], int(addr.max()) + 16)
        elif op == "buffer_store_dwordx4":
            src = list(vrange(a[0]))
            data = v if a[0].startswith("v") else acc
            voff = reg(a[1])
            for ln in range(64):
                o = int(voff[ln])
                if o + 16 <= ops["onb"]:
                    for i, rr in enumerate(src):
                        out[o + 4 * i:o + 4 * i + 4] = np.frombuffer(np.uint32(data[rr][ln]).tobytes(),
                                                                      dtype=np.uint8)
                else:
                    assert o >= ops["onb"], "a store straddles the end of the rows"
        else:
            pytest.fail("no model for %s" % t)
    return cleared


def _run_turn(g, off, O, inv, ops, lds_size, out_bytes):
    """The turn on the model. Returns the output bytes (unwritten: 0xEE) and the LDS range the output rows
    went through."""
    pre, lead, items, _ = g.turn_work(off)
    v, acc, sreg = {}, {}, {}
    lds = np.zeros(lds_size, dtype=np.uint8)
    out = np.full(out_bytes, 0xEE, dtype=np.uint8)
    touched = [1 << 40, -1]
    cleared = _run_vector(list(pre) + list(lead) + [x for it in items for x in it["ins"]], O, inv, ops, lds, out,
                          touched, v, acc, sreg)
    assert cleared == set(range(2 * g.DB)), "O not cleared block by block"
    return out, touched


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("layout,nrows,off", [("bhnd", 64, 0), ("bhnd", 64, 1), ("bnhd", 64, 0), ("bnhd", 64, 1),
                                              ("bhnd", 37, 1), ("bnhd", 5, 0), ("bhnd", 0, 1)])
def test_turn_writes_previous_item_rows(layout, nrows, off, d):
    """The turn packs the finished item's O (the AGPR layout of the 32 x 32 products) as bf16(O / l) into the
    wave's Q slot and stores the rows from there: every row below the descriptor's end reaches memory at row * stride + column * 2, nothing else is
    written, and the rows go through the wave's own Q slot only."""
    g = _gen(d)
    TB, RB, DB = g.TILE_B, g.ROWB, g.DB
    rng = np.random.default_rng(5)
    H, wave = 3, 2
    stride = RB if layout == "bhnd" else H * RB
    qsb = 4 * TB + wave * TB
    onb = (nrows - 1) * stride + RB if nrows > 0 else 0
    O = rng.standard_normal((2 * DB, 16, 64)).astype(np.float32) * 3
    inv = (np.float32(0.37), np.float32(1.9))
    ops = {"wq": 4 * TB + wave * TB, "qsb": qsb, "ostr": stride, "onb": onb, **{"ka%d" % ks: 0 for ks in range(g.KS)}}
    out, touched = _run_turn(g, off, O.copy(), inv, ops, 10 * TB, 64 * stride + RB)
    assert touched[0] >= qsb and touched[1] <= qsb + TB, "output rows outside the wave's Q slot"
    want = np.full(64 * stride + RB, 0xEE, dtype=np.uint8)
    for k in range(2 * DB):
        qb, db = divmod(k, DB)
        for r in range(16):
            for ln in range(64):
                l32, hf = ln % 32, ln // 32
                q, dcol = qb * 32 + l32, db * 32 + (r // 4) * 8 + hf * 4 + r % 4
                if q >= nrows:
                    continue
                b = int(_bf16_bits(np.float32(O[k][r][ln]) * inv[qb]))
                o = q * stride + dcol * 2
                want[o:o + 2] = np.frombuffer(np.uint16(b).tobytes(), dtype=np.uint8)
    assert np.array_equal(out, want)
