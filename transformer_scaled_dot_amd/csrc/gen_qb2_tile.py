"""Generate attn_qb2_tile.inc: the tile steps of the 64-rows-per-wave attention
kernel for 128-wide heads, as inline-asm blocks with a fixed instruction
schedule.

A wave owns two 32-row query blocks (qb = 0, 1). One steady-state step for
key tile t:
  * S(t+1)^T = K(t+1) Q^T           32 MFMAs (8 k-steps x 2 key blocks x 2 qb)
  * P(t) = exp2(S(t) * c - mref)    rounded to bf16; row sums added to l
  * O^T += V(t)^T P(t)^T            32 MFMAs (4 key chunks x 4 d-blocks x 2 qb)
  * the row max of S(t+1)           for the next step's reference update
interleaved so that about five VALU instructions and one or two LDS reads sit
between consecutive MFMAs (a wave alone on its SIMD has no partner wave to
hide latencies). The first step of a wave computes only S(0) and its row max;
the last one only P and P.V. Lane layouts are those of the C++ kernel
(attn_fwd_bf16.hip): S^T has one query per lane, P goes from the score
accumulator to the P.V MFMA in the permuted key order, V^T operands come from
pairs of ds_read_b64_tr_b16.

The whole tile loop of a wave (S(0), then one step per key tile with the DMA,
the mask, the reference update, the rescale and the barrier) is ONE asm
statement, so the schedule inside it is exactly the one emitted here. O and
Q^T are bound to fixed AGPRs through the constraints; everything else the loop
works on lives in fixed registers that the statement declares clobbered:
  a[0:127]    O[qb][db]         a[128:191]  Q^T[qb][ks]  (MFMA B operand)
  v[0:63]     S buffer 0        v[64:127]   S buffer 1   (S[qb][jb], 16 each)
  v[128:159]  P[qb][c]          v[160:175]  K operand staging (4 slots)
  v[176:191]  V operand staging v[192:199]  exp temporaries
  v[200:212]  row max, reference, rescale factors, DMA offsets
  s[88:97]    tile indices and DMA addresses
The per-lane and per-wave inputs (LDS addresses, DMA offsets, limits, l, the
tile counts, base addresses) are compiler-placed operands; because the fixed
ranges are clobbers, the compiler cannot place an operand inside them (a test
compiles the kernel and checks every substituted register).
For the schedule it emits, the generator checks that every MFMA operand read
has completed (lgkmcnt) before its MFMA, that no staging slot is rewritten
before its last reader has issued, that every P operand is written at least
two instructions before its first MFMA, and that the row max reads the new S
only after three further MFMAs (or 24 wait states) behind the last MFMA that
wrote it. The loop ends with 24 wait states so that O is complete when C++
code next reads it.

Run:  python gen_qb2_tile.py  (writes attn_qb2_tile.inc for 128-wide heads and attn_qb2_tile_d64.inc for
64-wide ones next to this file)
"""
from __future__ import annotations

import math
import os

QB = 2                 # query blocks of 32 rows per wave


def configure(d):
    """Head width of the generated code (128 or 64): sets the module's shape constants."""
    global D, KS, DB, TILE_B, CH, TSH, RSH, ROWB, CPR, QSLOT, SUFFIX
    assert d in (64, 128)
    D, KS, DB = d, d // 16, d // 32
    TILE_B = 64 * D * 2            # bytes of a 64-row K, V or Q tile
    CH = TILE_B // 4096            # 1 KiB DMA instructions per tile and wave (4 waves)
    TSH = TILE_B.bit_length() - 1  # log2 of the tile bytes
    ROWB = D * 2                   # bytes of a row
    RSH = ROWB.bit_length() - 1
    CPR = D // 8                   # 16-byte chunks per row
    QSLOT = 4 * TILE_B             # LDS offset of the Q slots (four 64-row blocks)
    SUFFIX = "" if D == 128 else "_d%d" % D


configure(128)
S_BUF = (0, 64)
P0, KST, VST, TMP, MXT = 128, 160, 176, 192, 200
MXT_Q = ((200, 201), (217, 218))   # row-max temporaries of qb 0 and qb 1
CLOB_END = 204         # v[128:203] are the block's scratch registers
O_A, Q_A = 0, 128
LSUM_A, ONES_A = 192, 224   # a[192:199]: row-sum accumulators (qb 0, 1); a[224:227]: their 0/1 operand
NKS = NVS = 4          # staging slots
LOOK = 5               # MFMAs between an operand's read and its first MFMA
SLOT_CYC = 26          # issue cycles between two MFMAs of a wave that keep the MFMA pipe busy (measured best)
ISSUE_CYC = 4          # issue cost of one instruction
EXP_CYC = 8            # of a v_exp_f32
WAIT_AHEAD = 3         # an LDS wait also covers the operands of up to this many following MFMAs ...
WAIT_KEEP = 2          # ... leaving at least this many younger reads in flight
O_WAIT = ["s_nop 7", "s_nop 7", "s_nop 7"]   # before reading O (or scores) written by the last MFMAs
ONES_BF16X2 = "0x3f803f80"


def vr(base, n):
    return "v[%d:%d]" % (base, base + n - 1)


def ar(base, n):
    return "a[%d:%d]" % (base, base + n - 1)


def s_reg(buf, qb, jb, r):
    return S_BUF[buf] + (qb * 2 + jb) * 16 + r


def gen(x_buf, y_buf, kslot, vslot, do_s, do_pv, do_max, mref=("%[mref0]", "%[mref1]"), mx=("%[mx0]", "%[mx1]"),
        dma_ins=(), ref_upd=False, diag=False, pre=(), lead=(), extra_items=(), extra_mfma=()):
    """Instruction list of one block.

    x_buf: S buffer holding S(t) (exp + P.V part), y_buf: buffer receiving the
    new scores; kslot / vslot: LDS tile slots (0 or 1) of the K and V tiles.
    dma_ins: groups of DMA instructions, one group issued behind each of the
    first MFMAs (every other one); ref_upd: also move the reference of the new
    scores (after their row max and after this block's row sums); diag: the new scores are those of the
    wave's causal diagonal tile (its first key is the wave's first row; tile start * 64 in s89): mask
    them (keys past each row's own) before their row max.
    pre: instructions placed before the block's first operand reads (which then do not wait for the LDS
    reads in pre: the first MFMA's operand wait covers them, LDS returning in order); lead: instructions
    placed behind the first operand reads, before the first MFMA; extra_items: further work (dicts as the
    softmax items: ins, name, after) filled into the MFMA shadows after the block's own, in order;
    extra_mfma: MFMAs issued after the block's own, each after the extra items it names under "needs".
    The block ends without waiting for its last MFMAs: code that reads O or
    the new scores next must wait 24 wait states first (O_WAIT)."""
    koff = kslot * TILE_B
    voff = 2 * TILE_B + vslot * TILE_B

    mfma = []
    if do_s:
        for i in range(4 * KS):
            ks, jb, qb = i // 4, (i // 2) % 2, i % 2
            kop = ks * 2 + jb
            dst = S_BUF[y_buf] + (qb * 2 + jb) * 16
            src_c = "0" if ks == 0 else vr(dst, 16)
            mfma.append(dict(op=("k", kop), kind="S", qb=qb, jb=jb,
                             text="v_mfma_f32_32x32x16_bf16 %s, %s, %s, %s" % (
                                 vr(dst, 16), vr(KST + 4 * (kop % NKS), 4), ar(Q_A + 4 * (qb * KS + ks), 4), src_c)))
    if do_pv:
        for j in range(8 * DB):
            c, db, qb = j // (2 * DB), (j // 2) % DB, j % 2
            vop = c * DB + db
            acc = O_A + (qb * DB + db) * 16
            pop = vr(P0 + 4 * (qb * 4 + c), 4)
            mfma.append(dict(op=("v", vop), kind="PV", qb=qb, c=c,
                             text="v_mfma_f32_32x32x16_bf16 %s, %s, %s, %s" % (
                                 ar(acc, 16), vr(VST + 4 * (vop % NVS), 4), pop, ar(acc, 16))))
            if db == 0:
                # row sums of the rounded weights, from the same P^T operand read as the 32 x 16 B operand
                # of a 16 x 16 x 32 product (half the matrix-pipe time of a 32 x 32 x 16 one): lane l
                # holds query l % 32 and 8 of its 16 keys, i.e. column l % 16 and k-group l / 16 of B.
                # The 0/1 A operand (ones_pattern) adds the k-groups of parity p = (row / 4) % 2 into
                # each row, so output row m, column n is the sum of query n + 16 p over the 16 keys,
                # and the four rows lane l holds (4 (l / 16) .. + 3) all carry its own query's sum.
                ls = ar(LSUM_A + 4 * qb, 4)
                mfma.append(dict(op=None, kind="SUM", qb=qb, c=c,
                                 text="v_mfma_f32_16x16x32_bf16 %s, %s, %s, %s" % (ls, ar(ONES_A, 4), pop, ls)))
    mfma += [dict(f, op=None, kind="X") for f in extra_mfma]
    first_use, last_use = {}, {}
    for m, f in enumerate(mfma):
        if f["op"] is None:
            continue
        first_use.setdefault(f["op"], m)
        last_use[f["op"]] = m

    reads = {}
    for kop in range(2 * KS):
        ks, jb = kop // 2, kop % 2
        reads[("k", kop)] = ["ds_read_b128 %s, %s offset:%d" % (
            vr(KST + 4 * (kop % NKS), 4), "%%[ka%d]" % ks, koff + jb * 32 * D * 2)]
    for vop in range(4 * DB):
        c, db = vop // DB, vop % DB
        dst = VST + 4 * (vop % NVS)
        reads[("v", vop)] = ["ds_read_b64_tr_b16 %s, %%[va%d_%d] offset:%d" % (vr(dst + 2 * h, 2), db, h,
                                                                               voff + c * 16 * D * 2) for h in range(2)]
    read_at = {}
    for op, fu in first_use.items():
        read_at.setdefault(max(fu - LOOK, 0), []).append(op)
    for kind, nslots in (("k", NKS), ("v", NVS)):
        for o in sorted(o for o in first_use if o[0] == kind):
            nxt = (kind, o[1] + nslots)
            if nxt in first_use:
                assert max(first_use[nxt] - LOOK, 0) > last_use[o], ("staging slot reused too early", o, nxt)

    items = []
    if do_pv:
        # half-chunks of 4 scores (one per lane and row block): 4 fma, 4 exp, 2 packs into P.
        # Consecutive half-chunks use the two halves of v[192:199] in turn, and a half-chunk starts
        # only once the one two before it (same registers) is complete, so two can interleave.
        k = 0
        for c in range(4):
            for qb in range(QB):
                jb = c // 2
                dl = min(m for m, f in enumerate(mfma) if f["kind"] in ("PV", "SUM") and f["qb"] == qb and f["c"] == c)
                for h in range(2):
                    r0 = (c % 2) * 8 + 4 * h
                    tb = TMP + 4 * (k % 2)
                    fma = ["v_fma_f32 v%d, v%d, %%[c], -%s" % (tb + u, s_reg(x_buf, qb, jb, r0 + u), mref[qb])
                           for u in range(4)]
                    ex = ["v_exp_f32 v%d, v%d" % (tb + u, tb + u) for u in range(4)]
                    p = P0 + 4 * (qb * 4 + c) + 2 * h
                    cvt = ["v_cvt_pk_bf16_f32 v%d, v%d, v%d" % (p + w, tb + 2 * w, tb + 2 * w + 1) for w in range(2)]
                    seq = [fma[0], fma[1], ex[0], fma[2], ex[1], fma[3], ex[2], ex[3], cvt[0], cvt[1]]
                    items.append(dict(ins=seq, deadline=dl - 1, ready=0, p=P0 + 4 * (qb * 4 + c),
                                      name="exp %d" % k, after=["exp %d" % (k - 2)] if k >= 2 else []))
                    k += 1
    s_last = max((m for m, f in enumerate(mfma) if f["kind"] == "S"), default=None)
    if do_max:
        assert do_s
        for qb in range(QB):
            t0, t1 = MXT_Q[qb]
            chains = []
            for jb, m in ((0, t0), (1, t1)):
                vals = [s_reg(y_buf, qb, jb, r) for r in range(16)]
                ch = ["v_max3_f32 v%d, v%d, v%d, v%d" % (m, vals[0], vals[1], vals[2])]
                rest = vals[3:]
                while rest:
                    a_, b_ = rest[0], rest[1] if len(rest) > 1 else rest[0]
                    ch.append("v_max3_f32 v%d, v%d, v%d, v%d" % (m, m, a_, b_))
                    rest = rest[2:]
                chains.append(ch)
            ins = [x for pair in zip(*chains) for x in pair]   # the two chains alternate
            ins += ["v_max_f32 v%d, v%d, v%d" % (t0, t0, t1), "v_mov_b32 v%d, v%d" % (t1, t0), "s_nop 1",
                    "v_permlane32_swap_b32 v%d, v%d" % (t0, t1), "v_max_f32 %s, v%d, v%d" % (mx[qb], t0, t1)]
            if diag:
                items.append(dict(ins=diag_mask(y_buf, qb), deadline=len(mfma) + 8, ready=s_last + 4, p=None,
                                  name="diag q%d" % qb))
            items.append(dict(ins=ins, deadline=len(mfma) + 8, ready=s_last + 4, p=None, name="max q%d" % qb,
                              after=["diag q%d" % qb] if diag else []))
    if ref_upd:
        assert do_max
        for qb in range(QB):
            items.append(dict(ins=ref_check(qb), deadline=len(mfma) + 8, ready=s_last + 4, p=None,
                              name="ref q%d" % qb, after=["max q%d" % qb]))

    for n, it in enumerate(extra_items):
        items.append(dict(it, deadline=len(mfma) + 1000, ready=it.get("ready", 0), p=None))

    def cost(t):
        if t.startswith("v_exp"):
            return EXP_CYC
        return ISSUE_CYC

    out = list(pre) if pre else ["s_waitcnt lgkmcnt(0)"]
    issued, pos, p_done = [], {}, {}
    waited = [-1]       # LDS reads up to this index are known complete (LDS returns in order)
    queue = [dict(it, k=0, order=n) for n, it in enumerate(items)]
    by_name = {it["name"]: it for it in queue}

    def done(name):
        it = by_name[name]
        return it["k"] == len(it["ins"])

    def ready(it, m):
        return it["k"] < len(it["ins"]) and it["ready"] <= m and all(done(a_) for a_ in it.get("after", ()))

    dma_at = {2 * i: list(g) for i, g in enumerate(dma_ins)}
    for g in dma_at.values():
        assert len(g) == 2 and g[0].startswith("s_add_u32 m0") and "lds" in g[1]
    assert len(mfma) > 2 * (len(dma_ins) - 1) or not dma_ins

    # cycles of each slot (between two MFMA issues) left for the VALU work once the fixed
    # instructions (operand reads, DMA, waits) are in
    n_reads = [sum(len(reads[op]) for op in read_at.get(m + 1, [])) for m in range(len(mfma))]
    avail = [(SLOT_CYC if mfma[m]["kind"] != "SUM" else SLOT_CYC // 2) -
             ISSUE_CYC * (n_reads[m] + 1 + (2 if m + 1 in dma_at else 0)) for m in range(len(mfma))]

    def emit_reads(slot):
        for op in read_at.get(slot, []):
            for t in reads[op]:
                out.append(t)
                issued.append(op)
            pos[op] = len(issued) - 1

    def emit(it):
        t = it["ins"][it["k"]]
        out.append(t)
        it["k"] += 1
        if t.startswith("v_cvt_pk_bf16_f32"):
            p_done[int(t.split()[1][1:].rstrip(",")) // 4 * 4] = len(out) - 1  # the operand's last pack
        return cost(t)

    # the softmax half-chunks run at a steady pace that meets every P deadline: per slot, rate_c cycles
    # of their instructions, rate_e of their exps (cumulative targets); the row max and the reference
    # check use what the slots have left
    rate_c = rate_e = 0.0
    cum_c = cum_e = 0
    for it in sorted((it for it in queue if it["name"].startswith("exp")), key=lambda x: x["deadline"]):
        cum_c += sum(cost(t) for t in it["ins"])
        cum_e += sum(1 for t in it["ins"] if t.startswith("v_exp"))
        if it["deadline"] >= 0:
            rate_c = max(rate_c, cum_c / (it["deadline"] + 1))
            rate_e = max(rate_e, cum_e / (it["deadline"] + 1))
    prog = {"c": 0, "e": 0}

    emit_reads(0)
    out += list(lead)
    for m, f in enumerate(mfma):
        if f["kind"] in ("PV", "SUM"):
            p = P0 + 4 * (f["qb"] * 4 + f["c"])
            # nothing to overlap with yet (first P.V MFMAs of a block without S): finish that P operand here
            def force(it):
                for a_ in it.get("after", ()):
                    force(by_name[a_])
                while it["k"] < len(it["ins"]):
                    emit(it)
            for it in queue:
                if it["p"] == p:
                    force(it)
            # at least two instructions between the last write of P and the MFMA that reads it
            gap = sum(1 for t in out[p_done[p] + 1:] if not t.startswith("s_waitcnt"))
            if gap < 2:
                out.append("s_nop %d" % (1 - gap))
        for name in f.get("needs", ()):
            def force_named(it):
                for a_ in it.get("after", ()):
                    force_named(by_name[a_])
                while it["k"] < len(it["ins"]):
                    emit(it)
            force_named(by_name[name])
        if f["op"] is not None and pos[f["op"]] > waited[0]:
            # wait once for this operand and for those of the next MFMAs already read (they have had
            # at least as long to arrive), rather than once per operand
            upto = max([pos[f["op"]]] + [pos[g["op"]] for g in mfma[m + 1:m + 1 + WAIT_AHEAD]
                                         if g["op"] is not None and g["op"] in pos
                                         and pos[g["op"]] <= len(issued) - 1 - WAIT_KEEP])
            outstanding_after = len(issued) - 1 - upto
            assert 0 <= outstanding_after <= 15
            out.append("s_waitcnt lgkmcnt(%d)" % outstanding_after)
            waited[0] = upto
        dma = dma_at.pop(m, None)
        if dma:  # the MFMA is the wait state the LDS DMA needs after its M0 write
            out.append(dma[0])
        out.append(f["text"])
        if dma:
            out.append(dma[1])
        emit_reads(m + 1)
        # fill the slot: the half-chunks up to their pace (earliest deadline first), then the rest
        # within the slot's cycles
        spent = 0
        while True:
            pick = None
            for it in sorted((it for it in queue if ready(it, m)), key=lambda x: (x["deadline"], x["order"])):
                t = it["ins"][it["k"]]
                if it["name"].startswith("exp"):
                    if prog["c"] >= rate_c * (m + 1) - 1e-9:
                        continue
                    if t.startswith("v_exp") and prog["e"] + 1 > math.ceil(rate_e * (m + 1) - 1e-9):
                        continue
                elif spent + cost(t) > avail[m]:
                    continue
                pick = it
                break
            if pick is None:
                break
            t = pick["ins"][pick["k"]]
            if pick["name"].startswith("exp"):
                prog["c"] += cost(t)
                prog["e"] += t.startswith("v_exp")
            spent += emit(pick)
        if do_s:  # with the S part in front, every P operand is ready ahead of its MFMAs
            for it in queue:
                assert it["k"] == len(it["ins"]) or m < it["deadline"], ("deadline missed", it["name"], m)
    # what is left (the row max when few MFMAs follow the S part) runs after the last MFMA issued
    assert not dma_at
    rest = [it for it in sorted(queue, key=lambda x: x["order"]) if it["k"] < len(it["ins"])]
    if rest and s_last is not None and len(mfma) - 1 - s_last < 3:
        out += ["s_nop 7", "s_nop 7", "s_nop 7"]
    while rest:
        it = next(x for x in rest if all(done(a_) for a_ in x.get("after", ())))
        while it["k"] < len(it["ins"]):
            emit(it)
        rest.remove(it)
    return out


def o_binding():
    outs = []
    for qb in range(QB):
        for db in range(DB):
            b = O_A + (qb * DB + db) * 16
            outs.append('"+{a[%d:%d]}"(o[%d][%d])' % (b, b + 15, qb, db))
    return outs


def q_binding():
    return ['"{a[%d:%d]}"(q[%d][%d])' % (Q_A + 4 * (qb * KS + ks), Q_A + 4 * (qb * KS + ks) + 3, qb, ks)
            for qb in range(QB) for ks in range(KS)]


def ka_binding():
    return ['[ka%d] "v"(ka[%d])' % (ks, ks) for ks in range(KS)]


def va_binding():
    return ['[va%d_%d] "v"(va[%d][%d])' % (db, h, db, h) for db in range(DB) for h in range(2)]


# ---------------------------------------------------------------------------
# The whole tile loop of a wave as one asm statement (so that no C++ control
# flow sits between the blocks). Registers of the loop beyond the blocks':
MREF_V = (204, 205)     # reference max of the current tile, per qb
ALPHA_V = (206, 207)    # rescale factors
NINF_V = 208            # -inf for the mask
TMPL = 209              # v[209:214] scratch of the loop (mask limit, reference update: three per qb)
MX_V = (202, 203)       # row max of the current scores, per qb
KRES, VRES = 80, 84     # s[80:83] / s[84:87]: buffer descriptors of the K and V tiles being fetched
SREG = 88               # s[88:97] scratch SGPRs
UFLAG = (92, 94)        # s[92:93] / s[94:95]: rows whose reference moved, per qb
THR_S = 96              # the slack (8) in an SGPR
NKVB_S = 97             # the next item's kv_end in bytes
DIAG_S = ((98, 99), (90, 91))   # lane masks of the in-block diagonal mask, per qb
TF_S = 100              # the first step that is not a common step
MCP_V = (215, 216)      # reference + slack, per qb
LOOP_CLOB_V = list(range(0, 219))   # S buffers, P, staging and the loop's own registers
LOOP_CLOB_S = list(range(KRES, SREG + 13))
BUF_WORD3 = "0x20000"   # 32-bit data format, no stride: byte-addressed, range-checked raw buffer


def tile_res(res, tile_sreg, base_lo, base_hi):
    """Buffer descriptor of one K or V tile of the head: base = head + tile * 16 KiB, size = the bytes of
    the tile's rows below kv_end (0 past the end), so that rows past kv_end read as out of range and
    never touch memory."""
    return ["s_lshl_b32 s%d, %s, %d" % (SREG + 1, tile_sreg, TSH),
            "s_add_u32 s%d, %s, s%d" % (res, base_lo, SREG + 1),
            "s_addc_u32 s%d, %s, 0" % (res + 1, base_hi),
            "s_lshl_b32 s%d, %%[kve], %d" % (res + 2, RSH),
            "s_sub_i32 s%d, s%d, s%d" % (res + 2, res + 2, SREG + 1),
            "s_max_i32 s%d, s%d, 0" % (res + 2, res + 2),
            "s_mov_b32 s%d, %s" % (res + 3, BUF_WORD3)]


def dma_groups(res, slot_off):
    """The CH loads of one tile (each 64 lanes x 16 B into 1 KiB of LDS at M0), one group each."""
    return [["s_add_u32 m0, %%[lbw], %d" % (slot_off + j * 4096),
             "buffer_load_dwordx4 %%[vo%d], s[%d:%d], 0 offen lds" % (j, res, res + 3)] for j in range(CH)]


def step_dma(parity):
    """K(t+2) into K slot t % 2 and V(t+1) into V slot (t+1) % 2, as groups."""
    return dma_groups(KRES, parity * TILE_B) + dma_groups(VRES, 2 * TILE_B + (1 - parity) * TILE_B)


def ref_check(qb):
    """Rows of qb whose new tile max exceeds the reference by more than the slack (flags only)."""
    return ["v_mul_f32 v%d, v%d, %%[c]" % (TMPL + 3 * qb, MX_V[qb]),
            "v_cmp_gt_f32_e64 s[%d:%d], v%d, v%d" % (UFLAG[qb], UFLAG[qb] + 1, TMPL + 3 * qb, MCP_V[qb])]


def ref_update(qb, thr):
    """Move the reference of qb's rows to the new tile max where it exceeds the old reference by more than
    the slack (thr = 8); alpha = exp2(old - new) (1 where it stays)."""
    t0, t1, t2 = TMPL + 3 * qb, TMPL + 3 * qb + 1, TMPL + 3 * qb + 2
    u = "s[%d:%d]" % (UFLAG[qb], UFLAG[qb] + 1)
    return ["v_mul_f32 v%d, v%d, %%[c]" % (t0, MX_V[qb]),
            "v_add_f32 v%d, %s, %%[mc%d]" % (t1, thr, qb),
            "v_cmp_gt_f32_e64 %s, v%d, v%d" % (u, t0, t1),
            "v_cndmask_b32_e64 v%d, %%[mc%d], v%d, %s" % (t1, qb, t0, u),
            "v_sub_f32 v%d, %%[mc%d], v%d" % (t2, qb, t1),
            "v_exp_f32 v%d, v%d" % (t2, t2),
            "v_mov_b32 %%[mc%d], v%d" % (qb, t1),
            "v_max_f32 v%d, 0xff7fffff, v%d" % (MREF_V[qb], t1),
            "v_cndmask_b32_e64 v%d, 1.0, v%d, %s" % (ALPHA_V[qb], t2, u),
            "v_add_f32 v%d, %s, %%[mc%d]" % (MCP_V[qb], thr, qb)]


def diag_mask(buf, qb):
    """-inf for the keys past each row's own on the wave's causal diagonal tile (tile and wave start at the
    same key/row, a multiple of 64): block (qb 0, keys 32..63) is all masked, (qb 1, keys 0..31) all
    visible, the two 32 x 32 diagonal blocks are compared against the row's limit (lim - tile start,
    the lane half folded into lim)."""
    t, m = TMPL + 3 * qb, "s[%d:%d]" % DIAG_S[qb]
    o = ["v_subrev_u32 v%d, s%d, %%[lim%d]" % (t, SREG + 1, qb)]
    jb = qb  # the diagonal block of this row block
    for r in range(16):
        off = jb * 32 + (r >> 2) * 8 + (r & 3)
        sr = s_reg(buf, qb, jb, r)
        o += ["v_cmp_gt_i32_e64 %s, %d, v%d" % (m, off, t), "v_cndmask_b32_e64 v%d, v%d, v%d, %s" % (sr, sr, NINF_V, m)]
    if qb == 0:
        o += ["v_mov_b32 v%d, v%d" % (s_reg(buf, 0, 1, r), NINF_V) for r in range(16)]
    return o


def max_chain(buf, qb, dst):
    o = []
    for jb in range(2):
        m = MXT + jb
        vals = [s_reg(buf, qb, jb, r) for r in range(16)]
        o.append("v_max3_f32 v%d, v%d, v%d, v%d" % (m, vals[0], vals[1], vals[2]))
        rest = vals[3:]
        while rest:
            a, b = rest[0], rest[1] if len(rest) > 1 else rest[0]
            o.append("v_max3_f32 v%d, v%d, v%d, v%d" % (m, m, a, b))
            rest = rest[2:]
    o += ["v_max_f32 v%d, v%d, v%d" % (MXT, MXT, MXT + 1), "v_mov_b32 v%d, v%d" % (MXT + 1, MXT), "s_nop 1",
          "v_permlane32_swap_b32 v%d, v%d" % (MXT, MXT + 1), "v_max_f32 v%d, v%d, v%d" % (dst, MXT, MXT + 1)]
    return o


def res_advance(res):
    """Move a tile descriptor on by one tile; the size stays clamped at 0."""
    return ["s_add_u32 s%d, s%d, 0x%x" % (res, res, TILE_B), "s_addc_u32 s%d, s%d, 0" % (res + 1, res + 1),
            "s_sub_i32 s%d, s%d, 0x%x" % (res + 2, res + 2, TILE_B), "s_max_i32 s%d, s%d, 0" % (res + 2, res + 2)]


def mask_tile(tile_sreg, buf):
    """Scores of tile T (index in tile_sreg) in buffer buf: -inf for keys past each row's last visible key,
    then the row max again."""
    o = ["s_lshl_b32 s%d, %s, 6" % (SREG + 1, tile_sreg), "v_mov_b32 v%d, 0xff800000" % NINF_V]
    for qb in range(QB):
        o.append("v_subrev_u32 v%d, s%d, %%[lim%d]" % (TMPL, SREG + 1, qb))
        for jb in range(2):
            for r in range(16):
                off = jb * 32 + (r >> 2) * 8 + (r & 3)
                sr = s_reg(buf, qb, jb, r)
                o += ["v_cmp_gt_i32 vcc, %d, v%d" % (off, TMPL), "v_cndmask_b32 v%d, v%d, v%d, vcc" % (sr, sr, NINF_V)]
        o += max_chain(buf, qb, MX_V[qb])
    return o


def full_ref():
    o = ["s_mov_b32 s%d, 0x41000000" % THR_S]
    for qb in range(QB):
        o += ref_update(qb, "s%d" % THR_S)
    return o


def rescale():
    """O *= alpha and l *= alpha per row (l: the first register of each row-sum accumulator, the one read
    at the end)."""
    o = list(O_WAIT)
    for qb in range(QB):
        a = LSUM_A + 4 * qb
        o += ["v_accvgpr_read_b32 v%d, a%d" % (P0, a), "v_mul_f32 v%d, v%d, v%d" % (P0, P0, ALPHA_V[qb]),
              "v_accvgpr_write_b32 a%d, v%d" % (a, P0)]
    for qb in range(QB):
        for r in range(16 * DB):
            a = O_A + qb * 16 * DB + r
            t = P0 + (r % 16)
            o += ["v_accvgpr_read_b32 v%d, a%d" % (t, a), "v_mul_f32 v%d, v%d, v%d" % (t, t, ALPHA_V[qb]),
                  "v_accvgpr_write_b32 a%d, v%d" % (a, t)]
    return o + ["s_nop 1"]


# ---------------------------------------------------------------------------
# The turn between two items of a workgroup: the finished item's output O / l is packed to bf16 while the new
# item's Q rows go from the wave's Q slot into the Q AGPRs and its first scores S(0) are computed, so that the
# matrix pipe keeps working across the item boundary. The packed rows are written into the wave's Q slot (its Q
# rows have been read by then: LDS executes a wave's operations in order), 64 rows of 256 bytes with their 16-byte
# chunks XOR-swizzled by row, read back as whole rows and stored (non-temporal: the output is not read again,
# so it should not push the K/V tiles other workgroups share out of the L2). O is cleared by MFMAs of zero
# operands. Registers of the turn (free while S(0) is computed: the other score buffer, P, the V staging and the
# exp temporaries):
TURN_ZERO_V = 176       # v[176:179] = 0: operands of the MFMAs that clear O
TURN_WB_V = 180         # the lane's write address for chunk 0 (chunk c: XOR c << 4; row block qb: + 8 KiB)
TURN_RB_V = 181         # v[181:184]: the lane's read addresses for rows 4 j + (lane >> 4), j = 0..3
TURN_SB_V = 185         # the lane's byte offset in its output row group (row (lane >> 4), chunk lane & 15)
TURN_T_V = (186, 187)   # address temporaries (of the set-up)
TURN_L_V = 188          # v188 lane id, v189 lane & 15, v190 lane >> 4, v191 scratch
TURN_QA_V = 192         # v[192:199]: LDS addresses of the new Q rows, one per k-step
OUT_RES = KRES          # s[80:83]: the output rows' buffer descriptor (the K stream's is set after the turn)


def zero_o(k):
    return "v_mfma_f32_32x32x16_bf16 a[%d:%d], v[%d:%d], v[%d:%d], 0" % (
        O_A + 16 * k, O_A + 16 * k + 15, TURN_ZERO_V, TURN_ZERO_V + 3, TURN_ZERO_V, TURN_ZERO_V + 3)


def turn_work(off):
    """(pre, lead, items, zero MFMAs) of the turn for an item whose first scores go to buffer `off`: the finished
    item's packed rows go to the other score buffer (8 registers per 32 x 32 block of O, as qb2_out_bf16
    packs them), the pack temporaries alternate between the two halves of P. In the slot a row is ROWB bytes of
    CPR 16-byte chunks, chunk c of row r at chunk position c XOR (r mod CPR); one 16-byte read per lane covers
    RPR = 64 / CPR rows (row i RPR + lane / CPR, chunk lane mod CPR), whose positions repeat every NPAT reads."""
    pkb = S_BUF[1 - off]
    L, T0, T1 = TURN_L_V, TURN_T_V[0], TURN_T_V[1]
    RPR = 64 // CPR
    NPAT = max(CPR // RPR, 1)
    NRD = 32 // RPR                   # reads (and stores) per 32-row block
    pre = ["v_add_u32 v%d, %%[wq], %%[ka%d]" % (TURN_QA_V + ks, ks) for ks in range(KS)]
    pre += ["ds_read_b128 a[%d:%d], v%d offset:%d" % (Q_A + 4 * (qb * KS + ks), Q_A + 4 * (qb * KS + ks) + 3,
                                                      TURN_QA_V + ks, qb * 32 * D * 2)
            for qb in range(QB) for ks in range(KS)]
    pre += ["s_mov_b32 s%d, %%[obl]" % OUT_RES, "s_mov_b32 s%d, %%[obh]" % (OUT_RES + 1),
            "s_mov_b32 s%d, %%[onb]" % (OUT_RES + 2), "s_mov_b32 s%d, %s" % (OUT_RES + 3, BUF_WORD3)]
    pre += ["v_mov_b32 v%d, 0" % r for r in range(TURN_ZERO_V, TURN_ZERO_V + 4)]
    # lane id, lane mod CPR (chunk of a read), lane / CPR (row of a read)
    pre += ["v_mbcnt_lo_u32_b32 v%d, -1, 0" % L, "v_mbcnt_hi_u32_b32 v%d, -1, v%d" % (L, L),
            "v_and_b32 v%d, %d, v%d" % (L + 1, CPR - 1, L), "v_lshrrev_b32 v%d, %d, v%d" % (L + 2, CPR.bit_length() - 1, L)]
    # write address: slot + (lane & 31) * ROWB + (lane >> 5) * 8 + (((lane & 31) mod CPR) << 4); the slot is
    # 256-byte aligned, so the chunk bits hold (lane & 31) mod CPR and chunk c is that address XOR (c << 4)
    pre += ["v_and_b32 v%d, 31, v%d" % (T0, L), "v_lshlrev_b32 v%d, %d, v%d" % (T0, RSH, T0),
            "v_lshrrev_b32 v%d, 5, v%d" % (T1, L), "v_lshl_add_u32 v%d, v%d, 3, v%d" % (T0, T1, T0),
            "v_lshl_add_u32 v%d, v%d, 4, v%d" % (T0, L + 1, T0), "v_add_u32 v%d, %%[qsb], v%d" % (TURN_WB_V, T0)]
    # read address of pattern j: row r = j RPR + lane / CPR, chunk (lane mod CPR) XOR (r mod CPR)
    for j in range(NPAT):
        pre += ["v_add_u32 v%d, %d, v%d" % (T0, RPR * j, L + 2), "v_and_b32 v%d, %d, v%d" % (T1, CPR - 1, T0),
                "v_xor_b32 v%d, v%d, v%d" % (T1, T1, L + 1),
                "v_lshlrev_b32 v%d, 4, v%d" % (T1, T1), "v_lshl_add_u32 v%d, v%d, %d, v%d" % (T0, T0, RSH, T1),
                "v_add_u32 v%d, %%[qsb], v%d" % (TURN_RB_V + j, T0)]
    pre += ["v_mul_u32_u24 v%d, %%[ostr], v%d" % (T0, L + 2),
            "v_lshl_add_u32 v%d, v%d, 4, v%d" % (TURN_SB_V, L + 1, T0)]

    packs = []
    for k in range(QB * DB):
        qb, t, pk = k // DB, P0 + 16 * (k % 2), pkb + 8 * k
        ins = ["v_accvgpr_read_b32 v%d, a%d" % (t + r, O_A + 16 * k + r) for r in range(16)]
        ins += ["v_mul_f32 v%d, v%d, %%[inv%d]" % (t + r, t + r, qb) for r in range(16)]
        ins += ["v_cvt_pk_bf16_f32 v%d, v%d, v%d" % (pk + j, t + 2 * j, t + 2 * j + 1) for j in range(8)]
        packs.append(ins)
    # block 0 is packed ahead of the first MFMA (while the Q and first K reads are in flight)
    lead = packs[0]
    items = [dict(ins=packs[k], name="pack %d" % k, after=["pack %d" % (k - 2)] if k >= 3 else [])
             for k in range(1, QB * DB)]
    # one 32-row block at a time: its packed registers into the slot, read back as whole rows into the same
    # registers (LDS executes a wave's operations in order), then stored. Addresses of the writes and the
    # stores' offsets: the exp temporaries (block 0; free once the Q reads are issued), then the K operand
    # registers (block 1; free once the last S(0) MFMA has issued, four MFMAs before: ready)
    for qb in range(QB):
        tmp = [TMP + i for i in range(8)] if qb == 0 else list(range(KST, KST + 16))
        ready = 0 if qb == 0 else 4 * KS + 4
        rows = pkb + 8 * DB * qb          # the row block's packed registers (8 per 32 x 32 block)
        w = []
        for c in range(CPR):
            db, rg = c // 4, c % 4
            src = rows + 8 * db + 2 * rg
            a = tmp[c % len(tmp)]
            w += ["v_xor_b32 v%d, 0x%x, v%d" % (a, c << 4, TURN_WB_V),
                  "ds_write_b64 v%d, v[%d:%d] offset:%d" % (a, src, src + 1, qb * 32 * ROWB)]
        after = ["pack %d" % k for k in range(qb * DB, (qb + 1) * DB) if k > 0]
        after += ["store 0"] if qb else []
        items.append(dict(ins=w, name="write %d" % qb, after=after, ready=ready))
        rd = ["ds_read_b128 v[%d:%d], v%d offset:%d" % (rows + 4 * i, rows + 4 * i + 3, TURN_RB_V + (i % NPAT),
                                                        (qb * NRD + i) // NPAT * NPAT * 1024) for i in range(NRD)]
        items.append(dict(ins=rd, name="read %d" % qb, after=["write %d" % qb], ready=ready))
        st = ["s_waitcnt lgkmcnt(0)"]
        for i in range(NRD):
            a = tmp[i]
            st += ["v_mad_u32_u24 v%d, %d, %%[ostr], v%d" % (a, qb * 32 + RPR * i, TURN_SB_V),
                   "buffer_store_dwordx4 v[%d:%d], v%d, s[%d:%d], 0 offen nt" % (rows + 4 * i, rows + 4 * i + 3, a,
                                                                                OUT_RES, OUT_RES + 3)]
            if (i + 1) % (NRD // DB) == 0:
                # the row block's 32 x 32 blocks of O are cleared between its stores
                st.append(zero_o(qb * DB + i // (NRD // DB)))
        items.append(dict(ins=st, name="store %d" % qb, after=["read %d" % qb], ready=ready))
    # priority (the scheduler takes ready items in list order): block 0's packing, its staging, the first
    # block of qb 1 packed while block 0's rows come back from LDS, its stores, then the rest
    by = {it["name"]: it for it in items}
    order = (["pack %d" % k for k in range(1, DB)] + ["write 0", "read 0", "pack %d" % DB, "store 0"] +
             ["pack %d" % k for k in range(DB + 1, 2 * DB)] + ["write 1", "read 1", "store 1"])
    by["store 0"]["after"] = ["read 0", "pack %d" % DB]
    items = [by[n] for n in order]
    return pre, lead, items, []


def first_tile(off, turn=False):
    """S(0) of the wave, its mask where needed, its reference (O and l are still 0: no rescale). Tiles of
    the item take the slots and score buffers of parity (t + off) % 2: K(0) is in K slot off.
    turn: also the turn (the finished item's output, the new Q rows, O cleared), in the MFMA shadows of
    S(0), or on its own when the wave has no tile."""
    tag = ("t%d" if turn else "f%d") % off
    kw = {}
    if turn:
        pre, lead, items, zero = turn_work(off)
        kw = dict(pre=pre, lead=lead, extra_items=items, extra_mfma=zero)
    o = ["s_cmp_le_i32 %[ntw], 0", "s_cbranch_scc1 " + ("L_%s_only_%%=" % tag if turn else "L_first_done_%=")]
    o += gen(x_buf=1 - off, y_buf=off, kslot=off, vslot=off, do_s=True, do_pv=False, do_max=True,
             mx=("v%d" % MX_V[0], "v%d" % MX_V[1]), **kw)
    o += ["s_mov_b32 s%d, 0" % SREG, "s_cmp_eq_u32 %[dg], 0", "s_cbranch_scc1 L_%s_mask_%%=" % tag,
          "s_cmp_lt_i32 s%d, %%[tm]" % SREG, "s_cbranch_scc1 L_%s_ref_%%=" % tag, "L_%s_mask_%%=:" % tag]
    o += mask_tile("s%d" % SREG, off)
    o += ["L_%s_ref_%%=:" % tag] + full_ref() + ["s_branch L_first_done_%="]
    if turn:
        o += ["L_%s_only_%%=:" % tag]
        o += gen(x_buf=1 - off, y_buf=off, kslot=off, vslot=off, do_s=False, do_pv=False, do_max=False, **kw)
        o += ["s_branch L_first_done_%="]
    return o


def q_next_dma():
    """The next item's Q rows into the Q slots when this item has fewer than five tiles (else the general
    steps fetch them block by block, q_block_dma), issued once every wave has its own Q rows (after the barrier
    that follows S(0)): its four 64-row blocks, a quarter of each by every wave (the K/V tiles' DMA offsets),
    through descriptors covering each block's rows below N_q (rows past it read as zeros). nqr = the rows from
    the next item's first row to N_q; 0: no next item."""
    o = ["s_cmp_le_i32 %[nqr], 0", "s_cbranch_scc1 L_qdma_done_%=", "s_cmp_ge_i32 %[nt], 5",
         "s_cbranch_scc1 L_qdma_done_%="]
    for qw in range(4):
        o += ["s_add_u32 s%d, %%[nql], %d" % (KRES, qw * TILE_B), "s_addc_u32 s%d, %%[nqh], 0" % (KRES + 1),
              "s_sub_i32 s%d, %%[nqr], %d" % (KRES + 2, 64 * qw), "s_max_i32 s%d, s%d, 0" % (KRES + 2, KRES + 2),
              "s_min_i32 s%d, s%d, 64" % (KRES + 2, KRES + 2), "s_lshl_b32 s%d, s%d, %d" % (KRES + 2, KRES + 2, RSH),
              "s_mov_b32 s%d, %s" % (KRES + 3, BUF_WORD3)]
        for j in range(CH):
            o += ["s_add_u32 m0, %%[lbw], %d" % (QSLOT + qw * TILE_B + j * 4096), "s_nop 0",
                  "buffer_load_dwordx4 %%[vo%d], s[%d:%d], 0 offen nt lds" % (j, KRES, KRES + 3)]
    return o + ["L_qdma_done_%=:"]


def stream_res(res, x, base_lo, base_hi, nbase_lo, nbase_hi):
    """Descriptor of tile x (a constant) of the stream this item's tiles continue into the next item's:
    tile x of this item when x < nt, else tile x - nt of the next one."""
    o = ["s_mov_b32 s%d, %d" % (SREG, x)] + tile_res(res, "s%d" % SREG, base_lo, base_hi)
    o += ["s_cmp_ge_i32 s%d, %%[nt]" % SREG, "s_cbranch_scc0 L_sr%d_%d_%%=" % (res, x),
          "s_sub_i32 s%d, s%d, %%[nt]" % (SREG, SREG)]
    o += next_res(res, "s%d" % SREG, nbase_lo, nbase_hi) + ["L_sr%d_%d_%%=:" % (res, x)]
    return o


def next_res(res, tile_sreg, base_lo, base_hi):
    """Descriptor of tile (tile_sreg) of the next item (size from its kv_end: 0 when there is none)."""
    return ["s_lshl_b32 s%d, %s, %d" % (SREG + 1, tile_sreg, TSH),
            "s_add_u32 s%d, %s, s%d" % (res, base_lo, SREG + 1),
            "s_addc_u32 s%d, %s, 0" % (res + 1, base_hi),
            "s_lshl_b32 s%d, %%[nkve], %d" % (res + 2, RSH),
            "s_sub_i32 s%d, s%d, s%d" % (res + 2, res + 2, SREG + 1),
            "s_max_i32 s%d, s%d, 0" % (res + 2, res + 2),
            "s_mov_b32 s%d, %s" % (res + 3, BUF_WORD3)]


def res_advance_fast(res):
    """res_advance while the tile stays below the item's last (the size cannot reach 0)."""
    return ["s_add_u32 s%d, s%d, 0x%x" % (res, res, TILE_B), "s_addc_u32 s%d, s%d, 0" % (res + 1, res + 1),
            "s_sub_i32 s%d, s%d, 0x%x" % (res + 2, res + 2, TILE_B)]


def iteration(parity):
    """Step of tile t (S(t) in buffer `parity`, its reference applied). Returns the straight-line part and
    the out-of-line parts, which end by branching back. The straight-line part is the common step (t below
    the bound kept in s[TF_S]: the step computes S(t+1), needs no mask, and its fetches stay inside the item); every other
    step -- past the item's last tiles, the wave's last step, the diagonal or masked tile, waves without
    work -- takes the general path out of line, as do the rare reference moves."""
    P = parity
    tag = "p%d" % P
    nxt = "s%d" % SREG
    mref = ("v%d" % MREF_V[0], "v%d" % MREF_V[1])
    mx = ("v%d" % MX_V[0], "v%d" % MX_V[1])
    groups = step_dma(P)
    uf = "s[%d:%d], s[%d:%d]" % (UFLAG[0], UFLAG[0] + 1, UFLAG[1], UFLAG[1] + 1)
    full = lambda **kw: gen(x_buf=P, y_buf=1 - P, kslot=1 - P, vslot=P, do_s=True, do_pv=True, do_max=True,
                            mref=mref, mx=mx, dma_ins=groups, ref_upd=True, **kw)
    # common step (t < tf); the steps nt - 5 .. that fetch the next item's Q rows take a copy of it, out of line
    o = ["s_cmp_lt_i32 %%[t], s%d" % TF_S, "s_cbranch_scc0 L_slow_%s_%%=" % tag,
         "s_add_i32 s%d, %%[t], 5" % SREG, "s_cmp_ge_i32 s%d, %%[nt]" % SREG, "s_cbranch_scc1 L_qst_%s_%%=" % tag]
    o += res_advance_fast(KRES) + res_advance_fast(VRES)
    o += full()
    o += ["s_or_b64 vcc, %s" % uf, "s_cbranch_vccnz L_move_%s_%%=" % tag,
          "L_after_%s_%%=:" % tag, "s_waitcnt vmcnt(0)", "s_barrier"]
    tails = ["L_qst_%s_%%=:" % tag] + res_advance_fast(KRES) + res_advance_fast(VRES) + full()
    tails += ["s_or_b64 vcc, %s" % uf, "s_cbranch_vccnz L_move_%s_%%=" % tag, "s_branch L_after_%s_%%=" % tag]
    # general step: descriptors to K(t+2) and V(t+1) of the stream (past this item's last tile, the next
    # item's first tiles, so that they are in their slots when this item ends)
    ool = ["L_slow_%s_%%=:" % tag, "s_cmp_ge_i32 %[t], %[nt]", "s_cbranch_scc1 L_end_%="]
    ool += res_advance(KRES) + res_advance(VRES)
    ool += ["s_add_i32 %s, %%[t], 2" % nxt, "s_cmp_eq_i32 %s, %%[nt]" % nxt,
            "s_cselect_b32 s%d, %%[nkhl], s%d" % (KRES, KRES), "s_cselect_b32 s%d, %%[nkhh], s%d" % (KRES + 1, KRES + 1),
            "s_cselect_b32 s%d, s%d, s%d" % (KRES + 2, NKVB_S, KRES + 2)]
    ool += ["s_add_i32 %s, %%[t], 1" % nxt, "s_cmp_eq_i32 %s, %%[nt]" % nxt,
            "s_cselect_b32 s%d, %%[nvhl], s%d" % (VRES, VRES), "s_cselect_b32 s%d, %%[nvhh], s%d" % (VRES + 1, VRES + 1),
            "s_cselect_b32 s%d, s%d, s%d" % (VRES + 2, NKVB_S, VRES + 2)]
    ool += ["s_cmp_ge_i32 %[t], %[ntw]", "s_cbranch_scc1 L_nocomp_%s_%%=" % tag,
            "s_cmp_lt_i32 %s, %%[ntw]" % nxt, "s_cbranch_scc0 L_last_%s_%%=" % tag,
            "s_cmp_eq_u32 %s, %%[dg]" % nxt, "s_cbranch_scc1 L_diag_%s_%%=" % tag]
    ool += full()
    # tile t+1 masked: mask, row max, reference and rescale out of line; otherwise the block's check
    # says whether any row's reference must move (rare: then the update and the rescale)
    ool += ["s_cmp_ge_i32 %s, %%[tm]" % nxt, "s_cbranch_scc1 L_mask_%s_%%=" % tag,
            "s_or_b64 vcc, %s" % uf, "s_cbranch_vccnz L_move_%s_%%=" % tag, "s_branch L_after_%s_%%=" % tag]
    ool += ["L_mask_%s_%%=:" % tag] + mask_tile(nxt, 1 - P) + full_ref()
    ool += ["s_or_b64 vcc, %s" % uf, "s_cbranch_vccz L_after_%s_%%=" % tag] + rescale()
    ool += ["s_branch L_after_%s_%%=" % tag]
    ool += ["L_move_%s_%%=:" % tag] + full_ref() + rescale() + ["s_branch L_after_%s_%%=" % tag]
    # the step whose new scores are the wave's causal diagonal tile: masked inside the block
    ool += ["L_diag_%s_%%=:" % tag, "s_lshl_b32 s%d, %s, 6" % (SREG + 1, nxt)]
    ool += full(diag=True)
    ool += ["s_or_b64 vcc, %s" % uf, "s_cbranch_vccnz L_move_%s_%%=" % tag, "s_branch L_after_%s_%%=" % tag]
    ool += ["L_last_%s_%%=:" % tag]
    ool += gen(x_buf=P, y_buf=1 - P, kslot=1 - P, vslot=P, do_s=False, do_pv=True, do_max=False, mref=mref, mx=mx,
               dma_ins=groups)
    ool += ["s_branch L_after_%s_%%=" % tag, "L_nocomp_%s_%%=:" % tag]
    for g in groups:
        ool += g
    ool += ["s_branch L_after_%s_%%=" % tag]
    ool += tails
    ool = [x.replace("L_after_%s_%%=" % tag, "L_qchk_%s_%%=" % tag) if "branch" in x else x for x in ool]
    ool += q_block_dma(tag)
    o += ["L_cont_%s_%%=:" % tag]
    return o, ool


def q_block_dma(tag):
    """End of a step that is not a plain common one: in items of five or more tiles, the steps nt - 5 .. nt - 2
    each fetch one
    64-row block of the next item's Q rows (block t - nt + 5) into its Q slot, behind the step's own K/V
    fetches, and end by waiting for all but those four loads: the block has until the next step's end to
    arrive, and the last one is in before this item's loop ends. Every wave fetches a quarter of each block,
    so every Q slot is complete once all waves have passed that barrier."""
    qw, t = UFLAG[0], UFLAG[0] + 1
    o = ["L_qchk_%s_%%=:" % tag, "s_sub_i32 s%d, %%[t], %%[nt]" % qw, "s_add_i32 s%d, s%d, 5" % (qw, qw),
         "s_cmp_lt_u32 s%d, 4" % qw, "s_cbranch_scc0 L_after_%s_%%=" % tag,
         "s_cmp_lt_i32 %[nt], 5", "s_cbranch_scc1 L_after_%s_%%=" % tag,
         "s_cmp_le_i32 %[nqr], 0", "s_cbranch_scc1 L_after_%s_%%=" % tag]
    o += ["s_lshl_b32 s%d, s%d, %d" % (t, qw, TSH), "s_add_u32 s%d, %%[nql], s%d" % (SREG, t),
          "s_addc_u32 s%d, %%[nqh], 0" % (SREG + 1), "s_lshl_b32 s%d, s%d, 6" % (t, qw),
          "s_sub_i32 s%d, %%[nqr], s%d" % (SREG + 2, t), "s_max_i32 s%d, s%d, 0" % (SREG + 2, SREG + 2),
          "s_min_i32 s%d, s%d, 64" % (SREG + 2, SREG + 2), "s_lshl_b32 s%d, s%d, %d" % (SREG + 2, SREG + 2, RSH),
          "s_mov_b32 s%d, %s" % (SREG + 3, BUF_WORD3),
          "s_lshl_b32 s%d, s%d, %d" % (t, qw, TSH), "s_add_u32 s%d, s%d, %%[lbw]" % (t, t)]
    for j in range(CH):
        o += ["s_add_u32 m0, s%d, %d" % (t, QSLOT + j * 4096), "s_nop 0",
              "buffer_load_dwordx4 %%[vo%d], s[%d:%d], 0 offen nt lds" % (j, SREG, SREG + 3)]
    return o + ["s_waitcnt vmcnt(%d)" % CH, "s_barrier", "s_branch L_cont_%s_%%=" % tag]


def ones_pattern():
    """v0 = the A operand of the row-sum products for this lane: eight bf16 ones where the lane's k-group
    parity ((l / 16) % 2) equals its row's parity (((l % 16) / 4) % 2), zeros elsewhere."""
    return ["v_mbcnt_lo_u32_b32 v0, -1, 0", "v_mbcnt_hi_u32_b32 v0, -1, v0", "v_lshrrev_b32 v1, 4, v0",
            "v_lshrrev_b32 v0, 2, v0", "v_xor_b32 v0, v0, v1", "v_and_b32 v0, 1, v0", "v_cmp_eq_u32 vcc, 0, v0",
            "v_mov_b32 v1, %s" % ONES_BF16X2, "v_cndmask_b32 v0, 0, v1, vcc"]


def loop_body():
    o = ones_pattern()
    o += ["v_accvgpr_write_b32 a%d, v0" % (ONES_A + i) for i in range(4)]
    o += ["v_accvgpr_write_b32 a%d, 0" % (LSUM_A + i) for i in range(4 * QB)]
    o += ["s_nop 3", "s_lshl_b32 s%d, %%[nkve], %d" % (NKVB_S, RSH), "v_mov_b32 v%d, 0xff800000" % NINF_V]
    # S(0) with the item's parity, with the turn from the previous item (tn != 0) or without
    o += ["s_cmp_eq_u32 %[tn], 0", "s_cbranch_scc1 L_plain_%="]
    o += ["s_cmp_eq_u32 %[off], 0", "s_cbranch_scc0 L_turn1_%="] + first_tile(0, True)
    o += ["L_turn1_%=:"] + first_tile(1, True)
    o += ["L_plain_%=:", "s_cmp_eq_u32 %[off], 0", "s_cbranch_scc0 L_first1_%="] + first_tile(0)
    o += ["L_first1_%=:"] + first_tile(1) + ["L_first_done_%=:"]
    # step 0 fetches K(2) into the slot K(0) came from, and the next item's Q rows go where this item's were
    # read from: no wave may still be reading either
    o += ["s_barrier"] + q_next_dma()
    # descriptors one tile behind: each step first moves them to K(t+2) and V(t+1) of the stream
    o += stream_res(KRES, 1, "%[khl]", "%[khh]", "%[nkhl]", "%[nkhh]")
    o += stream_res(VRES, 0, "%[vhl]", "%[vhh]", "%[nvhl]", "%[nvhh]")
    # steps t < tf are common steps: tf = min(nt - 2, ntw - 1, t_diag - 1, t_mask - 1)
    o += ["s_add_i32 s%d, %%[nt], -2" % TF_S]
    for x in ("%[ntw]", "%[dg]", "%[tm]"):
        o += ["s_add_i32 s%d, %s, -1" % (SREG + 1, x), "s_min_i32 s%d, s%d, s%d" % (TF_S, TF_S, SREG + 1)]
    i0, ool0 = iteration(0)
    i1, ool1 = iteration(1)
    o += ["s_cmp_eq_u32 %[off], 0", "s_cbranch_scc0 L_mid_%="]
    # (tf <= nt - 2: a common step never ends the loop; the general one checks t against nt first)
    o += ["L_top_%=:"] + i0
    o += ["s_add_i32 %[t], %[t], 1", "L_mid_%=:"] + i1
    o += ["s_add_i32 %[t], %[t], 1", "s_branch L_top_%="]
    o += ool0 + ool1
    o += ["L_end_%=:"] + list(O_WAIT)
    o += ["v_accvgpr_read_b32 %%[l%d], a%d" % (qb, LSUM_A + 4 * qb) for qb in range(QB)]
    return o


def render_loop():
    body = loop_body()
    # Q^T is read and written: the turn loads the new item's rows into the same AGPRs
    outs = (o_binding() + ['"+' + b[1:] for b in q_binding()] +
            ['[l0] "+v"(l0)', '[l1] "+v"(l1)', '[mc0] "+v"(mc0)', '[mc1] "+v"(mc1)', '[t] "+s"(t)'])
    ins = (ka_binding() + va_binding() +
           ['[vo%d] "v"(vo[%d])' % (j, j) for j in range(CH)] +
           ['[lim0] "v"(lim0)', '[lim1] "v"(lim1)', '[c] "s"(c_log2)', '[nt] "s"(ntiles)', '[ntw] "s"(ntiles_w)',
            '[tm] "s"(t_mask)', '[kve] "s"(kv_end)', '[khl] "s"(kh_lo)', '[khh] "s"(kh_hi)',
            '[vhl] "s"(vh_lo)', '[vhh] "s"(vh_hi)', '[lbw] "s"(lbw)', '[off] "s"(off)', '[nkhl] "s"(nkh_lo)',
            '[nkhh] "s"(nkh_hi)', '[nvhl] "s"(nvh_lo)', '[nvhh] "s"(nvh_hi)', '[nkve] "s"(nkv_end)',
            '[dg] "s"(t_diag)', '[tn] "s"(turn)', '[inv0] "v"(inv0)', '[inv1] "v"(inv1)', '[obl] "s"(ob_lo)',
            '[obh] "s"(ob_hi)', '[onb] "s"(ob_bytes)', '[ostr] "s"(ob_stride)',
            '[wq] "s"(qslot)', '[qsb] "s"(qslot_lds)', '[nql] "s"(nq_lo)', '[nqh] "s"(nq_hi)', '[nqr] "s"(nq_rows)'])
    clob = (['"a%d"' % r for r in range(LSUM_A, ONES_A + 4)] + ['"v%d"' % r for r in LOOP_CLOB_V] +
            ['"s%d"' % r for r in LOOP_CLOB_S] +
            ['"vcc"', '"m0"', '"scc"', '"memory"'])
    return [
        "// S(0) of the wave and its reference, then its tile loop: for t = 0 .. ntiles-1 (the same count in",
        "// every wave of the workgroup, one barrier per tile), while t < ntiles_w the step with S(t+1) and",
        "// its reference (t + 1 < ntiles_w) or the last step, the DMA of K(t+2) and V(t+1) issued inside it;",
        "// then the mask of S(t+1) where it needs one and the rescale of O where a reference moved (both",
        "// out of line: the common path runs straight through). Tiles use the slots and score buffers of",
        "// parity (t + off) % 2; the fetches continue past the item's last tile into the next item's first",
        "// tiles (K(0), K(1), V(0) of the item given by nkh/nvh/nkv_end; nkv_end = 0: none). t_diag: the",
        "// wave's causal diagonal tile, masked inside its step (else out of range; t_mask then covers it).",
        "// K and V are read through range-checked buffer descriptors: rows at or past kv_end are not read.",
        "// turn != 0: before S(0), the item's Q rows are read from the wave's Q slot (qslot: its offset from the",
        "// K operand addresses; qslot_lds: its LDS address, 256-byte aligned) into q, and o (the previous item's",
        "// output, unnormalised) is packed as O / l (inv0, inv1: 1 / l of the wave's two row blocks) in bf16 into",
        "// that slot and stored from there to the rows of the buffer descriptor (ob_lo, ob_hi, ob_bytes), row r of",
        "// the wave at byte r * ob_stride; o is then cleared. turn == 0: q and o (= 0) are given. The next item's Q rows (nq_rows rows from address nq, 0: none) are fetched into the Q slots",
        "// after the barrier behind S(0) (items of fewer than five tiles) or one 64-row block per step at steps",
        "// nt - 5 .. nt - 2.",
        "__device__ __forceinline__ void qb2_loop%s(f32x16 (&o)[2][%d], bf16x8 (&q)[2][%d], const uint32_t (&ka)[%d],"
        % (SUFFIX, DB, KS, KS),
        "                                         const uint32_t (&va)[%d][2], const uint32_t (&vo)[%d]," % (DB, CH),
        "                                         int32_t lim0, int32_t lim1, float c_log2,",
        "                                         float &l0, float &l1, float &mc0, float &mc1,",
        "                                         int32_t t, int32_t ntiles, int32_t ntiles_w, int32_t t_mask,",
        "                                         int32_t kv_end, uint32_t kh_lo, uint32_t kh_hi,",
        "                                         uint32_t vh_lo, uint32_t vh_hi, uint32_t lbw, int32_t off,",
        "                                         uint32_t nkh_lo, uint32_t nkh_hi, uint32_t nvh_lo, uint32_t nvh_hi,",
        "                                         int32_t nkv_end, int32_t t_diag, int32_t turn, float inv0,",
        "                                         float inv1, uint32_t ob_lo, uint32_t ob_hi, uint32_t ob_bytes,",
        "                                         uint32_t ob_stride, uint32_t qslot, uint32_t qslot_lds,",
        "                                         uint32_t nq_lo, uint32_t nq_hi, int32_t nq_rows)",
        "{",
        "#pragma clang diagnostic push",
        "#pragma clang diagnostic ignored \"-Winline-asm\"",
        "    asm volatile(",
        "\n".join('        "%s\\n"' % x for x in body),
        "        : " + ",\n          ".join(outs),
        "        : " + ",\n          ".join(ins),
        "        : " + ", ".join(clob) + ");",
        "#pragma clang diagnostic pop",
        "}",
        "",
    ]


def render():
    lines = [
        "// Generated by gen_qb2_tile.py; edit the generator, not this file.",
        "// Tile steps of the 64-rows-per-wave kernel for %d-wide heads (see the" % D,
        "// generator for the schedule and the register plan).",
        "",
    ]
    # Q^T read from the wave's Q slot straight into its AGPRs (qa[ks]: LDS address of k-step ks of the first
    # query block, the second block 32 rows further) and O = 0 (each 32 x 32 block by one MFMA of zero
    # operands, 16 AGPRs per instruction) while the reads are in flight
    qrd = ["ds_read_b128 a[%d:%d], %%[qa%d] offset:%d" % (Q_A + 4 * (qb * KS + ks), Q_A + 4 * (qb * KS + ks) + 3, ks,
                                                           qb * 32 * D * 2) for qb in range(QB) for ks in range(KS)]
    zero = ["v_mov_b32 v%d, 0" % r for r in range(ZERO_V, ZERO_V + 4)] + ["s_nop 4"]
    zero += ["v_mfma_f32_32x32x16_bf16 a[%d:%d], v[%d:%d], v[%d:%d], 0" % (b, b + 15, ZERO_V, ZERO_V + 3, ZERO_V,
                                                                           ZERO_V + 3)
             for b in range(O_A, O_A + 16 * QB * DB, 16)]
    lines += [
        "__device__ __forceinline__ void qb2_init%s(f32x16 (&o)[2][%d], bf16x8 (&q)[2][%d], const uint32_t (&qa)[%d])"
        % (SUFFIX, DB, KS, KS),
        "{",
        "    asm volatile(",
        "\n".join('        "%s\\n"' % t for t in qrd + zero + ["s_waitcnt lgkmcnt(0)"] + list(O_WAIT)),
        "        : " + ",\n          ".join(
            ['"={a[%d:%d]}"(o[%d][%d])' % (O_A + (qb * DB + db) * 16, O_A + (qb * DB + db) * 16 + 15, qb, db)
             for qb in range(QB) for db in range(DB)] +
            ['"={a[%d:%d]}"(q[%d][%d])' % (Q_A + 4 * (qb * KS + ks), Q_A + 4 * (qb * KS + ks) + 3, qb, ks)
             for qb in range(QB) for ks in range(KS)]),
        "        : " + ",\n          ".join(['[qa%d] "v"(qa[%d])' % (ks, ks) for ks in range(KS)]),
        "        : " + ", ".join('"v%d"' % r for r in range(ZERO_V, ZERO_V + 4)) + ", \"memory\");",
        "}",
        "",
    ]
    lines += render_loop()
    lines += [""] + render_out_bf16()
    return "\n".join(lines)


ZERO_V = 0         # v[0:3] = 0: operands of the MFMAs that clear O
OUT_TMP_V = 0      # v[0:31]: two sets of 16 products
OUT_PK_V = 32      # v[32:95]: the packed rows, 8 registers per 32 x 32 block of O
OUT_INV_V = 96     # v96, v97: 1/l of each query block


def render_out_bf16():
    """O / l as bf16 pairs straight from the O AGPRs: per 32 x 32 block of O (qb, db), the 16 values a lane
    holds are read, scaled by the reciprocal of their row's sum and packed two by two (element 2j in the
    low half of pair j)."""
    ins = ["v_mov_b32 v%d, %%[inv0]" % OUT_INV_V, "v_mov_b32 v%d, %%[inv1]" % (OUT_INV_V + 1)]
    for k in range(QB * DB):
        qb, b, t, pk = k // DB, O_A + 16 * k, OUT_TMP_V + 16 * (k % 2), OUT_PK_V + 8 * k
        ins += ["v_accvgpr_read_b32 v%d, a%d" % (t + r, b + r) for r in range(16)]
        ins += ["v_mul_f32 v%d, v%d, v%d" % (t + r, t + r, OUT_INV_V + qb) for r in range(16)]
        ins += ["v_cvt_pk_bf16_f32 v%d, v%d, v%d" % (pk + j, t + 2 * j, t + 2 * j + 1) for j in range(8)]
    outs = ['"={v[%d:%d]}"(pk[%d][%d])' % (OUT_PK_V + 8 * k, OUT_PK_V + 8 * k + 7, k // DB, k % DB)
            for k in range(QB * DB)]
    inps = ['"{a[%d:%d]}"(o[%d][%d])' % (O_A + 16 * k, O_A + 16 * k + 15, k // DB, k % DB) for k in range(QB * DB)]
    inps += ['[inv0] "v"(inv0)', '[inv1] "v"(inv1)']
    clob = ['"v%d"' % r for r in list(range(OUT_TMP_V, OUT_TMP_V + 32)) + [OUT_INV_V, OUT_INV_V + 1]]
    return [
        "__device__ __forceinline__ void qb2_out_bf16%s(const f32x16 (&o)[2][%d], float inv0, float inv1," % (SUFFIX, DB),
        "                                             u32x8 (&pk)[2][%d])" % DB,
        "{",
        "    asm volatile(",
        "\n".join('        "%s\\n"' % t for t in ins),
        "        : " + ",\n          ".join(outs),
        "        : " + ",\n          ".join(inps),
        "        : " + ", ".join(clob) + ");",
        "}",
        "",
    ]


OUTPUTS = {128: "attn_qb2_tile.inc", 64: "attn_qb2_tile_d64.inc"}


if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    for d, name in OUTPUTS.items():
        configure(d)
        text = render()
        with open(os.path.join(here, name), "w", encoding="utf-8") as f:
            f.write(text)
        print("wrote", name)
    configure(128)
