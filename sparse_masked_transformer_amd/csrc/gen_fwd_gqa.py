"""Generator of the gfx950 assembly kernel for grouped-query sliding-window
attention forward, bf16, head size 128 (build step: writes a .s file).

The operation is the masked attention of Learn: Sparse & Sliding-Window
Attention, §3 equation, A = softmax(Q K^T * scale + log M) V, with M the
sliding window j in [i - W + 1, i] (the swa_mask of "Attention Variants
Compared"), computed with the tiled online softmax ("Flash style softmax",
same page): running maximum, running sum and running weighted sum per query
row while the key tiles of the window stream through LDS.

Work decomposition
  Workgroup = 4 waves = the 4 query heads h0 .. h0+3 of one key/value head
  (grouped-query attention), on the same 64 query rows.  Each wave owns 64
  rows of its head (two row groups of 32), so the K and V tiles staged in
  LDS serve all four heads, and every wave needs exactly the same key tiles
  (the band of its 64 rows): no wave idles on a tile its rows cannot see.
  One workgroup per CU (LDS holds four 64-key stages), one wave per SIMD.

Registers (512 per lane: 256 VGPRs + 256 AGPRs)
  AGPR  a[0:127]    O^T accumulators, two row groups x 4 blocks of 32 values
        a[128:191]  Q^T fragments (B operand of S^T = K Q^T), 2 x 8
        a[192:223]  K fragment ring (A operand), 8 slots
        a[224:255]  V^T fragment ring (A operand of O^T += V^T P^T), 8 slots
  VGPR  v[0:191]    three score buffers of 64 values: the tile whose scores
                    are being computed, the tile whose softmax is running
                    (its probabilities packed to bf16 in place), and the tile
                    whose probabilities feed the P V product
        v[192:255]  addressing, softmax state, temporaries

Software pipeline (one iteration per 64-key tile j)
  matrix cores: S(j+1) = K(j+1) Q^T (32 MFMAs) interleaved with
                O += V(j-1)^T P(j-1) (32 MFMAs)
  vector ALU:   row maxima of S(j), then p = exp2(s * c - m), the row sums
                and the bf16 packing of P(j), spread between the MFMAs
  LDS:          the fragments of both products, a few pairs ahead
  DMA:          tile j+2 into the fourth stage (buffer_load ... lds)
The running maximum moves only when a tile's maximum exceeds it by more than
8 (log2 units); O is then rescaled at the end of the iteration, after the
products of the old maximum have been accumulated.

Hazards: every instruction records the registers it reads and writes; a
final pass inserts the wait states gfx950 requires between producers and
consumers (MFMA results, VALU -> MFMA operands, transcendental results,
SGPRs written by the VALU, M0 before LDS-DMA) and the s_waitcnt each load's
consumer needs.
"""
import os
import sys

# ---------------------------------------------------------------------------
# sizes
D = 128                       # head size (q, k, v)
KROW = 2 * D + 16             # padded LDS row of K, bytes
VROW = 2 * D + 64             # padded LDS row of V, bytes
KTILE = 64 * KROW             # 17408
VTILE = 64 * VROW             # 20480
STAGE = KTILE + VTILE         # 37888
NSTAGE = 4
LDS_BYTES = NSTAGE * STAGE    # 151552
KCH, VCH = KTILE // 1024, VTILE // 1024   # 17, 20 chunks of 1 KiB
SLACK = 8.0
KARG_BYTES = 80
NAME = "swa_fwd_gqa_d128"

# magic multipliers: floor(x / 272) and floor(x / 320) as (x * M) >> 24
M272, M320 = 61681, 52429
for _x in range(KTILE):
    assert (_x * M272) >> 24 == _x // KROW
for _x in range(VTILE):
    assert (_x * M320) >> 24 == _x // VROW


# ---------------------------------------------------------------------------
# instruction IR
class R:
    """A register range: file 'v', 'a' or 's', first index, count."""

    def __init__(self, f, i, n=1):
        self.f, self.i, self.n = f, i, n

    def __str__(self):
        if self.n == 1:
            return f"{self.f}{self.i}"
        return f"{self.f}[{self.i}:{self.i + self.n - 1}]"

    def regs(self):
        return frozenset((self.f, k) for k in range(self.i, self.i + self.n))

    def sub(self, k, n=1):
        assert 0 <= k and k + n <= self.n
        return R(self.f, self.i + k, n)


def v(i, n=1):
    return R("v", i, n)


def a(i, n=1):
    return R("a", i, n)


def s(i, n=1):
    return R("s", i, n)


VCC = frozenset({("s", "vcc")})
M0 = frozenset({("s", "m0")})
SCC = frozenset({("s", "scc")})
EMPTY = frozenset()


def regs_of(*xs):
    out = set()
    for x in xs:
        if isinstance(x, R):
            out |= x.regs()
        elif isinstance(x, frozenset):
            out |= x
    return frozenset(out)


class I:
    """kind: mfma valu trans perm vcmp rfl salu lds dma vmem vstore smem
    wait barrier branch label nop raw"""

    def __init__(self, text, kind, reads=EMPTY, writes=EMPTY, srcab=EMPTY, srcc=EMPTY, lds_read=False,
                 vm_load=False, dests=EMPTY):
        self.text, self.kind = text, kind
        self.reads, self.writes = frozenset(reads), frozenset(writes)
        self.srcab, self.srcc = frozenset(srcab), frozenset(srcc)
        self.lds_read = lds_read      # increments lgkmcnt, writes `dests` when it returns
        self.vm_load = vm_load        # increments vmcnt
        self.dests = frozenset(dests)


class Prog:
    def __init__(self):
        self.ins = []
        self.nlabel = 0

    def add(self, x):
        self.ins.append(x)
        return x

    def label(self, name):
        self.add(I(f"{name}:", "label"))

    def new_label(self, hint):
        self.nlabel += 1
        return f".L{hint}_{self.nlabel}"

    def comment(self, text):
        self.add(I(f"  ; {text}", "raw"))

    # ---- scalar
    def salu(self, op, dst, *srcs, reads_scc=False, writes_scc=True):
        txt = f"  {op} {dst}" + "".join(f", {x}" for x in srcs)
        rd = regs_of(*[x for x in srcs if isinstance(x, R)])
        if reads_scc:
            rd |= SCC
        wr = regs_of(dst) if isinstance(dst, R) else (M0 if dst == "m0" else (VCC if dst == "vcc" else EMPTY))
        if writes_scc:
            wr |= SCC
        rd |= frozenset(("s", x) for x in srcs if x in ("m0", "vcc"))
        return self.add(I(txt, "salu", rd, wr))

    def scmp(self, op, x, y):
        return self.add(I(f"  {op} {x}, {y}", "salu", regs_of(*[z for z in (x, y) if isinstance(z, R)])
                          | (VCC if "vcc" in (x, y) else EMPTY), SCC))

    def branch(self, op, target):
        rd = SCC if "scc" in op else (VCC if "vcc" in op else EMPTY)
        self.add(I(f"  {op} {target}", "branch", rd))

    def smem(self, op, dst, base, off):
        self.add(I(f"  {op} {dst}, {base}, {off}", "smem", regs_of(base), regs_of(dst)))

    # ---- vector
    def valu(self, op, dst, *srcs, kind="valu", extra=""):
        txt = f"  {op} {dst}" + "".join(f", {x}" for x in srcs) + (f" {extra}" if extra else "")
        rd = set()
        for x in srcs:
            if isinstance(x, R):
                rd |= x.regs()
            elif isinstance(x, str) and x.startswith("-") and len(x) > 1 and x[1] in "vs":
                pass
        rd = frozenset(rd) | self._neg_regs(srcs)
        wr = regs_of(dst) if isinstance(dst, R) else (VCC if dst == "vcc" else EMPTY)
        if "vcc" in srcs:
            rd |= VCC
        return self.add(I(txt, kind, rd, wr))

    @staticmethod
    def _neg_regs(srcs):
        out = set()
        for x in srcs:
            if isinstance(x, NegR):
                out |= x.r.regs()
        return frozenset(out)

    def mfma(self, dst, ra, rb, rc):
        c = "0" if rc is None else str(rc)
        rd = regs_of(ra, rb) | (rc.regs() if rc is not None else EMPTY)
        self.add(I(f"  v_mfma_f32_32x32x16_bf16 {dst}, {ra}, {rb}, {c}", "mfma", rd, dst.regs(),
                   srcab=regs_of(ra, rb), srcc=(rc.regs() if rc is not None else EMPTY)))

    def ds_read(self, op, dst, addr, off):
        self.add(I(f"  {op} {dst}, {addr} offset:{off}", "lds", addr.regs(), dst.regs(), lds_read=True,
                   dests=dst.regs()))

    def buf_load(self, dst, voff, rsrc, soff, off=0):
        o = f" offset:{off}" if off else ""
        self.add(I(f"  buffer_load_dwordx4 {dst}, {voff}, {rsrc}, {soff} offen{o}", "vmem",
                   regs_of(voff, rsrc, soff if isinstance(soff, R) else None), dst.regs(), vm_load=True,
                   dests=dst.regs()))

    def dma(self, voff, rsrc, soff):
        self.add(I(f"  buffer_load_dwordx4 {voff}, {rsrc}, {soff} offen lds", "dma",
                   regs_of(voff, rsrc, soff) | M0, EMPTY, vm_load=True))

    def buf_store(self, op, data, voff, rsrc, off=0):
        o = f" offset:{off}" if off else ""
        self.add(I(f"  {op} {data}, {voff}, {rsrc}, 0 offen{o}", "vstore", regs_of(data, voff, rsrc), EMPTY))

    def waitcnt(self, vm=None, lgkm=None):
        parts = []
        if vm is not None:
            parts.append(f"vmcnt({vm})")
        if lgkm is not None:
            parts.append(f"lgkmcnt({lgkm})")
        self.add(I("  s_waitcnt " + " ".join(parts), "wait"))

    def barrier(self):
        self.add(I("  s_barrier", "barrier"))


class NegR:
    def __init__(self, r):
        self.r = r

    def __str__(self):
        return f"-{self.r}"


# ---------------------------------------------------------------------------
# hazard and wait-count resolution
MFMA_RAW = 12      # MFMA 32x32x16 result -> any other reader
MFMA_WAR_C = 8     # MFMA reading srcC -> VALU overwriting it
VALU_TO_MFMA = 2
TRANS_TO_USE = 1
VALU_TO_PERM = 2
VALU_TO_RFL = 4    # VALU writes a VGPR -> v_readfirstlane reads it (stale without)
VALU_SGPR_TO_VALU = 2
VALU_SGPR_TO_VMEM = 5
M0_TO_DMA = 1


def _need(p, x):
    """Wait states required between producer p and consumer x."""
    n = 0
    if p.kind == "mfma":
        if x.kind == "mfma":
            if x.srcab & p.writes:
                n = max(n, MFMA_RAW)
            if x.srcc & p.writes and x.srcc != p.writes:
                n = max(n, MFMA_RAW)
            if (x.writes & p.writes) and x.srcc != p.writes:
                n = max(n, MFMA_RAW)
        else:
            if x.reads & p.writes:
                n = max(n, MFMA_RAW)
            if x.writes & p.writes or x.dests & p.writes:
                n = max(n, MFMA_RAW)
            if x.writes & p.srcc or x.dests & p.srcc:
                n = max(n, MFMA_WAR_C)
            if x.dests & p.srcab:
                n = max(n, 4)
    elif p.kind in ("valu", "trans", "perm", "vcmp", "rfl"):
        vw = frozenset(r for r in p.writes if r[0] in "va")
        sw = frozenset(r for r in p.writes if r[0] == "s" and r[1] not in ("scc",))
        if x.kind == "mfma" and (x.srcab | x.srcc) & vw:
            n = max(n, VALU_TO_MFMA)
        if p.kind == "trans" and x.kind in ("valu", "trans", "perm", "vcmp") and x.reads & vw:
            n = max(n, TRANS_TO_USE)
        if x.kind == "perm" and x.reads & vw:
            n = max(n, VALU_TO_PERM)
        if x.kind == "rfl" and x.reads & vw:
            n = max(n, VALU_TO_RFL)
        if sw and x.reads & sw:
            if x.kind in ("vmem", "dma", "vstore", "smem", "lds"):
                n = max(n, VALU_SGPR_TO_VMEM)
            else:
                n = max(n, VALU_SGPR_TO_VALU)
    elif p.kind == "salu":
        if x.kind == "dma" and (p.writes & M0):
            n = max(n, M0_TO_DMA)
        if x.kind in ("vmem", "dma", "vstore") and (p.writes & x.reads - M0 - SCC):
            n = max(n, 1)
    return n


def _max_need(p):
    if p.kind == "mfma":
        return MFMA_RAW
    if p.kind in ("vcmp", "rfl"):
        return VALU_SGPR_TO_VMEM
    if p.kind in ("valu", "trans", "perm"):
        return VALU_TO_MFMA
    if p.kind == "salu":
        return 1
    return 0


def _nops(n):
    out = []
    while n > 0:
        k = min(n, 8)
        out.append(I(f"  s_nop {k - 1}", "nop"))
        n -= k
    return out


def resolve(ins):
    """Insert s_nop for hazards and s_waitcnt for load consumers."""
    out = []
    hist = []           # (wait-state index, instruction)
    ws = 0
    pend_lgkm = []      # dest register sets of outstanding LDS reads, in order
    pend_vm = []        # dest register sets (or empty for LDS-DMA) of outstanding vector loads

    def emit(x):
        nonlocal ws
        out.append(x)
        hist.append((ws, x))
        ws += 1
        while hist and ws - hist[0][0] > 24:
            hist.pop(0)

    def flush():
        nonlocal ws
        req = 0
        for pws, p in hist:
            req = max(req, _max_need(p) - (ws - pws - 1))
        if req > 0:
            for y in _nops(req):
                out.append(y)
            ws += req

    for x in ins:
        if x.kind == "raw":
            out.append(x)
            continue
        if x.kind in ("label", "branch"):
            # control flow: no load may be pending into registers, and every
            # hazard window is closed before it
            if pend_lgkm:
                out.append(I("  s_waitcnt lgkmcnt(0)", "wait"))
                ws += 1
                pend_lgkm = []
            if any(d for d in pend_vm):
                out.append(I("  s_waitcnt vmcnt(0)", "wait"))
                ws += 1
                pend_vm = []
            flush()
            out.append(x)
            ws += 1
            hist = []
            continue
        if x.kind == "wait":
            # explicit waits: parse and retire the matching pending loads
            t = x.text
            if "vmcnt(" in t:
                k = int(t.split("vmcnt(")[1].split(")")[0])
                pend_vm = pend_vm[len(pend_vm) - k:] if k < len(pend_vm) else pend_vm
                if k == 0:
                    pend_vm = []
            if "lgkmcnt(" in t:
                k = int(t.split("lgkmcnt(")[1].split(")")[0])
                pend_lgkm = pend_lgkm[len(pend_lgkm) - k:] if k < len(pend_lgkm) else pend_lgkm
                if k == 0:
                    pend_lgkm = []
            emit(x)
            continue
        # loads in flight whose destination x reads or overwrites
        touch = x.reads | x.writes | x.dests
        lg = [i for i, d in enumerate(pend_lgkm) if d & touch]
        vm = [i for i, d in enumerate(pend_vm) if d & touch]
        if lg or vm:
            parts = []
            if vm:
                k = len(pend_vm) - 1 - max(vm)
                k = min(k, 63)
                parts.append(f"vmcnt({k})")
                pend_vm = pend_vm[len(pend_vm) - k:] if k > 0 else []
            if lg:
                k = len(pend_lgkm) - 1 - max(lg)
                k = min(k, 15)
                parts.append(f"lgkmcnt({k})")
                pend_lgkm = pend_lgkm[len(pend_lgkm) - k:] if k > 0 else []
            emit(I("  s_waitcnt " + " ".join(parts), "wait"))
        req = 0
        for pws, p in hist:
            n = _need(p, x)
            if n:
                req = max(req, n - (ws - pws - 1))
        if req > 0:
            for y in _nops(req):
                out.append(y)
            ws += req
        emit(x)
        if x.lds_read:
            pend_lgkm.append(x.dests)
            if len(pend_lgkm) > 15:
                raise ValueError("more than 15 LDS reads in flight")
        if x.vm_load:
            pend_vm.append(x.dests)
    return out


# ---------------------------------------------------------------------------
# register map
S_BUF = [0, 64, 128]                 # three score buffers of 64 VGPRs
V_TID, V_KLANE, V_VLANE = v(192), v(193), v(194)
V_DK = [v(195 + i) for i in range(5)]
V_DV = [v(200 + i) for i in range(5)]
V_QOFF = [v(205), v(206)]
V_M = [v(207), v(208)]               # running maximum (scaled, log2 units)
V_MTHR = [v(209), v(210)]            # running maximum + slack
V_L = [[v(211), v(212)], [v(213), v(214)]]   # running sums, two partials per row group
V_ALPHA = [v(215), v(216)]
V_MOLD = [v(245), v(246)]            # running maximum before this tile
V_LT = [[v(247), v(248)], [v(249), v(250)]]   # this tile's row sums (two partials per row group)
V_KADDR, V_VADDR = v(217), v(218)
V_IBASE = [v(219), v(220)]           # row - 4 * (lane / 32), for the per-cell mask
V_T = [v(222 + i) for i in range(16)]  # even start: pairs of them are 64-bit tuples
V_OOFF = [v(238), v(239)]           # (spare since the output goes through LDS)
V_OWL, V_ORDL, V_OST = v(251), v(252), v(253)   # epilogue lane bases: LDS write, LDS read, global store
V_OW, V_ORD = v(254), v(255)
V_LOFF = [v(240), v(241)]
V_COL, V_HL, V_LANE = v(242), v(243), v(244)

A_O = [a(0, 64), a(64, 64)]          # O^T per row group: block db at 16 db
A_Q = [a(128, 32), a(160, 32)]       # Q^T fragments per row group: ks at 4 ks
A_KR = a(192, 32)                    # K fragment ring: slot at 4 slot
A_VR = a(224, 32)                    # V fragment ring

# SGPRs
S_KARG = s(0, 2)
S_WG = s(2)
S_Q, S_K, S_V, S_OUT, S_LSE = s(4, 2), s(6, 2), s(8, 2), s(10, 2), s(12, 2)
S_N, S_W, S_G, S_NHB, S_NRB, S_C = s(14), s(15), s(16), s(17), s(18), s(19)
S_TOTAL, S_HKV, S_HQ = s(20), s(21), s(22)
S_WAVE, S_LID, S_HB, S_RB, S_BG, S_R0, S_TLO, S_T, S_J = (s(24), s(25), s(26), s(27), s(28), s(29),
                                                          s(30), s(31), s(32))
S_RSK, S_RSV, S_RSQ, S_RSO, S_RSL = s(36, 4), s(40, 4), s(44, 4), s(48, 4), s(52, 4)
S_WAVE1K, S_SOFF, S_SB, S_SBK, S_SBV, S_K0 = s(56), s(57), s(58), s(59), s(60), s(61)
S_WM1, S_NINF, S_ONES = s(63), s(64), s(65)
S_SBW = s(62)                        # DMA stage base + 1024 * wave
S_NB = s(33)                         # N * 256: bytes per head, first offset past the rows
S_FLAG = s(68, 2)
S_CMP = [s(70, 2), s(72, 2)]
S_MV = [s(74, 2), s(76, 2)]
S_X = [s(78 + i) for i in range(14)]  # scalar temporaries s78..s91


# ---------------------------------------------------------------------------
# build options.  Row sums: over the bf16-rounded probabilities (v_dot2), the
# values the P V product accumulates, so the weights of a row sum to exactly
# one after the division (a near one-hot row gives its value row exactly);
# fp32_sums sums the unrounded values instead (the weights then sum to one
# only within 2^-8, which on peaky rows costs up to ~0.02 of output error)
OPT = {"fp32_sums": False}


# ---------------------------------------------------------------------------
# optional register dumps (a development aid: off in the library build)
DEBUG = {"on": False, "dumps": True, "n": 0, "tags": []}
S_DBG = s(92, 4)


def dump(P, tag, regs):
    """Store each 32-bit register of `regs` (VGPR or AGPR ranges) of every
    lane to the debug buffer: dump k, register r, global wave w, lane l at
    dword ((k * 256 + r) * waves + w) * 64 + l."""
    if not (DEBUG["on"] and DEBUG["dumps"]):
        return
    k = DEBUG["n"]
    DEBUG["n"] += 1
    DEBUG["tags"].append((tag, sum(x.n for x in regs)))
    r = 0
    for rng in regs:
        for i in range(rng.n):
            src = rng.sub(i)
            if src.f == "a":
                P.add(I(f"  v_accvgpr_read_b32 {V_T[15]}, {src}", "valu", src.regs(), V_T[15].regs()))
                src = V_T[15]
            # offset = ((k*256 + r) * waves + gwave) * 256 + lane * 4; waves
            # and gwave in S_X[0] / S_X[1] (set at kernel entry)
            P.salu("s_mul_i32", S_X[2], S_DBGW, str(k * 256 + r))
            P.salu("s_add_u32", S_X[2], S_X[2], S_DBGG)
            P.salu("s_lshl_b32", S_X[2], S_X[2], "8")
            P.add(I(f"  buffer_store_dword {src}, {V_DBGL}, {S_DBG}, {S_X[2]} offen", "vstore",
                    regs_of(src, V_DBGL, S_DBG, S_X[2]), EMPTY))
            r += 1


def dump_lds(P, tag, nbytes):
    """Dump LDS bytes 0 .. nbytes-1 (stage 0) as registers of 64 dwords."""
    if not (DEBUG["on"] and DEBUG["dumps"]):
        return
    k = DEBUG["n"]
    DEBUG["n"] += 1
    DEBUG["tags"].append((tag, nbytes // 256))
    for r in range(nbytes // 256):
        P.ds_read("ds_read_b32", V_T[14], V_DBGL, r * 256)
        P.salu("s_mul_i32", S_X[2], S_DBGW, str(k * 256 + r))
        P.salu("s_add_u32", S_X[2], S_X[2], S_DBGG)
        P.salu("s_lshl_b32", S_X[2], S_X[2], "8")
        P.add(I(f"  buffer_store_dword {V_T[14]}, {V_DBGL}, {S_DBG}, {S_X[2]} offen", "vstore",
                regs_of(V_T[14], V_DBGL, S_DBG, S_X[2]), EMPTY))


S_DBGW, S_DBGG = s(66), s(67)   # total waves, this wave's global index (debug only)
V_DBGL = v(221)                 # lane * 4 (debug only)


# ---------------------------------------------------------------------------
# building blocks
def udiv(P, x, d, q, r, t0, t1):
    """q = x / d, r = x % d for wave-uniform 0 <= x < 2^24, 1 <= d < 2^24
    (SGPRs); float estimate, then one correction each way."""
    P.valu("v_cvt_f32_u32", t0, x)
    P.valu("v_cvt_f32_u32", t1, d)
    P.valu("v_rcp_f32", t1, t1, kind="trans")
    P.valu("v_mul_f32", t0, t0, t1)
    P.valu("v_cvt_u32_f32", t0, t0)
    P.add(I(f"  v_readfirstlane_b32 {q}, {t0}", "rfl", t0.regs(), q.regs()))
    P.salu("s_mul_i32", r, q, d)
    P.salu("s_sub_i32", r, x, r)
    for _ in range(2):   # the estimate is within 2 of the quotient
        P.scmp("s_cmp_lt_i32", r, "0")
        P.salu("s_cselect_b32", S_X[12], "-1", "0", reads_scc=True, writes_scc=False)
        P.salu("s_add_i32", q, q, S_X[12])
        P.salu("s_and_b32", S_X[13], S_X[12], d)
        P.salu("s_add_i32", r, r, S_X[13])
    for _ in range(2):
        P.scmp("s_cmp_ge_i32", r, d)
        P.salu("s_cselect_b32", S_X[12], "-1", "0", reads_scc=True, writes_scc=False)
        P.salu("s_sub_i32", q, q, S_X[12])
        P.salu("s_and_b32", S_X[13], S_X[12], d)
        P.salu("s_sub_i32", r, r, S_X[13])


def rsrc(P, dst, base, idx, bytes_per_idx_sgpr, num_sgpr):
    """dst = raw buffer descriptor over base + idx * bytes_per_idx, num bytes."""
    P.salu("s_mul_i32", S_X[0], idx, bytes_per_idx_sgpr)
    P.salu("s_mul_hi_u32", S_X[1], idx, bytes_per_idx_sgpr)
    P.salu("s_add_u32", dst.sub(0), base.sub(0), S_X[0])
    P.salu("s_addc_u32", dst.sub(1), base.sub(1), S_X[1], reads_scc=True)
    P.salu("s_and_b32", dst.sub(1), dst.sub(1), "0xffff")
    P.salu("s_mov_b32", dst.sub(2), num_sgpr, writes_scc=False)
    P.salu("s_mov_b32", dst.sub(3), "0x00020000", writes_scc=False)


def dma_ops():
    """This wave's LDS-DMA loads of the tile whose key offset (bytes) is
    S_SOFF into the stage at LDS byte S_SB, as a list of emitters (each sets
    M0 and issues one load; S_SBW = S_SB + 1024 * wave).  K chunks wave + 4 jk
    (jk < 4) and chunk 16 (every wave writes the same bytes), V chunks
    wave + 4 jv."""
    ops = []
    for jk in range(5):
        def op(P, jk=jk):
            if jk < 4:
                P.salu("s_add_u32", "m0", S_SBW, str(jk * 4096))
            else:
                P.salu("s_add_u32", "m0", S_SB, str(16 * 1024))
            P.dma(V_DK[jk], S_RSK, S_SOFF)
        ops.append(op)
    for jv in range(5):
        def op(P, jv=jv):
            P.salu("s_add_u32", "m0", S_SBW, str(KTILE + jv * 4096))
            P.dma(V_DV[jv], S_RSV, S_SOFF)
        ops.append(op)
    return ops


def dma_tile(P):
    P.salu("s_add_u32", S_SBW, S_SB, S_WAVE1K)
    for op in dma_ops():
        op(P)


def qk_pair(P, qi, sbuf):
    """MFMAs of K fragment qi (key half kb, channels 16 ks .. 16 ks + 15)
    for both row groups: S^T[rg][kb] (+)= K Q^T."""
    kb, ks = divmod(qi, 8)
    slot = A_KR.sub(4 * (qi % 8), 4)
    for rg in range(2):
        dst = v(sbuf + 32 * rg + 16 * kb, 16)
        P.mfma(dst, slot, A_Q[rg].sub(4 * ks, 4), None if ks == 0 else dst)


def qk_read(P, qi):
    kb, ks = divmod(qi, 8)
    P.ds_read("ds_read_b128", A_KR.sub(4 * (qi % 8), 4), V_KADDR, kb * 32 * KROW + ks * 32)


def pv_pair(P, pi, pbuf):
    """MFMAs of V^T fragment pi (key half kb, keys 16 hf .. 16 hf + 15 of it,
    values 32 db .. 32 db + 31) for both row groups: O^T += V^T P^T."""
    kb, rest = divmod(pi, 8)
    hf, db = divmod(rest, 4)
    slot = A_VR.sub(4 * (pi % 8), 4)
    for rg in range(2):
        o = A_O[rg].sub(16 * db, 16)
        P.mfma(o, slot, v(pbuf + 32 * rg + 16 * kb + 4 * hf, 4), o)


def pv_read(P, pi):
    kb, rest = divmod(pi, 8)
    hf, db = divmod(rest, 4)
    slot = A_VR.sub(4 * (pi % 8), 4)
    off = (kb * 32 + hf * 16) * VROW + db * 64
    P.ds_read("ds_read_b64_tr_b16", slot.sub(0, 2), V_VADDR, off)
    P.ds_read("ds_read_b64_tr_b16", slot.sub(2, 2), V_VADDR, off + 8 * VROW)


def max_ops(sbuf, rg, track_flag):
    """Row maximum of the tile's 32 scores per lane (both key halves), the
    lazy update of the running maximum, alpha and the rescaled sums.  Returns
    a list of emit callbacks (one instruction each)."""
    sv = [v(sbuf + 32 * rg + k) for k in range(32)]
    t, t1, t2, t3 = V_T[8 + 4 * rg], V_T[9 + 4 * rg], V_T[10 + 4 * rg], V_T[11 + 4 * rg]
    acc = [t, t1, t2, t3]
    ops = []
    # four independent chains over 8 scores each (short dependency chains),
    # interleaved, then combined
    for step in range(4):
        for c in range(4):
            b = 8 * c
            if step == 0:
                ops.append(lambda P, c=c, b=b: P.valu("v_max3_f32", acc[c], sv[b], sv[b + 1], sv[b + 2]))
            elif step < 3:
                k = b + 1 + 2 * step
                ops.append(lambda P, c=c, k=k: P.valu("v_max3_f32", acc[c], acc[c], sv[k], sv[k + 1]))
            else:
                ops.append(lambda P, c=c, b=b: P.valu("v_max_f32", acc[c], acc[c], sv[b + 7]))
    ops.append(lambda P: P.valu("v_max3_f32", t, t, t1, t2))
    ops.append(lambda P: P.valu("v_max_f32", t, t, t3))
    ops.append(lambda P: P.valu("v_mov_b32", t1, t))
    ops.append(lambda P: P.add(I(f"  v_permlane32_swap_b32 {t}, {t1}", "perm", regs_of(t, t1), regs_of(t, t1))))
    ops.append(lambda P: P.valu("v_max_f32", t, t, t1))
    ops.append(lambda P: P.valu("v_mul_f32", t, S_C, t))                     # tile max, scaled
    ops.append(lambda P: P.add(I(f"  v_cmp_gt_f32 {S_CMP[rg]}, {t}, {V_MTHR[rg]}", "vcmp",
                                 regs_of(t, V_MTHR[rg]), S_CMP[rg].regs())))
    ops.append(lambda P: P.valu("v_max_f32", t2, V_M[rg], t))                # candidate maximum
    # (compare and select in one op: merged op lists must not split an SCC
    # producer from its consumer)
    def moved(P):
        P.scmp("s_cmp_lg_u64", S_CMP[rg], "0")
        P.salu("s_cselect_b64", S_MV[rg], "-1", "0", reads_scc=True, writes_scc=False)
    ops.append(moved)
    ops.append(lambda P: P.valu("v_mov_b32", V_MOLD[rg], V_M[rg]))
    ops.append(lambda P: P.valu("v_cndmask_b32", V_M[rg], V_M[rg], t2, S_MV[rg]))  # moved (any lane) ? new : old
    ops.append(lambda P: P.salu("s_or_b64", S_FLAG, S_FLAG, S_MV[rg]))
    return ops


def exp_ops(sbuf, rg, kb):
    """p = exp2(s * c - m) for 16 scores, packed in place to bf16 pairs (the
    B operand of the P V product), row sums of the packed values."""
    base = sbuf + 32 * rg + 16 * kb
    sv = [v(base + k) for k in range(16)]
    ops = []
    for k in range(16):
        ops.append(lambda P, k=k: P.valu("v_fma_f32", sv[k], sv[k], S_C, NegR(V_M[rg])))
    for k in range(16):
        op = (lambda P, k=k: P.valu("v_exp_f32", sv[k], sv[k], kind="trans"))
        op.cost = 2.0
        ops.append(op)
    lt = V_LT[rg]
    if OPT["fp32_sums"]:
        if kb == 0:
            ops.append(lambda P: P.valu("v_add_f32", lt[0], sv[0], sv[2]))
            ops.append(lambda P: P.valu("v_add_f32", lt[1], sv[1], sv[3]))
            first = 4
        else:
            first = 0
        for k in range(first, 16):
            ops.append(lambda P, k=k: P.valu("v_add_f32", lt[k % 2], lt[k % 2], sv[k]))
    for i in range(8):
        ops.append(lambda P, i=i: P.valu("v_cvt_pk_bf16_f32", sv[i], sv[2 * i], sv[2 * i + 1]))
    if not OPT["fp32_sums"]:
        for i in range(8):
            a = i % 2            # (the key half kb = 0 initializes both partials)
            if kb == 0 and i < 2:
                ops.append(lambda P, i=i, a=a: P.valu("v_dot2_f32_bf16", lt[a], sv[i], S_ONES, "0"))
            else:
                ops.append(lambda P, i=i, a=a: P.valu("v_dot2_f32_bf16", lt[a], sv[i], S_ONES, lt[a]))
    return ops


def merge_rr(lists):
    """Round-robin merge of op lists (the i-th op of each list, in turn)."""
    out = []
    for i in range(max(len(x) for x in lists)):
        for x in lists:
            if i < len(x):
                out.append(x[i])
    return out


def mask_block(P, sbuf):
    """Per-cell window mask of tile j (key offset S_K0) on score buffer sbuf:
    key j attends row i iff 0 <= i - j <= W - 1.  One 32-bit word per lane
    and key half (bit kc set iff the lane's key kc attends), then one
    bit-field select per score."""
    tb, tlo, thi, tm1, tm2, tk = V_T[0], V_T[1], V_T[2], V_T[3], V_T[4], V_T[5]
    for rg in range(2):
        for kb in range(2):
            P.salu("s_add_u32", S_X[3], S_K0, str(32 * kb))
            P.valu("v_subrev_u32", tb, S_X[3], V_IBASE[rg])                  # base = i - 4 hl - key0
            P.valu("v_subrev_u32", tlo, S_WM1, tb)                            # base - (W - 1)
            P.valu("v_max_i32", tlo, "0", tlo)
            P.valu("v_min_i32", thi, "31", tb)
            P.valu("v_lshlrev_b32_e64", tm1, thi, "2")
            P.valu("v_add_u32", tm1, "-1", tm1)                                # (2 << hi) - 1
            P.valu("v_lshlrev_b32_e64", tm2, tlo, "-1")                        # ~0 << lo
            P.valu("v_and_b32", tm1, tm1, tm2)
            P.add(I(f"  v_cmp_le_i32 vcc, {tlo}, {thi}", "vcmp", regs_of(tlo, thi), VCC))
            P.valu("v_cndmask_b32", tm1, "0", tm1, "vcc")
            for r in range(16):
                kc = (r % 4) + 8 * (r // 4)
                sr = v(sbuf + 32 * rg + 16 * kb + r)
                P.valu("v_bfe_i32", tk, tm1, str(kc), "1")
                P.valu("v_bitop3_b32", sr, sr, S_NINF, tk, extra="bitop3:0xe4")


def rescale_block(P, with_o=True):
    """The running maximum moved (rare): alpha = exp2(m_old - m_new), the
    threshold follows the maximum, the running sum and (once a P V product
    has been accumulated) O are rescaled, after every product of the old
    maximum."""
    tmp = V_T
    for rg in range(2):
        P.valu("v_sub_f32", tmp[0], V_MOLD[rg], V_M[rg])
        P.valu("v_exp_f32", V_ALPHA[rg], tmp[0], kind="trans")
        P.valu("v_add_f32", V_MTHR[rg], str(SLACK), V_M[rg])
        P.valu("v_mul_f32", V_L[rg][0], V_L[rg][0], V_ALPHA[rg])
    if not with_o:
        return
    for rg in range(2):
        for k0 in range(0, 64, 8):
            for k in range(8):
                P.add(I(f"  v_accvgpr_read_b32 {tmp[k]}, {A_O[rg].sub(k0 + k)}", "valu",
                        A_O[rg].sub(k0 + k).regs(), tmp[k].regs()))
            for k in range(8):
                P.valu("v_mul_f32", tmp[k], tmp[k], V_ALPHA[rg])
            for k in range(8):
                P.add(I(f"  v_accvgpr_write_b32 {A_O[rg].sub(k0 + k)}, {tmp[k]}", "valu",
                        tmp[k].regs(), A_O[rg].sub(k0 + k).regs()))


# ---------------------------------------------------------------------------
PREFETCH = 6   # MFMA pairs whose fragments are read ahead


def interleave(P, pairs, valu_ops, extra_ops=()):
    """pairs: list of (read_fn, mfma_fn) in order; valu_ops, extra_ops: lists
    of emitters.  Reads run PREFETCH pairs ahead; VALU work is spread evenly
    between the MFMAs, the extra ops (LDS-DMA loads) one every few MFMAs."""
    n_mfma = 2 * len(pairs)
    for k in range(min(PREFETCH, len(pairs))):
        pairs[k][0](P)
    extra = list(extra_ops)
    every = max(1, (n_mfma - 8) // max(1, len(extra))) if extra else 0
    # issue cost of each op (transcendentals take two VALU slots)
    costs = [getattr(op, "cost", 1.0) for op in valu_ops]
    total = sum(costs)
    vi = 0
    done = 0
    spent = 0.0
    for p_idx, (rd, mf) in enumerate(pairs):
        for half in range(2):
            mf(P, half)
            done += 1
            if extra and done % every == 0:
                extra.pop(0)(P)
            target = total * done / n_mfma
            while vi < len(valu_ops) and spent + 0.5 * costs[vi] <= target:
                valu_ops[vi](P)
                spent += costs[vi]
                vi += 1
            if half == 0 and p_idx + PREFETCH < len(pairs):
                pairs[p_idx + PREFETCH][0](P)
    while vi < len(valu_ops):
        valu_ops[vi](P)
        vi += 1
    while extra:
        extra.pop(0)(P)


def make_pairs(has_qk, has_pv, sbuf_next, pbuf):
    qk = [((lambda P, qi=qi: qk_read(P, qi)),
           (lambda P, half, qi=qi: qk_pair_half(P, qi, sbuf_next, half))) for qi in range(16)]
    pv = [((lambda P, pi=pi: pv_read(P, pi)),
           (lambda P, half, pi=pi: pv_pair_half(P, pi, pbuf, half))) for pi in range(16)]
    if has_qk and has_pv:
        out = []
        for k in range(16):
            out.append(pv[k])
            out.append(qk[k])
        return out
    return qk if has_qk else (pv if has_pv else [])


def qk_pair_half(P, qi, sbuf, rg):
    kb, ks = divmod(qi, 8)
    slot = A_KR.sub(4 * (qi % 8), 4)
    dst = v(sbuf + 32 * rg + 16 * kb, 16)
    P.mfma(dst, slot, A_Q[rg].sub(4 * ks, 4), None if ks == 0 else dst)


def pv_pair_half(P, pi, pbuf, rg):
    kb, rest = divmod(pi, 8)
    hf, db = divmod(rest, 4)
    slot = A_VR.sub(4 * (pi % 8), 4)
    o = A_O[rg].sub(16 * db, 16)
    P.mfma(o, slot, v(pbuf + 32 * rg + 16 * kb + 4 * hf, 4), o)


def stage_base(P, dst, jsgpr, add):
    """dst = ((j + add) & 3) * STAGE"""
    P.salu("s_add_u32", dst, jsgpr, str(add & 0xffffffff) if add >= 0 else str(add))
    P.salu("s_and_b32", dst, dst, "3")
    P.salu("s_mul_i32", dst, dst, str(STAGE))


def iteration(P, phase, has_qk, has_pv, first):
    """One tile j (S_J) of the pipeline; buffers by phase = j % 3."""
    sb_cur, sb_next, sb_prev = S_BUF[phase], S_BUF[(phase + 1) % 3], S_BUF[(phase + 2) % 3]
    P.comment(f"iteration phase {phase} qk={has_qk} pv={has_pv}")
    P.waitcnt(vm=0)
    P.barrier()
    if has_pv:
        settle_previous(P)
    # DMA of tile j + 2 into stage (j + 2) & 3; past the band (j + 2 >= T)
    # the offset is N rows, out of the descriptor's range: the loads read
    # zeros without touching memory, into a stage nothing reads
    if has_qk:
        P.salu("s_add_u32", S_X[4], S_J, "2")
        P.salu("s_add_u32", S_X[5], S_TLO, S_X[4])
        P.salu("s_lshl_b32", S_X[5], S_X[5], "14")
        P.scmp("s_cmp_lt_u32", S_X[4], S_T)
        P.salu("s_cselect_b32", S_SOFF, S_X[5], S_NB, reads_scc=True, writes_scc=False)
        stage_base(P, S_SB, S_J, 2)
        P.salu("s_add_u32", S_SBW, S_SB, S_WAVE1K)
    if has_qk:
        stage_base(P, S_SBK, S_J, 1)
        P.valu("v_add_u32", V_KADDR, S_SBK, V_KLANE)
    if has_pv:
        stage_base(P, S_SBV, S_J, -1 + 4)
        P.valu("v_add_u32", V_VADDR, S_SBV, V_VLANE)
    # per-cell mask of tile j unless every cell attends
    P.salu("s_add_u32", S_X[6], S_TLO, S_J)
    P.salu("s_lshl_b32", S_K0, S_X[6], "6")                 # key0 of tile j
    P.salu("s_add_u32", S_X[7], S_K0, "63")
    P.salu("s_add_u32", S_X[8], S_K0, S_W)                  # key0 + W >= r0 + 64 ?
    P.salu("s_add_u32", S_X[9], S_R0, "64")
    P.scmp("s_cmp_le_u32", S_X[7], S_R0)
    P.salu("s_cselect_b32", S_X[10], "1", "0", reads_scc=True, writes_scc=False)
    P.scmp("s_cmp_ge_u32", S_X[8], S_X[9])
    P.salu("s_cselect_b32", S_X[11], "1", "0", reads_scc=True, writes_scc=False)
    P.salu("s_and_b32", S_X[10], S_X[10], S_X[11])
    P.scmp("s_cmp_eq_u32", S_X[10], "1")
    skip = P.new_label("full")
    P.branch("s_cbranch_scc1", skip)
    mask_block(P, sb_cur)
    P.label(skip)
    dump(P, f"masked{phase}{int(has_qk)}{int(has_pv)}", [v(sb_cur, 64)])
    P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)
    valu = merge_rr([max_ops(sb_cur, 0, has_pv), max_ops(sb_cur, 1, has_pv)])
    # (blocks in the order (rg, kb) = (0,0), (1,0), (0,1), (1,1): a key half
    # 1 op accumulates into the partial its key half 0 op initialized two
    # ops earlier)
    valu += merge_rr([exp_ops(sb_cur, rg, kb) for kb in range(2) for rg in range(2)])
    pairs = make_pairs(has_qk, has_pv, sb_next, sb_prev)
    interleave(P, pairs, valu, dma_ops() if has_qk else [])
    dump(P, f"soft{phase}{int(has_qk)}{int(has_pv)}", [v(sb_cur, 64), V_M[0], V_M[1], V_L[0][0], V_L[0][1],
                                                        V_L[1][0], V_L[1][1], V_ALPHA[0], V_ALPHA[1]])
    if not has_pv:
        # first tile: nothing accumulated yet (O = 0, l = 0), so the moved
        # maximum only moves the threshold; this tile's sums are merged at
        # the start of the next step
        for rg in range(2):
            P.valu("v_add_f32", V_MTHR[rg], str(SLACK), V_M[rg])
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)


def settle_previous(P):
    """Between the P V products of the previous tile and of this one: if the
    previous tile moved the running maximum, rescale l and O (rare), then add
    the previous tile's row sums to l."""
    skip = P.new_label("norescale")
    P.scmp("s_cmp_eq_u64", S_FLAG, "0")
    P.branch("s_cbranch_scc1", skip)
    rescale_block(P, with_o=True)
    P.label(skip)
    for rg in range(2):
        P.valu("v_add_f32", V_L[rg][0], V_L[rg][0], V_LT[rg][0])
        P.valu("v_add_f32", V_L[rg][0], V_L[rg][0], V_LT[rg][1])


def epilogue(P, phase):
    """O += V(T-1)^T P(T-1), then O / l -> bf16 rows, and the log-sum-exp."""
    pbuf = S_BUF[phase]
    P.waitcnt(vm=0)
    P.barrier()
    settle_previous(P)
    stage_base(P, S_SBV, S_J, 0)
    P.valu("v_add_u32", V_VADDR, S_SBV, V_VLANE)
    pairs = make_pairs(False, True, None, pbuf)
    interleave(P, pairs, [])
    dump(P, f"O{phase}", [A_O[0], A_O[1]])
    t = V_T
    for rg in range(2):
        l, l2, inv = t[0], t[1], t[2 + rg]
        P.valu("v_add_f32", l, V_L[rg][0], V_L[rg][1])
        P.valu("v_mov_b32", l2, l)
        P.add(I(f"  v_permlane32_swap_b32 {l}, {l2}", "perm", regs_of(l, l2), regs_of(l, l2)))
        P.valu("v_add_f32", l, l, l2)                       # the row's sum over both lane halves
        P.valu("v_rcp_f32", inv, l, kind="trans")
        # log-sum-exp, natural log: (m + log2 l) * ln 2
        skip = P.new_label("nolse")
        P.scmp("s_cmp_eq_u64", S_LSE, "0")
        P.branch("s_cbranch_scc1", skip)
        P.valu("v_log_f32", l2, l, kind="trans")
        P.valu("v_add_f32", l2, V_M[rg], l2)
        P.valu("v_mul_f32", l2, "0x3f317218", l2)
        P.buf_store("buffer_store_dword", l2, V_LOFF[rg], S_RSL)
        P.label(skip)
    # O / l -> bf16, staged through LDS so the global stores are whole rows
    # (16 lanes x 16 bytes per 256-byte row) instead of 8-byte pieces of 32
    # rows.  Each wave uses its own 64 x 272-byte region in the two stages
    # that do not hold the last V tile (the only one other waves may still
    # read): stages 0-1 if that tile is in stage 2 or 3, else stages 2-3.
    P.salu("s_and_b32", S_X[0], S_J, "3")
    P.scmp("s_cmp_ge_u32", S_X[0], "2")
    P.salu("s_cselect_b32", S_X[1], "0", str(2 * STAGE), reads_scc=True, writes_scc=False)
    P.salu("s_mul_i32", S_X[2], S_WAVE, str(64 * KROW))
    P.salu("s_add_u32", S_X[1], S_X[1], S_X[2])                    # this wave's region
    P.valu("v_add_u32", V_OW, S_X[1], V_OWL)
    P.valu("v_add_u32", V_ORD, S_X[1], V_ORDL)
    for rg in range(2):
        inv = t[2 + rg]
        for db in range(4):
            for r4 in range(4):
                x = [t[4 + k] for k in range(4)]
                for k in range(4):
                    P.add(I(f"  v_accvgpr_read_b32 {x[k]}, {A_O[rg].sub(16 * db + 4 * r4 + k)}", "valu",
                            A_O[rg].sub(16 * db + 4 * r4 + k).regs(), x[k].regs()))
                for k in range(4):
                    P.valu("v_mul_f32", x[k], x[k], inv)
                pk0, pk1 = t[8 + 2 * (r4 % 2)], t[9 + 2 * (r4 % 2)]
                P.valu("v_cvt_pk_bf16_f32", pk0, x[0], x[1])
                P.valu("v_cvt_pk_bf16_f32", pk1, x[2], x[3])
                # row 32 rg + col, values 32 db + 8 r4 + 4 hl .. +3
                P.add(I(f"  ds_write_b64 {V_OW}, {v(pk0.i, 2)} offset:{rg * 32 * KROW + db * 64 + r4 * 16}", "lds",
                        regs_of(V_OW, v(pk0.i, 2)), EMPTY))
    ob = S_BUF[(phase + 1) % 3]                                     # free score buffer

    def rd(kk):
        # rows 4 kk + lane / 16, bytes 16 (lane % 16) .. +15 of each
        P.ds_read("ds_read_b128", v(ob + 4 * kk, 4), V_ORD, kk * 4 * KROW)
    for kk in range(8):
        rd(kk)
    for kk in range(16):
        P.salu("s_mov_b32", S_X[3 + (kk % 4)], str(kk * 1024), writes_scc=False)
        P.add(I(f"  buffer_store_dwordx4 {v(ob + 4 * kk, 4)}, {V_OST}, {S_RSO}, {S_X[3 + (kk % 4)]} offen",
                "vstore", regs_of(v(ob + 4 * kk, 4), V_OST, S_RSO, S_X[3 + (kk % 4)]), EMPTY))
        if kk + 8 < 16:
            rd(kk + 8)
    P.add(I("  s_endpgm", "branch"))


def prologue(P):
    P.smem("s_load_dwordx16", s(4, 16), S_KARG, "0x0")
    P.smem("s_load_dwordx4", s(20, 4), S_KARG, "0x40")
    P.valu("v_and_b32", V_TID, "0x3ff", v(0))
    P.valu("v_lshrrev_b32", V_T[0], "6", V_TID)
    P.add(I(f"  v_readfirstlane_b32 {S_WAVE}, {V_T[0]}", "rfl", V_T[0].regs(), S_WAVE.regs()))
    P.valu("v_and_b32", V_LANE, "63", V_TID)
    P.valu("v_and_b32", V_COL, "31", V_LANE)
    P.valu("v_lshrrev_b32", V_HL, "5", V_LANE)
    if DEBUG["on"]:
        P.smem("s_load_dwordx2", s(92, 2), S_KARG, "0x50")
        P.smem("s_load_dword", s(94), S_KARG, "0x58")
    P.waitcnt(lgkm=0)
    if DEBUG["on"]:
        P.salu("s_and_b32", S_DBG.sub(1), S_DBG.sub(1), "0xffff")
        P.salu("s_mov_b32", S_DBG.sub(3), "0x00020000", writes_scc=False)
        P.salu("s_lshl_b32", S_DBGW, S_TOTAL, "2")
        P.salu("s_lshl_b32", S_DBGG, S_WG, "2")
        P.salu("s_add_u32", S_DBGG, S_DBGG, S_WAVE)
        P.valu("v_lshlrev_b32", V_DBGL, "2", V_LANE)
    # workgroup -> logical id: consecutive ids go to the 8 XCDs in turn; each
    # XCD gets a contiguous run of logical ids
    P.salu("s_and_b32", S_X[0], S_TOTAL, "7")
    P.salu("s_and_b32", S_X[1], S_WG, "7")
    P.salu("s_lshr_b32", S_X[2], S_TOTAL, "3")
    P.salu("s_mul_i32", S_X[1], S_X[1], S_X[2])
    P.salu("s_lshr_b32", S_X[3], S_WG, "3")
    P.salu("s_add_u32", S_X[1], S_X[1], S_X[3])
    P.scmp("s_cmp_eq_u32", S_X[0], "0")
    P.salu("s_cselect_b32", S_LID, S_X[1], S_WG, reads_scc=True, writes_scc=False)
    # lid -> (head block, row block, batch * kv head).  Row blocks in
    # ascending order: the first blocks of a head have short bands, so the
    # first workgroups on the CUs end at different times and the later ones'
    # loads and stores do not all hit memory at once (measured 5% faster
    # than longest first)
    udiv(P, S_LID, S_NHB, S_X[4], S_HB, V_T[1], V_T[2])        # S_X[4] = rest
    udiv(P, S_X[4], S_NRB, S_BG, S_RB, V_T[1], V_T[2])         # row block
    P.salu("s_lshl_b32", S_R0, S_RB, "6")
    done = ".Ldone"
    P.scmp("s_cmp_ge_u32", S_R0, S_N)
    P.branch("s_cbranch_scc1", done)
    # band of rows r0 .. r0+63: key tiles t_lo .. t_hi
    P.salu("s_sub_i32", S_X[0], S_R0, S_W)
    P.salu("s_add_i32", S_X[0], S_X[0], "1")
    P.salu("s_max_i32", S_X[0], S_X[0], "0")
    P.salu("s_lshr_b32", S_TLO, S_X[0], "6")
    P.salu("s_add_u32", S_X[1], S_R0, "63")
    P.salu("s_sub_u32", S_X[2], S_N, "1")
    P.salu("s_min_u32", S_X[1], S_X[1], S_X[2])
    P.salu("s_lshr_b32", S_X[1], S_X[1], "6")
    P.salu("s_sub_u32", S_T, S_X[1], S_TLO)
    P.salu("s_add_u32", S_T, S_T, "1")
    # descriptors
    P.salu("s_lshl_b32", S_X[6], S_N, "8")                     # bytes per head (N rows of 256 B)
    rsrc(P, S_RSK, S_K, S_BG, S_X[6], S_X[6])
    rsrc(P, S_RSV, S_V, S_BG, S_X[6], S_X[6])
    P.salu("s_mul_i32", S_X[7], S_BG, S_G)                     # query head = bg * G + 4 hb + wave
    P.salu("s_lshl_b32", S_X[8], S_HB, "2")
    P.salu("s_add_u32", S_X[7], S_X[7], S_X[8])
    P.salu("s_add_u32", S_X[7], S_X[7], S_WAVE)
    rsrc(P, S_RSQ, S_Q, S_X[7], S_X[6], S_X[6])
    rsrc(P, S_RSO, S_OUT, S_X[7], S_X[6], S_X[6])
    P.salu("s_lshl_b32", S_X[9], S_N, "2")
    rsrc(P, S_RSL, S_LSE, S_X[7], S_X[9], S_X[9])
    P.salu("s_lshl_b32", S_WAVE1K, S_WAVE, "10")
    P.salu("s_lshl_b32", S_NB, S_N, "8")
    P.salu("s_sub_u32", S_WM1, S_W, "1")
    P.salu("s_mov_b32", S_NINF, "0xff800000", writes_scc=False)
    P.salu("s_mov_b32", S_ONES, "0x3f803f80", writes_scc=False)
    # per-lane addressing
    t = V_T
    P.valu("v_mul_u32_u24", V_KLANE, str(KROW), V_COL)
    P.valu("v_lshlrev_b32", t[0], "4", V_HL)
    P.valu("v_add_u32", V_KLANE, V_KLANE, t[0])
    P.valu("v_lshrrev_b32", t[0], "4", V_LANE)                 # grp
    P.valu("v_and_b32", t[1], "15", V_LANE)                    # sl
    P.valu("v_lshrrev_b32", t[2], "1", t[0])                   # grp >> 1
    P.valu("v_lshlrev_b32", t[2], "2", t[2])
    P.valu("v_lshrrev_b32", t[3], "2", t[1])                   # sl >> 2
    P.valu("v_add_u32", t[2], t[2], t[3])
    P.valu("v_mul_u32_u24", t[2], str(VROW), t[2])
    P.valu("v_and_b32", t[3], "1", t[0])
    P.valu("v_lshlrev_b32", t[3], "5", t[3])                   # 16 * (grp & 1) * 2
    P.valu("v_and_b32", t[4], "3", t[1])
    P.valu("v_lshlrev_b32", t[4], "3", t[4])                   # 4 * (sl & 3) * 2
    P.valu("v_add_u32", t[2], t[2], t[3])
    P.valu("v_add_u32", t[2], t[2], t[4])
    P.valu("v_add_u32", V_VLANE, str(KTILE), t[2])
    for rg in range(2):
        P.valu("v_add_u32", t[5], S_R0, V_COL)
        if rg:
            P.valu("v_add_u32", t[5], "32", t[5])              # row
        P.valu("v_lshlrev_b32", t[6], "8", t[5])               # row * 256
        P.valu("v_lshlrev_b32", t[7], "4", V_HL)
        P.valu("v_add_u32", V_QOFF[rg], t[6], t[7])
        P.valu("v_lshlrev_b32", t[7], "3", V_HL)
        P.valu("v_add_u32", V_OOFF[rg], t[6], t[7])
        P.valu("v_lshlrev_b32", V_LOFF[rg], "2", t[5])
        P.valu("v_lshlrev_b32", t[7], "2", V_HL)
        P.valu("v_sub_u32", V_IBASE[rg], t[5], t[7])
    # epilogue: LDS write base (row col, values 4 hl: col * 272 + 8 hl), LDS
    # read base (row lane / 16, bytes 16 (lane % 16)), global store offset
    P.valu("v_mul_u32_u24", V_OWL, str(KROW), V_COL)
    P.valu("v_lshlrev_b32", t[0], "3", V_HL)
    P.valu("v_add_u32", V_OWL, V_OWL, t[0])
    P.valu("v_lshrrev_b32", t[0], "4", V_LANE)
    P.valu("v_and_b32", t[1], "15", V_LANE)
    P.valu("v_lshlrev_b32", t[1], "4", t[1])
    P.valu("v_mul_u32_u24", V_ORDL, str(KROW), t[0])
    P.valu("v_add_u32", V_ORDL, V_ORDL, t[1])
    P.valu("v_add_u32", t[0], S_R0, t[0])
    P.valu("v_lshlrev_b32", t[0], "8", t[0])
    P.valu("v_add_u32", V_OST, t[0], t[1])
    # DMA lane offsets: K chunk wave + 4 jk (jk < 4) or 16, V chunk wave + 4 jv
    P.valu("v_lshlrev_b32", t[8], "4", V_LANE)                 # 16 lane
    P.valu("v_mov_b32", t[9], S_WAVE1K)
    for jk in range(5):
        if jk < 4:
            P.valu("v_add_u32", t[10], t[9], t[8])
            P.valu("v_add_u32", t[10], str(jk * 4096), t[10])
        else:
            P.valu("v_add_u32", t[10], str(16 * 1024), t[8])
        _chunk_src(P, V_DK[jk], t[10], M272, KROW, t)
    for jv in range(5):
        P.valu("v_add_u32", t[10], t[9], t[8])
        P.valu("v_add_u32", t[10], str(jv * 4096), t[10])
        _chunk_src(P, V_DV[jv], t[10], M320, VROW, t)
    # softmax state
    for rg in range(2):
        P.valu("v_mov_b32", V_M[rg], "0xf149f2ca")             # -1e30
        P.valu("v_mov_b32", V_MTHR[rg], "0xf149f2ca")
        for k in range(2):
            P.valu("v_mov_b32", V_L[rg][k], "0")
        for k in range(64):
            P.add(I(f"  v_accvgpr_write_b32 {A_O[rg].sub(k)}, 0", "valu", EMPTY, A_O[rg].sub(k).regs()))
    # Q fragments
    for rg in range(2):
        for ks in range(8):
            P.buf_load(A_Q[rg].sub(4 * ks, 4), V_QOFF[rg], S_RSQ, "0", 32 * ks)
    # stage tiles 0 and 1 (tile 1 also when the band has one tile: its rows
    # are read, or are past N and read as zeros, and never used)
    P.salu("s_lshl_b32", S_SOFF, S_TLO, "14")
    P.salu("s_mov_b32", S_SB, "0", writes_scc=False)
    dma_tile(P)
    P.salu("s_add_u32", S_SOFF, S_SOFF, str(1 << 14))
    P.salu("s_mov_b32", S_SB, str(STAGE), writes_scc=False)
    dma_tile(P)
    P.waitcnt(vm=10)
    P.barrier()
    # S(0) = K(0) Q^T
    P.salu("s_mov_b32", S_J, "0", writes_scc=False)
    P.valu("v_add_u32", V_KADDR, "0", V_KLANE)
    dump_lds(P, "lds0", STAGE)
    dump(P, "q", [A_Q[0], A_Q[1]])
    pairs = make_pairs(True, False, S_BUF[0], None)
    interleave(P, pairs, [])
    dump(P, "s0", [v(S_BUF[0], 64)])


def _chunk_src(P, dst, pos, magic, rowb, t):
    """dst = source byte offset of tile byte `pos`: row * 256 + column, the
    column of padding bytes replaced by 0."""
    P.salu("s_mov_b32", S_X[11], str(magic), writes_scc=False)
    P.valu("v_mul_lo_u32", t[11], pos, S_X[11])
    P.valu("v_lshrrev_b32", t[11], "24", t[11])                # row
    P.valu("v_mul_u32_u24", t[12], str(rowb), t[11])
    P.valu("v_sub_u32", t[12], pos, t[12])                     # column byte
    P.add(I(f"  v_cmp_gt_u32 vcc, {2 * D}, {t[12]}", "vcmp", t[12].regs(), VCC))
    P.valu("v_cndmask_b32", t[12], "0", t[12], "vcc")
    P.valu("v_lshlrev_b32", t[11], "8", t[11])
    P.valu("v_add_u32", dst, t[11], t[12])


def kernel_text():
    P = Prog()
    prologue(P)
    # T == 1: softmax of S(0) only
    P.scmp("s_cmp_le_u32", S_T, "1")
    P.branch("s_cbranch_scc1", ".Lsingle")
    iteration(P, 0, True, False, True)                         # j = 0
    P.salu("s_mov_b32", S_J, "1", writes_scc=False)
    P.salu("s_add_u32", S_X[0], S_J, "1")
    P.scmp("s_cmp_ge_u32", S_X[0], S_T)
    P.branch("s_cbranch_scc1", ".Llast1")
    P.label(".Lmid1")
    for ph in (1, 2, 0):
        iteration(P, ph, True, True, False)
        P.salu("s_add_u32", S_J, S_J, "1")
        P.salu("s_add_u32", S_X[0], S_J, "1")
        P.scmp("s_cmp_ge_u32", S_X[0], S_T)                   # j == T - 1 (>=: a bound)
        P.branch("s_cbranch_scc1", f".Llast{(ph + 1) % 3}")
    P.branch("s_branch", ".Lmid1")
    for ph in range(3):
        P.label(f".Llast{ph}")
        iteration(P, ph, False, True, False)
        epilogue(P, ph)
    P.label(".Lsingle")
    iteration(P, 0, False, False, True)
    epilogue(P, 0)
    P.label(done_label())
    P.add(I("  s_endpgm", "branch"))
    body = resolve(P.ins)
    lines = [x.text for x in body]
    return "\n".join(lines)


def done_label():
    return ".Ldone"


def render():
    body = kernel_text()
    karg = KARG_BYTES + (16 if DEBUG["on"] else 0)
    head = f""".amdgcn_target "amdgcn-amd-amdhsa--gfx950"
.text
.globl {NAME}
.p2align 8
.type {NAME},@function
{NAME}:
"""
    tail = f"""
.Lfunc_end:
.size {NAME}, .Lfunc_end-{NAME}

.rodata
.p2align 6
.amdhsa_kernel {NAME}
  .amdhsa_group_segment_fixed_size {LDS_BYTES}
  .amdhsa_private_segment_fixed_size 0
  .amdhsa_kernarg_size {karg}
  .amdhsa_user_sgpr_count 2
  .amdhsa_user_sgpr_kernarg_segment_ptr 1
  .amdhsa_system_sgpr_workgroup_id_x 1
  .amdhsa_system_vgpr_workitem_id 0
  .amdhsa_next_free_vgpr 512
  .amdhsa_next_free_sgpr 96
  .amdhsa_accum_offset 256
  .amdhsa_reserve_vcc 1
  .amdhsa_float_denorm_mode_32 3
  .amdhsa_float_denorm_mode_16_64 3
  .amdhsa_dx10_clamp 1
  .amdhsa_ieee_mode 1
.end_amdhsa_kernel

.amdgpu_metadata
---
amdhsa.version: [ 1, 2 ]
amdhsa.kernels:
  - .name: {NAME}
    .symbol: {NAME}.kd
    .kernarg_segment_size: {karg}
    .group_segment_fixed_size: {LDS_BYTES}
    .private_segment_fixed_size: 0
    .kernarg_segment_align: 8
    .wavefront_size: 64
    .sgpr_count: 96
    .vgpr_count: 512
    .agpr_count: 256
    .max_flat_workgroup_size: 256
    .args:
      - {{ .offset: 0, .size: {karg}, .value_kind: by_value }}
...
.end_amdgpu_metadata
"""
    return head + body + tail


def main(out_path):
    text = render()
    with open(out_path, "w") as f:
        f.write(text)
    return out_path


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.getcwd(), NAME + ".s"))
