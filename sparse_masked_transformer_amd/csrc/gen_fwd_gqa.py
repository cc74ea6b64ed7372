"""Generator of the gfx950 assembly kernel for grouped-query sliding-window
attention forward, bf16, head size 128 (build step: writes a .s file).

The operation is the masked attention of Learn: Sparse & Sliding-Window
Attention, §3 equation, A = softmax(Q K^T * scale + log M) V, with M the
sliding window j in [i - W + 1, i] (the swa_mask of "Attention Variants
Compared"), computed with the tiled online softmax ("Flash style softmax",
same page): running maximum, running sum and running weighted sum per query
row while the key tiles of the window stream through LDS.

Work decomposition
  Item = the 4 query heads h0 .. h0+3 of one key/value head (grouped-query
  attention) on the same 64 query rows; its 8 waves: wave w takes head
  h0 + (w & 3) and rows 32 (w >> 2) .. +31 of the block, so the K and V
  tiles staged in LDS serve all four heads and every wave needs the same key
  tiles (the band of the 64 rows).  One workgroup per CU (LDS holds four
  64-key stages), two waves per SIMD: while one wave waits on a dependency
  or an LDS read, the other issues.
  Persistent grid: workgroup g takes items g, g + grid, g + 2 grid, ...
  (grid a multiple of 8, so all of them run on one XCD, whose items are a
  contiguous run of row blocks of one head: neighbouring bands share K and
  V tiles in that XCD's L2).  In the last step of an item the workgroup
  already loads the next item's Q fragments and first two tiles, into the
  two stages the current item no longer reads; the output of the current
  item is staged through the stage of its last-but-one tile.

Registers (256 per lane: 128 VGPRs + 128 AGPRs, two waves per SIMD)
  AGPR  a[0:63]     O^T accumulators, 4 blocks of 32 values
        a[64:95]    Q^T fragments (B operand of S^T = K Q^T), 8
        a[96:111]   K fragment ring (A operand), 4 slots
        a[112:127]  V^T fragment ring (A operand of O^T += V^T P^T), 4 slots
  VGPR  v[0:63]     two score buffers of 32 values: the tile whose scores
                    are being computed and the tile whose softmax is running
        v[64:79]    the probabilities that feed the P V product, bf16 pairs
        v[80:126]   addressing, softmax state, temporaries

Software pipeline (one iteration per 64-key tile j)
  matrix cores: O += V(j-1)^T P(j-1) (16 MFMAs: four, then two per QK MFMA)
                and S(j+1) = K(j+1) Q^T (16 MFMAs, the last ten after the
                P V product)
  vector ALU:   (first two tiles of an item, and its last: row maxima of
                S(j)), then p = exp2(s * c - m), the bf16
                packing of P(j) into the P buffer (once the P V product has
                read it) and the row sums, spread evenly between the MFMAs
  LDS:          the fragments of both products, three ahead of their MFMA;
                the first three V fragments of the next step are read before
                the next barrier (their tile is already in LDS)
  DMA:          tile j+2 into the fourth stage (buffer_load ... lds), and
                the scalar set-up of the next step, spread between the MFMAs
The running maximum moves only when a tile's maximum exceeds it by more than
SLACK = 32 (log2 units); O is then rescaled at the start of the next
iteration, after the products of the old maximum have been accumulated.
Every row of an item attends a key of its first two tiles, so from the
third tile on the step takes no row maximum: it checks instead that no
row's sum of p exceeds 2^SLACK and, only if one does, computes the tile
again with its maximum (outputs are those of the step with maxima).

Variants (build options, the plain kernel's code unchanged by them) for
the dilated window and the global tokens of Learn: Sparse & Sliding-Window
Attention, §3b
  dilated (DIL): with dilation r, each residue class of the rows mod r is
  walked as a plain window over every r-th row (row pitch 256 r bytes);
  global tokens (GLB): the tiles of the global columns left of an item's
  band are walked ahead of it and the global columns ORed into the cell
  mask.

Hazards: every instruction records the registers it reads and writes; a
final pass inserts the wait states gfx950 requires between producers and
consumers (MFMA results, VALU -> MFMA operands, transcendental results,
SGPRs written by the VALU, M0 before LDS-DMA) and the s_waitcnt each load's
consumer needs.
"""
import os
import struct
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
# the running maximum m moves only when a tile's maximum exceeds it by more
# than SLACK (log2 units), so every p = exp2(s c - m) is at most 2^SLACK:
# bf16 P keeps its relative precision at any magnitude, and the fp32 sums
# of p and of p v stay finite for |v| up to 2^(128 - SLACK - 10) over 2^10
# keys.  With 32 a move is rare even on sharply peaked rows.
SLACK = 32.0
OROW = 144                    # LDS row of the output staging (half a row of values + 16)
EPI_STORES = 8                # output stores of an item's epilogue (the log-sum-exp store aside)
assert 8 * 32 * OROW <= STAGE
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

    def buf_load(self, dst, voff, rsrc, soff, off=0, track=True):
        """track=False: no automatic wait before the destination's readers
        (the caller places an explicit s_waitcnt; the load may then stay in
        flight across labels and branches)."""
        o = f" offset:{off}" if off else ""
        self.add(I(f"  buffer_load_dwordx4 {dst}, {voff}, {rsrc}, {soff} offen{o}", "vmem",
                   regs_of(voff, rsrc, soff if isinstance(soff, R) else None), dst.regs(), vm_load=True,
                   dests=dst.regs() if track else EMPTY))

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
            if x.dests & p.srcab or x.writes & p.srcab:
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


def check_scc(ins):
    """Every reader of SCC reads the flag its producer of that kind set: a
    select or a conditional branch the last compare, an add with carry the
    last add (no other SCC writer between them, no label or branch)."""
    last = None
    for x in ins:
        if x.kind in ("label", "branch") and not (x.kind == "branch" and "scc" in x.text):
            last = None
            continue
        op = x.text.split()[0] if x.text.strip() else ""
        if SCC <= x.reads:
            want = ("s_add_u32", "s_addc_u32") if op == "s_addc_u32" else ("s_cmp", "s_bitcmp")
            if last is None or not last.startswith(want):
                raise ValueError(f"{x.text.strip()} reads SCC set by {last}")
        if SCC <= x.writes:
            last = op


def resolve(ins):
    """Insert s_nop for hazards and s_waitcnt for load consumers."""
    check_scc(ins)
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
# register map: 256 per lane (VGPRs v0..v127, AGPRs a0..a127), two waves per
# SIMD
NW = 8                               # waves per workgroup
S_BUF = [0, 32]                      # two score buffers of 32 VGPRs: tile j, tile j + 1
P_BUF = 64                           # probabilities of one tile, bf16 pairs: 16 VGPRs
V_TID, V_KLANE, V_VLANE, V_KADDR, V_VADDR = v(80), v(81), v(82), v(83), v(84)
V_DK = [v(85), v(86)]                # LDS-DMA source offsets per lane: K chunks wave, wave + 8
V_DV = [v(88), v(89)]                # V chunks wave, wave + 8
V_DX = v(87)                         # the wave's fifth chunk (V 16 + wave, or K 16)
V_M = v(91)                          # running maximum (scaled, log2 units)
V_MTHR = v(92)                       # running maximum + slack
V_ALPHA = v(93)
V_MOLD = v(94)                       # running maximum before this tile
V_L = [v(95), v(96)]                 # running sum, two partials
V_LT = [v(97), v(98)]                # this tile's row sums, two partials
V_IBASE = v(99)                      # row - 4 * (lane / 32), for the per-cell mask
V_LOFF, V_QOFF = v(100), v(101)
V_COL, V_HL = v(102), v(103)
V_T = [v(104 + i) for i in range(16)]  # even start: pairs of them are 64-bit tuples
V_OWL, V_ORDL, V_OST, V_OW, V_ORD = v(120), v(121), v(122), v(123), v(124)
V_LANE = v(125)
V_QLANE = v(127)                     # (lane % 32) * 256 + 16 (lane / 32): Q load offset within the rows

A_O = a(0, 64)                       # O^T: block db at 16 db
A_Q = a(64, 32)                      # Q^T fragments: ks at 4 ks
A_KR = a(96, 16)                     # K fragment ring: 4 slots
A_VR = a(112, 16)                    # V^T fragment ring: 4 slots
RING = 4

# SGPRs
S_KARG = s(0, 2)
S_WG = s(2)
S_Q, S_K, S_V, S_OUT, S_LSE = s(4, 2), s(6, 2), s(8, 2), s(10, 2), s(12, 2)
S_N, S_W, S_G, S_NHB, S_NRB, S_C = s(14), s(15), s(16), s(17), s(18), s(19)
S_TOTAL, S_STRIDE, S_VID = s(20), s(21), s(22)   # row-block items, items per pass (grid size), item
S_BASE = s(3)                        # stage of the next item's first tile
S_WH, S_WR, S_R0W = s(23), s(34), s(35)   # wave & 3 (head), wave >> 2 (row half), its first row
S_WAVE, S_LID, S_HB, S_RB, S_BG, S_R0, S_TLO, S_T, S_J = (s(24), s(25), s(26), s(27), s(28), s(29),
                                                          s(30), s(31), s(32))
S_RSK, S_RSV, S_RSQ, S_RSO, S_RSL = s(36, 4), s(40, 4), s(44, 4), s(48, 4), s(52, 4)
S_WAVE1K, S_SOFF, S_SB = s(56), s(57), s(58)
S_R0W32 = s(59)                      # this wave's first row + 32
S_K0P = [s(61), s(76)]               # key0 of the tile, by iteration phase
S_FULL = [s(77), s(60)]              # 1 if every cell of the tile attends this wave's rows, by phase
S_WM1, S_NINF, S_ONES = s(63), s(64), s(65)
S_SBW = s(62)                        # DMA stage base + 1024 * wave
S_XOFF = s(72)                       # LDS offset of the wave's fifth chunk within a stage
S_HALF1 = s(73)                      # 1 if key half 1 of the item's last tile lies past the wave's rows
S_RSE = s(96, 4)                     # its descriptor: V on waves 0-3, K on waves 4-7
S_NB = s(33)                         # N * 256: bytes per head, first offset past the rows
S_FLAG = s(68, 2)
S_CMP = s(70, 2)
S_MV = s(74, 2)
S_X = [s(78 + i) for i in range(14)]  # scalar temporaries s78..s91


# ---------------------------------------------------------------------------
# build options.  Row sums: over the bf16-rounded probabilities (v_dot2), the
# values the P V product accumulates, so the weights of a row sum to exactly
# one after the division (a near one-hot row gives its value row exactly);
# fp32_sums sums the unrounded values instead (the weights then sum to one
# only within 2^-8, which on peaky rows costs up to ~0.02 of output error)
OPT = {"fp32_sums": False}

# the dilated variant (dilation r > 1, window only): the rows i with
# i % r == c form residue class c, on which the dilated window is a plain
# window of W keys; the kernel runs each class as its own sequence of
# N_c = ceil((N - c) / r) rows, reading every r-th row (a row pitch of
# 256 r bytes from byte 256 c).  Off in the plain kernel, whose code is
# unchanged by the option.
DIL = {"on": False}
S_DIL, S_PITCH, S_TILEB, S_CLS, S_NC, S_NCLS = s(66), s(67), s(92), s(93), s(94), s(95)

# the global-token variant (n_global G > 0, dilation 1, window only): keys
# j < G attend every row i >= j, and rows i < G attend every key j <= i.
# An item whose band starts past the global columns walks their tiles
# first (the prefix tiles 0 .. NP-1), then its band; an item holding
# global rows starts its band at key 0.  Step s of an item is tile s while
# s < NP, else tile t_lo + s - NP.  Off in the plain kernel.
GLB = {"on": False}
S_NGLB, S_PB = s(66), s(67)          # G; NP + the item's stage base (the first band step)
V_GB = v(126)                        # G - 4 (lane / 32): the global columns of the lane's keys
V_WM1L = v(80)                       # W - 1, or 2^30 on a global row (every earlier key attends)


# ---------------------------------------------------------------------------
# optional register dumps (a development aid: off in the library build)
DEBUG = {"on": False, "dumps": True, "n": 0, "tags": []}
S_DBG = s(92, 4)
S_DBGW, S_DBGG = s(66), s(67)   # total waves, this wave's global index (debug only)
V_DBGL = v(126)                 # lane * 4 (debug only)


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


# ---------------------------------------------------------------------------
# building blocks
def udiv(P, x, d, q, r, t0, t1):
    """q = x / d, r = x % d for wave-uniform 0 <= x < 2^24, 1 <= d < 2^24
    (SGPRs); float estimate, then corrections each way."""
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


def rsrc_add(P, dst, off):
    """Move a raw buffer descriptor's base up by `off` bytes (SGPR)."""
    P.salu("s_add_u32", dst.sub(0), dst.sub(0), off)
    P.salu("s_addc_u32", dst.sub(1), dst.sub(1), "0", reads_scc=True)
    P.salu("s_and_b32", dst.sub(1), dst.sub(1), "0xffff")


def class_rows(P, dst, pitch, row_bytes):
    """dst = (N_c - 1) * pitch + row_bytes: the bytes from a class's first
    row to the end of its last (the descriptor range of the class)."""
    P.salu("s_sub_u32", dst, S_NC, "1")
    P.salu("s_mul_i32", dst, dst, pitch)
    P.salu("s_add_u32", dst, dst, str(row_bytes))


def dma_ops():
    """This wave's LDS-DMA loads of the tile whose key offset (bytes) is
    S_SOFF into the stage at LDS byte S_SB, as a list of emitters (each sets
    M0 and issues one 1 KiB load).  The padded K tile is 17 chunks of 1 KiB
    and the V tile 20: K chunks wave and wave + 8, V chunks wave and
    wave + 8, and a fifth chunk through the wave's own descriptor, V chunk
    16 + wave on waves 0-3 and K chunk 16 on waves 4-7 (the four of them
    write the same bytes)."""
    ops = []
    for jk in range(2):
        def op(P, jk=jk):
            P.salu("s_add_u32", "m0", S_SBW, str(jk * 8192))
            P.dma(V_DK[jk], S_RSK, S_SOFF)
        ops.append(op)
    for jv in range(2):
        def op(P, jv=jv):
            P.salu("s_add_u32", "m0", S_SBW, str(KTILE + jv * 8192))
            P.dma(V_DV[jv], S_RSV, S_SOFF)
        ops.append(op)

    def op(P):
        P.salu("s_add_u32", "m0", S_SB, S_XOFF)
        P.dma(V_DX, S_RSE, S_SOFF)
    ops.append(op)
    return ops


def dma_bases(P):
    P.salu("s_add_u32", S_SBW, S_SB, S_WAVE1K)


def dma_tile(P):
    dma_bases(P)
    for op in dma_ops():
        op(P)


# K fragments in issue order n = 0..15: key half kb = n % 2, channels
# 16 ks .. 16 ks + 15 with ks = n / 2 (the two key halves' accumulation
# chains alternate); V^T fragments n = 0..15: key step n / 4 (key half
# kb, keys 16 hf .. 16 hf + 15 of it), values 32 db .. 32 db + 31 with
# db = n % 4 (four O^T blocks in turn).  Ring slot n % 4.
def qk_read(P, n):
    kb, ks = n % 2, n // 2
    P.ds_read("ds_read_b128", A_KR.sub(4 * (n % RING), 4), V_KADDR, kb * 32 * KROW + ks * 32)


def qk_mfma(P, n, sbuf):
    """S^T[kb] (+)= K Q^T for K fragment n."""
    kb, ks = n % 2, n // 2
    dst = v(sbuf + 16 * kb, 16)
    P.mfma(dst, A_KR.sub(4 * (n % RING), 4), A_Q.sub(4 * ks, 4), None if ks == 0 else dst)


def qk_half(P, sbuf, kb):
    """S^T[kb] = K Q^T for key half kb alone (the 8 K fragments n with
    n % 2 == kb, ring slots by position)."""
    ns = [n for n in range(16) if n % 2 == kb]

    def slot(i):
        return A_KR.sub(4 * (i % RING), 4)

    def rd(i):
        P.ds_read("ds_read_b128", slot(i), V_KADDR, kb * 32 * KROW + (ns[i] // 2) * 32)

    def mm(i):
        ks = ns[i] // 2
        dst = v(sbuf + 16 * kb, 16)
        P.mfma(dst, slot(i), A_Q.sub(4 * ks, 4), None if ks == 0 else dst)
    for i in range(AHEAD):
        rd(i)
    for i in range(len(ns)):
        mm(i)
        if i + AHEAD < len(ns):
            rd(i + AHEAD)


def pv_read(P, n):
    kstep, db = divmod(n, 4)
    kb, hf = divmod(kstep, 2)
    slot = A_VR.sub(4 * (n % RING), 4)
    off = (kb * 32 + hf * 16) * VROW + db * 64
    P.ds_read("ds_read_b64_tr_b16", slot.sub(0, 2), V_VADDR, off)
    P.ds_read("ds_read_b64_tr_b16", slot.sub(2, 2), V_VADDR, off + 8 * VROW)


def pv_mfma(P, n):
    """O^T[db] += V^T P^T for V^T fragment n."""
    kstep, db = divmod(n, 4)
    kb, hf = divmod(kstep, 2)
    o = A_O.sub(16 * db, 16)
    P.mfma(o, A_VR.sub(4 * (n % RING), 4), v(P_BUF + 8 * kb + 4 * hf, 4), o)


def max_ops(sbuf):
    """Row maximum of the tile's 32 scores per lane (both key halves), the
    lazy update of the running maximum and the flag of a moved maximum.
    Returns a list of emit callbacks (one instruction each)."""
    sv = [v(sbuf + k) for k in range(32)]
    t, t1, t2, t3 = V_T[8], V_T[9], V_T[10], V_T[11]
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
    ops.append(lambda P: P.add(I(f"  v_cmp_gt_f32 {S_CMP}, {t}, {V_MTHR}", "vcmp",
                                 regs_of(t, V_MTHR), S_CMP.regs())))
    ops.append(lambda P: P.valu("v_max_f32", t2, V_M, t))                    # candidate maximum

    # (compare and select in one op: merged op lists must not split an SCC
    # producer from its consumer)
    def moved(P):
        P.scmp("s_cmp_lg_u64", S_CMP, "0")
        P.salu("s_cselect_b64", S_MV, "-1", "0", reads_scc=True, writes_scc=False)
    ops.append(moved)
    ops.append(lambda P: P.valu("v_mov_b32", V_MOLD, V_M))
    ops.append(lambda P: P.valu("v_cndmask_b32", V_M, V_M, t2, S_MV))       # moved (any lane) ? new : old
    ops.append(lambda P: P.salu("s_or_b64", S_FLAG, S_FLAG, S_MV))
    return ops


def exp_ops(sbuf, kb):
    """p = exp2(s * c - m) for the 16 scores of key half kb, in place."""
    sv = [v(sbuf + 16 * kb + k) for k in range(16)]
    ops = []
    for k in range(16):
        ops.append(lambda P, k=k: P.valu("v_fma_f32", sv[k], sv[k], S_C, NegR(V_M)))
    for k in range(16):
        op = (lambda P, k=k: P.valu("v_exp_f32", sv[k], sv[k], kind="trans"))
        op.cost = 2.0
        ops.append(op)
    if OPT["fp32_sums"]:
        lt = V_LT
        if kb == 0:
            ops.append(lambda P: P.valu("v_add_f32", lt[0], sv[0], sv[2]))
            ops.append(lambda P: P.valu("v_add_f32", lt[1], sv[1], sv[3]))
            first = 4
        else:
            first = 0
        for k in range(first, 16):
            ops.append(lambda P, k=k: P.valu("v_add_f32", lt[k % 2], lt[k % 2], sv[k]))
    return ops


def pack_ops(sbuf, kb, vlast=None):
    """The probabilities of key half kb packed to bf16 pairs into the P
    buffer (the B operand of the P V product), and the row sums of the
    packed values.  vlast: the last V^T fragment of the current P V product
    that reads key half kb (8 kb + 7 at value head size 128)."""
    sv = [v(sbuf + 16 * kb + k) for k in range(16)]
    pv = [v(P_BUF + 8 * kb + i) for i in range(8)]
    lt = V_LT
    ops = []
    # (the P buffer's key half kb is read by the V fragments 8 kb .. 8 kb + 7
    # of the current P V product)
    for i in range(8):
        ops.append(after(lambda P, i=i: P.valu("v_cvt_pk_bf16_f32", pv[i], sv[2 * i], sv[2 * i + 1]),
                         "v", 8 * kb + 7 if vlast is None else vlast))
    if not OPT["fp32_sums"]:
        for i in range(8):
            a_ = i % 2            # (key half 0 initializes both partials)
            if kb == 0 and i < 2:
                ops.append(lambda P, i=i, a_=a_: P.valu("v_dot2_f32_bf16", lt[a_], pv[i], S_ONES, "0"))
            else:
                ops.append(lambda P, i=i, a_=a_: P.valu("v_dot2_f32_bf16", lt[a_], pv[i], S_ONES, lt[a_]))
    return ops


def merge_rr(lists):
    """Round-robin merge of op lists (the i-th op of each list, in turn)."""
    out = []
    for i in range(max(len(x) for x in lists)):
        for x in lists:
            if i < len(x):
                out.append(x[i])
    return out


def mask_block(P, sbuf, k0):
    """Per-cell window mask of tile j (key offset in k0) on score buffer sbuf:
    key j attends row i iff 0 <= i - j <= W - 1.  One 32-bit word per lane
    and key half (bit kc set iff the lane's key kc attends), then one
    bit-field select per score."""
    tb, tlo, thi, tm1, tm2, tk = V_T[0], V_T[1], V_T[2], V_T[3], V_T[4], V_T[5]
    for kb in range(2):
        P.salu("s_add_u32", S_X[3], k0, str(32 * kb))
        P.valu("v_subrev_u32", tb, S_X[3], V_IBASE)                      # base = i - 4 hl - key0
        if GLB["on"]:
            P.valu("v_sub_u32", tlo, tb, V_WM1L)                          # base - (W - 1)
        else:
            P.valu("v_subrev_u32", tlo, S_WM1, tb)                        # base - (W - 1)
        P.valu("v_max_i32", tlo, "0", tlo)
        P.valu("v_min_i32", thi, "31", tb)
        P.valu("v_lshlrev_b32_e64", tm1, thi, "2")
        P.valu("v_add_u32", tm1, "-1", tm1)                                # (2 << hi) - 1
        P.valu("v_lshlrev_b32_e64", tm2, tlo, "-1")                        # ~0 << lo
        P.valu("v_and_b32", tm1, tm1, tm2)
        P.add(I(f"  v_cmp_le_i32 vcc, {tlo}, {thi}", "vcmp", regs_of(tlo, thi), VCC))
        P.valu("v_cndmask_b32", tm1, "0", tm1, "vcc")
        if GLB["on"]:
            # or the global columns kc < G - 4 hl - key0, within kc <= hi
            tg, tg2 = V_T[6], V_T[7]
            P.valu("v_subrev_u32", tg, S_X[3], V_GB)
            P.valu("v_min_i32", tg, "32", tg)
            P.valu("v_add_u32", tg2, "-1", tg)
            P.valu("v_lshlrev_b32_e64", tg2, tg2, "2")
            P.valu("v_add_u32", tg2, "-1", tg2)                            # (1 << g) - 1, g = 1..32
            P.add(I(f"  v_cmp_lt_i32 vcc, 0, {tg}", "vcmp", regs_of(tg), VCC))
            P.valu("v_cndmask_b32", tg2, "0", tg2, "vcc")
            P.valu("v_lshlrev_b32_e64", tm2, thi, "2")
            P.valu("v_add_u32", tm2, "-1", tm2)                            # (2 << hi) - 1
            P.valu("v_and_b32", tg2, tg2, tm2)
            P.add(I(f"  v_cmp_le_i32 vcc, 0, {thi}", "vcmp", regs_of(thi), VCC))
            P.valu("v_cndmask_b32", tg2, "0", tg2, "vcc")
            P.valu("v_or_b32", tm1, tm1, tg2)
        for r in range(16):
            kc = (r % 4) + 8 * (r // 4)
            sr = v(sbuf + 16 * kb + r)
            P.valu("v_bfe_i32", tk, tm1, str(kc), "1")
            P.valu("v_bitop3_b32", sr, sr, S_NINF, tk, extra="bitop3:0xe4")


def rescale_block(P, with_o=True, o=None):
    """The running maximum moved (rare): alpha = exp2(m_old - m_new), the
    threshold follows the maximum, the running sum and (once a P V product
    has been accumulated) O are rescaled, after every product of the old
    maximum.  o: the O accumulators (A_O by default)."""
    o = A_O if o is None else o
    tmp = V_T
    P.valu("v_sub_f32", tmp[0], V_MOLD, V_M)
    P.valu("v_exp_f32", V_ALPHA, tmp[0], kind="trans")
    P.valu("v_add_f32", V_MTHR, str(SLACK), V_M)
    P.valu("v_mul_f32", V_L[0], V_L[0], V_ALPHA)
    P.valu("v_mul_f32", V_L[1], V_L[1], V_ALPHA)
    if not with_o:
        return
    for k0 in range(0, o.n, 8):
        for k in range(8):
            P.add(I(f"  v_accvgpr_read_b32 {tmp[k]}, {o.sub(k0 + k)}", "valu",
                    o.sub(k0 + k).regs(), tmp[k].regs()))
        for k in range(8):
            P.valu("v_mul_f32", tmp[k], tmp[k], V_ALPHA)
        for k in range(8):
            P.add(I(f"  v_accvgpr_write_b32 {o.sub(k0 + k)}, {tmp[k]}", "valu",
                    tmp[k].regs(), o.sub(k0 + k).regs()))


# ---------------------------------------------------------------------------
AHEAD = RING - 1   # fragments of each kind read ahead of their MFMA


def after(op, kind, n):
    """Mark op to run only after the MFMA of fragment (kind, n) is issued."""
    op.after = (kind, n)
    return op


def interleave(P, order, sbuf_next, valu_ops, extra_ops=(), v_ready=0):
    """order: the MFMAs as ("k", n) (QK fragment n into sbuf_next) or ("v",
    n) (PV fragment n).  Fragment reads of each kind run AHEAD fragments
    ahead of their MFMA (the first v_ready V fragments are already read).
    valu_ops keep their order and are spread evenly (by issue cost) over
    all the MFMAs; an op marked with after() waits for that MFMA (when it
    is part of this order).  extra_ops (the LDS-DMA loads and the scalar
    set-up of the next step) go one every few MFMAs."""
    nk = sum(1 for x in order if x[0] == "k")
    nv = len(order) - nk
    rd = {"k": lambda n: qk_read(P, n), "v": lambda n: pv_read(P, n)}
    cnt = {"k": nk, "v": nv}
    issued = {"k": 0, "v": v_ready if nv else 0}

    def read_upto(kind, last):
        while issued[kind] <= min(last, cnt[kind] - 1):
            rd[kind](issued[kind])
            issued[kind] += 1
    for kind in ("v", "k"):
        read_upto(kind, AHEAD - 1)
    index = {x: i for i, x in enumerate(order)}
    costs = [getattr(op, "cost", 1.0) for op in valu_ops]
    total = sum(costs)
    placed = {}
    vi, spent = 0, 0.0
    for m in range(len(order)):
        target = total * (m + 1) / len(order)
        while vi < len(valu_ops) and spent + 0.5 * costs[vi] <= target:
            need = index.get(getattr(valu_ops[vi], "after", None), -1)
            if need > m:
                break
            placed.setdefault(m, []).append(valu_ops[vi])
            spent += costs[vi]
            vi += 1
    tail = valu_ops[vi:]
    extra = list(extra_ops)
    every = max(1, (len(order) - 4) // max(1, len(extra))) if extra else 0
    for m, (kind, n) in enumerate(order):
        read_upto(kind, n)
        if kind == "k":
            qk_mfma(P, n, sbuf_next)
        else:
            pv_mfma(P, n)
        read_upto(kind, n + AHEAD)
        if extra and (m + 1) % every == 0:
            extra.pop(0)(P)
        for op in placed.get(m, []):
            op(P)
    for op in tail:
        op(P)
    while extra:
        extra.pop(0)(P)


def mfma_order(has_qk, has_pv):
    if has_qk and has_pv:
        # four P V products first (their first fragments were read before
        # the barrier; the K fragments of the new tile are read after it),
        # then two P V products per QK product until the P V products are
        # done: the VALU work that must follow them (the packing of P) then
        # has the last ten QK products to hide behind
        out = [("v", 0), ("v", 1), ("v", 2), ("v", 3)]
        for k in range(6):
            out += [("k", k), ("v", 4 + 2 * k), ("v", 5 + 2 * k)]
        return out + [("k", k) for k in range(6, 16)]
    if has_qk:
        return [("k", k) for k in range(16)]
    if has_pv:
        return [("v", k) for k in range(16)]
    return []


def stage_base(P, dst, jsgpr, add):
    """dst = ((j + add) & 3) * STAGE"""
    P.salu("s_add_u32", dst, jsgpr, str(add & 0xffffffff) if add >= 0 else str(add))
    P.salu("s_and_b32", dst, dst, "3")
    P.salu("s_mul_i32", dst, dst, str(STAGE))


def setup_ops(pn):
    """Scalar set-up of iteration i = j + 1 (S_J = j), as emitters: the DMA
    of tile i + 2 (offset, stage, M0 bases), key0 of tile i and whether
    every cell of tile i attends this wave's rows.  Runs after this
    iteration's DMA loads (it overwrites their offset and bases)."""
    def o1(P):
        P.salu("s_add_u32", S_X[9], S_J, "1")                  # i
        P.salu("s_add_u32", S_X[4], S_X[9], "2")               # tile i + 2
        P.salu("s_add_u32", S_X[5], S_TLO, S_X[4])
        if GLB["on"]:
            P.salu("s_sub_u32", S_X[6], S_X[4], S_BASE)        # a prefix step: tile = step
            P.scmp("s_cmp_lt_u32", S_X[4], S_PB)
            P.salu("s_cselect_b32", S_X[5], S_X[6], S_X[5], reads_scc=True, writes_scc=False)
        if DIL["on"]:
            P.salu("s_mul_i32", S_X[5], S_X[5], S_TILEB)
        else:
            P.salu("s_lshl_b32", S_X[5], S_X[5], "14")

    # past the band (i + 2 >= T) the offset is N rows, out of the
    # descriptor's range: the loads read zeros without touching memory,
    # into a stage nothing reads
    def o2(P):
        P.scmp("s_cmp_lt_u32", S_X[4], S_T)
        P.salu("s_cselect_b32", S_SOFF, S_X[5], S_NB, reads_scc=True, writes_scc=False)

    def o3(P):
        P.salu("s_and_b32", S_SB, S_X[4], "3")
        P.salu("s_mul_i32", S_SB, S_SB, str(STAGE))
        P.salu("s_add_u32", S_SBW, S_SB, S_WAVE1K)

    def o4(P):
        P.salu("s_add_u32", S_X[6], S_TLO, S_X[9])
        if GLB["on"]:
            P.salu("s_sub_u32", S_X[7], S_X[9], S_BASE)
            P.scmp("s_cmp_lt_u32", S_X[9], S_PB)
            P.salu("s_cselect_b32", S_X[6], S_X[7], S_X[6], reads_scc=True, writes_scc=False)
        P.salu("s_lshl_b32", S_K0P[pn], S_X[6], "6")           # key0 of tile i
        P.salu("s_add_u32", S_X[7], S_K0P[pn], "63")
        P.salu("s_add_u32", S_X[8], S_K0P[pn], S_W)

    def o5(P):
        P.scmp("s_cmp_le_u32", S_X[7], S_R0W)                  # last key <= first row
        P.salu("s_cselect_b32", S_X[10], "1", "0", reads_scc=True, writes_scc=False)

    def o6(P):
        P.scmp("s_cmp_ge_u32", S_X[8], S_R0W32)                # key0 + W >= last row + 1
        P.salu("s_cselect_b32", S_X[11], "1", "0", reads_scc=True, writes_scc=False)
        P.salu("s_and_b32", S_FULL[pn], S_X[10], S_X[11])
    return [o1, o2, o3, o4, o5, o6]


def v_prefetch_ops():
    """The first AHEAD V^T fragments of the next P V product (tile j, in
    stage j & 3, visible since an earlier barrier), read before the next
    barrier."""
    def addr(P):
        P.salu("s_and_b32", S_X[12], S_J, "3")
        P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
        P.valu("v_add_u32", V_VADDR, S_X[12], V_VLANE)
    # (after the last V read of this step, which uses the same address
    # register, and after the MFMAs that read the ring slots it refills)
    return [after(op, "v", 15) for op in [addr] + [(lambda P, n=n: pv_read(P, n)) for n in range(AHEAD)]]


def k_addr_next(P):
    """LDS address of the K fragments of the next QK product (tile j + 2)."""
    P.salu("s_add_u32", S_X[12], S_J, "2")
    P.salu("s_and_b32", S_X[12], S_X[12], "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)


def iteration(P, phase, has_qk, has_pv, first, exact=True):
    """One tile j (S_J) of the pipeline; score buffers by phase = j % 2.  The
    last step of an item (no QK product) also starts the loads of the
    workgroup's next item.  With exact=False the step takes no row maximum:
    p = exp2(s c - m) with the running maximum m as it stands, and only if
    some row's sum of this tile's p exceeds 2^SLACK (then a p may exceed
    it: the tile's maximum may lie more than SLACK above m) is the tile
    redone with its maximum (max_redo)."""
    sb_cur, sb_next = S_BUF[phase], S_BUF[1 - phase]
    P.comment(f"iteration phase {phase} qk={has_qk} pv={has_pv}")
    # the first step waits for tile 1 of its item, not for the previous
    # item's output stores (the last EPI_STORES vector memory operations)
    P.waitcnt(vm=EPI_STORES if first else 0)
    P.barrier()
    if has_pv:
        settle_previous(P)
    if first and has_qk and not GLB["on"]:
        first_step(P)
        return
    # per-cell mask of tile j unless every cell of this wave's 32 rows attends
    P.scmp("s_cmp_eq_u32", S_FULL[phase], "1")
    skip = P.new_label("full")
    P.branch("s_cbranch_scc1", skip)
    mask_block(P, sb_cur, S_K0P[phase])
    P.label(skip)
    dump(P, f"masked{phase}{int(has_qk)}{int(has_pv)}", [v(sb_cur, 32)])
    P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)
    if not has_qk:
        # the last tile: where its key half 1 lies past the wave's rows (before
        # the next item's loads replace the row) that half takes no softmax
        # (its p are 0; the epilogue skips its P V fragments)
        P.scmp("s_cmp_ge_u32", S_K0P[phase], S_R0W)
        P.salu("s_cselect_b32", S_HALF1, "1", "0", reads_scc=True, writes_scc=False)
        half, joined = P.new_label("lasthalf"), P.new_label("lastdone")
        P.scmp("s_cmp_eq_u32", S_HALF1, "1")
        P.branch("s_cbranch_scc1", half)
        item_loads(P, first=False)
        valu = (max_ops(sb_cur) + merge_rr([exp_ops(sb_cur, 0), exp_ops(sb_cur, 1)]) + pack_ops(sb_cur, 0)
                + v_prefetch_ops() + pack_ops(sb_cur, 1))
        interleave(P, mfma_order(False, has_pv), sb_next, valu, [], v_ready=AHEAD)
        P.branch("s_branch", joined)
        P.label(half)
        item_loads(P, first=False)
        valu = max_ops(sb_cur) + exp_ops(sb_cur, 0) + pack_ops(sb_cur, 0) + v_prefetch_ops()
        interleave(P, mfma_order(False, has_pv), sb_next, valu, [], v_ready=AHEAD)
        P.label(joined)
    else:
        valu = ((max_ops(sb_cur) if exact else []) + merge_rr([exp_ops(sb_cur, 0), exp_ops(sb_cur, 1)])
                + pack_ops(sb_cur, 0) + v_prefetch_ops() + pack_ops(sb_cur, 1))
        extra = dma_ops() + setup_ops(1 - phase)
        interleave(P, mfma_order(has_qk, has_pv), sb_next, valu, extra, v_ready=AHEAD)
    if not exact:
        max_redo(P, phase)
    if has_qk:
        k_addr_next(P)
    dump(P, f"soft{phase}{int(has_qk)}{int(has_pv)}", [v(sb_cur, 32), v(P_BUF, 16), V_M, V_L[0], V_L[1],
                                                        V_LT[0], V_LT[1]])
    if not has_pv:
        # first tile: nothing accumulated yet (O = 0, l = 0), so the moved
        # maximum only moves the threshold; this tile's sums are merged at
        # the start of the next step
        P.valu("v_add_f32", V_MTHR, str(SLACK), V_M)
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)


def first_step(P):
    """Step 0 of an item (S(1) = K(1) Q^T, the DMA of tile 2, the softmax of
    tile 0, with its row maximum).  Where key half 0 of tile 0 lies before
    the window of the wave's first row (item_start then computed key half 1
    alone), that half takes no softmax: its P values and row sums are
    cleared for the P V product of step 1."""
    sb = S_BUF[0]
    half, joined = P.new_label("firsthalf"), P.new_label("firstdone")
    P.salu("s_add_u32", S_X[12], S_K0P[0], S_W)
    P.salu("s_add_u32", S_X[12], S_X[12], "31")
    P.scmp("s_cmp_le_u32", S_X[12], S_R0W)
    P.branch("s_cbranch_scc1", half)
    for kind in ("full", "half"):
        if kind == "half":
            P.label(half)
        P.scmp("s_cmp_eq_u32", S_FULL[0], "1")
        skip = P.new_label("full")
        P.branch("s_cbranch_scc1", skip)
        mask_block(P, sb, S_K0P[0])
        P.label(skip)
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)
        if kind == "full":
            valu = (max_ops(sb) + merge_rr([exp_ops(sb, 0), exp_ops(sb, 1)]) + pack_ops(sb, 0)
                    + v_prefetch_ops() + pack_ops(sb, 1))
        else:
            valu = ([lambda P, k=k: P.valu("v_mov_b32", V_LT[k], "0") for k in range(2)]
                    + max_ops(sb) + exp_ops(sb, 1) + pack_ops(sb, 1)
                    + [lambda P, i=i: P.valu("v_mov_b32", v(P_BUF + i), "0") for i in range(8)]
                    + v_prefetch_ops())
        interleave(P, mfma_order(True, False), S_BUF[1], valu, dma_ops() + setup_ops(1), v_ready=AHEAD)
        if kind == "full":
            P.branch("s_branch", joined)
    P.label(joined)
    k_addr_next(P)
    P.valu("v_add_f32", V_MTHR, str(SLACK), V_M)
    P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)


def max_redo(P, phase, qk=None, stage=None, mask=None):
    """After a step without the row maximum: if any lane's sum of the tile's
    p exceeds 2^SLACK, recompute S(j) = K(j) Q^T (tile j is still in its
    stage, the Q fragments in place), mask it, and take the step's softmax
    again with the row maximum.  Every wave of the branch starts and ends
    with no LDS read in flight (the next step's first V^T fragments, read
    during this step, are waited for here), so both paths join in the same
    state.  qk(P, sbuf) emits the kernel's QK product into sbuf and stage
    is its LDS stage size (this kernel's by default); mask(P, phase), when
    given, masks the recomputed tile in place of this kernel's mask."""
    sb_cur = S_BUF[phase]
    if qk is None:
        def qk(P, sbuf):
            interleave(P, mfma_order(True, False), sbuf, [])
    stage = STAGE if stage is None else stage
    t = V_T[15]
    P.valu("v_add_f32", t, V_LT[0], V_LT[1])
    two_slack = struct.unpack("<I", struct.pack("<f", 2.0 ** SLACK))[0]
    P.salu("s_mov_b32", S_X[13], hex(two_slack), writes_scc=False)   # 2^SLACK
    P.add(I(f"  v_cmp_lt_f32 {S_CMP}, {S_X[13]}, {t}", "vcmp", regs_of(S_X[13], t), S_CMP.regs()))
    P.waitcnt(lgkm=0)
    P.scmp("s_cmp_eq_u64", S_CMP, "0")
    skip = P.new_label("nomax")
    P.branch("s_cbranch_scc1", skip)
    P.salu("s_and_b32", S_X[12], S_J, "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(stage))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)
    qk(P, sb_cur)
    if mask is not None:
        mask(P, phase)
    else:
        P.scmp("s_cmp_eq_u32", S_FULL[phase], "1")
        full = P.new_label("full")
        P.branch("s_cbranch_scc1", full)
        mask_block(P, sb_cur, S_K0P[phase])
        P.label(full)
    for op in (max_ops(sb_cur) + merge_rr([exp_ops(sb_cur, 0), exp_ops(sb_cur, 1)]) + pack_ops(sb_cur, 0)
               + pack_ops(sb_cur, 1)):
        op(P)
    P.waitcnt(lgkm=0)
    P.label(skip)


def settle_previous(P, o=None):
    """Between the P V products of the previous tile and of this one: if the
    previous tile moved the running maximum, rescale l and O (rare), then add
    the previous tile's row sums to l.  o: the O accumulators (A_O by
    default)."""
    skip = P.new_label("norescale")
    P.scmp("s_cmp_eq_u64", S_FLAG, "0")
    P.branch("s_cbranch_scc1", skip)
    rescale_block(P, with_o=True, o=o)
    P.label(skip)
    P.valu("v_add_f32", V_L[0], V_L[0], V_LT[0])
    P.valu("v_add_f32", V_L[1], V_L[1], V_LT[1])


def epilogue(P, phase):
    """O += V(T-1)^T P(T-1), then O / l -> bf16 rows, and the log-sum-exp.
    Ends the workgroup, or goes on with its next item (whose loads are in
    flight)."""
    # (the next item's loads are not waited for: the barrier only orders
    # this item's last reads of the stage the output is staged in)
    P.barrier()
    settle_previous(P)
    # key half 1 of the last tile past the wave's last row: its p are 0, so
    # its P V products are skipped
    whole, done = P.new_label("pvlast"), P.new_label("pvdone")
    P.scmp("s_cmp_eq_u32", S_HALF1, "0")
    P.branch("s_cbranch_scc1", whole)
    interleave(P, [("v", n) for n in range(8)], None, [], v_ready=AHEAD)
    P.branch("s_branch", done)
    P.label(whole)
    interleave(P, mfma_order(False, True), None, [], v_ready=AHEAD)
    P.label(done)
    dump(P, f"O{phase}", [A_O])
    t = V_T
    l, l2, inv = t[0], t[1], t[2]
    P.valu("v_add_f32", l, V_L[0], V_L[1])
    P.valu("v_mov_b32", l2, l)
    P.add(I(f"  v_permlane32_swap_b32 {l}, {l2}", "perm", regs_of(l, l2), regs_of(l, l2)))
    P.valu("v_add_f32", l, l, l2)                       # the row's sum over both lane halves
    P.valu("v_rcp_f32", inv, l, kind="trans")
    # log-sum-exp, natural log: (m + log2 l) * ln 2
    skip = P.new_label("nolse")
    P.scmp("s_cmp_eq_u64", S_LSE, "0")
    P.branch("s_cbranch_scc1", skip)
    P.valu("v_log_f32", l2, l, kind="trans")
    P.valu("v_add_f32", l2, V_M, l2)
    P.valu("v_mul_f32", l2, "0x3f317218", l2)
    P.buf_store("buffer_store_dword", l2, V_LOFF, S_RSL)
    P.label(skip)
    # O / l -> bf16, staged through LDS so the global stores are 128-byte
    # runs of rows instead of 8-byte pieces of 32 rows.  The staging area is
    # the stage of tile T-2 (no wave reads it after the barrier above; the
    # stage of tile T-1 is still being read and the next two hold the next
    # item's first tiles): 8 waves x 32 rows x 144 bytes, half a row at a
    # time (values 0..63, then 64..127).
    P.salu("s_add_u32", S_X[0], S_J, "-1")
    P.salu("s_and_b32", S_X[0], S_X[0], "3")
    P.salu("s_mul_i32", S_X[0], S_X[0], str(STAGE))
    P.salu("s_mul_i32", S_X[2], S_WAVE, str(32 * OROW))
    P.salu("s_add_u32", S_X[1], S_X[0], S_X[2])                    # this wave's region
    P.valu("v_add_u32", V_OW, S_X[1], V_OWL)
    P.valu("v_add_u32", V_ORD, S_X[1], V_ORDL)
    for half in range(2):
        for db in (2 * half, 2 * half + 1):
            for r4 in range(4):
                x = [t[4 + k] for k in range(4)]
                for k in range(4):
                    P.add(I(f"  v_accvgpr_read_b32 {x[k]}, {A_O.sub(16 * db + 4 * r4 + k)}", "valu",
                            A_O.sub(16 * db + 4 * r4 + k).regs(), x[k].regs()))
                for k in range(4):
                    P.valu("v_mul_f32", x[k], x[k], inv)
                pk0, pk1 = t[8 + 2 * (r4 % 2)], t[9 + 2 * (r4 % 2)]
                P.valu("v_cvt_pk_bf16_f32", pk0, x[0], x[1])
                P.valu("v_cvt_pk_bf16_f32", pk1, x[2], x[3])
                # row col, values 32 db + 8 r4 + 4 hl .. +3
                P.add(I(f"  ds_write_b64 {V_OW}, {v(pk0.i, 2)} offset:{(db - 2 * half) * 64 + r4 * 16}",
                        "lds", regs_of(V_OW, v(pk0.i, 2)), EMPTY))
        # rows 8 kk + lane / 8, bytes 16 (lane % 8) .. +15 of the half row
        # (the next half's writes follow these reads: LDS operations of a
        # wave execute in order)
        ob = S_BUF[0] + 16 * half                                   # free score buffer
        for kk in range(4):
            P.ds_read("ds_read_b128", v(ob + 4 * kk, 4), V_ORD, kk * 8 * OROW)
        for kk in range(4):
            if DIL["on"]:
                P.salu("s_mul_i32", S_X[3 + kk], S_PITCH, str(8 * kk))
                P.salu("s_add_u32", S_X[3 + kk], S_X[3 + kk], str(half * 128))
            else:
                P.salu("s_mov_b32", S_X[3 + kk], str(kk * 8 * 256 + half * 128), writes_scc=False)
            P.add(I(f"  buffer_store_dwordx4 {v(ob + 4 * kk, 4)}, {V_OST}, {S_RSO}, {S_X[3 + kk]} offen",
                    "vstore", regs_of(v(ob + 4 * kk, 4), V_OST, S_RSO, S_X[3 + kk]), EMPTY))
    P.scmp("s_cmp_lt_u32", S_VID, S_TOTAL)
    P.branch("s_cbranch_scc1", ".Litem")
    P.add(I("  s_endpgm", "branch"))


def query_head(P, dst):
    """dst = bg * G + 4 hb + (wave & 3): this wave's query head (S_X[8] is
    its temporary)."""
    P.salu("s_mul_i32", dst, S_BG, S_G)
    P.salu("s_lshl_b32", S_X[8], S_HB, "2")
    P.salu("s_add_u32", dst, dst, S_X[8])
    P.salu("s_add_u32", dst, dst, S_WH)


def item_loads(P, first):
    """Start the workgroup's next item (S_VID + S_STRIDE; S_VID itself for
    the first): its row block, band and K, V, Q descriptors, then the loads
    of its Q fragments and of its tiles 0 and 1 into stages S_J + 1 and
    S_J + 2 (mod 4), which no wave reads any more once the last step of the
    current item has begun.  Nothing here waits for these loads.  The
    item's step counter then starts at S_BASE = (S_J + 1) & 3, so tile t
    of every item is in stage (S_BASE + t) & 3."""
    skip = None
    if not first:
        P.salu("s_add_u32", S_VID, S_VID, S_STRIDE)
        P.scmp("s_cmp_ge_u32", S_VID, S_TOTAL)
        skip = P.new_label("nonext")
        P.branch("s_cbranch_scc1", skip)
    P.salu("s_add_u32", S_BASE, S_J, "1")
    P.salu("s_and_b32", S_BASE, S_BASE, "3")
    # item -> logical id: items i, i + 8, ... (the workgroup's own id and its
    # steps by the grid size, a multiple of 8) run on XCD i % 8, which takes a
    # contiguous run of logical ids
    P.salu("s_and_b32", S_X[0], S_TOTAL, "7")
    P.salu("s_and_b32", S_X[1], S_VID, "7")
    P.salu("s_lshr_b32", S_X[2], S_TOTAL, "3")
    P.salu("s_mul_i32", S_X[1], S_X[1], S_X[2])
    P.salu("s_lshr_b32", S_X[3], S_VID, "3")
    P.salu("s_add_u32", S_X[1], S_X[1], S_X[3])
    P.scmp("s_cmp_eq_u32", S_X[0], "0")
    P.salu("s_cselect_b32", S_LID, S_X[1], S_VID, reads_scc=True, writes_scc=False)
    # lid -> (head block, row block, batch * kv head), row blocks ascending
    udiv(P, S_LID, S_NHB, S_X[4], S_HB, V_T[1], V_T[2])        # S_X[4] = rest
    if DIL["on"]:
        # rest -> (batch * kv head, residue class, row block of the class)
        udiv(P, S_X[4], S_NRB, S_X[5], S_RB, V_T[1], V_T[2])
        udiv(P, S_X[5], S_NCLS, S_BG, S_CLS, V_T[1], V_T[2])
        P.salu("s_sub_u32", S_X[6], S_N, S_CLS)                # rows of the class: ceil((N - c) / r)
        P.salu("s_add_u32", S_X[6], S_X[6], S_DIL)
        P.salu("s_sub_u32", S_X[6], S_X[6], "1")
        udiv(P, S_X[6], S_DIL, S_NC, S_X[7], V_T[1], V_T[2])
    else:
        udiv(P, S_X[4], S_NRB, S_BG, S_RB, V_T[1], V_T[2])     # row block
    P.salu("s_lshl_b32", S_R0, S_RB, "6")
    P.salu("s_lshl_b32", S_R0W, S_WR, "5")
    P.salu("s_add_u32", S_R0W, S_R0W, S_R0)                    # this wave's first row
    # band of rows r0 .. r0+63: key tiles t_lo .. t_hi
    P.salu("s_sub_i32", S_X[0], S_R0, S_W)
    P.salu("s_add_i32", S_X[0], S_X[0], "1")
    P.salu("s_max_i32", S_X[0], S_X[0], "0")
    P.salu("s_lshr_b32", S_TLO, S_X[0], "6")
    if GLB["on"]:
        P.scmp("s_cmp_lt_u32", S_R0, S_NGLB)                   # global rows: the band starts at key 0
        P.salu("s_cselect_b32", S_TLO, "0", S_TLO, reads_scc=True, writes_scc=False)
    P.salu("s_add_u32", S_X[1], S_R0, "63")
    P.salu("s_sub_u32", S_X[2], S_NC if DIL["on"] else S_N, "1")
    P.salu("s_min_u32", S_X[1], S_X[1], S_X[2])
    if DIL["on"]:
        # (a last row block past its class's rows walks one tile of zeros)
        P.salu("s_max_u32", S_X[1], S_X[1], S_R0)
    P.salu("s_lshr_b32", S_X[1], S_X[1], "6")
    P.salu("s_sub_u32", S_T, S_X[1], S_TLO)
    P.salu("s_add_u32", S_T, S_T, "1")
    # descriptors
    P.salu("s_lshl_b32", S_X[6], S_N, "8")                     # bytes per head (N rows of 256 B)
    if DIL["on"]:
        query_head(P, S_X[7])                                  # (uses S_X[8] as a temporary)
        class_rows(P, S_X[8], S_PITCH, 256)                    # the class's rows: (N_c - 1) pitch + 256
        P.salu("s_lshl_b32", S_X[9], S_CLS, "8")
        P.salu("s_mul_i32", S_NB, S_NC, S_PITCH)               # past the class's rows
        rsrc(P, S_RSK, S_K, S_BG, S_X[6], S_X[8])
        rsrc_add(P, S_RSK, S_X[9])
        rsrc(P, S_RSV, S_V, S_BG, S_X[6], S_X[8])
        rsrc_add(P, S_RSV, S_X[9])
        rsrc(P, S_RSQ, S_Q, S_X[7], S_X[6], S_X[8])
        rsrc_add(P, S_RSQ, S_X[9])
    else:
        rsrc(P, S_RSK, S_K, S_BG, S_X[6], S_X[6])
        rsrc(P, S_RSV, S_V, S_BG, S_X[6], S_X[6])
        query_head(P, S_X[7])
        rsrc(P, S_RSQ, S_Q, S_X[7], S_X[6], S_X[6])
    # the fifth DMA chunk's descriptor: V on waves 0-3, K on waves 4-7
    P.scmp("s_cmp_lt_u32", S_WAVE, "4")
    for h in (0, 2):
        P.salu("s_cselect_b64", S_RSE.sub(h, 2), S_RSV.sub(h, 2), S_RSK.sub(h, 2), reads_scc=True,
               writes_scc=False)
    # Q fragments
    if DIL["on"]:
        P.salu("s_mul_i32", S_X[9], S_R0W, S_PITCH)
    else:
        P.salu("s_lshl_b32", S_X[9], S_R0W, "8")
    P.valu("v_add_u32", V_QOFF, S_X[9], V_QLANE)
    for ks in range(8):
        P.buf_load(A_Q.sub(4 * ks, 4), V_QOFF, S_RSQ, "0", 32 * ks, track=False)
    # tiles 0 and 1 (tile 1 also when the band has one tile: its rows are
    # read, or are past N and read as zeros, and never used)
    if GLB["on"]:
        # prefix tiles NP = min(ceil(G / 64), t_lo); tiles of steps 0 and 1
        P.salu("s_add_u32", S_X[0], S_NGLB, "63")
        P.salu("s_lshr_b32", S_X[0], S_X[0], "6")
        P.salu("s_min_u32", S_X[10], S_X[0], S_TLO)            # NP
        P.scmp("s_cmp_gt_u32", S_X[10], "0")
        P.salu("s_cselect_b32", S_X[0], "0", S_TLO, reads_scc=True, writes_scc=False)
        P.salu("s_sub_u32", S_X[1], S_TLO, S_X[10])
        P.salu("s_add_u32", S_X[1], S_X[1], "1")
        P.scmp("s_cmp_gt_u32", S_X[10], "1")
        P.salu("s_cselect_b32", S_X[1], "1", S_X[1], reads_scc=True, writes_scc=False)
        P.salu("s_lshl_b32", S_SOFF, S_X[0], "14")
        P.salu("s_lshl_b32", S_X[1], S_X[1], "14")
    elif DIL["on"]:
        P.salu("s_mul_i32", S_SOFF, S_TLO, S_TILEB)
    else:
        P.salu("s_lshl_b32", S_SOFF, S_TLO, "14")
    P.salu("s_mul_i32", S_SB, S_BASE, str(STAGE))
    dma_tile(P)
    if GLB["on"]:
        P.salu("s_mov_b32", S_SOFF, S_X[1], writes_scc=False)
    else:
        P.salu("s_add_u32", S_SOFF, S_SOFF, S_TILEB if DIL["on"] else str(1 << 14))
    P.salu("s_add_u32", S_X[0], S_BASE, "1")
    P.salu("s_and_b32", S_X[0], S_X[0], "3")
    P.salu("s_mul_i32", S_SB, S_X[0], str(STAGE))
    dma_tile(P)
    # step counter from S_BASE: first tile and band end shifted to match
    if GLB["on"]:
        P.salu("s_add_u32", S_T, S_T, S_X[10])                 # prefix steps first
        P.salu("s_sub_u32", S_TLO, S_TLO, S_X[10])
        P.salu("s_add_u32", S_PB, S_X[10], S_BASE)
    P.salu("s_sub_u32", S_TLO, S_TLO, S_BASE)
    P.salu("s_add_u32", S_T, S_T, S_BASE)
    if skip:
        P.label(skip)


def item_start(P):
    """Set-up of an item once the previous one's epilogue is issued: output
    descriptors, the row-dependent lane offsets, the softmax state and the
    scalar set-up of step 0; then, with Q and tile 0 in, S(0) = K(0) Q^T."""
    P.label(".Litem")
    P.salu("s_lshl_b32", S_X[6], S_N, "8")
    query_head(P, S_X[7])
    if DIL["on"]:
        P.salu("s_lshl_b32", S_X[9], S_N, "2")
        class_rows(P, S_X[8], S_PITCH, 256)
        P.salu("s_lshl_b32", S_X[10], S_CLS, "8")
        rsrc(P, S_RSO, S_OUT, S_X[7], S_X[6], S_X[8])
        rsrc_add(P, S_RSO, S_X[10])
        P.salu("s_lshl_b32", S_X[11], S_DIL, "2")              # log-sum-exp pitch 4 r
        class_rows(P, S_X[8], S_X[11], 4)
        P.salu("s_lshl_b32", S_X[10], S_CLS, "2")
        rsrc(P, S_RSL, S_LSE, S_X[7], S_X[9], S_X[8])
        rsrc_add(P, S_RSL, S_X[10])
    else:
        rsrc(P, S_RSO, S_OUT, S_X[7], S_X[6], S_X[6])
        P.salu("s_lshl_b32", S_X[9], S_N, "2")
        rsrc(P, S_RSL, S_LSE, S_X[7], S_X[9], S_X[9])
    P.salu("s_add_u32", S_R0W32, S_R0W, "32")
    t = V_T
    P.valu("v_add_u32", t[5], S_R0W, V_COL)                    # row
    if DIL["on"]:
        P.valu("v_mul_u32_u24", V_LOFF, S_X[11], t[5])
    else:
        P.valu("v_lshlrev_b32", V_LOFF, "2", t[5])
    P.valu("v_lshlrev_b32", t[7], "2", V_HL)
    P.valu("v_sub_u32", V_IBASE, t[5], t[7])
    if GLB["on"]:
        P.add(I(f"  v_cmp_gt_u32 vcc, {S_NGLB}, {t[5]}", "vcmp", regs_of(S_NGLB, t[5]), VCC))
        P.valu("v_mov_b32", t[6], "0x40000000")
        P.valu("v_mov_b32", t[8], S_WM1)
        P.valu("v_cndmask_b32", V_WM1L, t[8], t[6], "vcc")
    # output store offset: row r0w + lane / 8, bytes 16 (lane % 8) of a half row
    P.valu("v_lshrrev_b32", t[0], "3", V_LANE)
    P.valu("v_add_u32", t[0], S_R0W, t[0])
    if DIL["on"]:
        P.valu("v_mul_u32_u24", t[0], S_PITCH, t[0])
    else:
        P.valu("v_lshlrev_b32", t[0], "8", t[0])
    P.valu("v_and_b32", t[1], "7", V_LANE)
    P.valu("v_lshlrev_b32", t[1], "4", t[1])
    P.valu("v_add_u32", V_OST, t[0], t[1])
    # softmax state
    P.valu("v_mov_b32", V_M, "0xf149f2ca")             # -1e30
    P.valu("v_mov_b32", V_MTHR, "0xf149f2ca")
    for k in range(2):
        P.valu("v_mov_b32", V_L[k], "0")
    for k in range(64):
        P.add(I(f"  v_accvgpr_write_b32 {A_O.sub(k)}, 0", "valu", EMPTY, A_O.sub(k).regs()))
    # set-up of step 0 (as if from a step j = -1)
    P.salu("s_sub_u32", S_J, S_BASE, "1")
    for op in setup_ops(0):
        op(P)
    # Q and tile 0 in: all but tile 1's loads and the previous item's output
    # stores, issued after them
    P.waitcnt(vm=len(dma_ops()) + EPI_STORES)
    P.barrier()
    # S(0) = K(0) Q^T
    P.salu("s_mov_b32", S_J, S_BASE, writes_scc=False)
    P.salu("s_mul_i32", S_X[12], S_BASE, str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)
    dump_lds(P, "lds0", STAGE)
    dump(P, "q", [A_Q])
    if GLB["on"]:
        interleave(P, mfma_order(True, False), S_BUF[0], [])
    else:
        # key half 0 of tile 0 before the window of the wave's first row
        # (every key + W - 1 < the row): its scores are masked to -inf
        # whatever they hold, so only key half 1 is computed
        whole, done = P.new_label("qk0"), P.new_label("qk0done")
        P.salu("s_add_u32", S_X[12], S_K0P[0], S_W)
        P.salu("s_add_u32", S_X[12], S_X[12], "31")
        P.scmp("s_cmp_gt_u32", S_X[12], S_R0W)
        P.branch("s_cbranch_scc1", whole)
        qk_half(P, S_BUF[0], 1)
        P.branch("s_branch", done)
        P.label(whole)
        interleave(P, mfma_order(True, False), S_BUF[0], [])
        P.label(done)
    P.salu("s_add_u32", S_X[12], S_BASE, "1")                  # QK(1) reads the next stage
    P.salu("s_and_b32", S_X[12], S_X[12], "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)
    dump(P, "s0", [v(S_BUF[0], 32)])


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
    if GLB["on"]:
        P.salu("s_mov_b32", S_NGLB, s(22), writes_scc=False)   # (shares an argument dword, as below)
    if DIL["on"]:
        # (the dilation and the class count share the argument dwords of
        # the item and workgroup registers set below)
        P.salu("s_mov_b32", S_DIL, s(22), writes_scc=False)
        P.salu("s_mov_b32", S_NCLS, s(23), writes_scc=False)
        P.salu("s_lshl_b32", S_PITCH, S_DIL, "8")
        P.salu("s_lshl_b32", S_TILEB, S_PITCH, "6")
    P.salu("s_and_b32", S_WH, S_WAVE, "3")
    P.salu("s_lshr_b32", S_WR, S_WAVE, "2")
    if DEBUG["on"]:
        P.salu("s_and_b32", S_DBG.sub(1), S_DBG.sub(1), "0xffff")
        P.salu("s_mov_b32", S_DBG.sub(3), "0x00020000", writes_scc=False)
        P.salu("s_lshl_b32", S_DBGW, S_TOTAL, "3")
        P.salu("s_lshl_b32", S_DBGG, S_WG, "3")
        P.salu("s_add_u32", S_DBGG, S_DBGG, S_WAVE)
        P.valu("v_lshlrev_b32", V_DBGL, "2", V_LANE)
    P.salu("s_mov_b32", S_VID, S_WG, writes_scc=False)
    P.salu("s_lshl_b32", S_WAVE1K, S_WAVE, "10")
    # the fifth chunk's LDS offset: KTILE + 1024 (16 + wave) on waves 0-3,
    # 1024 * 16 on waves 4-7
    P.salu("s_lshl_b32", S_XOFF, S_WH, "10")
    P.salu("s_add_u32", S_XOFF, S_XOFF, str(KTILE + 16 * 1024))
    P.scmp("s_cmp_lt_u32", S_WAVE, "4")
    P.salu("s_cselect_b32", S_XOFF, S_XOFF, str(16 * 1024), reads_scc=True, writes_scc=False)
    P.salu("s_lshl_b32", S_NB, S_N, "8")
    P.salu("s_sub_u32", S_WM1, S_W, "1")
    P.salu("s_mov_b32", S_NINF, "0xff800000", writes_scc=False)
    P.salu("s_mov_b32", S_ONES, "0x3f803f80", writes_scc=False)
    # per-lane addressing (the same for every item)
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
    # Q rows: row col of the wave's 32, bytes 16 hl of each 32-byte group
    if DIL["on"]:
        P.valu("v_mul_u32_u24", t[0], S_PITCH, V_COL)
    else:
        P.valu("v_lshlrev_b32", t[0], "8", V_COL)
    P.valu("v_lshlrev_b32", t[1], "4", V_HL)
    P.valu("v_add_u32", V_QLANE, t[0], t[1])
    if GLB["on"]:
        P.valu("v_lshlrev_b32", t[0], "2", V_HL)
        P.valu("v_sub_u32", V_GB, S_NGLB, t[0])
    # output staging: LDS write base (row col, values 4 hl: col * 144 +
    # 8 hl), LDS read base (row lane / 8, bytes 16 (lane % 8))
    P.valu("v_mul_u32_u24", V_OWL, str(OROW), V_COL)
    P.valu("v_lshlrev_b32", t[0], "3", V_HL)
    P.valu("v_add_u32", V_OWL, V_OWL, t[0])
    P.valu("v_lshrrev_b32", t[0], "3", V_LANE)
    P.valu("v_and_b32", t[1], "7", V_LANE)
    P.valu("v_lshlrev_b32", t[1], "4", t[1])
    P.valu("v_mul_u32_u24", V_ORDL, str(OROW), t[0])
    P.valu("v_add_u32", V_ORDL, V_ORDL, t[1])
    # DMA lane offsets: K chunks wave + 8 jk (jk < 2) and 16, V chunks
    # wave + 8 jv (jv < 2) and 16 + (wave & 3)
    P.valu("v_lshlrev_b32", t[8], "4", V_LANE)                 # 16 lane
    P.valu("v_mov_b32", t[9], S_WAVE1K)
    for jk in range(2):
        P.valu("v_add_u32", t[10], t[9], t[8])
        P.valu("v_add_u32", t[10], str(jk * 8192), t[10])
        _chunk_src(P, V_DK[jk], t[10], M272, KROW, t)
    for jv in range(2):
        P.valu("v_add_u32", t[10], t[9], t[8])
        P.valu("v_add_u32", t[10], str(jv * 8192), t[10])
        _chunk_src(P, V_DV[jv], t[10], M320, VROW, t)
    # the fifth chunk: K chunk 16 on waves 4-7, V chunk 16 + wave on waves 0-3
    P.valu("v_add_u32", t[10], str(16 * 1024), t[8])
    _chunk_src(P, t[14], t[10], M272, KROW, t)
    P.salu("s_lshl_b32", S_X[10], S_WH, "10")
    P.valu("v_add_u32", t[10], S_X[10], t[8])
    P.valu("v_add_u32", t[10], str(16 * 1024), t[10])
    _chunk_src(P, V_DX, t[10], M320, VROW, t)
    P.scmp("s_cmp_lt_u32", S_WAVE, "4")
    P.salu("s_cselect_b64", "vcc", "-1", "0", reads_scc=True, writes_scc=False)
    P.valu("v_cndmask_b32", V_DX, t[14], V_DX, "vcc")
    # the first item's loads (stage base 0), all of them in before its set-up
    P.salu("s_mov_b32", S_J, "-1", writes_scc=False)
    item_loads(P, first=True)
    P.waitcnt(vm=0)


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
    if DIL["on"]:
        P.valu("v_mul_u32_u24", t[11], S_PITCH, t[11])
    else:
        P.valu("v_lshlrev_b32", t[11], "8", t[11])
    P.valu("v_add_u32", dst, t[11], t[12])


def kernel_text():
    P = Prog()
    prologue(P)
    item_start(P)
    # T == 1: softmax of S(0) only
    P.salu("s_add_u32", S_X[0], S_J, "1")
    P.scmp("s_cmp_ge_u32", S_X[0], S_T)
    P.branch("s_cbranch_scc1", ".Lsingle")
    iteration(P, 0, True, False, True)                         # j = 0
    P.salu("s_add_u32", S_J, S_J, "1")
    P.salu("s_add_u32", S_X[0], S_J, "1")
    P.scmp("s_cmp_ge_u32", S_X[0], S_T)
    P.branch("s_cbranch_scc1", ".Llast1")
    # j = 1 with the row maximum too: every row of the item attends a key of
    # tiles 0 and 1, so from j = 2 on the running maximum is finite
    iteration(P, 1, True, True, False)
    P.salu("s_add_u32", S_J, S_J, "1")
    P.salu("s_add_u32", S_X[0], S_J, "1")
    P.scmp("s_cmp_ge_u32", S_X[0], S_T)
    P.branch("s_cbranch_scc1", ".Llast0")
    P.label(".Lmid0")
    for ph in (0, 1):
        iteration(P, ph, True, True, False, exact=False)
        P.salu("s_add_u32", S_J, S_J, "1")
        P.salu("s_add_u32", S_X[0], S_J, "1")
        P.scmp("s_cmp_ge_u32", S_X[0], S_T)                   # j == T - 1 (>=: a bound)
        P.branch("s_cbranch_scc1", f".Llast{1 - ph}")
    P.branch("s_branch", ".Lmid0")
    for ph in range(2):
        P.label(f".Llast{ph}")
        iteration(P, ph, False, True, False)
        epilogue(P, ph)
    P.label(".Lsingle")
    iteration(P, 0, False, False, True)
    epilogue(P, 0)
    body = resolve(P.ins)
    lines = [x.text for x in body]
    return "\n".join(lines)


def kernel_name():
    return NAME + ("_dil" if DIL["on"] else "") + ("_glb" if GLB["on"] else "")


def render():
    name = kernel_name()
    body = kernel_text()
    karg = KARG_BYTES + (16 if DEBUG["on"] else 0)
    head = f""".amdgcn_target "amdgcn-amd-amdhsa--gfx950"
.text
.globl {name}
.p2align 8
.type {name},@function
{name}:
"""
    tail = f"""
.Lfunc_end:
.size {name}, .Lfunc_end-{name}

.rodata
.p2align 6
.amdhsa_kernel {name}
  .amdhsa_group_segment_fixed_size {LDS_BYTES}
  .amdhsa_private_segment_fixed_size 0
  .amdhsa_kernarg_size {karg}
  .amdhsa_user_sgpr_count 2
  .amdhsa_user_sgpr_kernarg_segment_ptr 1
  .amdhsa_system_sgpr_workgroup_id_x 1
  .amdhsa_system_vgpr_workitem_id 0
  .amdhsa_next_free_vgpr 256
  .amdhsa_next_free_sgpr 100
  .amdhsa_accum_offset 128
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
  - .name: {name}
    .symbol: {name}.kd
    .kernarg_segment_size: {karg}
    .group_segment_fixed_size: {LDS_BYTES}
    .private_segment_fixed_size: 0
    .kernarg_segment_align: 8
    .wavefront_size: 64
    .sgpr_count: 100
    .vgpr_count: 256
    .agpr_count: 128
    .max_flat_workgroup_size: {64 * NW}
    .args:
      - {{ .offset: 0, .size: {karg}, .value_kind: by_value }}
...
.end_amdgpu_metadata
"""
    return head + body + tail


def main(out_path, dilated=False, global_tokens=False):
    """Write the kernel (the dilated or the global-token variant) to
    out_path; returns its name."""
    assert not (dilated and global_tokens)
    DIL["on"], GLB["on"] = dilated, global_tokens
    try:
        text = render()
        name = kernel_name()
    finally:
        DIL["on"] = GLB["on"] = False
    with open(out_path, "w") as f:
        f.write(text)
    return name


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else os.path.join(os.getcwd(), NAME + ".s"))
