"""Generator of the gfx950 assembly kernel for multi-head local + strided
attention forward, bf16, head size 64 (build step: writes a .s file).

The operation is the masked attention of Learn: Sparse & Sliding-Window
Attention, §3 equation, A = softmax(Q K^T * scale + log M) V, with M the
sliding window j in [i - W + 1, i] ORed with the stride pattern (j mod s ==
0 and j <= i; the swa_mask and strided_mask of "Attention Variants
Compared"), computed with the tiled online softmax of the same page.  The
stride s is 0 (a plain window) or a power of two from 64 to 2^18, so that a
64-key tile at a multiple of 64 holds at most one stride key, its first.

Work decomposition
  Item = 128 query rows of two consecutive (batch, head) pairs bh0, bh0 + 1
  (B * H even; the key/value head of a query head is itself).  Wave w takes
  head bh0 + (w >> 2) and rows 32 g .. +31 with g = w & 3 for the first
  head and 3 - (w & 3) for the second, so the two waves of a SIMD (w and
  w + 4) hold rows from both ends of the block and every SIMD's pair does
  about the same work in each step (masked tiles, dead tiles).  LDS stages (four) hold per
  64-key tile the K and V tiles of both heads (K: 64 rows of 128 bytes,
  padded to 144; V: 32 pairs of rows at a pitch of 320 bytes, so that any
  four consecutive rows fall on disjoint LDS banks for the transposed
  reads; 38,912 bytes per stage, 155,648 in all): one workgroup per CU, two
  waves per SIMD.  Per tile a wave issues 8 MFMAs of S^T = K Q^T and 8
  of O^T += V^T P^T.
  An item walks first its prefix, the stride keys below its band (keys
  0, s, 2 s, ... below the band's first key: every row of the item attends
  them), gathered 64 at a time into a tile by LDS-DMA with a row pitch of
  s rows, then the band tiles of its 128 rows.  The stride keys inside the
  band enter through the cell mask of the band's partial tiles.
  Persistent grid as in gen_fwd_gqa.py: workgroup g takes items g, g + grid,
  ..., each XCD a contiguous run of items (row blocks ascending per pair of
  heads); the last step of an item loads the next item's Q fragments and
  first two tiles.  Epilogue: O / l -> bf16 rows staged through LDS,
  128-byte row stores, and the optional log-sum-exp.

The softmax, the row maxima and the P V building blocks are those of
gen_fwd_gqa.py (imported with their register assignments), as in
gen_fwd_diff.py.
"""
import os
import struct
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gen_fwd_gqa as g                      # noqa: E402
from gen_fwd_gqa import (I, Prog, v, s, regs_of, EMPTY, resolve,  # noqa: E402
                         udiv, rsrc, max_ops, exp_ops, pack_ops, merge_rr,
                         settle_previous, after, AHEAD, RING, SLACK,
                         S_BUF, P_BUF, V_KLANE, V_VLANE, V_KADDR, V_VADDR, V_M, V_MTHR, V_L, V_LT,
                         V_IBASE, V_COL, V_HL, V_T, V_LANE, A_KR, A_VR, S_C, S_NINF, S_ONES, S_WM1,
                         S_FLAG, S_CMP, S_X)

# ---------------------------------------------------------------------------
# sizes
D = 64                        # head size (q, k, v)
ROW = 2 * D + 16              # padded LDS row of a K tile, bytes
KTILE = 64 * ROW              # 9216: 9 chunks of 1 KiB
VPAIR = 4 * D + 64            # LDS pitch of a pair of V rows (two rows of 128 bytes, 64 bytes of padding)
VTILE = 32 * VPAIR            # 10240: 10 chunks
STAGE = 2 * KTILE + 2 * VTILE  # K of both heads, then V of both heads
NSTAGE = 4
LDS_BYTES = NSTAGE * STAGE    # 155648
TILE_OFF = (0, KTILE, 2 * KTILE, 2 * KTILE + VTILE)   # K0, K1, V0, V1 within a stage
# the chunks past 8 of each tile (K0 8, K1 8, V0 8, V0 9, V1 8, V1 9): the
# fifth DMA load of waves 0..5; waves 6 and 7 repeat those of waves 0 and 1
FIFTH = [(0, 8), (1, 8), (2, 8), (2, 9), (3, 8), (3, 9), (0, 8), (1, 8)]
OROW = 2 * D + 16             # LDS row of the output staging
EPI_STORES = 4                # output stores of a wave per item (the log-sum-exp store aside)
KARG_BYTES = 80
NAME = "swa_fwd_mha_d64_str"
assert 8 * 32 * OROW <= STAGE and LDS_BYTES <= 160 * 1024
assert KTILE % 1024 == 0 and VTILE % 1024 == 0

# floor(x / 144) and floor(x / 320) as (x * M) >> 24 over a tile
M144 = -(-(1 << 24) // ROW)
M320 = -(-(1 << 24) // VPAIR)
for _x in range(VTILE):
    assert (_x * M144) >> 24 == _x // ROW and (_x * M320) >> 24 == _x // VPAIR

# ---------------------------------------------------------------------------
# registers (the ones shared with the imported building blocks keep their
# numbers: score and P buffers, softmax state, temporaries, the fragment
# rings, S_C, S_NINF, S_ONES, S_WM1, S_FLAG and the flag temporaries, S_X)
# LDS-DMA source offsets per lane: K chunk w, V chunk w and the wave's
# fifth chunk, for the rows of a band tile (pitch 128 bytes), of a prefix
# tile (pitch s rows) and of the tile being loaded
V_DBK, V_DBV, V_DB5 = v(85), v(86), v(80)
V_DPK, V_DPV, V_DP5 = v(87), v(88), v(124)
V_DCK, V_DCV, V_DC5 = v(89), v(90), v(126)
V_HL0 = v(100)                       # 1 on the lanes of the first key quad (lane < 32), else 0
V_LOFF = v(101)                      # log-sum-exp store offset: row * 4
V_OWL, V_ORDL, V_OST = v(120), v(121), v(122)
V_QLANE = v(127)                     # (lane % 32) * 128 + 16 (lane / 32)

A_O = g.a(0, 32)                     # O^T: block db at 16 db (values 32 db .. +31)
A_Q = g.a(64, 16)                    # Q^T fragments: ks at 4 ks

S_KARG, S_WG, S_BASE = s(0, 2), s(2), s(3)
S_Q, S_K, S_V, S_OUT, S_LSE = s(4, 2), s(6, 2), s(8, 2), s(10, 2), s(12, 2)
S_N, S_W, S_TOTAL, S_STRIDE, S_NRB = s(14), s(15), s(16), s(17), s(18)
assert S_C.i == 19
S_SSTR, S_LGS, S_NPRE, S_PEND = s(20), s(21), s(22), s(23)
S_WAVE, S_PPART, S_SBIT, S_VID = s(24), s(25), s(26), s(27)
S_BH, S_R0W, S_TLO, S_T, S_J, S_NB, S_R0W32, S_WAVE1K = (s(28), s(29), s(30), s(31), s(32), s(33), s(34),
                                                          s(35))
S_RSK0, S_RSK1, S_RSV0, S_RSV1, S_RSQ, S_RSO = s(36, 4), s(40, 4), s(44, 4), s(48, 4), s(52, 4), s(56, 4)
S_FULL = [s(77), s(60)]              # by phase: 1 full, 0 / 4 band partial (4: key0 is a stride key),
S_K0P = [s(61), s(76)]               # 2 partial prefix tile; key0 (prefix: 64 x prefix index)
S_SBW, S_SOFF, S_SB, S_XOFF = s(62), s(66), s(67), s(72)
assert (S_WM1.i, S_NINF.i, S_ONES.i, S_FLAG.i) == (63, 64, 65, 68)
S_RSL, S_RSE = s(92, 4), s(96, 4)    # log-sum-exp; the wave's fifth DMA chunk
S_FIFTH = s(73)                      # the tile (0..3: K0, K1, V0, V1) of the wave's fifth chunk


# ---------------------------------------------------------------------------
# building blocks of this kernel
def dma_ops():
    """This wave's LDS-DMA loads of the tile at key offset S_SOFF into the
    stage at S_SB, with lane offsets V_DCK / V_DCV / V_DC5 (band or prefix
    rows).  The stage holds the K tiles of heads 0 and 1 (9 chunks of 1 KiB
    each) and their V tiles (10 chunks each): wave w loads chunk w of each,
    and a fifth chunk (FIFTH) through its own descriptor."""
    ops = []
    for k, rs in enumerate((S_RSK0, S_RSK1, S_RSV0, S_RSV1)):
        def op(P, k=k, rs=rs):
            P.salu("s_add_u32", "m0", S_SBW, str(TILE_OFF[k]))
            P.dma(V_DCK if k < 2 else V_DCV, rs, S_SOFF)
        ops.append(op)

    def op(P):
        P.salu("s_add_u32", "m0", S_SB, S_XOFF)
        P.dma(V_DC5, S_RSE, S_SOFF)
    ops.append(op)
    return ops


def dma_tile(P):
    P.salu("s_add_u32", S_SBW, S_SB, S_WAVE1K)
    for op in dma_ops():
        op(P)


# K fragments n = 0..7: key half kb = n % 2, channels 16 ks .. +15 with
# ks = n / 2.  V^T fragments n = 0..7: key step n / 2 (key half kb, keys
# 16 hf .. +15 of it), values 32 db .. +31 with db = n % 2.  Ring slot n % 4.
def qk_read(P, n):
    kb, ks = n % 2, n // 2
    P.ds_read("ds_read_b128", A_KR.sub(4 * (n % RING), 4), V_KADDR, kb * 32 * ROW + ks * 32)


def qk_mfma(P, n, sbuf):
    kb, ks = n % 2, n // 2
    dst = v(sbuf + 16 * kb, 16)
    P.mfma(dst, A_KR.sub(4 * (n % RING), 4), A_Q.sub(4 * ks, 4), None if ks == 0 else dst)


def pv_read(P, n):
    kstep, db = divmod(n, 2)
    kb, hf = divmod(kstep, 2)
    slot = A_VR.sub(4 * (n % RING), 4)
    off = (kb * 32 + hf * 16) // 2 * VPAIR + db * 64
    P.ds_read("ds_read_b64_tr_b16", slot.sub(0, 2), V_VADDR, off)
    P.ds_read("ds_read_b64_tr_b16", slot.sub(2, 2), V_VADDR, off + 4 * VPAIR)


def pv_mfma(P, n):
    kstep, db = divmod(n, 2)
    kb, hf = divmod(kstep, 2)
    o = A_O.sub(16 * db, 16)
    P.mfma(o, A_VR.sub(4 * (n % RING), 4), v(P_BUF + 8 * kb + 4 * hf, 4), o)


NV = 8                                # V^T fragments per tile


def pack(sbuf, kb):
    return pack_ops(sbuf, kb, vlast=4 * kb + 3)


def interleave(P, order, sbuf_next, valu_ops, extra_ops=(), v_ready=0):
    """The MFMAs of `order` (("k", n): QK fragment n into sbuf_next; ("v",
    n): PV fragment n) with their fragment reads AHEAD ahead, the VALU ops
    spread evenly by issue cost (after() constraints kept) and the extra
    ops (DMA loads, scalar set-up) one every few MFMAs."""
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
    every = max(1, (len(order) - 2) // max(1, len(extra))) if extra else 0
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
        out = [("v", 0), ("v", 1), ("v", 2), ("v", 3)]
        for k in range(4):
            out += [("k", k), ("v", 4 + k)]
        return out + [("k", k) for k in range(4, 8)]
    if has_qk:
        return [("k", k) for k in range(8)]
    if has_pv:
        return [("v", k) for k in range(NV)]
    return []


def band_mask(P, sbuf, k0, full):
    """Per-cell mask of band tile j (key offset in k0) on score buffer sbuf:
    key j attends row i iff 0 <= i - j <= W - 1, or j is a stride key and
    j <= i.  The only stride key of the tile is its first (bit 2 of `full`
    set), which only lanes of the first key quad (lane < 32) hold, as key
    kc = 0 of key half 0.  One 32-bit word per lane and key half (bit kc set
    iff the lane's key kc attends), then one bit-field select per score."""
    tb, tlo, thi, tm1, tm2, tk, tg = V_T[0], V_T[1], V_T[2], V_T[3], V_T[4], V_T[5], V_T[6]
    for kb in range(2):
        P.salu("s_add_u32", S_X[3], k0, str(32 * kb))
        P.valu("v_subrev_u32", tb, S_X[3], V_IBASE)                      # base = i - 4 hl - key0
        P.valu("v_subrev_u32", tlo, S_WM1, tb)                            # base - (W - 1)
        P.valu("v_max_i32", tlo, "0", tlo)
        P.valu("v_min_i32", thi, "31", tb)
        P.valu("v_lshlrev_b32_e64", tm1, thi, "2")
        P.valu("v_add_u32", tm1, "-1", tm1)                                # (2 << hi) - 1
        P.valu("v_lshlrev_b32_e64", tm2, tlo, "-1")                        # ~0 << lo
        P.valu("v_and_b32", tm1, tm1, tm2)
        P.add(I(f"  v_cmp_le_i32 vcc, {tlo}, {thi}", "vcmp", regs_of(tlo, thi), g.VCC))
        P.valu("v_cndmask_b32", tm1, "0", tm1, "vcc")
        if kb == 0:
            # the stride key (bit 0 on the lanes of the first key quad), if
            # it does not lie past the row
            P.salu("s_lshr_b32", S_X[4], full, "2")
            P.valu("v_and_b32", tg, S_X[4], V_HL0)
            P.add(I(f"  v_cmp_le_i32 vcc, 0, {tb}", "vcmp", regs_of(tb), g.VCC))
            P.valu("v_cndmask_b32", tg, "0", tg, "vcc")
            P.valu("v_or_b32", tm1, tm1, tg)
        select(P, sbuf, kb, tm1, tk)


def select(P, sbuf, kb, word, tk):
    for r in range(16):
        kc = (r % 4) + 8 * (r // 4)
        sr = v(sbuf + 16 * kb + r)
        P.valu("v_bfe_i32", tk, word, str(kc), "1")
        P.valu("v_bitop3_b32", sr, sr, S_NINF, tk, extra="bitop3:0xe4")


def prefix_mask(P, sbuf, k0):
    """Mask of the item's last prefix tile when it is partial: its key kc
    (prefix index k0 + kc) exists iff k0 + kc < the item's prefix count."""
    tb, thi, tm1, tk = V_T[0], V_T[2], V_T[3], V_T[5]
    P.valu("v_lshlrev_b32", V_T[7], "2", V_HL)                          # 4 hl
    for kb in range(2):
        P.salu("s_sub_u32", S_X[3], S_NPRE, k0)
        P.salu("s_sub_u32", S_X[3], S_X[3], str(1 + 32 * kb))            # count - 1 - 32 kb
        P.valu("v_sub_u32", tb, S_X[3], V_T[7])
        P.valu("v_min_i32", thi, "31", tb)
        P.valu("v_lshlrev_b32_e64", tm1, thi, "2")
        P.valu("v_add_u32", tm1, "-1", tm1)                                # (2 << hi) - 1
        P.add(I(f"  v_cmp_le_i32 vcc, 0, {thi}", "vcmp", regs_of(thi), g.VCC))
        P.valu("v_cndmask_b32", tm1, "0", tm1, "vcc")
        select(P, sbuf, kb, tm1, tk)


def mask(P, phase):
    """The cell mask of tile j (phase j % 2) by its kind: none for a full
    tile, the band mask, or the prefix mask."""
    sb = S_BUF[phase]
    done, pre = P.new_label("masked"), P.new_label("premask")
    P.scmp("s_cmp_eq_u32", S_FULL[phase], "1")
    P.branch("s_cbranch_scc1", done)
    P.scmp("s_cmp_eq_u32", S_FULL[phase], "2")
    P.branch("s_cbranch_scc1", pre)
    band_mask(P, sb, S_K0P[phase], S_FULL[phase])
    P.branch("s_branch", done)
    P.label(pre)
    prefix_mask(P, sb, S_K0P[phase])
    P.label(done)


def tile_src(P, q, off_band, off_pre):
    """For step q of the item (SGPR): the key offset of its tile into
    S_SOFF (past the item's tiles: N rows, outside the descriptors, so the
    loads read zeros into a stage nothing reads) and its lane offsets into
    V_DCK / V_DCV / V_DC5.  off_band / off_pre are scalar temporaries."""
    P.salu("s_add_u32", off_band, S_TLO, q)
    P.salu("s_lshl_b32", off_band, off_band, "13")                    # band tile: 64 rows of 128 bytes
    P.salu("s_sub_u32", off_pre, q, S_BASE)
    P.salu("s_add_u32", S_X[11], S_LGS, "13")
    P.salu("s_lshl_b32", off_pre, off_pre, S_X[11])                   # prefix tile: 64 rows, pitch s rows
    P.scmp("s_cmp_lt_u32", q, S_PEND)
    P.salu("s_cselect_b32", S_SOFF, off_pre, off_band, reads_scc=True, writes_scc=False)
    P.salu("s_cselect_b64", s(S_X[2].i, 2), "-1", "0", reads_scc=True, writes_scc=False)
    for dc, db, dp in ((V_DCK, V_DBK, V_DPK), (V_DCV, V_DBV, V_DPV), (V_DC5, V_DB5, V_DP5)):
        P.valu("v_cndmask_b32", dc, db, dp, s(S_X[2].i, 2))
    P.scmp("s_cmp_lt_u32", q, S_T)
    P.salu("s_cselect_b32", S_SOFF, S_SOFF, S_NB, reads_scc=True, writes_scc=False)


def tile_kind(i, pn):
    """For step i (SGPR): key0 of its tile into S_K0P[pn] (prefix: 64 x its
    prefix index) and its kind into S_FULL[pn]: a band tile is full when
    every cell attends this wave's 32 rows, else partial (0, or 4 when its
    first key is a stride key); a prefix tile is full unless it is the
    item's last and partial (2)."""
    def o1(P):
        P.salu("s_add_u32", S_X[6], S_TLO, i)
        P.salu("s_lshl_b32", S_X[6], S_X[6], "6")                     # band key0
        P.salu("s_sub_u32", S_X[7], i, S_BASE)
        P.salu("s_lshl_b32", S_X[7], S_X[7], "6")                     # 64 x prefix index
        P.scmp("s_cmp_lt_u32", i, S_PEND)
        P.salu("s_cselect_b32", S_K0P[pn], S_X[7], S_X[6], reads_scc=True, writes_scc=False)
        P.salu("s_cselect_b32", S_X[10], "1", "0", reads_scc=True, writes_scc=False)

    def o2(P):
        P.salu("s_add_u32", S_X[7], S_K0P[pn], "63")
        P.scmp("s_cmp_le_u32", S_X[7], S_R0W)                         # last key <= first row
        P.salu("s_cselect_b32", S_X[8], "1", "0", reads_scc=True, writes_scc=False)
        P.salu("s_add_u32", S_X[7], S_K0P[pn], S_W)
        P.scmp("s_cmp_ge_u32", S_X[7], S_R0W32)                       # key0 + W >= last row + 1
        P.salu("s_cselect_b32", S_X[8], S_X[8], "0", reads_scc=True, writes_scc=False)

    def o3(P):
        P.salu("s_add_u32", S_X[7], S_SSTR, "-1")
        P.salu("s_and_b32", S_X[7], S_K0P[pn], S_X[7])
        P.scmp("s_cmp_eq_u32", S_X[7], "0")                           # key0 a multiple of s
        P.salu("s_cselect_b32", S_X[7], S_SBIT, "0", reads_scc=True, writes_scc=False)
        P.scmp("s_cmp_eq_u32", S_X[8], "1")
        P.salu("s_cselect_b32", S_X[8], "1", S_X[7], reads_scc=True, writes_scc=False)

    def o4(P):
        P.scmp("s_cmp_eq_u32", i, S_PPART)
        P.salu("s_cselect_b32", S_X[7], "2", "1", reads_scc=True, writes_scc=False)
        P.scmp("s_cmp_eq_u32", S_X[10], "1")
        P.salu("s_cselect_b32", S_FULL[pn], S_X[7], S_X[8], reads_scc=True, writes_scc=False)
    return [o1, o2, o3, o4]


def setup_ops(pn):
    """Scalar set-up of step i = j + 1 (S_J = j): the DMA of tile i + 2
    (offsets, lane offsets, stage, M0 bases), key0 and kind of tile i; after
    this step's DMA loads (they overwrite what those read)."""
    def o1(P):
        P.salu("s_add_u32", S_X[9], S_J, "1")                  # i
        P.salu("s_add_u32", S_X[4], S_X[9], "2")               # step i + 2

    def o2(P):
        tile_src(P, S_X[4], S_X[5], S_X[6])

    def o3(P):
        P.salu("s_and_b32", S_SB, S_X[4], "3")
        P.salu("s_mul_i32", S_SB, S_SB, str(STAGE))
        P.salu("s_add_u32", S_SBW, S_SB, S_WAVE1K)
    return [o1, o2, o3] + tile_kind(S_X[9], pn)


def v_prefetch_ops():
    """The first AHEAD V^T fragments of the next P V product, read before
    the next barrier."""
    def addr(P):
        P.salu("s_and_b32", S_X[12], S_J, "3")
        P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
        P.valu("v_add_u32", V_VADDR, S_X[12], V_VLANE)
    return [after(op, "v", NV - 1) for op in [addr] + [(lambda P, n=n: pv_read(P, n)) for n in range(AHEAD)]]


def k_addr_next(P):
    P.salu("s_add_u32", S_X[12], S_J, "2")
    P.salu("s_and_b32", S_X[12], S_X[12], "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)


def redo_previous(P, phase):
    """At the start of step j + 1 (phase `phase`): if a row's sum of the p
    of tile j, taken without the row maximum, exceeds 2^SLACK (flag S_CMP,
    set at the end of step j), compute S(j) = K(j) Q^T again (tile j is
    still in its stage, the Q fragments in place; its score buffer is free),
    mask it, and take its softmax again with the row maximum, before the
    running sum and O take in tile j.  Placed after the barrier, the check
    waits for nothing the step does not wait for anyway."""
    p = 1 - phase
    sb = S_BUF[p]
    skip = P.new_label("nomax")
    P.scmp("s_cmp_eq_u64", S_CMP, "0")
    P.branch("s_cbranch_scc1", skip)
    P.salu("s_add_u32", S_X[12], S_J, "-1")
    P.salu("s_and_b32", S_X[12], S_X[12], "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)
    interleave(P, mfma_order(True, False), sb, [])
    mask(P, p)
    for op in max_ops(sb) + merge_rr([exp_ops(sb, 0), exp_ops(sb, 1)]) + pack(sb, 0) + pack(sb, 1):
        op(P)
    P.salu("s_add_u32", S_X[12], S_J, "1")                     # the K fragments of this step's product
    P.salu("s_and_b32", S_X[12], S_X[12], "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)
    P.label(skip)


def sum_check(P):
    """S_CMP = the lanes whose sum of this tile's p exceeds 2^SLACK (a p
    may then exceed it: the tile's maximum may lie more than SLACK above
    the running maximum)."""
    t = V_T[15]
    P.valu("v_add_f32", t, V_LT[0], V_LT[1])
    two_slack = struct.unpack("<I", struct.pack("<f", 2.0 ** SLACK))[0]
    P.salu("s_mov_b32", S_X[13], hex(two_slack), writes_scc=False)
    P.add(I(f"  v_cmp_lt_f32 {S_CMP}, {S_X[13]}, {t}", "vcmp", regs_of(S_X[13], t), S_CMP.regs()))


def iteration(P, phase, has_qk, has_pv, first, exact=True):
    """One tile j of the pipeline, as in gen_fwd_gqa.  exact=False: no row
    maximum; the row sums are checked at the end of the step and, where
    one exceeds 2^SLACK, the step is redone at the start of the next
    (redo_previous).  Every step but an item's first starts with that
    check of its predecessor (an exact step clears the flag)."""
    sb_cur, sb_next = S_BUF[phase], S_BUF[1 - phase]
    P.comment(f"iteration phase {phase} qk={has_qk} pv={has_pv}")
    # the first step waits for tile 1 of its item, not for the previous
    # item's output stores (the last vector memory operations issued)
    P.waitcnt(vm=EPI_STORES if first else 0)
    P.barrier()
    if has_pv:
        redo_previous(P, phase)
        settle_previous(P, o=A_O)
    if not has_qk:
        last_step(P, phase, has_pv)
        return
    mask(P, phase)
    P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)
    valu = ((max_ops(sb_cur) if exact else []) + merge_rr([exp_ops(sb_cur, 0), exp_ops(sb_cur, 1)])
            + pack(sb_cur, 0) + v_prefetch_ops() + pack(sb_cur, 1))
    extra = dma_ops() + setup_ops(1 - phase)
    interleave(P, mfma_order(has_qk, has_pv), sb_next, valu, extra, v_ready=AHEAD)
    if has_qk:
        if exact:
            P.salu("s_mov_b64", S_CMP, "0", writes_scc=False)
        else:
            sum_check(P)
        k_addr_next(P)
    if not has_pv:
        P.valu("v_add_f32", V_MTHR, str(SLACK), V_M)
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)


def last_step(P, phase, has_pv):
    """The softmax of an item's last tile (with its row maximum), the P V
    product of the one before (has_pv), and the loads of the next item.
    Key halves of the tile that lie past every row of the wave (the tile is
    the diagonal's or the one after it) take no softmax: every key past
    the rows (2: the whole tile) gives p = 0, and the epilogue skips their
    P V fragments too; only key half 1 past the rows (1) keeps half 0."""
    sb_cur = S_BUF[phase]
    order = mfma_order(False, has_pv)
    dead, half, joined = P.new_label("lastdead"), P.new_label("lasthalf"), P.new_label("lastdone")
    P.salu("s_add_u32", S_X[0], S_R0W, "32")
    P.scmp("s_cmp_ge_u32", S_K0P[phase], S_X[0])
    P.branch("s_cbranch_scc1", dead)
    P.scmp("s_cmp_ge_u32", S_K0P[phase], S_R0W)
    P.branch("s_cbranch_scc1", half)
    for kind in ("full", "half", "dead"):
        if kind == "half":
            P.label(half)
        elif kind == "dead":
            P.label(dead)
        if kind != "dead":
            mask(P, phase)
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)
        if kind == "dead":
            for k in range(2):
                P.valu("v_mov_b32", V_LT[k], "0")
        item_loads(P, first=False)
        if kind == "full":
            valu = (max_ops(sb_cur) + merge_rr([exp_ops(sb_cur, 0), exp_ops(sb_cur, 1)]) + pack(sb_cur, 0)
                    + v_prefetch_ops() + pack(sb_cur, 1))
        elif kind == "half":
            valu = max_ops(sb_cur) + exp_ops(sb_cur, 0) + pack(sb_cur, 0) + v_prefetch_ops()
        else:
            valu = []
        interleave(P, order, None, valu, [], v_ready=AHEAD)
        if kind != "dead":
            P.branch("s_branch", joined)
    P.label(joined)
    if not has_pv:
        P.valu("v_add_f32", V_MTHR, str(SLACK), V_M)
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)


def epilogue(P, phase):
    """O += V(T-1)^T P(T-1), then O / l -> bf16 rows (staged through the
    stage of tile T-2, free after the barrier: the stage of tile T-1 is
    still being read and the next two hold the next item's first tiles),
    and the log-sum-exp.  Ends the workgroup, or goes on with its next
    item."""
    P.barrier()
    settle_previous(P, o=A_O)
    # the key halves of the last tile past the wave's rows (as in last_step;
    # the next item's loads have replaced S_R0W: lane 0's V_IBASE is the
    # wave's first row)
    dead, half, joined = P.new_label("pvdead"), P.new_label("pvhalf"), P.new_label("pvdone")
    P.add(I(f"  v_readfirstlane_b32 {S_X[13]}, {V_IBASE}", "rfl", V_IBASE.regs(), S_X[13].regs()))
    P.salu("s_add_u32", S_X[12], S_X[13], "32")
    P.scmp("s_cmp_ge_u32", S_K0P[phase], S_X[12])
    P.branch("s_cbranch_scc1", dead)
    P.scmp("s_cmp_ge_u32", S_K0P[phase], S_X[13])
    P.branch("s_cbranch_scc1", half)
    interleave(P, mfma_order(False, True), None, [], v_ready=AHEAD)
    P.branch("s_branch", joined)
    P.label(half)
    interleave(P, [("v", n) for n in range(4)], None, [], v_ready=AHEAD)
    P.label(dead)
    P.label(joined)
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
    P.salu("s_add_u32", S_X[0], S_J, "-1")
    P.salu("s_and_b32", S_X[0], S_X[0], "3")
    P.salu("s_mul_i32", S_X[0], S_X[0], str(STAGE))
    P.salu("s_mul_i32", S_X[2], S_WAVE, str(32 * OROW))
    P.salu("s_add_u32", S_X[1], S_X[0], S_X[2])                    # this wave's region
    ow, ord_ = t[12], t[13]
    P.valu("v_add_u32", ow, S_X[1], V_OWL)
    P.valu("v_add_u32", ord_, S_X[1], V_ORDL)
    for db in range(2):
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
            P.add(I(f"  ds_write_b64 {ow}, {v(pk0.i, 2)} offset:{db * 64 + r4 * 16}", "lds",
                    regs_of(ow, v(pk0.i, 2)), EMPTY))
    # rows 8 kk + lane / 8, bytes 16 (lane % 8) .. +15
    ob = S_BUF[0]
    for kk in range(4):
        P.ds_read("ds_read_b128", v(ob + 4 * kk, 4), ord_, kk * 8 * OROW)
    for kk in range(4):
        P.salu("s_mov_b32", S_X[3 + kk], str(kk * 8 * 128), writes_scc=False)
        P.add(I(f"  buffer_store_dwordx4 {v(ob + 4 * kk, 4)}, {V_OST}, {S_RSO}, {S_X[3 + kk]} offen",
                "vstore", regs_of(v(ob + 4 * kk, 4), V_OST, S_RSO, S_X[3 + kk]), EMPTY))
    P.scmp("s_cmp_lt_u32", S_VID, S_TOTAL)
    P.branch("s_cbranch_scc1", ".Litem")
    P.add(I("  s_endpgm", "branch"))


def item_loads(P, first):
    """Start the workgroup's next item (S_VID + S_STRIDE; S_VID itself for
    the first): pair of heads, row block, prefix and band, descriptors,
    then the loads of its Q fragments and of its tiles 0 and 1 into stages
    S_J + 1 and S_J + 2 (mod 4), not waited for here.  Its step counter
    starts at S_BASE = (S_J + 1) & 3; step q < S_PEND is prefix tile
    q - S_BASE, a later one band tile S_TLO + q."""
    skip = None
    if not first:
        P.salu("s_add_u32", S_VID, S_VID, S_STRIDE)
        P.scmp("s_cmp_ge_u32", S_VID, S_TOTAL)
        skip = P.new_label("nonext")
        P.branch("s_cbranch_scc1", skip)
    P.salu("s_add_u32", S_BASE, S_J, "1")
    P.salu("s_and_b32", S_BASE, S_BASE, "3")
    # item -> logical id (each XCD a contiguous run), then (pair of heads,
    # 128-row block), row blocks ascending
    lid, pair, rb = S_X[9], S_X[10], S_X[11]
    P.salu("s_and_b32", S_X[0], S_TOTAL, "7")
    P.salu("s_and_b32", S_X[1], S_VID, "7")
    P.salu("s_lshr_b32", S_X[2], S_TOTAL, "3")
    P.salu("s_mul_i32", S_X[1], S_X[1], S_X[2])
    P.salu("s_lshr_b32", S_X[3], S_VID, "3")
    P.salu("s_add_u32", S_X[1], S_X[1], S_X[3])
    P.scmp("s_cmp_eq_u32", S_X[0], "0")
    P.salu("s_cselect_b32", lid, S_X[1], S_VID, reads_scc=True, writes_scc=False)
    udiv(P, lid, S_NRB, pair, rb, V_T[1], V_T[2])
    P.salu("s_lshl_b32", S_X[8], pair, "1")                    # bh0
    P.salu("s_lshr_b32", S_X[0], S_WAVE, "2")
    P.salu("s_add_u32", S_BH, S_X[8], S_X[0])                  # this wave's head
    P.salu("s_lshl_b32", S_X[5], rb, "7")                      # r0
    # row group (w & 3) for the first head, 3 - (w & 3) for the second: the
    # two waves of a SIMD take rows from both ends of the block
    P.salu("s_lshr_b32", S_X[1], S_WAVE, "2")
    P.salu("s_mul_i32", S_X[1], S_X[1], "3")
    P.salu("s_and_b32", S_X[0], S_WAVE, "3")
    P.salu("s_xor_b32", S_X[0], S_X[0], S_X[1])
    P.salu("s_lshl_b32", S_X[0], S_X[0], "5")
    P.salu("s_add_u32", S_R0W, S_X[5], S_X[0])                 # this wave's first row
    # band of rows r0 .. r0+127: key tiles t_lo .. t_hi
    tlo = S_X[6]
    P.salu("s_sub_i32", S_X[0], S_X[5], S_W)
    P.salu("s_add_i32", S_X[0], S_X[0], "1")
    P.salu("s_max_i32", S_X[0], S_X[0], "0")
    P.salu("s_lshr_b32", tlo, S_X[0], "6")
    P.salu("s_add_u32", S_X[1], S_X[5], "127")
    P.salu("s_sub_u32", S_X[2], S_N, "1")
    P.salu("s_min_u32", S_X[1], S_X[1], S_X[2])
    P.salu("s_lshr_b32", S_X[1], S_X[1], "6")
    P.salu("s_sub_u32", S_T, S_X[1], tlo)
    P.salu("s_add_u32", S_T, S_T, "1")                         # band tiles
    # prefix: the stride keys below the band, ceil(64 t_lo / s) of them,
    # in ceil(count / 64) tiles
    P.salu("s_lshl_b32", S_X[0], tlo, "6")
    P.salu("s_add_u32", S_X[0], S_X[0], S_SSTR)
    P.salu("s_add_u32", S_X[0], S_X[0], "-1")
    P.salu("s_lshr_b32", S_X[0], S_X[0], S_LGS)
    P.scmp("s_cmp_eq_u32", S_SSTR, "0")
    P.salu("s_cselect_b32", S_NPRE, "0", S_X[0], reads_scc=True, writes_scc=False)
    P.salu("s_add_u32", S_X[1], S_NPRE, "63")
    P.salu("s_lshr_b32", S_X[1], S_X[1], "6")                  # prefix tiles
    P.salu("s_add_u32", S_PEND, S_BASE, S_X[1])
    P.salu("s_add_u32", S_T, S_T, S_PEND)                      # first step past the item
    P.salu("s_sub_i32", S_TLO, tlo, S_PEND)                    # band tile of step q: S_TLO + q
    P.salu("s_and_b32", S_X[2], S_NPRE, "63")
    P.salu("s_add_u32", S_X[3], S_PEND, "-1")
    P.scmp("s_cmp_eq_u32", S_X[2], "0")
    P.salu("s_cselect_b32", S_PPART, "-1", S_X[3], reads_scc=True, writes_scc=False)
    # descriptors: K and V of both heads, Q of this wave's head (rows of 128
    # bytes)
    nb = S_X[7]
    P.salu("s_lshl_b32", nb, S_N, "7")
    rsrc(P, S_RSK0, S_K, S_X[8], nb, nb)
    rsrc(P, S_RSV0, S_V, S_X[8], nb, nb)
    P.salu("s_add_u32", S_X[8], S_X[8], "1")
    rsrc(P, S_RSK1, S_K, S_X[8], nb, nb)
    rsrc(P, S_RSV1, S_V, S_X[8], nb, nb)
    # the fifth chunk's descriptor: that of its tile
    for h in (0, 2):
        P.scmp("s_cmp_eq_u32", S_FIFTH, "0")
        P.salu("s_cselect_b64", S_RSE.sub(h, 2), S_RSK0.sub(h, 2), S_RSK1.sub(h, 2), reads_scc=True,
               writes_scc=False)
        P.scmp("s_cmp_eq_u32", S_FIFTH, "2")
        P.salu("s_cselect_b64", S_RSE.sub(h, 2), S_RSV0.sub(h, 2), S_RSE.sub(h, 2), reads_scc=True,
               writes_scc=False)
        P.scmp("s_cmp_eq_u32", S_FIFTH, "3")
        P.salu("s_cselect_b64", S_RSE.sub(h, 2), S_RSV1.sub(h, 2), S_RSE.sub(h, 2), reads_scc=True,
               writes_scc=False)
    rsrc(P, S_RSQ, S_Q, S_BH, nb, nb)
    qoff = V_T[3]
    P.salu("s_lshl_b32", S_X[0], S_R0W, "7")
    P.valu("v_add_u32", qoff, S_X[0], V_QLANE)
    for ks in range(4):
        P.buf_load(A_Q.sub(4 * ks, 4), qoff, S_RSQ, "0", 32 * ks, track=False)
    # steps 0 and 1 (step 1 also when the item has one tile: read as data or
    # zeros, never used)
    for k in range(2):
        P.salu("s_add_u32", S_X[4], S_BASE, str(k))
        tile_src(P, S_X[4], S_X[5], S_X[6])
        P.salu("s_and_b32", S_SB, S_X[4], "3")
        P.salu("s_mul_i32", S_SB, S_SB, str(STAGE))
        dma_tile(P)
    if skip:
        P.label(skip)


def item_start(P):
    P.label(".Litem")
    P.salu("s_lshl_b32", S_X[7], S_N, "7")
    rsrc(P, S_RSO, S_OUT, S_BH, S_X[7], S_X[7])
    P.salu("s_lshl_b32", S_X[7], S_N, "2")
    rsrc(P, S_RSL, S_LSE, S_BH, S_X[7], S_X[7])
    P.salu("s_add_u32", S_R0W32, S_R0W, "32")
    t = V_T
    P.valu("v_add_u32", t[5], S_R0W, V_COL)                    # row
    P.valu("v_lshlrev_b32", V_LOFF, "2", t[5])
    P.valu("v_lshlrev_b32", t[7], "2", V_HL)
    P.valu("v_sub_u32", V_IBASE, t[5], t[7])
    # output store offset: row r0w + lane / 8, bytes 16 (lane % 8)
    P.valu("v_lshrrev_b32", t[0], "3", V_LANE)
    P.valu("v_add_u32", t[0], S_R0W, t[0])
    P.valu("v_lshlrev_b32", t[0], "7", t[0])
    P.valu("v_and_b32", t[1], "7", V_LANE)
    P.valu("v_lshlrev_b32", t[1], "4", t[1])
    P.valu("v_add_u32", V_OST, t[0], t[1])
    P.valu("v_mov_b32", V_M, "0xf149f2ca")             # -1e30
    P.valu("v_mov_b32", V_MTHR, "0xf149f2ca")
    for k in range(2):
        P.valu("v_mov_b32", V_L[k], "0")
    for k in range(A_O.n):
        P.add(I(f"  v_accvgpr_write_b32 {A_O.sub(k)}, 0", "valu", EMPTY, A_O.sub(k).regs()))
    P.salu("s_sub_u32", S_J, S_BASE, "1")
    for op in setup_ops(0):
        op(P)
    # Q and tile 0 in: all but tile 1's loads and the previous item's
    # output stores
    P.waitcnt(vm=len(dma_ops()) + EPI_STORES)
    P.barrier()
    P.salu("s_mov_b32", S_J, S_BASE, writes_scc=False)
    P.salu("s_mul_i32", S_X[12], S_BASE, str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)
    interleave(P, mfma_order(True, False), S_BUF[0], [])
    P.salu("s_add_u32", S_X[12], S_BASE, "1")
    P.salu("s_and_b32", S_X[12], S_X[12], "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)


def _chunk_src_v(P, dst, pos, shift, t):
    """dst = source byte offset of V tile byte `pos` (a VGPR): pair p =
    pos / 320 holds rows 2 p and 2 p + 1 in its first 256 bytes; a byte at
    w = pos % 320 is row 2 p + (w >> 7) & 1, column w & 127 (the padding
    bytes fetch row 2 p's first 64 bytes again, never read)."""
    P.salu("s_mov_b32", S_X[11], str(M320), writes_scc=False)
    P.valu("v_mul_lo_u32", t[11], pos, S_X[11])
    P.valu("v_lshrrev_b32", t[11], "24", t[11])                # pair
    P.valu("v_mul_u32_u24", t[12], str(VPAIR), t[11])
    P.valu("v_sub_u32", t[12], pos, t[12])                     # byte within the pair
    P.valu("v_bfe_u32", t[13], t[12], "7", "1")
    P.valu("v_lshl_add_u32", t[11], t[11], "1", t[13])         # row
    P.valu("v_and_b32", t[12], "127", t[12])                   # column byte
    P.valu("v_lshlrev_b32", t[11], shift, t[11])
    P.valu("v_add_u32", dst, t[11], t[12])


def _chunk_src(P, dst, pos, shift, t):
    """dst = source byte offset of K tile byte `pos` (a VGPR): row << shift
    plus the column byte, the columns of padding replaced by 0."""
    P.salu("s_mov_b32", S_X[11], str(M144), writes_scc=False)
    P.valu("v_mul_lo_u32", t[11], pos, S_X[11])
    P.valu("v_lshrrev_b32", t[11], "24", t[11])                # row
    P.valu("v_mul_u32_u24", t[12], str(ROW), t[11])
    P.valu("v_sub_u32", t[12], pos, t[12])                     # column byte
    P.add(I(f"  v_cmp_gt_u32 vcc, {2 * D}, {t[12]}", "vcmp", t[12].regs(), g.VCC))
    P.valu("v_cndmask_b32", t[12], "0", t[12], "vcc")
    P.valu("v_lshlrev_b32", t[11], shift, t[11])
    P.valu("v_add_u32", dst, t[11], t[12])


def prologue(P):
    P.smem("s_load_dwordx16", s(4, 16), S_KARG, "0x0")
    P.smem("s_load_dwordx4", s(20, 4), S_KARG, "0x40")
    P.valu("v_and_b32", V_T[0], "0x3ff", v(0))                # thread id
    P.valu("v_lshrrev_b32", V_T[1], "6", V_T[0])
    P.add(I(f"  v_readfirstlane_b32 {S_WAVE}, {V_T[1]}", "rfl", V_T[1].regs(), S_WAVE.regs()))
    P.valu("v_and_b32", V_LANE, "63", V_T[0])
    P.valu("v_and_b32", V_COL, "31", V_LANE)
    P.valu("v_lshrrev_b32", V_HL, "5", V_LANE)
    P.valu("v_xor_b32", V_HL0, "1", V_HL)
    P.waitcnt(lgkm=0)
    P.salu("s_mov_b32", S_VID, S_WG, writes_scc=False)
    P.salu("s_lshl_b32", S_WAVE1K, S_WAVE, "10")
    P.salu("s_lshl_b32", S_NB, S_N, "7")
    P.scmp("s_cmp_eq_u32", S_SSTR, "0")
    P.salu("s_cselect_b32", S_SBIT, "0", "4", reads_scc=True, writes_scc=False)
    # the fifth chunk (FIFTH): its tile and LDS offset in a stage
    for w, (k, c) in enumerate(FIFTH):
        P.scmp("s_cmp_eq_u32", S_WAVE, str(w))
        P.salu("s_cselect_b32", S_FIFTH, str(k), S_FIFTH if w else "0", reads_scc=True, writes_scc=False)
        P.salu("s_cselect_b32", S_XOFF, str(TILE_OFF[k] + 1024 * c), S_XOFF if w else "0", reads_scc=True,
               writes_scc=False)
    P.salu("s_sub_u32", S_WM1, S_W, "1")
    P.salu("s_mov_b32", S_NINF, "0xff800000", writes_scc=False)
    P.salu("s_mov_b32", S_ONES, "0x3f803f80", writes_scc=False)
    t = V_T
    # this wave's head: its K and V tiles
    P.salu("s_lshr_b32", S_X[1], S_WAVE, "2")
    P.salu("s_mul_i32", S_X[0], S_X[1], str(KTILE))
    # K fragment reads: row col, bytes 16 hl
    P.valu("v_mul_u32_u24", V_KLANE, str(ROW), V_COL)
    P.valu("v_lshlrev_b32", t[0], "4", V_HL)
    P.valu("v_add_u32", V_KLANE, V_KLANE, t[0])
    P.valu("v_add_u32", V_KLANE, S_X[0], V_KLANE)
    # V^T fragment reads: row r = 4 (grp / 2) + sl / 4 at (r / 2) * 320 +
    # (r % 2) * 128, bytes 32 (grp % 2) + 8 (sl % 4), grp = lane / 16,
    # sl = lane % 16
    P.salu("s_mul_i32", S_X[1], S_X[1], str(VTILE))
    P.valu("v_lshrrev_b32", t[0], "4", V_LANE)                 # grp
    P.valu("v_and_b32", t[1], "15", V_LANE)                    # sl
    P.valu("v_lshrrev_b32", t[2], "1", t[0])
    P.valu("v_lshlrev_b32", t[2], "2", t[2])
    P.valu("v_lshrrev_b32", t[3], "2", t[1])
    P.valu("v_add_u32", t[2], t[2], t[3])                      # r
    P.valu("v_lshrrev_b32", t[5], "1", t[2])
    P.valu("v_mul_u32_u24", t[5], str(VPAIR), t[5])
    P.valu("v_and_b32", t[2], "1", t[2])
    P.valu("v_lshlrev_b32", t[2], "7", t[2])
    P.valu("v_add_u32", t[2], t[2], t[5])
    P.valu("v_and_b32", t[3], "1", t[0])
    P.valu("v_lshlrev_b32", t[3], "5", t[3])
    P.valu("v_and_b32", t[4], "3", t[1])
    P.valu("v_lshlrev_b32", t[4], "3", t[4])
    P.valu("v_add_u32", t[2], t[2], t[3])
    P.valu("v_add_u32", t[2], t[2], t[4])
    P.valu("v_add_u32", t[2], S_X[1], t[2])
    P.valu("v_add_u32", V_VLANE, str(2 * KTILE), t[2])
    # Q rows of 128 bytes: row col, bytes 16 hl of each 32-byte group
    P.valu("v_lshlrev_b32", t[0], "7", V_COL)
    P.valu("v_lshlrev_b32", t[1], "4", V_HL)
    P.valu("v_add_u32", V_QLANE, t[0], t[1])
    # epilogue: output staging write (row col, 8 hl) and read (row lane / 8,
    # bytes 16 (lane % 8))
    P.valu("v_mul_u32_u24", t[0], str(OROW), V_COL)
    P.valu("v_lshlrev_b32", t[1], "3", V_HL)
    P.valu("v_add_u32", V_OWL, t[0], t[1])
    P.valu("v_lshrrev_b32", t[0], "3", V_LANE)
    P.valu("v_and_b32", t[1], "7", V_LANE)
    P.valu("v_lshlrev_b32", t[1], "4", t[1])
    P.valu("v_mul_u32_u24", V_ORDL, str(OROW), t[0])
    P.valu("v_add_u32", V_ORDL, V_ORDL, t[1])
    # DMA lane offsets: K chunk w, V chunk w and the fifth chunk, rows of a
    # band tile (pitch 128 bytes) and of a prefix tile (pitch s rows of 128
    # bytes)
    P.valu("v_lshlrev_b32", t[8], "4", V_LANE)                 # 16 lane
    P.valu("v_add_u32", t[10], S_WAVE1K, t[8])
    P.salu("s_add_u32", S_X[1], S_LGS, "7")
    _chunk_src(P, V_DBK, t[10], "7", t)
    _chunk_src(P, V_DPK, t[10], S_X[1], t)
    _chunk_src_v(P, V_DBV, t[10], "7", t)
    _chunk_src_v(P, V_DPV, t[10], S_X[1], t)
    # the fifth chunk: byte XOFF - TILE_OFF[FIFTH] + 16 lane of a K or V tile
    P.salu("s_mov_b32", S_X[2], "0", writes_scc=False)
    for k in (1, 2, 3):
        P.scmp("s_cmp_eq_u32", S_FIFTH, str(k))
        P.salu("s_cselect_b32", S_X[2], str(TILE_OFF[k]), S_X[2], reads_scc=True, writes_scc=False)
    P.salu("s_sub_u32", S_X[2], S_XOFF, S_X[2])
    P.valu("v_add_u32", t[9], S_X[2], t[8])
    _chunk_src(P, t[14], t[9], "7", t)
    _chunk_src_v(P, V_DB5, t[9], "7", t)
    P.scmp("s_cmp_lt_u32", S_FIFTH, "2")
    P.salu("s_cselect_b64", "vcc", "-1", "0", reads_scc=True, writes_scc=False)
    P.valu("v_cndmask_b32", V_DB5, V_DB5, t[14], "vcc")
    _chunk_src(P, t[14], t[9], S_X[1], t)
    _chunk_src_v(P, V_DP5, t[9], S_X[1], t)
    P.scmp("s_cmp_lt_u32", S_FIFTH, "2")
    P.salu("s_cselect_b64", "vcc", "-1", "0", reads_scc=True, writes_scc=False)
    P.valu("v_cndmask_b32", V_DP5, V_DP5, t[14], "vcc")
    P.salu("s_mov_b32", S_J, "-1", writes_scc=False)
    item_loads(P, first=True)
    P.waitcnt(vm=0)


def kernel_text():
    P = Prog()
    prologue(P)
    item_start(P)
    P.salu("s_add_u32", S_X[0], S_J, "1")
    P.scmp("s_cmp_ge_u32", S_X[0], S_T)
    P.branch("s_cbranch_scc1", ".Lsingle")
    iteration(P, 0, True, False, True)                         # j = 0
    P.salu("s_add_u32", S_J, S_J, "1")
    P.salu("s_add_u32", S_X[0], S_J, "1")
    P.scmp("s_cmp_ge_u32", S_X[0], S_T)
    P.branch("s_cbranch_scc1", ".Llast1")
    # j = 1 and 2 with the row maximum too: every row of the 128 attends a
    # key of tiles 0 .. 2 (a prefix tile's first key, or its band's), so
    # from j = 3 on the running maximum is finite
    for ph in (1, 0):
        iteration(P, ph, True, True, False)
        P.salu("s_add_u32", S_J, S_J, "1")
        P.salu("s_add_u32", S_X[0], S_J, "1")
        P.scmp("s_cmp_ge_u32", S_X[0], S_T)
        P.branch("s_cbranch_scc1", f".Llast{1 - ph}")
    P.label(".Lmid1")
    for ph in (1, 0):
        iteration(P, ph, True, True, False, exact=False)
        P.salu("s_add_u32", S_J, S_J, "1")
        P.salu("s_add_u32", S_X[0], S_J, "1")
        P.scmp("s_cmp_ge_u32", S_X[0], S_T)
        P.branch("s_cbranch_scc1", f".Llast{1 - ph}")
    P.branch("s_branch", ".Lmid1")
    for ph in range(2):
        P.label(f".Llast{ph}")
        iteration(P, ph, False, True, False)
        epilogue(P, ph)
    P.label(".Lsingle")
    iteration(P, 0, False, False, True)
    epilogue(P, 0)
    body = resolve(P.ins)
    return "\n".join(x.text for x in body)


def render():
    body = kernel_text()
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
  .amdhsa_kernarg_size {KARG_BYTES}
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
  - .name: {NAME}
    .symbol: {NAME}.kd
    .kernarg_segment_size: {KARG_BYTES}
    .group_segment_fixed_size: {LDS_BYTES}
    .private_segment_fixed_size: 0
    .kernarg_segment_align: 8
    .wavefront_size: 64
    .sgpr_count: 100
    .vgpr_count: 256
    .agpr_count: 128
    .max_flat_workgroup_size: 512
    .args:
      - {{ .offset: 0, .size: {KARG_BYTES}, .value_kind: by_value }}
...
.end_amdgpu_metadata
"""
    return head + body + tail


def main(out_path):
    """Write the kernel to out_path; returns its name."""
    with open(out_path, "w") as f:
        f.write(render())
    return NAME


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else NAME + ".s")
