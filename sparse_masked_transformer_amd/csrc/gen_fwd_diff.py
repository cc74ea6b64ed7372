"""Generator of the gfx950 assembly kernel for differential sliding-window
attention forward, bf16, query/key head size 64, value head size 128 (build
step: writes a .s file).

The operation is the differential attention of "Attention Variants — Sliding
Window, Sparse, Differential" (two attention maps from separate query/key
projections, the second subtracted from the first with weight lambda) over
the sliding window of Learn: Sparse & Sliding-Window Attention, §3 equation,
with one value cache read for both maps ("Attention Variants Compared", the
value cache of the differential variant):

  out = softmax(Q1 K1^T * scale + log M) V - lambda * softmax(Q2 K2^T * scale + log M) V

Each map is computed with the tiled online softmax ("Flash style softmax",
Attention Variants Compared), the same per-step code as the grouped-query
kernel of gen_fwd_gqa.py, whose instruction IR, hazard pass and softmax,
mask and P V building blocks this generator imports (with their register
assignments).

Work decomposition
  Item = 128 query rows of one query head.  Its 8 waves: wave w computes map
  1 + (w >> 2) (query and key projection 1 or 2) for rows 32 g .. +31, g =
  w & 3 for the first map and 3 - (w & 3) for the second, so waves w and
  w + 4 share a SIMD with rows from both ends of the item; the waves of the
  two maps on the same rows exchange through LDS.  LDS stages (four) hold,
  per 64-key tile, the K1 and K2 tiles (64 keys x 64 channels, rows padded
  to 144 bytes) and the V tile (64 keys x 128 values, rows padded to 320
  bytes): every key tile is read from HBM once for both maps.  Per tile a
  wave issues 8 MFMAs of S^T = K Q^T (head size 64) and 16 of O^T += V^T P^T.
  Persistent grid as in the grouped-query kernel: workgroup g takes items
  g, g + grid, ...; the last step of an item loads the next item's Q
  fragments and first two tiles.
  Epilogue: each wave of the second map writes lambda O2 / l2 (fp32) to LDS,
  half the values at a time, its partner wave of the first map reads it and
  forms O1 / l1 minus it, and the first map's waves store the bf16 rows
  through LDS.
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import gen_fwd_gqa as g                      # noqa: E402
from gen_fwd_gqa import (R, I, Prog, NegR, v, s, regs_of, EMPTY, VCC, resolve,  # noqa: E402,F401
                         udiv, rsrc, max_ops, exp_ops, pack_ops, merge_rr, mask_block,
                         settle_previous, after, AHEAD, RING, pv_read, pv_mfma, SLACK,
                         S_BUF, P_BUF, V_KADDR, V_VADDR, V_M, V_MTHR, V_L, V_LT, V_IBASE,
                         V_COL, V_HL, V_T, V_LANE, A_O, A_KR, A_VR, S_C, S_NINF, S_ONES,
                         S_WM1, S_FLAG, S_X, VROW, VTILE, M320)

# ---------------------------------------------------------------------------
# sizes
D = 64                        # query/key head size
DV = 128                      # value head size
KROW = 2 * D + 16             # padded LDS row of K1 / K2, bytes
KTILE = 64 * KROW             # 9216
STAGE = 2 * KTILE + VTILE     # 38912
NSTAGE = 4
LDS_BYTES = NSTAGE * STAGE    # 155648
XROW = 4 * 64 + 16            # LDS row of the map exchange (64 fp32 values) and of the output staging
EPI_STORES = 8                # output stores of a first-map wave per item
KARG_BYTES = 80
NAME = "diff_fwd_d64_dv128"
assert 32 * XROW * 4 <= STAGE
assert KTILE % 1024 == 0 and VTILE % 1024 == 0

# floor(x / 144) as (x * M144) >> 24 over a tile
M144 = -(-(1 << 24) // KROW)
for _x in range(KTILE):
    assert (_x * M144) >> 24 == _x // KROW

# ---------------------------------------------------------------------------
# registers (the ones shared with the imported building blocks keep their
# numbers: score and P buffers, softmax state, temporaries, O, the fragment
# rings, S_C, S_NINF, S_ONES, S_WM1, S_FLAG and the flag temporaries, S_X)
V_KLANE, V_VLANE = v(81), v(82)
V_DK = [v(85)]                       # LDS-DMA source offsets per lane: K chunk w (K1 and K2)
V_DV = [v(87), v(88)]                # V chunks w, w + 8
V_DX = v(86)                         # the wave's fifth chunk (V 16 + w, or K 8)
V_OWL, V_ORDL, V_OST, V_XCH = v(120), v(121), v(122), v(123)
V_QLANE = v(127)                     # (lane % 32) * 128 + 16 (lane / 32)

A_Q = g.a(64, 16)                    # Q^T fragments: ks at 4 ks

S_KARG, S_WG, S_BASE = s(0, 2), s(2), s(3)
S_Q1, S_K1, S_Q2, S_K2, S_V, S_OUT = s(4, 2), s(6, 2), s(8, 2), s(10, 2), s(12, 2), s(14, 2)
S_N, S_W, S_G = s(16), s(17), s(18)
assert S_C.i == 19
S_LAMBDA, S_TOTAL, S_STRIDE, S_NRB = s(20), s(21), s(22), s(23)
S_WAVE, S_LID, S_KV, S_RB, S_BG, S_R0, S_TLO, S_T, S_J = (s(24), s(25), s(26), s(27), s(28), s(29), s(30),
                                                          s(31), s(32))
S_NBK, S_MAP, S_R0W = s(33), s(34), s(35)
S_RSK1, S_RSV, S_RSQ, S_RSO, S_RSK2 = s(36, 4), s(40, 4), s(44, 4), s(48, 4), s(52, 4)
S_WAVE1K, S_SOFFK, S_SB, S_R0W32 = s(56), s(57), s(58), s(59)
S_K0P = [s(61), s(76)]
S_FULL = [s(77), s(60)]
S_SBW = s(62)
S_NBV, S_SOFFV = s(66), s(67)
S_XOFF, S_SOFFX, S_NBX, S_SHX = s(73), s(72), s(94), s(95)   # the fifth chunk: LDS offset in a stage,
S_RSE = s(96, 4)                     # key offset, offset past the rows, row shift, descriptor
S_VID, S_RGRP = s(92), s(93)


# ---------------------------------------------------------------------------
# building blocks of this kernel
def dma_ops():
    """This wave's LDS-DMA loads of the tile at key offset S_SOFFK (K1, K2)
    / S_SOFFV (V) into the stage at S_SB.  The padded K1 and K2 tiles are 9
    chunks of 1 KiB each and the V tile 20: K1 chunk w, K2 chunk w, V chunks
    w and w + 8, and a fifth chunk through the wave's own descriptor and
    offset (S_RSE, S_SOFFX): V chunk 16 + w on waves 0-3, K1 chunk 8 on
    waves 4 and 6, K2 chunk 8 on waves 5 and 7 (two waves write the same
    bytes)."""
    ops = []
    for rs, base in ((S_RSK1, 0), (S_RSK2, KTILE)):
        def op(P, rs=rs, base=base):
            P.salu("s_add_u32", "m0", S_SBW, str(base))
            P.dma(V_DK[0], rs, S_SOFFK)
        ops.append(op)
    for jv in range(2):
        def op(P, jv=jv):
            P.salu("s_add_u32", "m0", S_SBW, str(2 * KTILE + jv * 8192))
            P.dma(V_DV[jv], S_RSV, S_SOFFV)
        ops.append(op)

    def op(P):
        P.salu("s_add_u32", "m0", S_SB, S_XOFF)
        P.dma(V_DX, S_RSE, S_SOFFX)
    ops.append(op)
    return ops


def dma_tile(P):
    P.salu("s_add_u32", S_SBW, S_SB, S_WAVE1K)
    for op in dma_ops():
        op(P)


# K fragments n = 0..7: key half kb = n % 2, channels 16 ks .. +15 with
# ks = n / 2 (head size 64: four steps); V^T fragments as in gen_fwd_gqa.
def qk_read(P, n):
    kb, ks = n % 2, n // 2
    P.ds_read("ds_read_b128", A_KR.sub(4 * (n % RING), 4), V_KADDR, kb * 32 * KROW + ks * 32)


def qk_mfma(P, n, sbuf):
    kb, ks = n % 2, n // 2
    dst = v(sbuf + 16 * kb, 16)
    P.mfma(dst, A_KR.sub(4 * (n % RING), 4), A_Q.sub(4 * ks, 4), None if ks == 0 else dst)


def qk_half(P, sbuf, kb):
    """S^T[kb] = K Q^T for key half kb alone (the 4 K fragments n with
    n % 2 == kb, ring slots by position)."""
    ns = [n for n in range(8) if n % 2 == kb]

    def slot(i):
        return A_KR.sub(4 * (i % RING), 4)

    def rd(i):
        P.ds_read("ds_read_b128", slot(i), V_KADDR, kb * 32 * KROW + (ns[i] // 2) * 32)

    def mm(i):
        ks = ns[i] // 2
        dst = v(sbuf + 16 * kb, 16)
        P.mfma(dst, slot(i), A_Q.sub(4 * ks, 4), None if ks == 0 else dst)
    for i in range(min(AHEAD, len(ns))):
        rd(i)
    for i in range(len(ns)):
        mm(i)
        if i + AHEAD < len(ns):
            rd(i + AHEAD)


def first_tile_kind(P, dead, half):
    """Branch to `dead` if the item's first tile lies before the window of
    the wave's first row (every key + W - 1 < the row), to `half` if its key
    half 0 does; fall through otherwise."""
    P.salu("s_add_u32", S_X[12], S_K0P[0], S_W)
    P.salu("s_add_u32", S_X[13], S_X[12], "63")
    P.scmp("s_cmp_le_u32", S_X[13], S_R0W)
    P.branch("s_cbranch_scc1", dead)
    P.salu("s_add_u32", S_X[13], S_X[12], "31")
    P.scmp("s_cmp_le_u32", S_X[13], S_R0W)
    P.branch("s_cbranch_scc1", half)


def interleave(P, order, sbuf_next, valu_ops, extra_ops=(), v_ready=0):
    """The MFMAs of `order` (("k", n): QK fragment n into sbuf_next; ("v",
    n): PV fragment n) with their fragment reads AHEAD ahead, the VALU ops
    spread evenly by issue cost (after() constraints kept) and the extra
    ops (DMA loads, scalar set-up) one every few MFMAs; as in gen_fwd_gqa."""
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
        out = [("v", 0), ("v", 1), ("v", 2), ("v", 3)]
        for k in range(6):
            out += [("k", k), ("v", 4 + 2 * k), ("v", 5 + 2 * k)]
        return out + [("k", 6), ("k", 7)]
    if has_qk:
        return [("k", k) for k in range(8)]
    if has_pv:
        return [("v", k) for k in range(16)]
    return []


def setup_ops(pn):
    """Scalar set-up of step i = j + 1 (S_J = j): the DMA of tile i + 2
    (offsets, stage, M0 bases), key0 of tile i and whether every cell of
    tile i attends this wave's rows; after this step's DMA loads."""
    def o1(P):
        P.salu("s_add_u32", S_X[9], S_J, "1")                  # i
        P.salu("s_add_u32", S_X[4], S_X[9], "2")               # tile i + 2
        P.salu("s_add_u32", S_X[5], S_TLO, S_X[4])
        P.salu("s_lshl_b32", S_X[2], S_X[5], "14")             # V offset (256-byte rows)
        P.salu("s_lshl_b32", S_X[3], S_X[5], S_SHX)            # the fifth chunk's tensor
        P.salu("s_lshl_b32", S_X[5], S_X[5], "13")             # K offset (128-byte rows)

    # past the band the offsets are N rows, out of the descriptors' range:
    # the loads read zeros into a stage nothing reads
    def o2(P):
        P.scmp("s_cmp_lt_u32", S_X[4], S_T)
        P.salu("s_cselect_b32", S_SOFFK, S_X[5], S_NBK, reads_scc=True, writes_scc=False)
        P.salu("s_cselect_b32", S_SOFFV, S_X[2], S_NBV, reads_scc=True, writes_scc=False)
        P.salu("s_cselect_b32", S_SOFFX, S_X[3], S_NBX, reads_scc=True, writes_scc=False)

    def o3(P):
        P.salu("s_and_b32", S_SB, S_X[4], "3")
        P.salu("s_mul_i32", S_SB, S_SB, str(STAGE))
        P.salu("s_add_u32", S_SBW, S_SB, S_WAVE1K)

    def o4(P):
        P.salu("s_add_u32", S_X[6], S_TLO, S_X[9])
        P.salu("s_lshl_b32", S_K0P[pn], S_X[6], "6")           # key0 of tile i
        P.salu("s_add_u32", S_X[7], S_K0P[pn], "63")
        P.salu("s_add_u32", S_X[8], S_K0P[pn], S_W)

    def o5(P):
        P.scmp("s_cmp_le_u32", S_X[7], S_R0W)
        P.salu("s_cselect_b32", S_X[10], "1", "0", reads_scc=True, writes_scc=False)

    def o6(P):
        P.scmp("s_cmp_ge_u32", S_X[8], S_R0W32)
        P.salu("s_cselect_b32", S_X[11], "1", "0", reads_scc=True, writes_scc=False)
        P.salu("s_and_b32", S_FULL[pn], S_X[10], S_X[11])
    return [o1, o2, o3, o4, o5, o6]


def v_prefetch_ops():
    """The first AHEAD V^T fragments of the next P V product, read before
    the next barrier."""
    def addr(P):
        P.salu("s_and_b32", S_X[12], S_J, "3")
        P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
        P.valu("v_add_u32", V_VADDR, S_X[12], V_VLANE)
    return [after(op, "v", 15) for op in [addr] + [(lambda P, n=n: pv_read(P, n)) for n in range(AHEAD)]]


def k_addr_next(P):
    P.salu("s_add_u32", S_X[12], S_J, "2")
    P.salu("s_and_b32", S_X[12], S_X[12], "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)


def by_map(P, first_map, second_map):
    """Emit first_map(P) for the waves of the first map and second_map(P)
    for the others (a wave-uniform branch)."""
    other, done = P.new_label("map2"), P.new_label("mapped")
    P.scmp("s_cmp_lg_u32", S_MAP, "0")
    P.branch("s_cbranch_scc1", other)
    first_map(P)
    P.branch("s_branch", done)
    P.label(other)
    second_map(P)
    P.label(done)


def iteration(P, phase, has_qk, has_pv, first, exact=True):
    """One tile j of the pipeline, as in gen_fwd_gqa (exact=False: no row
    maximum unless a row's sum of p exceeds 2^SLACK)."""
    sb_cur, sb_next = S_BUF[phase], S_BUF[1 - phase]
    P.comment(f"iteration phase {phase} qk={has_qk} pv={has_pv}")
    if first:
        # tile 1 of the item in; the first map's waves have the previous
        # item's EPI_STORES output stores issued after it
        by_map(P, lambda P: P.waitcnt(vm=EPI_STORES), lambda P: P.waitcnt(vm=0))
    else:
        P.waitcnt(vm=0)
    P.barrier()
    if has_pv:
        settle_previous(P)
    if first and has_qk:
        first_step(P)
        return
    if not has_qk:
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)
        last_step(P, phase, has_pv)
    else:
        P.scmp("s_cmp_eq_u32", S_FULL[phase], "1")
        skip = P.new_label("full")
        P.branch("s_cbranch_scc1", skip)
        mask_block(P, sb_cur, S_K0P[phase])
        P.label(skip)
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)
        valu = ((max_ops(sb_cur) if exact else []) + merge_rr([exp_ops(sb_cur, 0), exp_ops(sb_cur, 1)])
                + pack_ops(sb_cur, 0) + v_prefetch_ops() + pack_ops(sb_cur, 1))
        extra = dma_ops() + setup_ops(1 - phase)
        interleave(P, mfma_order(has_qk, has_pv), sb_next, valu, extra, v_ready=AHEAD)
    if not exact:
        g.max_redo(P, phase, qk=lambda P, sb: interleave(P, mfma_order(True, False), sb, []), stage=STAGE)
    if has_qk:
        k_addr_next(P)
    if not has_pv:
        P.valu("v_add_f32", V_MTHR, str(SLACK), V_M)
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)


def first_step(P):
    """Step 0 of an item (S(1) = K(1) Q^T, the DMA of tile 2, the softmax of
    tile 0).  Where tile 0 lies before the window of every row of the wave,
    it takes no softmax (p = 0: the P buffer and the row sums are cleared
    for the P V product of step 1); where only its key half 0 does, that
    half takes none."""
    sb = S_BUF[0]
    dead, half, joined = P.new_label("firstdead"), P.new_label("firsthalf"), P.new_label("firstdone")
    first_tile_kind(P, dead, half)
    zero_lt = [lambda P, k=k: P.valu("v_mov_b32", V_LT[k], "0") for k in range(2)]

    def zero_p(lo, hi):
        return [lambda P, i=i: P.valu("v_mov_b32", v(P_BUF + i), "0") for i in range(lo, hi)]
    for kind in ("full", "half", "dead"):
        if kind == "half":
            P.label(half)
        elif kind == "dead":
            P.label(dead)
        if kind != "dead":
            P.scmp("s_cmp_eq_u32", S_FULL[0], "1")
            skip = P.new_label("full")
            P.branch("s_cbranch_scc1", skip)
            mask_block(P, sb, S_K0P[0])
            P.label(skip)
        P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)
        if kind == "full":
            valu = (max_ops(sb) + merge_rr([exp_ops(sb, 0), exp_ops(sb, 1)]) + pack_ops(sb, 0)
                    + v_prefetch_ops() + pack_ops(sb, 1))
        elif kind == "half":
            valu = zero_lt + max_ops(sb) + exp_ops(sb, 1) + pack_ops(sb, 1) + zero_p(0, 8) + v_prefetch_ops()
        else:
            valu = zero_lt + zero_p(0, 16) + v_prefetch_ops()
        interleave(P, mfma_order(True, False), S_BUF[1], valu, dma_ops() + setup_ops(1), v_ready=AHEAD)
        if kind != "dead":
            P.branch("s_branch", joined)
    P.label(joined)
    k_addr_next(P)
    P.valu("v_add_f32", V_MTHR, str(SLACK), V_M)
    P.salu("s_mov_b64", S_FLAG, "0", writes_scc=False)


def last_step(P, phase, has_pv):
    """The softmax of an item's last tile (with its row maximum), the P V
    product of the one before (has_pv), and the loads of the next item.
    Key halves of the tile that lie past every row of the wave take no
    softmax (their p are 0; the epilogue skips their P V fragments): the
    whole tile for the row groups it lies past, key half 1 where only that
    half does."""
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
            for k in range(2):
                P.valu("v_mov_b32", V_LT[k], "0")
        if kind != "dead":
            P.scmp("s_cmp_eq_u32", S_FULL[phase], "1")
            skip = P.new_label("full")
            P.branch("s_cbranch_scc1", skip)
            mask_block(P, sb_cur, S_K0P[phase])
            P.label(skip)
        item_loads(P, first=False)
        if kind == "full":
            valu = (max_ops(sb_cur) + merge_rr([exp_ops(sb_cur, 0), exp_ops(sb_cur, 1)]) + pack_ops(sb_cur, 0)
                    + v_prefetch_ops() + pack_ops(sb_cur, 1))
        elif kind == "half":
            valu = max_ops(sb_cur) + exp_ops(sb_cur, 0) + pack_ops(sb_cur, 0) + v_prefetch_ops()
        else:
            valu = []
        interleave(P, order, None, valu, [], v_ready=AHEAD)
        if kind != "dead":
            P.branch("s_branch", joined)
    P.label(joined)


def epilogue(P, phase):
    """O += V(T-1)^T P(T-1); then out = O1 / l1 - lambda O2 / l2 -> bf16.
    The second map's waves hand lambda O2 / l2 to their partner waves (same
    rows) through LDS, half the values at a time, in the stage of
    tile T-2 (free after the barrier; the stage of tile T-1 is still being
    read and the next two hold the next item's first tiles); the first
    map's waves stage the bf16 rows there for whole-row stores."""
    P.barrier()
    settle_previous(P)
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
    interleave(P, [("v", n) for n in range(8)], None, [], v_ready=AHEAD)
    P.label(dead)
    P.label(joined)
    t = V_T
    l, l2, inv = t[0], t[1], t[2]
    P.valu("v_add_f32", l, V_L[0], V_L[1])
    P.valu("v_mov_b32", l2, l)
    P.add(I(f"  v_permlane32_swap_b32 {l}, {l2}", "perm", regs_of(l, l2), regs_of(l, l2)))
    P.valu("v_add_f32", l, l, l2)
    P.valu("v_rcp_f32", inv, l, kind="trans")
    P.scmp("s_cmp_eq_u32", S_MAP, "0")
    P.salu("s_cselect_b32", S_X[0], "1.0", S_LAMBDA, reads_scc=True, writes_scc=False)
    P.valu("v_mul_f32", inv, S_X[0], inv)                         # 1 / l1, or lambda / l2
    # this row group's region: 32 rows x XROW bytes
    P.salu("s_add_u32", S_X[1], S_J, "-1")
    P.salu("s_and_b32", S_X[1], S_X[1], "3")
    P.salu("s_mul_i32", S_X[1], S_X[1], str(STAGE))
    P.salu("s_mul_i32", S_X[2], S_RGRP, str(32 * XROW))
    P.salu("s_add_u32", S_X[1], S_X[1], S_X[2])
    xch, ow, ord_ = t[12], t[13], t[14]
    P.valu("v_add_u32", xch, S_X[1], V_XCH)
    P.valu("v_add_u32", ow, S_X[1], V_OWL)
    P.valu("v_add_u32", ord_, S_X[1], V_ORDL)

    def acc4(P, db, r4, x):
        for k in range(4):
            P.add(I(f"  v_accvgpr_read_b32 {x[k]}, {A_O.sub(16 * db + 4 * r4 + k)}", "valu",
                    A_O.sub(16 * db + 4 * r4 + k).regs(), x[k].regs()))

    def put(half):
        # second map: lambda O2 / l2, values 32 db + 8 r4 + 4 hl .. +3 of row col
        def emit(P):
            for db in (2 * half, 2 * half + 1):
                for r4 in range(4):
                    x = [t[4 + k] for k in range(4)]
                    acc4(P, db, r4, x)
                    for k in range(4):
                        P.valu("v_mul_f32", x[k], x[k], inv)
                    P.add(I(f"  ds_write_b128 {xch}, {v(x[0].i, 4)} offset:{(db - 2 * half) * 128 + r4 * 32}",
                            "lds", regs_of(xch, v(x[0].i, 4)), EMPTY))
        return emit

    def take(half):
        # first map: O1 / l1 minus the partner's values -> bf16 pairs in the
        # free score buffer (v[16 half .. 16 half + 15])
        def emit(P):
            for db in (2 * half, 2 * half + 1):
                for r4 in range(4):
                    y = v(t[4].i, 4)
                    P.ds_read("ds_read_b128", y, xch, (db - 2 * half) * 128 + r4 * 32)
                    x = [t[8 + k] for k in range(4)]
                    acc4(P, db, r4, x)
                    for k in range(4):
                        P.valu("v_fma_f32", x[k], x[k], inv, NegR(y.sub(k)))
                    o = S_BUF[0] + 16 * half + 8 * (db - 2 * half) + 2 * r4
                    P.valu("v_cvt_pk_bf16_f32", v(o), x[0], x[1])
                    P.valu("v_cvt_pk_bf16_f32", v(o + 1), x[2], x[3])
        return emit

    def none(P):
        return None
    for half in range(2):
        by_map(P, none, put(half))
        P.barrier()
        by_map(P, take(half), none)
        if half == 0:
            P.barrier()

    def store(P):
        # rows col, values 32 db + 8 r4 + 4 hl .. +3 (bf16, 8 bytes), then
        # rows 4 kk + lane / 16, bytes 16 (lane % 16) .. +15 of each row
        for half in range(2):
            for db in (2 * half, 2 * half + 1):
                for r4 in range(4):
                    o = S_BUF[0] + 16 * half + 8 * (db - 2 * half) + 2 * r4
                    P.add(I(f"  ds_write_b64 {ow}, {v(o, 2)} offset:{db * 64 + r4 * 16}", "lds",
                            regs_of(ow, v(o, 2)), EMPTY))
        ob = S_BUF[1]
        for kk in range(8):
            P.ds_read("ds_read_b128", v(ob + 4 * kk, 4), ord_, kk * 4 * XROW)
        for kk in range(8):
            P.salu("s_mov_b32", S_X[3 + (kk % 4)], str(kk * 1024), writes_scc=False)
            P.add(I(f"  buffer_store_dwordx4 {v(ob + 4 * kk, 4)}, {V_OST}, {S_RSO}, {S_X[3 + (kk % 4)]} offen",
                    "vstore", regs_of(v(ob + 4 * kk, 4), V_OST, S_RSO, S_X[3 + (kk % 4)]), EMPTY))
    by_map(P, store, none)
    P.scmp("s_cmp_lt_u32", S_VID, S_TOTAL)
    P.branch("s_cbranch_scc1", ".Litem")
    P.add(I("  s_endpgm", "branch"))


def item_loads(P, first):
    """Start the workgroup's next item (S_VID + S_STRIDE; S_VID itself for
    the first): row block, band, descriptors, then the loads of its Q
    fragments and of its tiles 0 and 1 into stages S_J + 1 and S_J + 2
    (mod 4), not waited for here.  Its step counter starts at
    S_BASE = (S_J + 1) & 3."""
    skip = None
    if not first:
        P.salu("s_add_u32", S_VID, S_VID, S_STRIDE)
        P.scmp("s_cmp_ge_u32", S_VID, S_TOTAL)
        skip = P.new_label("nonext")
        P.branch("s_cbranch_scc1", skip)
    P.salu("s_add_u32", S_BASE, S_J, "1")
    P.salu("s_and_b32", S_BASE, S_BASE, "3")
    # item -> logical id (each XCD a contiguous run), then (query head of the
    # batch, 128-row block), row blocks ascending
    P.salu("s_and_b32", S_X[0], S_TOTAL, "7")
    P.salu("s_and_b32", S_X[1], S_VID, "7")
    P.salu("s_lshr_b32", S_X[2], S_TOTAL, "3")
    P.salu("s_mul_i32", S_X[1], S_X[1], S_X[2])
    P.salu("s_lshr_b32", S_X[3], S_VID, "3")
    P.salu("s_add_u32", S_X[1], S_X[1], S_X[3])
    P.scmp("s_cmp_eq_u32", S_X[0], "0")
    P.salu("s_cselect_b32", S_LID, S_X[1], S_VID, reads_scc=True, writes_scc=False)
    udiv(P, S_LID, S_NRB, S_BG, S_RB, V_T[1], V_T[2])          # b * Hq + h, row block
    udiv(P, S_BG, S_G, S_KV, S_X[4], V_T[1], V_T[2])           # b * Hkv + h / G
    P.salu("s_lshl_b32", S_R0, S_RB, "7")
    P.salu("s_lshl_b32", S_R0W, S_RGRP, "5")
    P.salu("s_add_u32", S_R0W, S_R0W, S_R0)                    # this wave's first row
    # band of rows r0 .. r0+127: key tiles t_lo .. t_hi
    P.salu("s_sub_i32", S_X[0], S_R0, S_W)
    P.salu("s_add_i32", S_X[0], S_X[0], "1")
    P.salu("s_max_i32", S_X[0], S_X[0], "0")
    P.salu("s_lshr_b32", S_TLO, S_X[0], "6")
    P.salu("s_add_u32", S_X[1], S_R0, "127")
    P.salu("s_sub_u32", S_X[2], S_N, "1")
    P.salu("s_min_u32", S_X[1], S_X[1], S_X[2])
    P.salu("s_lshr_b32", S_X[1], S_X[1], "6")
    P.salu("s_sub_u32", S_T, S_X[1], S_TLO)
    P.salu("s_add_u32", S_T, S_T, "1")
    # descriptors: K1, K2 and Q rows of 128 bytes, V rows of 256
    P.salu("s_lshl_b32", S_X[6], S_N, "7")
    rsrc(P, S_RSK1, S_K1, S_KV, S_X[6], S_X[6])
    rsrc(P, S_RSK2, S_K2, S_KV, S_X[6], S_X[6])
    P.salu("s_lshl_b32", S_X[7], S_N, "8")
    rsrc(P, S_RSV, S_V, S_KV, S_X[7], S_X[7])
    # the fifth DMA chunk's descriptor: V on waves 0-3, K1 on waves 4 and
    # 6, K2 on waves 5 and 7
    P.scmp("s_bitcmp1_b32", S_WAVE, "0")
    for h in (0, 2):
        P.salu("s_cselect_b64", S_RSE.sub(h, 2), S_RSK2.sub(h, 2), S_RSK1.sub(h, 2), reads_scc=True,
               writes_scc=False)
    P.scmp("s_cmp_lt_u32", S_WAVE, "4")
    for h in (0, 2):
        P.salu("s_cselect_b64", S_RSE.sub(h, 2), S_RSV.sub(h, 2), S_RSE.sub(h, 2), reads_scc=True,
               writes_scc=False)
    qsrc = s(S_X[8].i, 2)
    P.scmp("s_cmp_eq_u32", S_MAP, "0")
    P.salu("s_cselect_b64", qsrc, S_Q1, S_Q2, reads_scc=True, writes_scc=False)
    rsrc(P, S_RSQ, qsrc, S_BG, S_X[6], S_X[6])
    qoff = V_T[3]
    P.salu("s_lshl_b32", S_X[10], S_R0W, "7")
    P.valu("v_add_u32", qoff, S_X[10], V_QLANE)
    for ks in range(4):
        P.buf_load(A_Q.sub(4 * ks, 4), qoff, S_RSQ, "0", 32 * ks, track=False)
    # tiles 0 and 1 (tile 1 also when the band has one tile: read as data or
    # zeros, never used)
    P.salu("s_lshl_b32", S_SOFFK, S_TLO, "13")
    P.salu("s_lshl_b32", S_SOFFV, S_TLO, "14")
    P.salu("s_lshl_b32", S_SOFFX, S_TLO, S_SHX)
    P.salu("s_mul_i32", S_SB, S_BASE, str(STAGE))
    dma_tile(P)
    P.salu("s_add_u32", S_SOFFK, S_SOFFK, str(1 << 13))
    P.salu("s_add_u32", S_SOFFV, S_SOFFV, str(1 << 14))
    P.salu("s_add_u32", S_X[0], S_TLO, "1")
    P.salu("s_lshl_b32", S_SOFFX, S_X[0], S_SHX)
    P.salu("s_add_u32", S_X[0], S_BASE, "1")
    P.salu("s_and_b32", S_X[0], S_X[0], "3")
    P.salu("s_mul_i32", S_SB, S_X[0], str(STAGE))
    dma_tile(P)
    P.salu("s_sub_u32", S_TLO, S_TLO, S_BASE)
    P.salu("s_add_u32", S_T, S_T, S_BASE)
    if skip:
        P.label(skip)


def item_start(P):
    P.label(".Litem")
    P.salu("s_lshl_b32", S_X[7], S_N, "8")
    rsrc(P, S_RSO, S_OUT, S_BG, S_X[7], S_X[7])
    P.salu("s_add_u32", S_R0W32, S_R0W, "32")
    t = V_T
    P.valu("v_add_u32", t[5], S_R0W, V_COL)                    # row
    P.valu("v_lshlrev_b32", t[7], "2", V_HL)
    P.valu("v_sub_u32", V_IBASE, t[5], t[7])
    # output store offset: row r0w + lane / 16, bytes 16 (lane % 16)
    P.valu("v_lshrrev_b32", t[0], "4", V_LANE)
    P.valu("v_add_u32", t[0], S_R0W, t[0])
    P.valu("v_lshlrev_b32", t[0], "8", t[0])
    P.valu("v_and_b32", t[1], "15", V_LANE)
    P.valu("v_lshlrev_b32", t[1], "4", t[1])
    P.valu("v_add_u32", V_OST, t[0], t[1])
    P.valu("v_mov_b32", V_M, "0xf149f2ca")             # -1e30
    P.valu("v_mov_b32", V_MTHR, "0xf149f2ca")
    for k in range(2):
        P.valu("v_mov_b32", V_L[k], "0")
    for k in range(64):
        P.add(I(f"  v_accvgpr_write_b32 {A_O.sub(k)}, 0", "valu", EMPTY, A_O.sub(k).regs()))
    P.salu("s_sub_u32", S_J, S_BASE, "1")
    for op in setup_ops(0):
        op(P)
    # Q and tile 0 in: all but tile 1's loads and (first map) the previous
    # item's output stores
    by_map(P, lambda P: P.waitcnt(vm=len(dma_ops()) + EPI_STORES), lambda P: P.waitcnt(vm=len(dma_ops())))
    P.barrier()
    P.salu("s_mov_b32", S_J, S_BASE, writes_scc=False)
    P.salu("s_mul_i32", S_X[12], S_BASE, str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)
    # S(0), or of its key half 1 alone, or none (first_step)
    dead, half, joined = P.new_label("qk0dead"), P.new_label("qk0half"), P.new_label("qk0done")
    first_tile_kind(P, dead, half)
    interleave(P, mfma_order(True, False), S_BUF[0], [])
    P.branch("s_branch", joined)
    P.label(half)
    qk_half(P, S_BUF[0], 1)
    P.label(dead)
    P.label(joined)
    P.salu("s_add_u32", S_X[12], S_BASE, "1")
    P.salu("s_and_b32", S_X[12], S_X[12], "3")
    P.salu("s_mul_i32", S_X[12], S_X[12], str(STAGE))
    P.valu("v_add_u32", V_KADDR, S_X[12], V_KLANE)


def _chunk_src(P, dst, pos, magic, rowb, pitch_shift, data, t):
    """dst = source byte offset of tile byte `pos`: row * pitch + column, the
    columns of padding replaced by 0."""
    P.salu("s_mov_b32", S_X[11], str(magic), writes_scc=False)
    P.valu("v_mul_lo_u32", t[11], pos, S_X[11])
    P.valu("v_lshrrev_b32", t[11], "24", t[11])                # row
    P.valu("v_mul_u32_u24", t[12], str(rowb), t[11])
    P.valu("v_sub_u32", t[12], pos, t[12])                     # column byte
    P.add(I(f"  v_cmp_gt_u32 vcc, {data}, {t[12]}", "vcmp", t[12].regs(), VCC))
    P.valu("v_cndmask_b32", t[12], "0", t[12], "vcc")
    P.valu("v_lshlrev_b32", t[11], str(pitch_shift), t[11])
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
    P.waitcnt(lgkm=0)
    P.salu("s_and_b32", S_RGRP, S_WAVE, "3")
    P.salu("s_lshr_b32", S_MAP, S_WAVE, "2")
    P.salu("s_mov_b32", S_VID, S_WG, writes_scc=False)
    P.salu("s_lshl_b32", S_WAVE1K, S_WAVE, "10")
    P.salu("s_lshl_b32", S_NBK, S_N, "7")
    P.salu("s_lshl_b32", S_NBV, S_N, "8")
    # the fifth DMA chunk: V chunk 16 + w on waves 0-3 (LDS offset
    # 2 KTILE + 1024 (16 + w), rows of 256 bytes), K1 / K2 chunk 8 on even /
    # odd waves 4-7 (8 KiB into the K1 or K2 tile, rows of 128 bytes)
    P.salu("s_mov_b32", S_X[0], str(8 * 1024), writes_scc=False)
    P.scmp("s_bitcmp1_b32", S_WAVE, "0")
    P.salu("s_cselect_b32", S_X[0], str(KTILE + 8 * 1024), S_X[0], reads_scc=True, writes_scc=False)
    P.salu("s_lshl_b32", S_XOFF, S_RGRP, "10")
    P.salu("s_add_u32", S_XOFF, S_XOFF, str(2 * KTILE + 16 * 1024))
    P.scmp("s_cmp_lt_u32", S_WAVE, "4")
    P.salu("s_cselect_b32", S_XOFF, S_XOFF, S_X[0], reads_scc=True, writes_scc=False)
    P.salu("s_cselect_b32", S_SHX, "14", "13", reads_scc=True, writes_scc=False)
    P.salu("s_cselect_b32", S_NBX, S_NBV, S_NBK, reads_scc=True, writes_scc=False)
    P.salu("s_sub_u32", S_WM1, S_W, "1")
    P.salu("s_mov_b32", S_NINF, "0xff800000", writes_scc=False)
    P.salu("s_mov_b32", S_ONES, "0x3f803f80", writes_scc=False)
    t = V_T
    # K fragment reads: the wave's own map's K tile, row col, bytes 16 hl
    P.salu("s_mul_i32", S_X[0], S_MAP, str(KTILE))
    P.valu("v_mul_u32_u24", V_KLANE, str(KROW), V_COL)
    P.valu("v_lshlrev_b32", t[0], "4", V_HL)
    P.valu("v_add_u32", V_KLANE, V_KLANE, t[0])
    P.valu("v_add_u32", V_KLANE, S_X[0], V_KLANE)
    # V^T fragment reads (the layout of gen_fwd_gqa), after both K tiles
    P.valu("v_lshrrev_b32", t[0], "4", V_LANE)                 # grp
    P.valu("v_and_b32", t[1], "15", V_LANE)                    # sl
    P.valu("v_lshrrev_b32", t[2], "1", t[0])
    P.valu("v_lshlrev_b32", t[2], "2", t[2])
    P.valu("v_lshrrev_b32", t[3], "2", t[1])
    P.valu("v_add_u32", t[2], t[2], t[3])
    P.valu("v_mul_u32_u24", t[2], str(VROW), t[2])
    P.valu("v_and_b32", t[3], "1", t[0])
    P.valu("v_lshlrev_b32", t[3], "5", t[3])
    P.valu("v_and_b32", t[4], "3", t[1])
    P.valu("v_lshlrev_b32", t[4], "3", t[4])
    P.valu("v_add_u32", t[2], t[2], t[3])
    P.valu("v_add_u32", t[2], t[2], t[4])
    P.valu("v_add_u32", V_VLANE, str(2 * KTILE), t[2])
    # Q rows of 128 bytes: row col, bytes 16 hl of each 32-byte group
    P.valu("v_lshlrev_b32", t[0], "7", V_COL)
    P.valu("v_lshlrev_b32", t[1], "4", V_HL)
    P.valu("v_add_u32", V_QLANE, t[0], t[1])
    # epilogue: exchange (row col, 16 hl), output staging write (row col,
    # 8 hl) and read (row lane / 16, bytes 16 (lane % 16))
    P.valu("v_mul_u32_u24", t[0], str(XROW), V_COL)
    P.valu("v_lshlrev_b32", t[1], "4", V_HL)
    P.valu("v_add_u32", V_XCH, t[0], t[1])
    P.valu("v_lshlrev_b32", t[1], "3", V_HL)
    P.valu("v_add_u32", V_OWL, t[0], t[1])
    P.valu("v_lshrrev_b32", t[0], "4", V_LANE)
    P.valu("v_and_b32", t[1], "15", V_LANE)
    P.valu("v_lshlrev_b32", t[1], "4", t[1])
    P.valu("v_mul_u32_u24", V_ORDL, str(XROW), t[0])
    P.valu("v_add_u32", V_ORDL, V_ORDL, t[1])
    # DMA lane offsets: K chunks w and 8 (the same offsets serve K1 and K2),
    # V chunks w, w + 8 and 16 + (w & 3)
    P.valu("v_lshlrev_b32", t[8], "4", V_LANE)                 # 16 lane
    P.valu("v_add_u32", t[10], S_WAVE1K, t[8])
    _chunk_src(P, V_DK[0], t[10], M144, KROW, 7, 2 * D, t)
    for jv in range(2):
        P.valu("v_add_u32", t[10], S_WAVE1K, t[8])
        P.valu("v_add_u32", t[10], str(jv * 8192), t[10])
        _chunk_src(P, V_DV[jv], t[10], M320, VROW, 8, 2 * DV, t)
    # the fifth chunk: K chunk 8 on waves 4-7, V chunk 16 + w on waves 0-3
    P.valu("v_add_u32", t[10], str(8 * 1024), t[8])
    _chunk_src(P, t[14], t[10], M144, KROW, 7, 2 * D, t)
    P.salu("s_lshl_b32", S_X[0], S_RGRP, "10")
    P.valu("v_add_u32", t[10], S_X[0], t[8])
    P.valu("v_add_u32", t[10], str(16 * 1024), t[10])
    _chunk_src(P, V_DX, t[10], M320, VROW, 8, 2 * DV, t)
    P.scmp("s_cmp_lt_u32", S_WAVE, "4")
    P.salu("s_cselect_b64", "vcc", "-1", "0", reads_scc=True, writes_scc=False)
    P.valu("v_cndmask_b32", V_DX, t[14], V_DX, "vcc")
    # row groups: w & 3 for the first map's waves, 3 - (w & 3) for the
    # second's, so the two waves of a SIMD hold rows from both ends of an
    # item and meet about the same masked and dead tiles in each step (the
    # fifth DMA chunk above is V chunk 16 + (w & 3) on the first map's waves)
    P.salu("s_mul_i32", S_X[0], S_MAP, "3")
    P.salu("s_xor_b32", S_RGRP, S_RGRP, S_X[0])
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
    # key of tiles 0 .. 2, so from j = 3 on the running maximum is finite
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
