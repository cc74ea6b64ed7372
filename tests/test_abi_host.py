"""CPU tests of the C-ABI boundary (no GPU, no kernel launch).

The library must load and export every entry point include/*.h declares;
argument checks run on the host before any HIP call, so every rejection is
exercised here with fake (never dereferenced) pointers; the host-side block
mask sizing must agree exactly with the oracle's brute-force tile list.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("swa.h", "swa_probe.h")]
PKG = os.path.join(ROOT, "sparse_masked_transformer_amd")

FAKE = 0x7F0000000000  # 16-byte aligned; never dereferenced by a rejected call


@pytest.fixture(scope="module")
def swa():
    other = os.environ.get("SWA_ABI_LIBRARY")
    if other:
        # another build of the library (the sanitizer run): its host surface
        # through the ctypes layer alone, without PyTorch
        import importlib.util
        spec = importlib.util.spec_from_file_location("swa_abi_layer", os.path.join(PKG, "_abi.py"))
        m = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(m)
        return m.namespace(m.configure(ctypes.CDLL(other)), other)
    if not os.path.exists(os.path.join(PKG, "libswa.so")):
        subprocess.run([sys.executable, os.path.join(PKG, "build.py")], check=True)
    import sparse_masked_transformer_amd as m
    return m


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*\b([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ("swa_block_mask_build", "swa_attn_fwd", "swa_attn_decode", "swa_attn_decode_sinks",
              "diff_attn_fwd", "diff_attn_decode"):
        assert n in names
    assert "swa_probe_mfma_bf16" in names and "swa_probe_stream_read" in names
    assert len(names) == 14, names


def test_every_header_is_listed():
    assert sorted(os.path.basename(h) for h in HEADERS) == sorted(
        f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))


def test_probe_rejections(swa):
    lib = swa.lib
    P = ctypes.c_void_p
    assert lib.swa_probe_mfma_bf16(None, P(FAKE), 1, 1, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_mfma_bf16(P(FAKE + 8), P(FAKE), 1, 1, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_mfma_bf16(P(FAKE), P(FAKE), 0, 1, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_mfma_bf16(P(FAKE), P(FAKE), 1, 0, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_mfma_bf16(P(FAKE), P(FAKE), 1, (1 << 24) + 1, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_stream_read(None, 16, P(FAKE), 1, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_stream_read(P(FAKE), 0, P(FAKE), 1, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_stream_read(P(FAKE), 24, P(FAKE), 1, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_stream_read(P(FAKE + 4), 16, P(FAKE), 1, None) == swa.SWA_ERR_INVALID_ARG
    assert lib.swa_probe_stream_read(P(FAKE), 16, P(FAKE), 65536, None) == swa.SWA_ERR_INVALID_ARG


def test_library_exports_every_declared_symbol(swa):
    out = subprocess.run(["nm", "-D", "--defined-only", swa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(swa.lib, name)


def test_library_does_not_touch_the_oracle(swa):
    out = subprocess.run(["nm", "-D", swa.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "orc_" not in out
    deps = subprocess.run(["ldd", swa.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src, f


def test_strerror(swa):
    assert swa.swa_strerror(0) == "success"
    for code in (-1, -2, -3, -4, -5):
        assert swa.swa_strerror(code) not in ("success", "unknown status")
    assert swa.swa_strerror(-99) == "unknown status"


def test_tile_config(swa):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    cfg = lambda op, dt, d, dv: (swa.lib.swa_tile_config(op, dt, d, dv, ctypes.byref(bm), ctypes.byref(bn)),
                                 bm.value, bn.value)
    assert cfg(swa.SWA_OP_ATTN, swa.SWA_BF16, 128, 128) == (0, 128, 64)
    assert cfg(swa.SWA_OP_DIFF, swa.SWA_BF16, 64, 128) == (0, 128, 64)    # 32 rows per wave
    assert cfg(swa.SWA_OP_ATTN, swa.SWA_F32, 32, 32) == (0, 32, 64)
    assert cfg(swa.SWA_OP_DIFF, swa.SWA_F32, 64, 128) == (0, 32, 64)
    assert cfg(swa.SWA_OP_ATTN, swa.SWA_BF16, 48, 48)[0] == swa.SWA_ERR_INVALID_ARG
    assert cfg(swa.SWA_OP_ATTN, 7, 64, 64)[0] == swa.SWA_ERR_INVALID_ARG
    assert cfg(5, swa.SWA_BF16, 64, 64)[0] == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("N,W,s,bm,bn,dil,g", [
    (1, 1, 0, 128, 64, 1, 0), (37, 5, 3, 16, 16, 1, 0), (300, 64, 5, 128, 64, 1, 0),
    (511, 129, 64, 128, 64, 1, 0), (1000, 50, 130, 128, 64, 1, 0), (777, 200, 1, 64, 32, 1, 0),
    (4096, 1024, 0, 128, 64, 1, 0), (8192, 1024, 0, 128, 64, 1, 0), (16384, 256, 128, 128, 64, 1, 0),
    (640, 600, 700, 32, 128, 1, 0), (999, 7, 65, 64, 64, 1, 0), (2000, 3000, 3, 256, 16, 1, 0),
    # dilated windows (dilation <= bn) and global tokens
    (1000, 50, 0, 128, 64, 2, 0), (1000, 30, 0, 128, 64, 64, 0), (777, 40, 9, 64, 16, 16, 0),
    (1000, 50, 0, 128, 64, 1, 64), (1000, 50, 130, 128, 64, 1, 300), (700, 20, 3, 32, 32, 5, 17),
    (300, 4, 0, 128, 64, 3, 1000), (4096, 512, 0, 128, 64, 2, 64), (555, 8, 100, 16, 64, 7, 65)])
def test_mask_query_matches_oracle(swa, N, W, s, bm, bn, dil, g):
    nq, nnz = swa.swa_block_mask_query(N, W, s, bm, bn, dil, g)
    t = oracle.tile_list(N, W, s, bm, bn, dilation=dil, n_global=g)
    assert (nq, nnz) == (t["num_q_tiles"], t["nnz"])


def test_mask_query_rejects(swa):
    for args in [(0, 4, 0, 128, 64), (10, 0, 0, 128, 64), (10, 4, -1, 128, 64), (10, 4, 0, 100, 64),
                 (10, 4, 0, 128, 8), (swa.SWA_MAX_N + 1, 4, 0, 128, 64),
                 (10, 4, 0, 128, 64, 0, 0),        # dilation < 1
                 (10, 4, 0, 128, 64, 65, 0),       # dilation > bn
                 (10, 4, 0, 128, 16, 17, 0),
                 (10, 4, 0, 128, 64, 1, -1)]:      # negative global count
        with pytest.raises(swa.SwaError) as e:
            swa.swa_block_mask_query(*args)
        assert e.value.status == swa.SWA_ERR_INVALID_ARG


def fake_mask(swa, N, W, s, bm=128, bn=64, nq=None, nnz=None, null=False, dil=1, g=0):
    q, z = swa.swa_block_mask_query(N, W, s, bm, 64, dil, g)
    p = 0 if null else FAKE
    return swa.swa_block_mask_t(N, W, s, dil, g, bm, bn, q if nq is None else nq,
                                z if nnz is None else nnz, p, p, p, p, p, p)


def fwd(swa, q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, dt=1, B=1, Hq=4, Hkv=2, N=256, d=64,
        W=32, s=0, scale=0.125, mask=None, dil=1, g=0):
    mask = fake_mask(swa, N, W, s) if mask is None else mask
    return swa.lib.swa_attn_fwd(q, k, v, out, lse, dt, B, Hq, Hkv, N, d, W, s, dil, g, scale,
                                ctypes.byref(mask), None)


def test_fwd_rejections(swa):
    E, U = swa.SWA_ERR_INVALID_ARG, swa.SWA_ERR_UNSUPPORTED
    assert fwd(swa, q=0) == E
    assert fwd(swa, k=FAKE + 8) == E             # misaligned
    assert fwd(swa, lse=FAKE + 2) == E           # misaligned lse
    assert fwd(swa, dt=5) == E
    assert fwd(swa, B=0) == E
    assert fwd(swa, Hq=6, Hkv=4) == E            # Hq % Hkv != 0
    assert fwd(swa, N=0, mask=fake_mask(swa, 1, 32, 0)) == E
    assert fwd(swa, W=0, mask=fake_mask(swa, 256, 1, 0)) == E
    assert fwd(swa, s=-1, mask=fake_mask(swa, 256, 32, 0)) == E
    assert fwd(swa, scale=0.0) == E
    assert fwd(swa, scale=float("nan")) == E
    assert fwd(swa, scale=-0.5) == E
    assert fwd(swa, d=48) == U
    assert fwd(swa, mask=fake_mask(swa, 255, 32, 0)) == E          # built for another N
    assert fwd(swa, mask=fake_mask(swa, 256, 33, 0)) == E          # another window
    assert fwd(swa, mask=fake_mask(swa, 256, 32, 4)) == E          # another stride
    assert fwd(swa, mask=fake_mask(swa, 256, 32, 0, bm=256)) == E  # another tiling
    assert fwd(swa, mask=fake_mask(swa, 256, 32, 0, nnz=1)) == E   # wrong size
    assert fwd(swa, mask=fake_mask(swa, 256, 32, 0, null=True)) == E
    assert fwd(swa, dil=0) == E
    assert fwd(swa, g=-1) == E
    assert fwd(swa, dil=2) == E                                     # mask built for dilation 1
    assert fwd(swa, g=8) == E                                       # mask built without globals
    assert fwd(swa, dil=2, g=8, mask=fake_mask(swa, 256, 32, 0, dil=2)) == E
    assert fwd(swa, dil=2, mask=fake_mask(swa, 256, 32, 0, dil=2, g=8)) == E
    assert swa.lib.swa_attn_fwd(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 4, 2, 256, 64, 32, 0, 1, 0, 0.125,
                                None, None) == E
    assert fwd(swa, B=1 << 12, Hq=1 << 10, Hkv=1 << 10, N=1 << 12,
               mask=fake_mask(swa, 1 << 12, 32, 0)) == U   # flat row index beyond int32


def test_fwd_rejects_grids_beyond_one_dispatch(swa):
    """Row indices fit int32 but the launch would need 2^32 or more work-items:
    rejected on the host, nothing launched."""
    U = swa.SWA_ERR_UNSUPPORTED
    # bf16, ragged N = 130: 2 query tiles of 128 rows for each of 2^23 heads
    assert fwd(swa, B=1 << 10, Hq=1 << 13, Hkv=1 << 13, N=130,
               mask=fake_mask(swa, 130, 32, 0)) == U
    # fp32 (32-row tiles of 256 lanes): 2^30 rows -> 2^33 work-items
    assert fwd(swa, dt=0, B=1, Hq=1 << 9, Hkv=1, N=1 << 21,
               mask=fake_mask(swa, 1 << 21, 32, 0, bm=32)) == U
    m = fake_mask(swa, 1 << 21, 32, 0, bm=32)
    assert swa.lib.diff_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 1 << 9, 1, 1 << 21, 64,
                                 64, 32, 0, 1, 0, 0.125, 0.5, ctypes.byref(m), None) == U
    # bf16 differential attention: 512 lanes per workgroup (one wave group per
    # map), 2 query tiles for each of 2^22 heads -> 2^32 work-items
    m = fake_mask(swa, 130, 32, 0, bm=128)
    assert swa.lib.diff_attn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1 << 9, 1 << 13, 1 << 13, 130,
                                 64, 64, 32, 0, 1, 0, 0.125, 0.5, ctypes.byref(m), None) == U


def dec(swa, q=FAKE, kr=FAKE, vr=FAKE, out=FAKE, sl=None, ws=FAKE, wsb=None, dt=1, B=2, Hq=8,
        Hkv=2, N=10, d=128, W=64, s=0, scale=0.1):
    if wsb is None:
        wsb = swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, W)
    return swa.lib.swa_attn_decode(q, kr, vr, out, sl, ws, wsb, dt, B, Hq, Hkv, N, d, W, s, scale, None)


def test_decode_rejections(swa):
    E, U, WS = swa.SWA_ERR_INVALID_ARG, swa.SWA_ERR_UNSUPPORTED, swa.SWA_ERR_WORKSPACE
    assert swa.swa_attn_decode_workspace_bytes(2, 8, 2, 128, 64) > 0   # the cases below need one
    assert dec(swa, q=0) == E
    assert dec(swa, vr=FAKE + 4) == E
    assert dec(swa, sl=FAKE + 2) == E
    assert dec(swa, Hq=6, Hkv=4) == E
    assert dec(swa, W=0, wsb=1 << 20) == E
    assert dec(swa, N=-1) == E
    assert dec(swa, scale=0.0) == E
    assert dec(swa, d=96) == U
    assert dec(swa, s=3) == U                    # stride keys are not in the ring
    assert dec(swa, ws=0) == WS
    assert dec(swa, wsb=swa.swa_attn_decode_workspace_bytes(2, 8, 2, 128, 64) - 4) == WS
    assert dec(swa, ws=FAKE + 8) == WS


def test_decode_noalloc_rejections(swa):
    """The no-allocation decode runs every check of swa_attn_decode, plus the
    bound of its static scratch, before its first HIP call."""
    E, U, SC = swa.SWA_ERR_INVALID_ARG, swa.SWA_ERR_UNSUPPORTED, swa.SWA_ERR_SCRATCH

    def call(q=FAKE, vr=FAKE, sl=None, dt=1, B=2, Hq=8, Hkv=2, N=100, d=128, W=64, s=0, scale=0.1):
        return swa.lib.swa_attn_decode_noalloc(q, FAKE, vr, FAKE, sl, dt, B, Hq, Hkv, N, d, W, s, scale,
                                               None)
    assert call(q=0) == E
    assert call(vr=FAKE + 4) == E
    assert call(sl=FAKE + 2) == E
    assert call(Hq=6, Hkv=4) == E
    assert call(W=0) == E
    assert call(scale=float("inf")) == E
    assert call(d=96) == U
    assert call(s=3) == U
    # 1024 query heads on one key/value head: 64 blocks of 16, 8 splits of a
    # 4096-slot ring -> 8192 partials of 130 floats, beyond the 4 MiB scratch
    need = swa.swa_attn_decode_workspace_bytes(1, 1024, 1, 128, 4096)
    assert need > swa.SWA_DECODE_SCRATCH_BYTES
    assert call(B=1, Hq=1024, Hkv=1, W=4096) == SC
    assert swa.swa_strerror(SC) not in ("success", "unknown status")


def test_decode_rejects_grids_beyond_one_dispatch(swa):
    U = swa.SWA_ERR_UNSUPPORTED
    # a one-slot window gives one 64-lane workgroup per (sequence, key/value
    # head): 2^30 pairs -> 2^36 work-items
    assert dec(swa, B=1 << 15, Hq=1 << 15, Hkv=1 << 15, W=1, d=64, wsb=0) == U
    # fp32: 8 lanes per (sequence, query head), 2^29 of them -> 2^32 work-items
    assert dec(swa, dt=0, B=1 << 15, Hq=1 << 14, Hkv=1 << 14, W=1, d=64, wsb=0) == U
    # B * Hq beyond int32 (B * Hkv * window fits)
    assert dec(swa, B=1 << 16, Hq=1 << 16, Hkv=1 << 12, W=1, d=64, wsb=0) == U


def test_decode_sinks_rejections(swa):
    E, U, WS = swa.SWA_ERR_INVALID_ARG, swa.SWA_ERR_UNSUPPORTED, swa.SWA_ERR_WORKSPACE

    def call(ks=FAKE, vs=FAKE, S=4, ws=FAKE, wsb=None, Hq=8, Hkv=2, d=64, W=60, dt=1):
        if wsb is None:
            wsb = swa.swa_attn_decode_workspace_bytes(1, Hq, Hkv, d, W, max(S, 0))
        return swa.lib.swa_attn_decode_sinks(FAKE, ks, vs, S, FAKE, FAKE, FAKE, None, ws, wsb, dt, 1,
                                             Hq, Hkv, 100, d, W, 0.125, None)
    assert call(S=-1) == E
    assert call(ks=0) == E                       # sink slots without a sink buffer
    assert call(vs=FAKE + 8) == E
    assert call(S=swa.SWA_MAX_N + 1) == E
    assert call(d=48) == U
    assert call(ws=0) == WS
    assert call(wsb=swa.swa_attn_decode_workspace_bytes(1, 8, 2, 64, 60, 4) - 16) == WS


def test_diff_decode_rejections(swa):
    E, U = swa.SWA_ERR_INVALID_ARG, swa.SWA_ERR_UNSUPPORTED

    def call(q2=FAKE, d=64, dv=128, lam=0.5, dt=1, Hq=4, Hkv=4, scale=0.125):
        wsb = swa.swa_attn_decode_workspace_bytes(2, Hq, Hkv, dv, 256, 0, swa.SWA_OP_DIFF)
        return swa.lib.diff_attn_decode(FAKE, FAKE, q2, FAKE, FAKE, FAKE, None, FAKE, wsb, dt, 2, Hq,
                                        Hkv, 300, d, dv, 256, scale, lam, None)
    assert call(q2=0) == E
    assert call(q2=FAKE + 4) == E
    assert call(lam=float("nan")) == E
    assert call(scale=-1.0) == E
    assert call(dv=96) == U


def test_decode_workspace_bytes(swa):
    ATTN, DIFF = swa.SWA_OP_ATTN, swa.SWA_OP_DIFF
    ws = lambda *a: swa.lib.swa_attn_decode_workspace_bytes(*a)
    # 512 (sequence, key/value head) pairs of a 4096-slot ring fill the chip
    # with one workgroup each: the output is written directly, no workspace
    assert ws(ATTN, 64, 32, 8, 128, 4096, 0) == 0
    assert ws(ATTN, 64, 32, 8, 128, 4096, 4) == 0
    assert ws(DIFF, 32, 16, 16, 128, 4096, 0) == 0
    # one pair, 4 steps of 32 slots: 4 splits of one wave; 12 partials of
    # (max, sum) padded to 24 floats, then 12 x 32 partial outputs
    assert ws(ATTN, 1, 3, 1, 32, 100, 0) == (24 + 12 * 32) * 4
    # 4 pairs, 128 steps: 4 waves per workgroup, 16 splits (the cap); two maps
    parts = 2 * 4 * 16 * 2
    assert ws(DIFF, 2, 4, 2, 128, 4096, 0) == (parts * 2 + parts * 128) * 4
    # sink slots count as cache slots: 60 + 4 = 64 slots = 2 steps -> 2 splits
    parts = 1 * 8 * 2
    assert ws(ATTN, 1, 8, 2, 64, 60, 4) == (parts * 2 + parts * 64) * 4
    # 32 query heads on one key/value head: two blocks of 16, each a pair of
    # the plan; 4 steps -> 4 splits of one wave; 32 heads x 4 splits partials
    parts = 32 * 4
    assert ws(ATTN, 1, 32, 1, 32, 100, 0) == (parts * 2 + parts * 32) * 4
    # invalid sizes
    assert ws(ATTN, 0, 3, 1, 32, 100, 0) == 0
    assert ws(ATTN, 1, 3, 2, 32, 100, 0) == 0
    assert ws(7, 1, 3, 1, 32, 100, 0) == 0


def test_diff_rejections(swa):
    E, U = swa.SWA_ERR_INVALID_ARG, swa.SWA_ERR_UNSUPPORTED

    def call(d=64, dv=128, dt=1, lam=0.5, q2=FAKE, W=32, mask=None, dil=1, g=0):
        m = fake_mask(swa, 256, W, 0, bm=128) if mask is None else mask
        return swa.lib.diff_attn_fwd(FAKE, FAKE, q2, FAKE, FAKE, FAKE, dt, 1, 4, 4, 256, d, dv, W, 0,
                                     dil, g, 0.125, lam, ctypes.byref(m), None)
    assert call(q2=0) == E
    assert call(lam=float("inf")) == E
    assert call(d=96) == U
    assert call(mask=fake_mask(swa, 256, 31, 0, bm=128)) == E
    assert call(mask=fake_mask(swa, 256, 32, 0, bm=64)) == E         # another tiling
    assert call(dil=3) == E                                          # another dilation
    assert call(g=1) == E                                            # another global count


def test_block_mask_build_rejections(swa):
    E = swa.SWA_ERR_INVALID_ARG
    assert swa.lib.swa_block_mask_build(None, None) == E
    m = fake_mask(swa, 300, 20, 0, bm=128, bn=64)
    m.nnz += 1
    assert swa.lib.swa_block_mask_build(ctypes.byref(m), None) == E
    m = fake_mask(swa, 300, 20, 0, null=True)
    assert swa.lib.swa_block_mask_build(ctypes.byref(m), None) == E
    assert swa.lib.swa_mask_dense(20000, 4, 0, 1, 0, FAKE, None) == E
    assert swa.lib.swa_mask_dense(20, 4, 0, 1, 0, None, None) == E
    assert swa.lib.swa_mask_dense(20, 4, 0, 0, 0, FAKE, None) == E
    assert swa.lib.swa_mask_dense(20, 4, 0, 1, -2, FAKE, None) == E
