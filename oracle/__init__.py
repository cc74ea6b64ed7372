"""fp64 CPU oracle for masked causal attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never loads it and
shares no code with it.  The arithmetic lives in ``oracle.c`` (plain C,
double precision); this module only marshals numpy arrays through ctypes.

Each wrapper names the page passage its C function follows; see ``oracle.c``
for the definitions written out.
"""
import contextlib
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_ptr = ctypes.c_void_p


def _configure(lib):
    """Declare the C signatures of oracle.c on a loaded library."""
    lib.orc_allowed.restype = ctypes.c_int
    lib.orc_allowed.argtypes = [_i64] * 7
    lib.orc_mask_dense.restype = None
    lib.orc_mask_dense.argtypes = [_i64] * 5 + [_ptr]
    lib.orc_count_nonmasked.restype = _i64
    lib.orc_count_nonmasked.argtypes = [_i64] * 5 + [_ptr]
    lib.orc_tile_list.restype = _i64
    lib.orc_tile_list.argtypes = [_i64] * 7 + [_ptr] * 6 + [_i64]
    lib.orc_attention_row.restype = _dbl
    lib.orc_attention_row.argtypes = [_ptr] * 4 + [_i64] * 5 + [_dbl, _ptr, _ptr]
    lib.orc_tiled_softmax_dot.restype = None
    lib.orc_tiled_softmax_dot.argtypes = [_ptr] * 3 + [_i64] * 4 + [_dbl, _ptr]
    lib.orc_attn_rows.restype = None
    lib.orc_attn_rows.argtypes = [_ptr] * 3 + [_i64] * 10 + [_dbl, _ptr, _i64, _ptr, _ptr]
    lib.orc_attn_full.restype = None
    lib.orc_attn_full.argtypes = [_ptr] * 3 + [_i64] * 10 + [_dbl, _ptr, _ptr]
    lib.orc_diff_rows.restype = None
    lib.orc_diff_rows.argtypes = [_ptr] * 5 + [_i64] * 10 + [_dbl, _dbl, _ptr, _i64, _ptr]
    lib.orc_decode.restype = None
    lib.orc_decode.argtypes = [_ptr] * 6 + [_i64] * 7 + [_dbl, _ptr, _ptr]
    lib.orc_count_nsa.restype = _i64
    lib.orc_count_nsa.argtypes = [_i64] * 4
    lib.orc_kv_cache_bytes.restype = _i64
    lib.orc_kv_cache_bytes.argtypes = [_i64] * 5
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle.build import build
            build()
        _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Run the wrappers of this module against another build of oracle.c
    (the mutation tests compile deliberately broken copies on the CPU)."""
    global _lib
    saved = _lib
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data


def _p(a):
    return a.ctypes.data if a is not None else None


def allowed(i, j, n, window, stride=0, dilation=1, n_global=0):
    """Mask predicate of swa_mask / strided_mask ("Attention Variants Compared"),
    with Longformer's dilation and global tokens ("Learn: Sparse &
    Sliding-Window Attention" §3b) under the causal order."""
    return bool(_load().orc_allowed(i, j, n, window, stride, dilation, n_global))


def mask_dense(n, window, stride=0, dilation=1, n_global=0):
    """Dense 0/1 uint8 [n, n] mask (1 = attends)."""
    out = np.zeros((n, n), dtype=np.uint8)
    _load().orc_mask_dense(n, window, stride, dilation, n_global, out.ctypes.data)
    return out


def count_nonmasked(n, window, stride=0, dilation=1, n_global=0):
    """(total, per-row counts) of attended cells -- count_nonmasked(M)."""
    rows = np.zeros(n, dtype=np.int64)
    total = _load().orc_count_nonmasked(n, window, stride, dilation, n_global, rows.ctypes.data)
    return int(total), rows


def tile_list(n, window, stride, bm, bn, dilation=1, n_global=0):
    """Block mask as a CSR over query tiles (see orc_tile_list)."""
    nq, nk = -(-n // bm), -(-n // bn)
    cap = nq * nk
    row_ptr = np.zeros(nq + 1, dtype=np.int32)
    kv_tile = np.zeros(max(cap, 1), dtype=np.int32)
    kind = np.zeros(max(cap, 1), dtype=np.uint8)
    cells = np.zeros(max(cap, 1), dtype=np.int32)
    prefix_keys = np.zeros(nq, dtype=np.int32)
    band_begin = np.zeros(nq, dtype=np.int32)
    nnz = _load().orc_tile_list(n, window, stride, dilation, n_global, bm, bn,
                                row_ptr.ctypes.data, kv_tile.ctypes.data, kind.ctypes.data,
                                cells.ctypes.data, prefix_keys.ctypes.data, band_begin.ctypes.data,
                                cap)
    assert nnz >= 0
    return dict(row_ptr=row_ptr, kv_tile=kv_tile[:nnz].copy(), kind=kind[:nnz].copy(),
                cells=cells[:nnz].copy(), prefix_keys=prefix_keys, band_begin=band_begin,
                nnz=int(nnz), num_q_tiles=nq)


def attention_row(q, K, V, mask_row, scale):
    """attention_row(q, K, V, mask_row) -> (out, weights, lse)."""
    q, qp = _f32(q)
    K, kp = _f32(K)
    V, vp = _f32(V)
    m = np.ascontiguousarray(mask_row, dtype=np.uint8)
    n, d = K.shape
    dv = V.shape[1]
    out = np.zeros(dv, dtype=np.float64)
    w = np.zeros(n, dtype=np.float64)
    lse = _load().orc_attention_row(qp, kp, vp, m.ctypes.data, n, d, dv, d, dv, scale,
                                    out.ctypes.data, w.ctypes.data)
    return out, w, lse


def tiled_softmax_dot(q, K, V, scale, tile=4):
    """Flash-style tiled online softmax over all keys of K/V for one query."""
    q, qp = _f32(q)
    K, kp = _f32(K)
    V, vp = _f32(V)
    n, d = K.shape
    dv = V.shape[1]
    out = np.zeros(dv, dtype=np.float64)
    _load().orc_tiled_softmax_dot(qp, kp, vp, n, d, dv, tile, scale, out.ctypes.data)
    return out


def attn_rows(q, k, v, window, stride, scale, rows, with_lse=False, dilation=1, n_global=0):
    """Masked attention for selected flat rows (b*Hq + h)*N + i.

    q: [B, Hq, N, d]; k: [B, Hkv, N, d]; v: [B, Hkv, N, dv] (float32 values).
    Returns out [len(rows), dv] float64 (and lse [len(rows)])."""
    q, qp = _f32(q)
    k, kp = _f32(k)
    v, vp = _f32(v)
    B, Hq, N, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), dv), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    _load().orc_attn_rows(qp, kp, vp, B, Hq, Hkv, N, d, dv, window, stride, dilation, n_global,
                          scale, rows.ctypes.data, len(rows), out.ctypes.data, lse.ctypes.data)
    return (out, lse) if with_lse else out


def attn_full(q, k, v, window, stride, scale, with_lse=False, dilation=1, n_global=0):
    """Masked attention for every row: out [B, Hq, N, dv] float64."""
    q, qp = _f32(q)
    k, kp = _f32(k)
    v, vp = _f32(v)
    B, Hq, N, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    out = np.zeros((B, Hq, N, dv), dtype=np.float64)
    lse = np.zeros((B, Hq, N), dtype=np.float64)
    _load().orc_attn_full(qp, kp, vp, B, Hq, Hkv, N, d, dv, window, stride, dilation, n_global,
                          scale, out.ctypes.data, lse.ctypes.data)
    return (out, lse) if with_lse else out


def diff_rows(q1, k1, q2, k2, v, window, stride, scale, lam, rows, dilation=1, n_global=0):
    """Differential attention for selected flat rows: out [len(rows), dv]."""
    q1, q1p = _f32(q1)
    k1, k1p = _f32(k1)
    q2, q2p = _f32(q2)
    k2, k2p = _f32(k2)
    v, vp = _f32(v)
    B, Hq, N, d = q1.shape
    Hkv, dv = k1.shape[1], v.shape[3]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), dv), dtype=np.float64)
    _load().orc_diff_rows(q1p, k1p, q2p, k2p, vp, B, Hq, Hkv, N, d, dv, window, stride, dilation,
                          n_global, scale, lam, rows.ctypes.data, len(rows), out.ctypes.data)
    return out


def diff_full(q1, k1, q2, k2, v, window, stride, scale, lam, dilation=1, n_global=0):
    B, Hq, N, _ = q1.shape
    out = diff_rows(q1, k1, q2, k2, v, window, stride, scale, lam, np.arange(B * Hq * N),
                    dilation=dilation, n_global=n_global)
    return out.reshape(B, Hq, N, -1)


def decode(q, k_ring, v_ring, seq_len, scale, k_sink=None, v_sink=None, with_lse=False):
    """One decode step over a rolling KV window (optionally with sink slots).

    q: [B, Hq, d]; k_ring/v_ring: [B, Hkv, W, d|dv]; seq_len: [B] tokens so far
    (current one included); k_sink/v_sink: [B, Hkv, S, d|dv] or None."""
    q, qp = _f32(q)
    kr, krp = _f32(k_ring)
    vr, vrp = _f32(v_ring)
    B, Hq, d = q.shape
    Hkv, W, dv = kr.shape[1], kr.shape[2], vr.shape[3]
    if k_sink is not None:
        ks, ksp = _f32(k_sink)
        vs, vsp = _f32(v_sink)
        S = ks.shape[2]
    else:
        ks = vs = None
        ksp = vsp = None
        S = 0
    sl = np.ascontiguousarray(seq_len, dtype=np.int64)
    out = np.zeros((B, Hq, dv), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    _load().orc_decode(qp, krp, vrp, ksp, vsp, sl.ctypes.data, B, Hq, Hkv, W, S, d, dv, scale,
                       out.ctypes.data, lse.ctypes.data)
    return (out, lse) if with_lse else out


def diff_decode(q1, k1_ring, q2, k2_ring, v_ring, seq_len, scale, lam):
    """Differential attention for one decode step over a rolling window
    ("Attention Variants — Sliding Window, Sparse, Differential": the second
    map's attention output, weighted by lambda, is subtracted from the
    first's; both read the same values):
    decode(q1, K1, V) - lam * decode(q2, K2, V).  Shapes as decode()."""
    a = decode(q1, k1_ring, v_ring, seq_len, scale)
    b = decode(q2, k2_ring, v_ring, seq_len, scale)
    return a - lam * b


def count_nsa(n, l, k, w):
    """count_nsa(N, l, k, W): keys read per query by native sparse attention."""
    return int(_load().orc_count_nsa(n, l, k, w))


def kv_cache_bytes(N, n_layers, n_heads_kv, d_head, dtype=2):
    """kv_cache_bytes(N, n_layers, n_heads_kv, d_head, dtype=2): bytes of the
    keys and values kept for N positions ("Attention Variants Compared",
    task table)."""
    return int(_load().orc_kv_cache_bytes(N, n_layers, n_heads_kv, d_head, dtype))
