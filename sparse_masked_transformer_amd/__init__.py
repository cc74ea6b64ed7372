"""Python binding of libswa.so, the gfx950 masked causal attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/swa.h, and each function here
has the name of the C entry point it calls.  PyTorch provides device memory
and the current HIP stream.  Importing this package fails if the library has
not been built (``python sparse_masked_transformer_amd/build.py``); there is
no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with "
                      "`python sparse_masked_transformer_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

SWA_OK, SWA_ERR_INVALID_ARG, SWA_ERR_UNSUPPORTED, SWA_ERR_WORKSPACE, SWA_ERR_HIP = 0, -1, -2, -3, -4
SWA_F32, SWA_BF16 = 0, 1
SWA_OP_ATTN, SWA_OP_DIFF = 0, 1
SWA_MAX_N = 1 << 22

_p = ctypes.c_void_p
_i = ctypes.c_int
_i32p = ctypes.POINTER(ctypes.c_int32)


class swa_block_mask_t(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("window", ctypes.c_int32), ("stride", ctypes.c_int32),
                ("dilation", ctypes.c_int32), ("n_global", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("bn", ctypes.c_int32),
                ("num_q_tiles", ctypes.c_int32), ("nnz", ctypes.c_int32),
                ("row_ptr", _p), ("kv_tile", _p), ("kind", _p), ("cells", _p),
                ("prefix_keys", _p), ("band_begin", _p)]


_lib.swa_tile_config.restype = _i
_lib.swa_tile_config.argtypes = [_i, _i, _i, _i, _i32p, _i32p]
_lib.swa_block_mask_query.restype = _i
_lib.swa_block_mask_query.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i32p, _i32p]
_lib.swa_block_mask_build.restype = _i
_lib.swa_block_mask_build.argtypes = [ctypes.POINTER(swa_block_mask_t), _p]
_lib.swa_mask_dense.restype = _i
_lib.swa_mask_dense.argtypes = [_i, _i, _i, _i, _i, _p, _p]
_lib.swa_attn_fwd.restype = _i
_lib.swa_attn_fwd.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                              ctypes.c_float, ctypes.POINTER(swa_block_mask_t), _p]
_lib.swa_attn_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.swa_attn_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
_lib.swa_attn_decode.restype = _i
_lib.swa_attn_decode.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_size_t, _i, _i, _i, _i, _i, _i,
                                 _i, _i, ctypes.c_float, _p]
_lib.swa_attn_decode_sinks.restype = _i
_lib.swa_attn_decode_sinks.argtypes = [_p, _p, _p, _i, _p, _p, _p, _p, _p, ctypes.c_size_t, _i, _i,
                                       _i, _i, _i, _i, _i, ctypes.c_float, _p]
_lib.diff_attn_decode.restype = _i
_lib.diff_attn_decode.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _i, _i, _i, _i,
                                  _i, _i, _i, _i, ctypes.c_float, ctypes.c_float, _p]
_lib.diff_attn_fwd.restype = _i
_lib.diff_attn_fwd.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                               ctypes.c_float, ctypes.c_float, ctypes.POINTER(swa_block_mask_t), _p]
_lib.swa_strerror.restype = ctypes.c_char_p
_lib.swa_strerror.argtypes = [_i]

lib = _lib  # raw ctypes handle (the tests call the C functions directly)


class SwaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {swa_strerror(status)} ({status})")


def _check(status, where):
    if status != SWA_OK:
        raise SwaError(status, where)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor on the GPU")


def swa_strerror(status):
    return _lib.swa_strerror(status).decode()


def swa_tile_config(dtype, d, dv=None, op=SWA_OP_ATTN):
    """(bm, bn): query-tile rows and key-tile keys the kernel of `op` walks."""
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    code = SWA_BF16 if dtype == torch.bfloat16 else SWA_F32
    _check(_lib.swa_tile_config(op, code, d, dv or d, ctypes.byref(bm), ctypes.byref(bn)),
           "swa_tile_config")
    return bm.value, bn.value


def swa_block_mask_query(N, window, stride, bm, bn, dilation=1, n_global=0):
    """(num_q_tiles, nnz) of the block mask of (N, window, stride, dilation,
    n_global, bm, bn)."""
    nq, nnz = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.swa_block_mask_query(N, window, stride, dilation, n_global, bm, bn, ctypes.byref(nq),
                                     ctypes.byref(nnz)), "swa_block_mask_query")
    return nq.value, nnz.value


class BlockMask:
    """Device block mask (CSR over query tiles) plus its C struct."""

    def __init__(self, N, window, stride, bm, bn, device, dilation=1, n_global=0):
        nq, nnz = swa_block_mask_query(N, window, stride, bm, bn, dilation, n_global)
        i32 = dict(dtype=torch.int32, device=device)
        self.row_ptr = torch.empty(nq + 1, **i32)
        self.kv_tile = torch.empty(max(nnz, 1), **i32)
        self.kind = torch.empty(max(nnz, 1), dtype=torch.uint8, device=device)
        self.cells = torch.empty(max(nnz, 1), **i32)
        self.prefix_keys = torch.empty(nq, **i32)
        self.band_begin = torch.empty(nq, **i32)
        self.N, self.window, self.stride, self.bm, self.bn = N, window, stride, bm, bn
        self.dilation, self.n_global = dilation, n_global
        self.num_q_tiles, self.nnz = nq, nnz
        self.c = swa_block_mask_t(N, window, stride, dilation, n_global, bm, bn, nq, nnz,
                                  self.row_ptr.data_ptr(), self.kv_tile.data_ptr(),
                                  self.kind.data_ptr(), self.cells.data_ptr(),
                                  self.prefix_keys.data_ptr(), self.band_begin.data_ptr())

    def host(self):
        """Copy of the CSR arrays as numpy (synchronizes)."""
        n = self.nnz
        return dict(row_ptr=self.row_ptr.cpu().numpy(), kv_tile=self.kv_tile[:n].cpu().numpy(),
                    kind=self.kind[:n].cpu().numpy(), cells=self.cells[:n].cpu().numpy(),
                    prefix_keys=self.prefix_keys.cpu().numpy(),
                    band_begin=self.band_begin.cpu().numpy(), nnz=n, num_q_tiles=self.num_q_tiles)


def swa_block_mask_build(N, window, stride=0, bm=None, bn=None, device="cuda",
                         dtype=torch.bfloat16, d=128, dv=None, into=None, op=SWA_OP_ATTN,
                         dilation=1, n_global=0):
    """Build the block mask on the GPU (asynchronous on the current stream),
    into a new BlockMask or into `into` (same sizes, arrays reused).  bm/bn
    default to the tile shape of the kernel serving (op, dtype)."""
    if bm is None or bn is None:
        bm, bn = swa_tile_config(dtype, d, dv, op)
    key = (N, window, stride, dilation, n_global, bm, bn)
    if into is not None:
        if (into.N, into.window, into.stride, into.dilation, into.n_global, into.bm, into.bn) != key:
            raise ValueError("`into` was allocated for another mask")
        m = into
    else:
        m = BlockMask(N, window, stride, bm, bn, torch.device(device), dilation, n_global)
    _check(_lib.swa_block_mask_build(ctypes.byref(m.c), _stream(m.row_ptr)), "swa_block_mask_build")
    return m


def swa_mask_dense(N, window, stride=0, device="cuda", dilation=1, n_global=0):
    """Dense uint8 [N, N] mask computed on the GPU (debug export)."""
    out = torch.empty((N, N), dtype=torch.uint8, device=device)
    _check(_lib.swa_mask_dense(N, window, stride, dilation, n_global, _ptr(out), _stream(out)),
           "swa_mask_dense")
    return out


def swa_attn_fwd(q, k, v, window, stride, scale, mask, out=None, lse=None):
    """Masked attention forward.  q [B,Hq,N,d], k/v [B,Hkv,N,d]; returns out."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    _check(_lib.swa_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q), B, Hq,
                             Hkv, N, d, window, stride, mask.dilation, mask.n_global, float(scale),
                             ctypes.byref(mask.c), _stream(q)), "swa_attn_fwd")
    return out


def swa_attn_decode_workspace_bytes(B, Hq, Hkv, dv, window, n_sink=0, op=SWA_OP_ATTN):
    """Workspace bytes of a decode call (0: none needed)."""
    return int(_lib.swa_attn_decode_workspace_bytes(op, B, Hq, Hkv, dv, window, n_sink))


def _workspace(workspace, nbytes, device):
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def swa_attn_decode(q, k_ring, v_ring, seq_len, scale, workspace=None, out=None, N=0, stride=0):
    """One decode step.  q [B,Hq,d]; k_ring/v_ring [B,Hkv,W,d]; seq_len int32
    [B] on the GPU (or None: every sequence at length N); returns out."""
    for t, n in ((q, "q"), (k_ring, "k_ring"), (v_ring, "v_ring")):
        _need(t, n)
    B, Hq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    ws, ws_bytes = _workspace(workspace, swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, W), q.device)
    if out is None:
        out = torch.empty_like(q)
    _check(_lib.swa_attn_decode(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(out), _ptr(seq_len),
                                _ptr(ws), ws_bytes, _dtype_code(q), B, Hq, Hkv, N, d, W, stride,
                                float(scale), _stream(q)), "swa_attn_decode")
    return out


def swa_attn_decode_sinks(q, k_sink, v_sink, k_ring, v_ring, seq_len, scale, workspace=None,
                          out=None, N=0):
    """Decode step with sink slots.  k_sink/v_sink [B,Hkv,S,d] hold positions
    0..S-1; k_ring/v_ring [B,Hkv,W,d]; returns out [B,Hq,d]."""
    for t, n in ((q, "q"), (k_sink, "k_sink"), (v_sink, "v_sink"), (k_ring, "k_ring"),
                 (v_ring, "v_ring")):
        _need(t, n)
    B, Hq, d = q.shape
    Hkv, S, W = k_ring.shape[1], k_sink.shape[2], k_ring.shape[2]
    ws, ws_bytes = _workspace(workspace, swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, W, S),
                              q.device)
    if out is None:
        out = torch.empty_like(q)
    _check(_lib.swa_attn_decode_sinks(_ptr(q), _ptr(k_sink), _ptr(v_sink), S, _ptr(k_ring),
                                      _ptr(v_ring), _ptr(out), _ptr(seq_len), _ptr(ws), ws_bytes,
                                      _dtype_code(q), B, Hq, Hkv, N, d, W, float(scale), _stream(q)),
           "swa_attn_decode_sinks")
    return out


def diff_attn_decode(q1, k1_ring, q2, k2_ring, v_ring, seq_len, scale, lam, workspace=None,
                     out=None, N=0):
    """Differential decode step.  q1/q2 [B,Hq,d]; k1_ring/k2_ring [B,Hkv,W,d];
    v_ring [B,Hkv,W,dv]; returns out [B,Hq,dv]."""
    for t, n in ((q1, "q1"), (k1_ring, "k1_ring"), (q2, "q2"), (k2_ring, "k2_ring"),
                 (v_ring, "v_ring")):
        _need(t, n)
    B, Hq, d = q1.shape
    Hkv, W, dv = v_ring.shape[1], v_ring.shape[2], v_ring.shape[3]
    ws, ws_bytes = _workspace(workspace, swa_attn_decode_workspace_bytes(B, Hq, Hkv, dv, W, 0,
                                                                         SWA_OP_DIFF), q1.device)
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=q1.dtype, device=q1.device)
    _check(_lib.diff_attn_decode(_ptr(q1), _ptr(k1_ring), _ptr(q2), _ptr(k2_ring), _ptr(v_ring),
                                 _ptr(out), _ptr(seq_len), _ptr(ws), ws_bytes, _dtype_code(q1), B,
                                 Hq, Hkv, N, d, dv, W, float(scale), float(lam), _stream(q1)),
           "diff_attn_decode")
    return out


def diff_attn_fwd(q1, k1, q2, k2, v, window, stride, scale, lam, mask, out=None):
    """Differential attention: (softmax(q1 k1^T s + log M) - lam softmax(q2 k2^T s + log M)) v."""
    for t, n in ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v")):
        _need(t, n)
    B, Hq, N, d = q1.shape
    Hkv, dv = k1.shape[1], v.shape[3]
    if out is None:
        out = torch.empty((B, Hq, N, dv), dtype=q1.dtype, device=q1.device)
    _check(_lib.diff_attn_fwd(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(out),
                              _dtype_code(q1), B, Hq, Hkv, N, d, dv, window, stride, mask.dilation,
                              mask.n_global, float(scale), float(lam), ctypes.byref(mask.c),
                              _stream(q1)), "diff_attn_fwd")
    return out


__all__ = ["swa_tile_config", "swa_block_mask_query", "swa_block_mask_build", "swa_mask_dense",
           "swa_attn_fwd", "swa_attn_decode_workspace_bytes", "swa_attn_decode",
           "swa_attn_decode_sinks", "diff_attn_decode", "diff_attn_fwd",
           "swa_strerror", "SwaError", "BlockMask"]
