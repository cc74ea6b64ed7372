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

from ._abi import (SWA_OK, SWA_ERR_INVALID_ARG, SWA_ERR_UNSUPPORTED, SWA_ERR_WORKSPACE,  # noqa: E402
                   SWA_ERR_HIP, SWA_ERR_SCRATCH, SWA_DECODE_SCRATCH_BYTES, SWA_F32, SWA_BF16,
                   SWA_OP_ATTN, SWA_OP_DIFF, SWA_MAX_N, SwaError, swa_block_mask_t)
from . import _abi  # noqa: E402

_lib = _abi.configure(ctypes.CDLL(LIB_PATH))
lib = _lib  # raw ctypes handle (the tests call the C functions directly)


def _check(status, where):
    _abi.check(_lib, status, where)


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
    if not isinstance(t, torch.Tensor) or not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor on the GPU")


def _dims(t, name, n):
    _need(t, name)
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _expect(t, name, shape, dtype, device):
    """The kernels index every buffer from the sizes passed with it: a buffer
    of another shape, dtype or device would be read or written out of
    bounds, so it is rejected here, before the call."""
    _need(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _expect_mask(mask, device):
    if mask.row_ptr.device != device:
        raise ValueError(f"block mask is on {mask.row_ptr.device}, expected {device}")


def _expect_seq_len(seq_len, B, device):
    if seq_len is not None:
        _expect(seq_len, "seq_len", (B,), torch.int32, device)


def _expect_workspace(workspace, device):
    if workspace is not None:
        _need(workspace, "workspace")
        if workspace.device != device:
            raise ValueError(f"workspace is on {workspace.device}, expected {device}")


def swa_strerror(status):
    return _abi.strerror(_lib, status)


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
    return _abi.block_mask_query(_lib, N, window, stride, bm, bn, dilation, n_global)


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
    B, Hq, N, d = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[1]
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _expect(t, n, (B, Hkv, N, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", (B, Hq, N, d), q.dtype, dev)
    if lse is not None:
        _expect(lse, "lse", (B, Hq, N), torch.float32, dev)
    _expect_mask(mask, dev)
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
    B, Hq, d = _dims(q, "q", 3)
    _, Hkv, W, _ = _dims(k_ring, "k_ring", 4)
    dev = q.device
    for t, n in ((k_ring, "k_ring"), (v_ring, "v_ring")):
        _expect(t, n, (B, Hkv, W, d), q.dtype, dev)
    _expect_seq_len(seq_len, B, dev)
    _expect_workspace(workspace, dev)
    ws, ws_bytes = _workspace(workspace, swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, W), dev)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", (B, Hq, d), q.dtype, dev)
    _check(_lib.swa_attn_decode(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(out), _ptr(seq_len),
                                _ptr(ws), ws_bytes, _dtype_code(q), B, Hq, Hkv, N, d, W, stride,
                                float(scale), _stream(q)), "swa_attn_decode")
    return out


def swa_attn_decode_noalloc(q, k_ring, v_ring, seq_len, scale, out, N=0, stride=0):
    """swa_attn_decode with the library's static per-GPU scratch in place of a
    workspace: the call itself allocates nothing (`out` is required).  Calls
    that overlap in time on one GPU race on that scratch."""
    B, Hq, d = _dims(q, "q", 3)
    _, Hkv, W, _ = _dims(k_ring, "k_ring", 4)
    dev = q.device
    for t, n in ((k_ring, "k_ring"), (v_ring, "v_ring")):
        _expect(t, n, (B, Hkv, W, d), q.dtype, dev)
    _expect_seq_len(seq_len, B, dev)
    _expect(out, "out", (B, Hq, d), q.dtype, dev)
    _check(_lib.swa_attn_decode_noalloc(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(out), _ptr(seq_len),
                                        _dtype_code(q), B, Hq, Hkv, N, d, W, stride, float(scale),
                                        _stream(q)), "swa_attn_decode_noalloc")
    return out


def swa_attn_decode_sinks(q, k_sink, v_sink, k_ring, v_ring, seq_len, scale, workspace=None,
                          out=None, N=0):
    """Decode step with sink slots.  k_sink/v_sink [B,Hkv,S,d] hold positions
    0..S-1; k_ring/v_ring [B,Hkv,W,d]; returns out [B,Hq,d]."""
    B, Hq, d = _dims(q, "q", 3)
    _, Hkv, W, _ = _dims(k_ring, "k_ring", 4)
    S = _dims(k_sink, "k_sink", 4)[2]
    dev = q.device
    for t, n in ((k_ring, "k_ring"), (v_ring, "v_ring")):
        _expect(t, n, (B, Hkv, W, d), q.dtype, dev)
    for t, n in ((k_sink, "k_sink"), (v_sink, "v_sink")):
        _expect(t, n, (B, Hkv, S, d), q.dtype, dev)
    _expect_seq_len(seq_len, B, dev)
    _expect_workspace(workspace, dev)
    ws, ws_bytes = _workspace(workspace, swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, W, S), dev)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", (B, Hq, d), q.dtype, dev)
    _check(_lib.swa_attn_decode_sinks(_ptr(q), _ptr(k_sink), _ptr(v_sink), S, _ptr(k_ring),
                                      _ptr(v_ring), _ptr(out), _ptr(seq_len), _ptr(ws), ws_bytes,
                                      _dtype_code(q), B, Hq, Hkv, N, d, W, float(scale), _stream(q)),
           "swa_attn_decode_sinks")
    return out


def diff_attn_decode(q1, k1_ring, q2, k2_ring, v_ring, seq_len, scale, lam, workspace=None,
                     out=None, N=0):
    """Differential decode step.  q1/q2 [B,Hq,d]; k1_ring/k2_ring [B,Hkv,W,d];
    v_ring [B,Hkv,W,dv]; returns out [B,Hq,dv]."""
    B, Hq, d = _dims(q1, "q1", 3)
    _, Hkv, W, dv = _dims(v_ring, "v_ring", 4)
    dev, dt = q1.device, q1.dtype
    _expect(q2, "q2", (B, Hq, d), dt, dev)
    for t, n in ((k1_ring, "k1_ring"), (k2_ring, "k2_ring")):
        _expect(t, n, (B, Hkv, W, d), dt, dev)
    _expect(v_ring, "v_ring", (B, Hkv, W, dv), dt, dev)
    _expect_seq_len(seq_len, B, dev)
    _expect_workspace(workspace, dev)
    ws, ws_bytes = _workspace(workspace, swa_attn_decode_workspace_bytes(B, Hq, Hkv, dv, W, 0,
                                                                         SWA_OP_DIFF), dev)
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=dt, device=dev)
    _expect(out, "out", (B, Hq, dv), dt, dev)
    _check(_lib.diff_attn_decode(_ptr(q1), _ptr(k1_ring), _ptr(q2), _ptr(k2_ring), _ptr(v_ring),
                                 _ptr(out), _ptr(seq_len), _ptr(ws), ws_bytes, _dtype_code(q1), B,
                                 Hq, Hkv, N, d, dv, W, float(scale), float(lam), _stream(q1)),
           "diff_attn_decode")
    return out


def diff_attn_fwd(q1, k1, q2, k2, v, window, stride, scale, lam, mask, out=None):
    """Differential attention: (softmax(q1 k1^T s + log M) - lam softmax(q2 k2^T s + log M)) v."""
    B, Hq, N, d = _dims(q1, "q1", 4)
    Hkv = _dims(k1, "k1", 4)[1]
    dv = _dims(v, "v", 4)[3]
    dev, dt = q1.device, q1.dtype
    _expect(q2, "q2", (B, Hq, N, d), dt, dev)
    for t, n in ((k1, "k1"), (k2, "k2")):
        _expect(t, n, (B, Hkv, N, d), dt, dev)
    _expect(v, "v", (B, Hkv, N, dv), dt, dev)
    if out is None:
        out = torch.empty((B, Hq, N, dv), dtype=dt, device=dev)
    _expect(out, "out", (B, Hq, N, dv), dt, dev)
    _expect_mask(mask, dev)
    _check(_lib.diff_attn_fwd(_ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(out),
                              _dtype_code(q1), B, Hq, Hkv, N, d, dv, window, stride, mask.dilation,
                              mask.n_global, float(scale), float(lam), ctypes.byref(mask.c),
                              _stream(q1)), "diff_attn_fwd")
    return out


__all__ = ["swa_tile_config", "swa_block_mask_query", "swa_block_mask_build", "swa_mask_dense",
           "swa_attn_fwd", "swa_attn_decode_workspace_bytes", "swa_attn_decode", "swa_attn_decode_noalloc",
           "swa_attn_decode_sinks", "diff_attn_decode", "diff_attn_fwd",
           "swa_strerror", "SwaError", "BlockMask"]


# ---- measurement probes (include/swa_probe.h) ---------------------------------
def swa_probe_mfma_bf16(operands, out, workgroups, iters):
    """Dense bf16 MFMA loop: `operands` 512 x 8 bf16 (device), `out`
    workgroups * 512 float32.  FLOP per call: workgroups * 8 * iters * 32 * 32768."""
    _expect(operands, "operands", (512, 8), torch.bfloat16, operands.device)
    _expect(out, "out", (workgroups * 512,), torch.float32, operands.device)
    _check(_lib.swa_probe_mfma_bf16(_ptr(operands), _ptr(out), workgroups, iters, _stream(out)),
           "swa_probe_mfma_bf16")
    return out


def swa_probe_stream_read(buf, out, workgroups):
    """Streaming read of the contiguous device tensor `buf` with 16-byte loads;
    `out` workgroups * 256 int32."""
    _need(buf, "buf")
    _expect(out, "out", (workgroups * 256,), torch.int32, buf.device)
    _check(_lib.swa_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), workgroups,
                                      _stream(out)), "swa_probe_stream_read")
    return out
