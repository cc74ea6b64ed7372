"""ctypes layer of libswa.so: the status codes and constants of include/swa.h,
the block-mask struct, the C signatures and the calls that run on the host
only (error strings, block-mask and workspace sizing).  It imports no
PyTorch, so the host-side code of the library can also be exercised against
another build of it (the sanitizer run of the test suite does)."""
import ctypes
import types

SWA_OK, SWA_ERR_INVALID_ARG, SWA_ERR_UNSUPPORTED, SWA_ERR_WORKSPACE, SWA_ERR_HIP = 0, -1, -2, -3, -4
SWA_ERR_SCRATCH = -5
SWA_DECODE_SCRATCH_BYTES = 4 << 20
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


def configure(lib):
    """Set the result and argument types of every entry point of include/*.h."""
    sig = {
        "swa_tile_config": (_i, [_i, _i, _i, _i, _i32p, _i32p]),
        "swa_block_mask_query": (_i, [_i, _i, _i, _i, _i, _i, _i, _i32p, _i32p]),
        "swa_block_mask_build": (_i, [ctypes.POINTER(swa_block_mask_t), _p]),
        "swa_mask_dense": (_i, [_i, _i, _i, _i, _i, _p, _p]),
        "swa_attn_fwd": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                              ctypes.c_float, ctypes.POINTER(swa_block_mask_t), _p]),
        "swa_attn_decode_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i, _i, _i]),
        "swa_attn_decode": (_i, [_p, _p, _p, _p, _p, _p, ctypes.c_size_t, _i, _i, _i, _i, _i, _i,
                                 _i, _i, ctypes.c_float, _p]),
        "swa_attn_decode_noalloc": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
                                         ctypes.c_float, _p]),
        "swa_attn_decode_sinks": (_i, [_p, _p, _p, _i, _p, _p, _p, _p, _p, ctypes.c_size_t, _i, _i,
                                       _i, _i, _i, _i, _i, ctypes.c_float, _p]),
        "diff_attn_decode": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _i, _i, _i, _i,
                                  _i, _i, _i, _i, ctypes.c_float, ctypes.c_float, _p]),
        "diff_attn_fwd": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                               ctypes.c_float, ctypes.c_float, ctypes.POINTER(swa_block_mask_t), _p]),
        "swa_probe_mfma_bf16": (_i, [_p, _p, _i, _i, _p]),
        "swa_probe_stream_read": (_i, [_p, ctypes.c_size_t, _p, _i, _p]),
        "swa_strerror": (ctypes.c_char_p, [_i]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


class SwaError(RuntimeError):
    def __init__(self, status, where, lib=None):
        self.status = status
        text = lib.swa_strerror(status).decode() if lib is not None else "error"
        super().__init__(f"{where}: {text} ({status})")


def check(lib, status, where):
    if status != SWA_OK:
        raise SwaError(status, where, lib)


def strerror(lib, status):
    return lib.swa_strerror(status).decode()


def block_mask_query(lib, N, window, stride, bm, bn, dilation=1, n_global=0):
    """(num_q_tiles, nnz) of the block mask of (N, window, stride, dilation,
    n_global, bm, bn)."""
    nq, nnz = ctypes.c_int32(), ctypes.c_int32()
    check(lib, lib.swa_block_mask_query(N, window, stride, dilation, n_global, bm, bn, ctypes.byref(nq),
                                        ctypes.byref(nnz)), "swa_block_mask_query")
    return nq.value, nnz.value


def decode_workspace_bytes(lib, B, Hq, Hkv, dv, window, n_sink=0, op=SWA_OP_ATTN):
    return int(lib.swa_attn_decode_workspace_bytes(op, B, Hq, Hkv, dv, window, n_sink))


def namespace(lib, path):
    """The host-only surface of the binding over `lib` (a configured ctypes
    handle of some build of the library at `path`)."""
    ns = types.SimpleNamespace(lib=lib, LIB_PATH=path, swa_block_mask_t=swa_block_mask_t, SwaError=SwaError)
    for k, v in globals().items():
        if k.startswith("SWA_"):
            setattr(ns, k, v)
    ns.swa_strerror = lambda status: strerror(lib, status)
    ns.swa_block_mask_query = lambda *a, **kw: block_mask_query(lib, *a, **kw)
    ns.swa_attn_decode_workspace_bytes = lambda *a, **kw: decode_workspace_bytes(lib, *a, **kw)
    return ns
