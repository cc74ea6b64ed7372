"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers and names workloads; it holds none of the
attention arithmetic.  Every tensor is drawn from numpy's PCG64 generator
(``numpy.random.default_rng(seed)``, ``standard_normal`` in float32) in a
fixed order, then -- for bf16 workloads -- rounded to the nearest bf16 value
(round-to-nearest-even on the float32 bit pattern).  The rounded values are
returned as float32 arrays, which is what both the GPU path (after a lossless
narrowing to bf16) and the fp64 oracle (after a lossless widening) read.

Workloads (sizes as the method's published configurations name them):

=====================  =====================================================
tiny_swa_f32           B=1, H=2, N=256, d=32, W=64, fp32, seed 1
swa_prefill_bf16       B=1, Hq=32, Hkv=8, N=8192, d=128, W=1024, bf16, seed 2
local_strided_bf16     B=2, H=16, N=16384, d=64, W=256, stride 128, seed 3
window_decode_bf16     64 sequences at position 131072, ring W=4096,
                       Hq=32, Hkv=8, d=128, bf16, seed 4
diff_bf16              B=1, H=16, N=4096, d=64 per map, dv=128, W=1024,
                       lambda 0.5, scale 1/8, bf16, seed 5
sink_decode_bf16       window_decode_bf16 plus 4 sink slots (positions 0-3),
                       seed 6
diff_decode_bf16       32 sequences at position 131072, ring W=4096, H=16,
                       d=64 per map, dv=128, lambda 0.5, scale 1/8, bf16,
                       seed 7
global_prefill_bf16    swa_prefill_bf16 plus 64 global tokens (positions
                       0-63), seed 8
dilated_prefill_bf16   swa_prefill_bf16 with a window of 512 keys at
                       dilation 2 (the same 1023-token span), seed 9
=====================  =====================================================
"""
import math

import numpy as np

WORKLOADS = {
    "tiny_swa_f32": dict(kind="prefill", dtype="f32", B=1, Hq=2, Hkv=2, N=256, d=32, dv=32,
                         window=64, stride=0, scale=1.0 / math.sqrt(32), seed=1),
    "swa_prefill_bf16": dict(kind="prefill", dtype="bf16", B=1, Hq=32, Hkv=8, N=8192, d=128,
                             dv=128, window=1024, stride=0, scale=1.0 / math.sqrt(128), seed=2),
    "local_strided_bf16": dict(kind="prefill", dtype="bf16", B=2, Hq=16, Hkv=16, N=16384, d=64,
                               dv=64, window=256, stride=128, scale=1.0 / 8, seed=3),
    "window_decode_bf16": dict(kind="decode", dtype="bf16", B=64, Hq=32, Hkv=8, window=4096,
                               d=128, dv=128, position=131072, n_sink=0,
                               scale=1.0 / math.sqrt(128), seed=4),
    "diff_bf16": dict(kind="diff", dtype="bf16", B=1, Hq=16, Hkv=16, N=4096, d=64, dv=128,
                      window=1024, stride=0, scale=1.0 / 8, lam=0.5, seed=5),
    "sink_decode_bf16": dict(kind="decode", dtype="bf16", B=64, Hq=32, Hkv=8, window=4096,
                             d=128, dv=128, position=131072, n_sink=4,
                             scale=1.0 / math.sqrt(128), seed=6),
    "diff_decode_bf16": dict(kind="diff_decode", dtype="bf16", B=32, Hq=16, Hkv=16, window=4096,
                             d=64, dv=128, position=131072, scale=1.0 / 8, lam=0.5, seed=7),
    "global_prefill_bf16": dict(kind="prefill", dtype="bf16", B=1, Hq=32, Hkv=8, N=8192, d=128,
                                dv=128, window=1024, stride=0, n_global=64,
                                scale=1.0 / math.sqrt(128), seed=8),
    "dilated_prefill_bf16": dict(kind="prefill", dtype="bf16", B=1, Hq=32, Hkv=8, N=8192, d=128,
                                 dv=128, window=512, stride=0, dilation=2,
                                 scale=1.0 / math.sqrt(128), seed=9),
}


def round_bf16(x):
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs only: the largest finite pattern plus 0x8000 stays below 2**32
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).reshape(x.shape)


def _draw(rng, shape, dtype, scale=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a = (a * np.float32(scale)).astype(np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def workload(name, **override):
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    cfg["name"] = name
    return cfg


def prefill_inputs(cfg, q_scale=1.0):
    """q [B,Hq,N,d], k [B,Hkv,N,d], v [B,Hkv,N,dv], drawn in that order."""
    rng = np.random.default_rng(cfg["seed"])
    B, Hq, Hkv, N, d, dv = (cfg[x] for x in ("B", "Hq", "Hkv", "N", "d", "dv"))
    q = _draw(rng, (B, Hq, N, d), cfg["dtype"], q_scale)
    k = _draw(rng, (B, Hkv, N, d), cfg["dtype"])
    v = _draw(rng, (B, Hkv, N, dv), cfg["dtype"])
    return q, k, v


def diff_inputs(cfg):
    """q1, k1, q2, k2 [B,H,N,d] and v [B,Hkv,N,dv], drawn in that order."""
    rng = np.random.default_rng(cfg["seed"])
    B, Hq, Hkv, N, d, dv = (cfg[x] for x in ("B", "Hq", "Hkv", "N", "d", "dv"))
    q1 = _draw(rng, (B, Hq, N, d), cfg["dtype"])
    k1 = _draw(rng, (B, Hkv, N, d), cfg["dtype"])
    q2 = _draw(rng, (B, Hq, N, d), cfg["dtype"])
    k2 = _draw(rng, (B, Hkv, N, d), cfg["dtype"])
    v = _draw(rng, (B, Hkv, N, dv), cfg["dtype"])
    return q1, k1, q2, k2, v


def decode_inputs(cfg, seq_len=None):
    """q [B,Hq,d], k_ring / v_ring [B,Hkv,W,d|dv], seq_len [B] (int64), and,
    when n_sink > 0, k_sink / v_sink [B,Hkv,n_sink,d|dv]; drawn in that order.

    By default every sequence sits at `position` (0-based) with its current
    token already appended, so seq_len = position + 1."""
    rng = np.random.default_rng(cfg["seed"])
    B, Hq, Hkv, W, d, dv = (cfg[x] for x in ("B", "Hq", "Hkv", "window", "d", "dv"))
    S = cfg.get("n_sink", 0)
    q = _draw(rng, (B, Hq, d), cfg["dtype"])
    kr = _draw(rng, (B, Hkv, W, d), cfg["dtype"])
    vr = _draw(rng, (B, Hkv, W, dv), cfg["dtype"])
    ks = _draw(rng, (B, Hkv, S, d), cfg["dtype"]) if S else None
    vs = _draw(rng, (B, Hkv, S, dv), cfg["dtype"]) if S else None
    if seq_len is None:
        seq_len = np.full(B, cfg["position"] + 1, dtype=np.int64)
    return dict(q=q, k_ring=kr, v_ring=vr, k_sink=ks, v_sink=vs,
                seq_len=np.asarray(seq_len, dtype=np.int64))


def diff_decode_inputs(cfg, seq_len=None):
    """q1 [B,Hq,d], k1_ring [B,Hkv,W,d], q2, k2_ring, v_ring [B,Hkv,W,dv] and
    seq_len [B] (int64), drawn in that order; seq_len as in decode_inputs."""
    rng = np.random.default_rng(cfg["seed"])
    B, Hq, Hkv, W, d, dv = (cfg[x] for x in ("B", "Hq", "Hkv", "window", "d", "dv"))
    q1 = _draw(rng, (B, Hq, d), cfg["dtype"])
    k1 = _draw(rng, (B, Hkv, W, d), cfg["dtype"])
    q2 = _draw(rng, (B, Hq, d), cfg["dtype"])
    k2 = _draw(rng, (B, Hkv, W, d), cfg["dtype"])
    v = _draw(rng, (B, Hkv, W, dv), cfg["dtype"])
    if seq_len is None:
        seq_len = np.full(B, cfg["position"] + 1, dtype=np.int64)
    return dict(q1=q1, k1_ring=k1, q2=q2, k2_ring=k2, v_ring=v,
                seq_len=np.asarray(seq_len, dtype=np.int64))


def sample_rows(total, count, seed=1234, must=()):
    """Sorted distinct flat row indices: `must` plus a seeded uniform sample."""
    rng = np.random.default_rng(seed)
    pick = set(int(m) for m in must if 0 <= m < total)
    extra = rng.choice(total, size=min(count, total), replace=False)
    pick.update(int(x) for x in extra)
    return np.array(sorted(pick), dtype=np.int64)
