"""GPU parity: the HIP path against the fp64 oracle on the same seeded inputs.

Integer outputs (block mask, dense mask) must match bit for bit.  Attention
outputs must match within max-abs 2e-2 for bf16 inputs (fp32 accumulation,
bf16 output) and 1e-5 for fp32 inputs -- the tolerances the method's
target states.  Small cases span several tiles and a ragged tail; the
full-size workloads are checked on sampled rows, in the launch configuration
the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}
# log-sum-exp: bf16 kernels may sum the bf16-rounded probabilities (each
# within a relative 2^-8 of its exact value), so their log of the row sum is
# within ln(1 + 2^-8) < 4e-3 of the exact one; fp32 kernels sum in fp32
LSE_TOL = {"bf16": 4e-3, "f32": 1e-5}


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_masked_transformer_amd as m
    return m


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    return t.cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def max_err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def banner(msg):
    print(f"[case] {msg}", flush=True)


# --------------------------------------------------------------------------
# block mask and dense mask: bit-exact
# --------------------------------------------------------------------------

MASK_CASES = [(1, 1, 0), (5, 3, 0), (130, 7, 0), (300, 64, 5), (300, 1000, 0), (511, 129, 64),
              (1000, 50, 130), (777, 200, 1), (4096, 1024, 0), (8192, 1024, 0),
              (16384, 256, 128), (2048, 33, 3), (640, 600, 700)]


@pytest.mark.parametrize("N,W,s", MASK_CASES)
@pytest.mark.parametrize("bm", [128, 256])
def test_block_mask_bit_exact(swa, N, W, s, bm):
    banner(f"block mask N={N} W={W} s={s} bm={bm}")
    m = swa.swa_block_mask_build(N, W, s, bm=bm, bn=64)
    got = m.host()
    want = oracle.tile_list(N, W, s, m.bm, m.bn)
    assert got["nnz"] == want["nnz"] and got["num_q_tiles"] == want["num_q_tiles"]
    for key in ("row_ptr", "kv_tile", "kind", "cells", "prefix_keys", "band_begin"):
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)


MASK_EXT_CASES = [
    # N, W, stride, dilation, n_global, bm, bn
    (1000, 50, 0, 2, 0, 128, 64), (1000, 30, 0, 64, 0, 128, 64), (777, 40, 9, 16, 0, 64, 16),
    (1000, 50, 0, 1, 64, 128, 64), (1000, 50, 130, 1, 300, 128, 64), (700, 20, 3, 5, 17, 32, 32),
    (300, 4, 0, 3, 1000, 128, 64), (4096, 512, 0, 2, 64, 128, 64), (555, 8, 100, 7, 65, 16, 64),
    (8192, 512, 0, 2, 0, 128, 64), (8192, 1024, 0, 1, 64, 128, 64)]


@pytest.mark.parametrize("N,W,s,dil,g,bm,bn", MASK_EXT_CASES)
def test_block_mask_dilated_global_bit_exact(swa, N, W, s, dil, g, bm, bn):
    banner(f"block mask N={N} W={W} s={s} dilation={dil} globals={g} bm={bm} bn={bn}")
    m = swa.swa_block_mask_build(N, W, s, bm=bm, bn=bn, dilation=dil, n_global=g)
    got = m.host()
    want = oracle.tile_list(N, W, s, bm, bn, dilation=dil, n_global=g)
    assert got["nnz"] == want["nnz"] and got["num_q_tiles"] == want["num_q_tiles"]
    for key in ("row_ptr", "kv_tile", "kind", "cells", "prefix_keys", "band_begin"):
        np.testing.assert_array_equal(got[key], want[key], err_msg=key)


@pytest.mark.parametrize("N,W,s,dil,g", [(1, 1, 0, 1, 0), (64, 5, 0, 1, 0), (257, 17, 7, 1, 0),
                                         (1024, 100, 64, 1, 0), (3000, 3000, 0, 1, 0),
                                         (500, 20, 0, 3, 0), (500, 20, 33, 2, 9), (300, 4, 0, 1, 300)])
def test_dense_mask_bit_exact(swa, N, W, s, dil, g):
    banner(f"dense mask N={N} W={W} s={s} dilation={dil} globals={g}")
    got = swa.swa_mask_dense(N, W, s, dilation=dil, n_global=g).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.mask_dense(N, W, s, dil, g))


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------

def run_prefill(swa, cfg, q, k, v, with_lse=False):
    dt = cfg["dtype"]
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], cfg["stride"],
                                    dtype=torch.bfloat16 if dt == "bf16" else torch.float32, d=cfg["d"],
                                    dilation=cfg.get("dilation", 1), n_global=cfg.get("n_global", 0))
    qd, kd, vd = dev(q, dt), dev(k, dt), dev(v, dt)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda") if with_lse else None
    out = swa.swa_attn_fwd(qd, kd, vd, cfg["window"], cfg["stride"], cfg["scale"], mask, lse=lse)
    torch.cuda.synchronize()
    return (host(out), lse.cpu().numpy()) if with_lse else host(out)


PREFILL_CASES = [
    # B, Hq, Hkv, N, d, W, stride
    (1, 2, 2, 64, 64, 16, 0),
    (1, 4, 2, 300, 64, 17, 0),
    (2, 4, 1, 333, 128, 100, 0),
    (1, 8, 2, 517, 128, 64, 0),
    (1, 2, 2, 300, 128, 300, 0),
    (1, 2, 2, 300, 64, 1000, 0),
    (1, 2, 1, 200, 32, 1, 0),
    (1, 2, 2, 450, 64, 40, 7),
    (1, 2, 2, 700, 64, 64, 128),
    (2, 2, 2, 390, 128, 33, 100),
    (1, 4, 4, 300, 32, 20, 1),
    (1, 2, 2, 1000, 64, 128, 64),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,N,d,W,s", PREFILL_CASES)
def test_prefill_parity_small(swa, dtype, B, Hq, Hkv, N, d, W, s):
    banner(f"prefill {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} W={W} s={s}")
    cfg = dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dv=d, window=W, stride=s,
               scale=1.0 / math.sqrt(d), seed=N + d + W + s)
    q, k, v = synth.prefill_inputs(cfg)
    got, lse = run_prefill(swa, cfg, q, k, v, with_lse=True)
    want, want_lse = oracle.attn_full(q, k, v, W, s, cfg["scale"], with_lse=True)
    assert max_err(got, want) <= TOL[dtype]
    assert max_err(lse, want_lse) <= LSE_TOL[dtype]


PREFILL_EXT_CASES = [
    # B, Hq, Hkv, N, d, W, stride, dilation, n_global
    (1, 2, 2, 300, 64, 20, 0, 2, 0),
    (1, 4, 2, 517, 128, 64, 0, 3, 0),
    (1, 2, 2, 450, 64, 40, 7, 4, 0),
    (1, 2, 2, 700, 128, 16, 0, 64, 0),      # span 960 keys, one key in 64
    (1, 2, 2, 600, 64, 50, 0, 1, 16),
    (1, 2, 2, 600, 128, 50, 100, 1, 70),    # global columns and stride keys in the prefix
    (2, 2, 1, 333, 64, 30, 0, 2, 5),
    (1, 2, 2, 300, 32, 10, 0, 1, 300),      # every token global: full causal
    (1, 4, 4, 1000, 64, 128, 64, 2, 64),
    (1, 2, 2, 260, 32, 3, 5, 9, 130),       # global columns across whole tiles
    # dilation alone runs as plain windows on the residue classes
    (1, 2, 2, 385, 64, 9, 0, 3, 0),         # classes of 129, 128, 128 rows: empty last tiles
    (1, 2, 1, 40, 32, 3, 0, 64, 0),         # N < dilation: classes without rows
    (2, 4, 1, 1000, 128, 100, 0, 7, 0),
    (1, 2, 2, 300, 32, 1000, 0, 2, 0),      # window longer than every class
    # (window - 1) * dilation beyond the int32 range: every earlier lattice key attends
    (1, 2, 2, 200, 64, 2 ** 30, 0, 5, 0),
    (1, 2, 2, 150, 32, 2 ** 30, 7, 3, 0),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,N,d,W,s,dil,g", PREFILL_EXT_CASES)
def test_prefill_dilated_global_parity(swa, dtype, B, Hq, Hkv, N, d, W, s, dil, g):
    banner(f"prefill {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} W={W} s={s} dilation={dil} globals={g}")
    cfg = dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dv=d, window=W, stride=s, dilation=dil,
               n_global=g, scale=1.0 / math.sqrt(d), seed=N + d + W + s + dil + g)
    q, k, v = synth.prefill_inputs(cfg)
    got, lse = run_prefill(swa, cfg, q, k, v, with_lse=True)
    want, want_lse = oracle.attn_full(q, k, v, W, s, cfg["scale"], with_lse=True, dilation=dil,
                                      n_global=g)
    assert max_err(got, want) <= TOL[dtype]
    assert max_err(lse, want_lse) <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_peaky_scores(swa, dtype):
    # query scaled by 8: near one-hot softmax rows, large score range
    banner(f"prefill peaky {dtype}")
    cfg = dict(dtype=dtype, B=1, Hq=4, Hkv=2, N=400, d=64, dv=64, window=90, stride=33,
               scale=1.0 / 8, seed=77)
    q, k, v = synth.prefill_inputs(cfg, q_scale=8.0)
    got = run_prefill(swa, cfg, q, k, v)
    want = oracle.attn_full(q, k, v, 90, 33, cfg["scale"])
    assert max_err(got, want) <= TOL[dtype]


# every HIP kernel the boundary can pick for these shapes (the generated
# kernels have their own case): bf16 window and local+strided prefill at
# d = 32, 64 and 128 with fewer than 4 query heads per key/value head, the
# bf16 two-map kernel (with a stride, and at d = 32, dv = 64), and the fp32
# paths
NAN_TAIL_CASES = [
    # kind, B, Hq, Hkv, N, d, dv, W, stride
    ("prefill", 1, 2, 2, 333, 64, 64, 40, 7),
    ("prefill", 2, 4, 2, 200, 128, 128, 64, 0),
    ("prefill", 1, 2, 1, 130, 32, 32, 17, 0),
    ("diff", 1, 2, 2, 300, 64, 128, 70, 9),
    ("diff", 1, 4, 2, 190, 32, 64, 40, 0),
]


def nan_tail(x, dtype, extra=64):
    """x on the device as a view at the start of a larger buffer whose rows
    past it hold NaN (a cache allocated longer than the sequence)."""
    B, H, N, w = x.shape
    buf = torch.full((B * H * N + extra, w), float("nan"), device="cuda",
                     dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    buf[:B * H * N] = dev(x, dtype).reshape(-1, w)
    return buf[:B * H * N].view(B, H, N, w)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind,B,Hq,Hkv,N,d,dv,W,s", NAN_TAIL_CASES)
def test_rows_past_n_read_as_zeros(swa, dtype, kind, B, Hq, Hkv, N, d, dv, W, s):
    """Queries, keys and values past row N of the last head hold NaN inside
    the same allocation: the kernels must not let them into any output."""
    banner(f"NaN past N {kind} {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} dv={dv} W={W} s={s}")
    cfg = dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dv=dv, window=W, stride=s,
               scale=1.0 / math.sqrt(d), lam=0.5, seed=900 + N + d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if kind == "prefill":
        q, k, v = synth.prefill_inputs(cfg)
        mask = swa.swa_block_mask_build(N, W, s, dtype=tdt, d=d)
        out = swa.swa_attn_fwd(nan_tail(q, dtype), nan_tail(k, dtype), nan_tail(v, dtype), W, s, cfg["scale"],
                               mask)
        want = oracle.attn_full(q, k, v, W, s, cfg["scale"])
    else:
        ins = synth.diff_inputs(cfg)
        mask = swa.swa_block_mask_build(N, W, s, dtype=tdt, d=d, dv=dv, op=swa.SWA_OP_DIFF)
        out = swa.diff_attn_fwd(*(nan_tail(x, dtype) for x in ins), W, s, cfg["scale"], cfg["lam"], mask)
        want = oracle.diff_full(*ins, W, s, cfg["scale"], cfg["lam"])
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(np.isfinite(got))
    assert max_err(got, want) <= TOL[dtype]


def test_tiny_fp32_workload_full(swa):
    cfg = synth.workload("tiny_swa_f32")
    banner("workload tiny_swa_f32 (all rows)")
    q, k, v = synth.prefill_inputs(cfg)
    got = run_prefill(swa, cfg, q, k, v)
    want = oracle.attn_full(q, k, v, cfg["window"], cfg["stride"], cfg["scale"])
    assert max_err(got, want) <= TOL["f32"]


def threaded(fn, idx):
    """fn over index chunks on the host's threads (the oracle releases the
    GIL), concatenated in order."""
    import concurrent.futures
    import os
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = [c for c in np.array_split(np.asarray(idx), threads * 4) if len(c)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        return np.concatenate(list(ex.map(fn, chunks)))


def boundary_rows(B, H, N, step, extra):
    must = []
    for b in range(B):
        for h in range(H):
            for i in (0, 1, 63, 64, 127, 128, N // 2, N - 2, N - 1):
                must.append((b * H + h) * N + i)
    return synth.sample_rows(B * H * N, extra, seed=step, must=must)


@pytest.mark.parametrize("name", ["swa_prefill_bf16", "local_strided_bf16", "global_prefill_bf16",
                                  "dilated_prefill_bf16"])
def test_prefill_workload_all_rows(swa, name):
    """Every row of the workload at full size (every workgroup of the launch
    the benchmark times), against the oracle run on the host's threads."""
    cfg = synth.workload(name)
    banner(f"workload {name} (all rows)")
    q, k, v = synth.prefill_inputs(cfg)
    got = run_prefill(swa, cfg, q, k, v).reshape(-1, cfg["dv"])
    rows = np.arange(got.shape[0], dtype=np.int64)
    want = threaded(lambda r: oracle.attn_rows(q, k, v, cfg["window"], cfg["stride"], cfg["scale"], r,
                                               dilation=cfg.get("dilation", 1),
                                               n_global=cfg.get("n_global", 0)), rows)
    assert max_err(got, want) <= TOL["bf16"]


def test_prefill_longest_sequence(swa):
    # N at its maximum (2^22): the largest byte offsets the kernels form (row *
    # d * 2 and the tile offsets, up to 1 GiB at d=128) and stride keys near
    # the end of the sequence
    N = swa.SWA_MAX_N
    cfg = dict(dtype="bf16", B=1, Hq=1, Hkv=1, N=N, d=128, dv=128, window=128, stride=1 << 20,
               scale=1.0 / math.sqrt(128), seed=21)
    banner(f"prefill at N={N} (sampled rows)")
    q, k, v = synth.prefill_inputs(cfg)
    got = run_prefill(swa, cfg, q, k, v).reshape(-1, cfg["dv"])
    rows = synth.sample_rows(N, 192, seed=22, must=[0, 63, 64, 127, 128, (1 << 20) - 1, 1 << 20,
                                                   (1 << 20) + 1, 3 << 20, N - 129, N - 65, N - 2,
                                                   N - 1])
    want = oracle.attn_rows(q, k, v, cfg["window"], cfg["stride"], cfg["scale"], rows)
    assert max_err(got[rows], want) <= TOL["bf16"]
    assert np.all(np.isfinite(got[N - 4096:]))


def test_prefill_deterministic(swa):
    cfg = dict(dtype="bf16", B=1, Hq=8, Hkv=2, N=1500, d=128, dv=128, window=300, stride=0,
               scale=1.0 / math.sqrt(128), seed=5)
    banner("prefill determinism")
    q, k, v = synth.prefill_inputs(cfg)
    a = run_prefill(swa, cfg, q, k, v)
    b = run_prefill(swa, cfg, q, k, v)
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------------------
# differential attention
# --------------------------------------------------------------------------

def run_diff(swa, cfg, q1, k1, q2, k2, v):
    dt = cfg["dtype"]
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], cfg["stride"],
                                    dtype=torch.bfloat16 if dt == "bf16" else torch.float32,
                                    d=cfg["d"], dv=cfg["dv"], op=swa.SWA_OP_DIFF,
                                    dilation=cfg.get("dilation", 1), n_global=cfg.get("n_global", 0))
    out = swa.diff_attn_fwd(dev(q1, dt), dev(k1, dt), dev(q2, dt), dev(k2, dt), dev(v, dt),
                            cfg["window"], cfg["stride"], cfg["scale"], cfg["lam"], mask)
    torch.cuda.synchronize()
    return host(out)


# every bf16 head-size pair (d, dv) the two-map kernel instantiates
DIFF_CASES = [(1, 2, 2, 300, 64, 128, 70, 0), (1, 4, 2, 257, 64, 64, 300, 0),
              (2, 2, 2, 200, 32, 128, 50, 9), (1, 2, 1, 130, 32, 32, 1, 0),
              (1, 4, 2, 190, 32, 64, 40, 0), (1, 2, 2, 150, 64, 32, 100, 7),
              (1, 2, 2, 200, 128, 128, 64, 0), (1, 4, 2, 170, 128, 64, 90, 5),
              (1, 2, 1, 140, 128, 32, 30, 0)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,N,d,dv,W,s", DIFF_CASES)
def test_diff_parity_small(swa, dtype, B, Hq, Hkv, N, d, dv, W, s):
    banner(f"diff {dtype} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} dv={dv} W={W} s={s}")
    cfg = dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, dv=dv, window=W, stride=s,
               scale=1.0 / 8, lam=0.5, seed=N + W)
    ins = synth.diff_inputs(cfg)
    got = run_diff(swa, cfg, *ins)
    want = oracle.diff_full(*ins, W, s, cfg["scale"], cfg["lam"])
    assert max_err(got, want) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,d,dv,W,s,dil,g", [(300, 64, 128, 40, 0, 2, 8), (200, 32, 64, 30, 9, 3, 1),
                                              (260, 64, 64, 20, 0, 1, 100)])
def test_diff_dilated_global_parity(swa, dtype, N, d, dv, W, s, dil, g):
    banner(f"diff {dtype} N={N} d={d} dv={dv} W={W} s={s} dilation={dil} globals={g}")
    cfg = dict(dtype=dtype, B=1, Hq=2, Hkv=1, N=N, d=d, dv=dv, window=W, stride=s, dilation=dil,
               n_global=g, scale=1.0 / 8, lam=0.5, seed=N + W + dil)
    ins = synth.diff_inputs(cfg)
    got = run_diff(swa, cfg, *ins)
    want = oracle.diff_full(*ins, W, s, cfg["scale"], cfg["lam"], dilation=dil, n_global=g)
    assert max_err(got, want) <= TOL[dtype]


def test_diff_workload_all_rows(swa):
    cfg = synth.workload("diff_bf16")
    banner("workload diff_bf16 (all rows)")
    ins = synth.diff_inputs(cfg)
    got = run_diff(swa, cfg, *ins).reshape(-1, cfg["dv"])
    rows = np.arange(got.shape[0], dtype=np.int64)
    want = threaded(lambda r: oracle.diff_rows(*ins, cfg["window"], cfg["stride"], cfg["scale"], cfg["lam"], r),
                    rows)
    assert max_err(got, want) <= TOL["bf16"]


def test_diff_deterministic(swa):
    cfg = dict(dtype="bf16", B=1, Hq=4, Hkv=4, N=1000, d=64, dv=128, window=300, stride=0, scale=0.125,
               lam=0.5, seed=55)
    banner("diff determinism")
    ins = synth.diff_inputs(cfg)
    a = run_diff(swa, cfg, *ins)
    b = run_diff(swa, cfg, *ins)
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------------------
# decode over a rolling window
# --------------------------------------------------------------------------

def run_decode(swa, cfg, ins, pass_len=True):
    dt = cfg["dtype"]
    sl = torch.from_numpy(ins["seq_len"].astype(np.int32)).cuda() if pass_len else None
    out = swa.swa_attn_decode(dev(ins["q"], dt), dev(ins["k_ring"], dt), dev(ins["v_ring"], dt), sl,
                              cfg["scale"], N=int(ins["seq_len"][0]))
    torch.cuda.synchronize()
    return host(out)


LENS16 = [(i * 397) % 2100 for i in range(16)]   # 0 .. 2099, below, at and above the window

DECODE_CASES = [
    # B, Hq, Hkv, W, d, lengths   (bf16 work split: workgroups of 1-4 waves; splits)
    (2, 32, 1, 200, 64, [150, 900]),           # one key/value head for 32 query heads
    (1, 34, 2, 70, 128, [70]),                 # 17 per group: a second block of one head
    (3, 4, 1, 64, 64, [1, 30, 64]),            # 1 wave, 2 splits
    (2, 8, 2, 300, 128, [299, 1000]),          # 2 waves, 5 splits
    (4, 4, 4, 1000, 32, [0, 5, 999, 1001]),    # 4 waves, 8 splits
    (2, 16, 1, 512, 128, [513, 4096]),         # 16 heads per key/value head
    (1, 2, 2, 33, 64, [100]),
    (16, 16, 16, 1000, 64, LENS16),            # 4 waves, 2 splits, 4 steps per wave
    (64, 8, 8, 1000, 32, [(i * 131) % 1400 for i in range(64)]),  # 512 pairs: 4 waves, one split
    (64, 8, 8, 520, 32, [(i * 131) % 700 for i in range(64)]),    # 3 waves, 2 splits
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,W,d,lens", DECODE_CASES)
def test_decode_parity(swa, dtype, B, Hq, Hkv, W, d, lens):
    banner(f"decode {dtype} B={B} Hq={Hq} Hkv={Hkv} W={W} d={d} lens={lens}")
    cfg = dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, window=W, d=d, dv=d, position=0, n_sink=0,
               scale=1.0 / math.sqrt(d), seed=W + d)
    ins = synth.decode_inputs(cfg, seq_len=lens)
    got = run_decode(swa, cfg, ins)
    want = oracle.decode(ins["q"], ins["k_ring"], ins["v_ring"], ins["seq_len"], cfg["scale"])
    assert max_err(got, want) <= TOL[dtype]


def test_decode_longest_ring(swa):
    # a ring of 2^22 slots (the largest window the boundary accepts) at
    # d = 128: split across workgroups, byte offsets up to 1 GiB per ring
    # (the bound the ring's 32-bit lane offsets rely on); one sequence past
    # the ring's first wrap, one still filling it
    W = swa.SWA_MAX_N
    cfg = dict(dtype="bf16", B=2, Hq=2, Hkv=1, window=W, d=128, dv=128, position=0, n_sink=0,
               scale=1.0 / math.sqrt(128), seed=23)
    banner(f"decode with a ring of {W} slots")
    ins = synth.decode_inputs(cfg, seq_len=[W + 1000, W // 2 + 3])
    got = run_decode(swa, cfg, ins)
    want = oracle.decode(ins["q"], ins["k_ring"], ins["v_ring"], ins["seq_len"], cfg["scale"])
    assert max_err(got, want) <= TOL["bf16"]


def test_decode_default_length(swa):
    cfg = dict(dtype="bf16", B=2, Hq=4, Hkv=1, window=128, d=64, dv=64, position=500, n_sink=0,
               scale=0.125, seed=3)
    banner("decode seq_len=NULL")
    ins = synth.decode_inputs(cfg)
    got = run_decode(swa, cfg, ins, pass_len=False)
    want = oracle.decode(ins["q"], ins["k_ring"], ins["v_ring"], ins["seq_len"], cfg["scale"])
    assert max_err(got, want) <= TOL["bf16"]


def run_decode_sinks(swa, cfg, ins):
    dt = cfg["dtype"]
    sl = torch.from_numpy(ins["seq_len"].astype(np.int32)).cuda()
    out = swa.swa_attn_decode_sinks(dev(ins["q"], dt), dev(ins["k_sink"], dt), dev(ins["v_sink"], dt),
                                    dev(ins["k_ring"], dt), dev(ins["v_ring"], dt), sl, cfg["scale"])
    torch.cuda.synchronize()
    return host(out)


SINK_CASES = [
    # B, Hq, Hkv, W, n_sink, d, lengths
    (2, 48, 2, 80, 4, 64, [30, 400]),          # 24 query heads per key/value head
    (2, 8, 2, 64, 4, 128, [3, 200]),           # no sink yet outside the ring; 4 sinks
    (3, 4, 1, 100, 4, 64, [102, 104, 5000]),   # sinks partly still in the ring
    (1, 2, 2, 31, 1, 32, [40]),                # sink + ring = exactly one 32-slot step
    (2, 4, 2, 48, 8, 128, [57, 8]),
    (16, 16, 16, 1000, 4, 64, LENS16),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,W,S,d,lens", SINK_CASES)
def test_decode_sinks_parity(swa, dtype, B, Hq, Hkv, W, S, d, lens):
    banner(f"decode sinks {dtype} B={B} Hq={Hq} Hkv={Hkv} W={W} S={S} d={d} lens={lens}")
    cfg = dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, window=W, d=d, dv=d, position=0, n_sink=S,
               scale=1.0 / math.sqrt(d), seed=W + S)
    ins = synth.decode_inputs(cfg, seq_len=lens)
    got = run_decode_sinks(swa, cfg, ins)
    want = oracle.decode(ins["q"], ins["k_ring"], ins["v_ring"], ins["seq_len"], cfg["scale"],
                         k_sink=ins["k_sink"], v_sink=ins["v_sink"])
    assert max_err(got, want) <= TOL[dtype]


def run_diff_decode(swa, cfg, ins):
    dt = cfg["dtype"]
    sl = torch.from_numpy(ins["seq_len"].astype(np.int32)).cuda()
    out = swa.diff_attn_decode(dev(ins["q1"], dt), dev(ins["k1_ring"], dt), dev(ins["q2"], dt),
                               dev(ins["k2_ring"], dt), dev(ins["v_ring"], dt), sl, cfg["scale"],
                               cfg["lam"])
    torch.cuda.synchronize()
    return host(out)


DIFF_DECODE_CASES = [
    # B, Hq, Hkv, W, d, dv, lengths
    (2, 4, 2, 64, 64, 128, [1, 500]),
    (3, 2, 2, 300, 32, 64, [0, 299, 1000]),
    (1, 8, 1, 129, 32, 128, [129]),
    (2, 4, 4, 96, 64, 64, [50, 97]),
    (16, 16, 16, 1000, 64, 128, LENS16),
    (2, 40, 2, 90, 64, 128, [91, 20]),         # 20 query heads per key/value head
    # 2 d + dv > 256: one register stage in bf16
    (2, 4, 2, 100, 128, 128, [50, 300]),
    (1, 8, 2, 70, 128, 64, [140]),
    (3, 4, 4, 64, 128, 32, [1, 64, 65]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,W,d,dv,lens", DIFF_DECODE_CASES)
def test_diff_decode_parity(swa, dtype, B, Hq, Hkv, W, d, dv, lens):
    banner(f"diff decode {dtype} B={B} Hq={Hq} Hkv={Hkv} W={W} d={d} dv={dv} lens={lens}")
    cfg = dict(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, window=W, d=d, dv=dv, position=0, scale=0.125,
               lam=0.5, seed=W + d + dv)
    ins = synth.diff_decode_inputs(cfg, seq_len=lens)
    got = run_diff_decode(swa, cfg, ins)
    want = oracle.diff_decode(ins["q1"], ins["k1_ring"], ins["q2"], ins["k2_ring"], ins["v_ring"],
                              ins["seq_len"], cfg["scale"], cfg["lam"])
    assert max_err(got, want) <= TOL[dtype]


def test_diff_decode_f32_wide_heads(swa):
    # fp32 has no register-stage limit: d = dv = 128 with two maps
    cfg = dict(dtype="f32", B=2, Hq=4, Hkv=2, window=80, d=128, dv=128, position=0, scale=0.09,
               lam=0.8, seed=71)
    banner("diff decode f32 d=dv=128")
    ins = synth.diff_decode_inputs(cfg, seq_len=[81, 40])
    got = run_diff_decode(swa, cfg, ins)
    want = oracle.diff_decode(ins["q1"], ins["k1_ring"], ins["q2"], ins["k2_ring"], ins["v_ring"],
                              ins["seq_len"], cfg["scale"], cfg["lam"])
    assert max_err(got, want) <= TOL["f32"]


def test_sink_decode_workload(swa):
    cfg = synth.workload("sink_decode_bf16")
    banner("workload sink_decode_bf16 (all 64 sequences)")
    ins = synth.decode_inputs(cfg)
    got = run_decode_sinks(swa, cfg, ins)
    want = threaded(lambda b: oracle.decode(ins["q"][b], ins["k_ring"][b], ins["v_ring"][b], ins["seq_len"][b],
                                            cfg["scale"], k_sink=ins["k_sink"][b], v_sink=ins["v_sink"][b]),
                    np.arange(cfg["B"]))
    assert max_err(got, want) <= TOL["bf16"]


def test_diff_decode_workload(swa):
    cfg = synth.workload("diff_decode_bf16")
    banner("workload diff_decode_bf16 (all 32 sequences)")
    ins = synth.diff_decode_inputs(cfg)
    got = run_diff_decode(swa, cfg, ins)
    want = threaded(lambda b: oracle.diff_decode(*(ins[x][b] for x in ("q1", "k1_ring", "q2", "k2_ring",
                                                                       "v_ring", "seq_len")),
                                                 cfg["scale"], cfg["lam"]), np.arange(cfg["B"]))
    assert max_err(got, want) <= TOL["bf16"]


def test_decode_workload(swa):
    cfg = synth.workload("window_decode_bf16")
    banner("workload window_decode_bf16 (all 64 sequences)")
    ins = synth.decode_inputs(cfg)
    got = run_decode(swa, cfg, ins)
    want = threaded(lambda b: oracle.decode(ins["q"][b], ins["k_ring"][b], ins["v_ring"][b],
                                            ins["seq_len"][b], cfg["scale"]), np.arange(cfg["B"]))
    assert max_err(got, want) <= TOL["bf16"]


# Run-to-run determinism (a race canary): the split of a window over
# workgroups and its combine, sink slots and the two-map decode must give
# bitwise the same output every time.
@pytest.mark.parametrize("kind", ["window_split", "sinks", "diff"])
def test_decode_deterministic(swa, kind):
    banner(f"decode determinism {kind}")
    if kind == "diff":
        cfg = dict(dtype="bf16", B=1, Hq=4, Hkv=2, window=3000, d=64, dv=128, position=0, scale=0.125,
                   lam=0.5, seed=81)
        ins = synth.diff_decode_inputs(cfg, seq_len=[2900])
        run = lambda: run_diff_decode(swa, cfg, ins)
    else:
        # one sequence, one key/value head: the window is split over many
        # workgroups and the partial results combined
        cfg = dict(dtype="bf16", B=1, Hq=4, Hkv=1, window=4096, d=128, dv=128, position=0,
                   n_sink=4 if kind == "sinks" else 0, scale=1.0 / math.sqrt(128), seed=82)
        ins = synth.decode_inputs(cfg, seq_len=[100000])
        run = (lambda: run_decode_sinks(swa, cfg, ins)) if kind == "sinks" else (lambda: run_decode(swa, cfg, ins))
    a = run()
    b = run()
    np.testing.assert_array_equal(a, b)
