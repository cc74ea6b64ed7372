"""Seeded random sweep of the GPU path against the fp64 oracle.

The hand-picked parity cases pin the edges one at a time; this sweep draws
combinations of them (sequence length, window, stride, dilation, global
tokens, head sizes, grouped heads, batch, dtype, decode lengths and sink
slots) from a fixed seed, so every run checks the same configurations; three
more sweeps draw only shapes the generated kernels serve (grouped-query
prefill with a plain, dilated or global-token window; differential
attention at d = 64, dv = 128; multi-head prefill at d = 64 with a window
and a power-of-two stride or none).
Tolerances are the parity bar: max-abs 2e-2 for bf16 inputs, 1e-5 for fp32.
SWA_RANDOM_SCALE=k multiplies the number of drawn configurations by k (the
default run draws 48; k = 150 draws about 7,000, about a minute on one GPU).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}
SCALE = max(1, int(os.environ.get("SWA_RANDOM_SCALE", "1")))


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_masked_transformer_amd as m
    return m


def dev(x, dt):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16 if dt == "bf16" else torch.float32)
    return t.cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def max_err(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def tdtype(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def mask_pattern(rng, N):
    """(window, stride, dilation, n_global): each part on or off at random."""
    W = int(rng.integers(1, N + 41))
    s = 0 if rng.random() < 0.5 else int(rng.integers(1, N + 6))
    dil = 1 if rng.random() < 0.5 else int(rng.integers(2, 7))
    g = 0 if rng.random() < 0.6 else int(rng.integers(1, N + 4))
    return W, s, dil, g


def heads(rng, max_group=4):
    Hkv = int(rng.integers(1, 3))
    return Hkv * int(rng.choice([1, 2, max_group])), Hkv


def prefill_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 601))
        W, s, dil, g = mask_pattern(rng, N)
        Hq, Hkv = heads(rng)
        d = int(rng.choice([32, 64, 128]))
        out.append(dict(dtype="bf16" if i % 2 == 0 else "f32", B=int(rng.integers(1, 3)), Hq=Hq,
                        Hkv=Hkv, N=N, d=d, dv=d, window=W, stride=s, dilation=dil, n_global=g,
                        scale=1.0 / math.sqrt(d), seed=1000 + i))
    return out


def diff_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 401))
        W, s, dil, g = mask_pattern(rng, N)
        Hq, Hkv = heads(rng)
        out.append(dict(dtype="bf16" if i % 2 == 0 else "f32", B=1, Hq=Hq, Hkv=Hkv, N=N,
                        d=int(rng.choice([32, 64, 128])), dv=int(rng.choice([32, 64, 128])),
                        window=W, stride=s, dilation=dil, n_global=g, scale=0.125,
                        lam=float(rng.uniform(0.0, 1.0)), seed=2000 + i))
    return out


def decode_configs(n, seed, sinks):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        W = int(rng.integers(1, 301))
        B = int(rng.integers(1, 6))
        Hq, Hkv = heads(rng, max_group=int(rng.choice([8, 20, 33])))
        d = int(rng.choice([32, 64, 128]))
        lens = [int(x) for x in rng.integers(0, 3 * W + 10, size=B)]
        out.append(dict(dtype="bf16" if i % 2 == 0 else "f32", B=B, Hq=Hq, Hkv=Hkv, window=W, d=d,
                        dv=d, position=0, n_sink=int(rng.integers(1, 9)) if sinks else 0,
                        scale=1.0 / math.sqrt(d), seed=3000 + i + (100 if sinks else 0), lens=lens))
    return out


def diff_decode_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = "bf16" if i % 2 == 0 else "f32"
        d, dv = int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128]))
        W = int(rng.integers(1, 301))
        B = int(rng.integers(1, 5))
        Hq, Hkv = heads(rng, max_group=8)
        lens = [int(x) for x in rng.integers(0, 3 * W + 10, size=B)]
        out.append(dict(dtype=dt, B=B, Hq=Hq, Hkv=Hkv, window=W, d=d, dv=dv, position=0,
                        scale=0.125, lam=float(rng.uniform(0.0, 1.0)), seed=4000 + i, lens=lens))
    return out


def long_configs(n, seed):
    """Long sequences (1,000-30,000 tokens), checked on sampled rows: windows
    up to 4,096 keys or wider than the sequence, stride, dilation up to the
    key-tile size, global tokens, one or two maps."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1000, 30001))
        two = rng.random() < 0.3
        d = int(rng.choice([32, 64, 128]))
        out.append(dict(dtype="bf16" if rng.random() < 0.75 else "f32", B=1,
                        Hq=int(rng.choice([1, 2, 4])), Hkv=1, N=N, d=d,
                        dv=int(rng.choice([32, 64, 128])) if two else d,
                        window=int(rng.integers(1, 4097)) if rng.random() < 0.9 else N + 5,
                        stride=0 if rng.random() < 0.5 else int(rng.integers(1, 3000)),
                        dilation=1 if rng.random() < 0.6 else int(rng.integers(2, 65)),
                        n_global=0 if rng.random() < 0.7 else int(rng.integers(1, 300)),
                        two=two, scale=1.0 / math.sqrt(d), lam=float(rng.uniform(0, 1)),
                        seed=10000 + i))
    return out


def asm_prefill_configs(n, seed):
    """Shapes of the generated prefill kernel (bf16, d = 128, 4 or 8 query
    heads per key/value head, no stride): a plain, dilated or global-token
    window, with the log-sum-exp."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 1501))
        kind = int(rng.integers(0, 3))
        Hkv = int(rng.integers(1, 3))
        out.append(dict(dtype="bf16", B=int(rng.integers(1, 3)), Hq=Hkv * int(rng.choice([4, 8])), Hkv=Hkv,
                        N=N, d=128, dv=128, window=int(rng.integers(1, N + 41)), stride=0,
                        dilation=int(rng.integers(2, 9)) if kind == 1 else 1,
                        n_global=int(rng.integers(1, N + 4)) if kind == 2 else 0,
                        scale=1.0 / math.sqrt(128), seed=5000 + i))
    return out


def asm_diff_configs(n, seed):
    """Shapes of the generated differential kernel (bf16, d = 64, dv = 128,
    a window only), lambda from -1 to 2."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 1201))
        Hkv = int(rng.integers(1, 3))
        out.append(dict(dtype="bf16", B=int(rng.integers(1, 3)), Hq=Hkv * int(rng.choice([1, 2, 4])), Hkv=Hkv,
                        N=N, d=64, dv=128, window=int(rng.integers(1, N + 41)), stride=0, dilation=1,
                        n_global=0, scale=0.125, lam=float(rng.uniform(-1.0, 2.0)), seed=6000 + i))
    return out


def asm_str_configs(n, seed):
    """Shapes of the generated multi-head kernel (bf16, d = dv = 64, one query
    head per key/value head, B * H even): a window with no stride or a
    power-of-two stride from 64 to 2^18, with the log-sum-exp."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 3001))
        B, H = [(1, 2), (2, 1), (1, 4), (2, 2), (3, 2)][int(rng.integers(0, 5))]
        s = 0 if rng.random() < 0.25 else 1 << int(rng.integers(6, 19))
        out.append(dict(dtype="bf16", B=B, Hq=H, Hkv=H, N=N, d=64, dv=64, window=int(rng.integers(1, N + 41)),
                        stride=s, dilation=1, n_global=0, scale=0.125, seed=7000 + i))
    return out


def label(c):
    keys = ("dtype", "B", "Hq", "Hkv", "N", "d", "dv", "window", "stride", "dilation", "n_global",
            "n_sink", "two")
    return " ".join(f"{k}={c[k]}" for k in keys if k in c)


def banner(c):
    print(f"[case] {label(c)}", flush=True)


@pytest.mark.parametrize("cfg", prefill_configs(16 * SCALE, 11), ids=label)
def test_random_prefill(swa, cfg):
    banner(cfg)
    dt = cfg["dtype"]
    q, k, v = synth.prefill_inputs(cfg)
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], cfg["stride"], dtype=tdtype(dt),
                                    d=cfg["d"], dilation=cfg["dilation"], n_global=cfg["n_global"])
    out = swa.swa_attn_fwd(dev(q, dt), dev(k, dt), dev(v, dt), cfg["window"], cfg["stride"],
                           cfg["scale"], mask)
    want = oracle.attn_full(q, k, v, cfg["window"], cfg["stride"], cfg["scale"],
                            dilation=cfg["dilation"], n_global=cfg["n_global"])
    assert max_err(host(out), want) <= TOL[dt]


@pytest.mark.parametrize("cfg", asm_prefill_configs(12 * SCALE, 17), ids=label)
def test_random_asm_prefill(swa, cfg):
    banner(cfg)
    q, k, v = synth.prefill_inputs(cfg)
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], 0, d=128, dilation=cfg["dilation"],
                                    n_global=cfg["n_global"])
    lse = torch.empty((cfg["B"], cfg["Hq"], cfg["N"]), dtype=torch.float32, device="cuda")
    out = swa.swa_attn_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), cfg["window"], 0, cfg["scale"],
                           mask, lse=lse)
    want, want_lse = oracle.attn_full(q, k, v, cfg["window"], 0, cfg["scale"], with_lse=True,
                                      dilation=cfg["dilation"], n_global=cfg["n_global"])
    assert max_err(host(out), want) <= TOL["bf16"]
    assert max_err(host(lse), want_lse) <= 4e-3


@pytest.mark.parametrize("cfg", asm_diff_configs(8 * SCALE, 18), ids=label)
def test_random_asm_diff(swa, cfg):
    banner(cfg)
    ins = synth.diff_inputs(cfg)
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], 0, d=64, dv=128, op=swa.SWA_OP_DIFF)
    out = swa.diff_attn_fwd(*(dev(x, "bf16") for x in ins), cfg["window"], 0, cfg["scale"], cfg["lam"], mask)
    want = oracle.diff_full(*ins, cfg["window"], 0, cfg["scale"], cfg["lam"])
    assert max_err(host(out), want) <= TOL["bf16"]


@pytest.mark.parametrize("cfg", asm_str_configs(8 * SCALE, 19), ids=label)
def test_random_asm_str(swa, cfg):
    banner(cfg)
    q, k, v = synth.prefill_inputs(cfg)
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], cfg["stride"], d=64)
    lse = torch.empty((cfg["B"], cfg["Hq"], cfg["N"]), dtype=torch.float32, device="cuda")
    out = swa.swa_attn_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), cfg["window"], cfg["stride"],
                           cfg["scale"], mask, lse=lse)
    want, want_lse = oracle.attn_full(q, k, v, cfg["window"], cfg["stride"], cfg["scale"], with_lse=True)
    assert max_err(host(out), want) <= TOL["bf16"]
    assert max_err(host(lse), want_lse) <= 4e-3


@pytest.mark.parametrize("cfg", diff_configs(10 * SCALE, 12), ids=label)
def test_random_diff(swa, cfg):
    banner(cfg)
    dt = cfg["dtype"]
    ins = synth.diff_inputs(cfg)
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], cfg["stride"], dtype=tdtype(dt),
                                    d=cfg["d"], dv=cfg["dv"], op=swa.SWA_OP_DIFF,
                                    dilation=cfg["dilation"], n_global=cfg["n_global"])
    out = swa.diff_attn_fwd(*(dev(x, dt) for x in ins), cfg["window"], cfg["stride"], cfg["scale"],
                            cfg["lam"], mask)
    want = oracle.diff_full(*ins, cfg["window"], cfg["stride"], cfg["scale"], cfg["lam"],
                            dilation=cfg["dilation"], n_global=cfg["n_global"])
    assert max_err(host(out), want) <= TOL[dt]


@pytest.mark.parametrize("cfg", decode_configs(8 * SCALE, 13, sinks=False) +
                         decode_configs(6 * SCALE, 14, sinks=True),
                         ids=label)
def test_random_decode(swa, cfg):
    banner(cfg)
    dt = cfg["dtype"]
    ins = synth.decode_inputs(cfg, seq_len=cfg["lens"])
    sl = torch.from_numpy(ins["seq_len"].astype(np.int32)).cuda()
    if cfg["n_sink"] == 0:
        out = swa.swa_attn_decode(dev(ins["q"], dt), dev(ins["k_ring"], dt), dev(ins["v_ring"], dt), sl,
                                  cfg["scale"])
        want = oracle.decode(ins["q"], ins["k_ring"], ins["v_ring"], ins["seq_len"], cfg["scale"])
    else:
        out = swa.swa_attn_decode_sinks(dev(ins["q"], dt), dev(ins["k_sink"], dt), dev(ins["v_sink"], dt),
                                        dev(ins["k_ring"], dt), dev(ins["v_ring"], dt), sl, cfg["scale"])
        want = oracle.decode(ins["q"], ins["k_ring"], ins["v_ring"], ins["seq_len"], cfg["scale"],
                             k_sink=ins["k_sink"], v_sink=ins["v_sink"])
    assert max_err(host(out), want) <= TOL[dt]


@pytest.mark.parametrize("cfg", diff_decode_configs(8 * SCALE, 15), ids=label)
def test_random_diff_decode(swa, cfg):
    banner(cfg)
    dt = cfg["dtype"]
    ins = synth.diff_decode_inputs(cfg, seq_len=cfg["lens"])
    sl = torch.from_numpy(ins["seq_len"].astype(np.int32)).cuda()
    out = swa.diff_attn_decode(*(dev(ins[x], dt) for x in ("q1", "k1_ring", "q2", "k2_ring", "v_ring")),
                               sl, cfg["scale"], cfg["lam"])
    want = oracle.diff_decode(ins["q1"], ins["k1_ring"], ins["q2"], ins["k2_ring"], ins["v_ring"],
                              ins["seq_len"], cfg["scale"], cfg["lam"])
    assert max_err(host(out), want) <= TOL[dt]


@pytest.mark.parametrize("cfg", long_configs(6 * SCALE, 16), ids=label)
def test_random_long_sampled(swa, cfg):
    banner(cfg)
    dt, N, Hq, dv = cfg["dtype"], cfg["N"], cfg["Hq"], cfg["dv"]
    W, s, dil, g = cfg["window"], cfg["stride"], cfg["dilation"], cfg["n_global"]
    rng = np.random.default_rng(cfg["seed"])
    rows = np.unique(np.concatenate([rng.integers(0, Hq * N, size=48), [0, N - 1, Hq * N - 1]]))
    if cfg["two"]:
        ins = synth.diff_inputs(cfg)
        mask = swa.swa_block_mask_build(N, W, s, dtype=tdtype(dt), d=cfg["d"], dv=dv, op=swa.SWA_OP_DIFF,
                                        dilation=dil, n_global=g)
        out = swa.diff_attn_fwd(*(dev(x, dt) for x in ins), W, s, cfg["scale"], cfg["lam"], mask)
        want = oracle.diff_rows(*ins, W, s, cfg["scale"], cfg["lam"], rows, dilation=dil, n_global=g)
    else:
        q, k, v = synth.prefill_inputs(cfg)
        mask = swa.swa_block_mask_build(N, W, s, dtype=tdtype(dt), d=cfg["d"], dilation=dil, n_global=g)
        out = swa.swa_attn_fwd(dev(q, dt), dev(k, dt), dev(v, dt), W, s, cfg["scale"], mask)
        want = oracle.attn_rows(q, k, v, W, s, cfg["scale"], rows, dilation=dil, n_global=g)
    got = host(out).reshape(-1, dv)
    assert np.all(np.isfinite(got))
    assert max_err(got[rows], want) <= TOL[dt]
