"""GPU parity of the multi-head local + strided assembly kernel (the generated
gfx950 kernel that serves bf16, d = dv = 64, one query head per key/value
head, a window with an optional power-of-two stride pattern) against the
fp64 oracle.

The kernel works on items of 128 query rows of two consecutive (batch,
head) pairs, a workgroup per compute unit taking items in turn; an item
walks the stride keys below its band (gathered 64 at a time, the last group
partial) and then its band.  The cases cover one-tile bands, ragged sequence
ends, windows around the 64-key tile size and beyond N, strides from 64 to
2^18 (one, several and many gathered tiles per item, and a stride past N),
no stride at all, pairs of heads that straddle two batch entries, chains of
several items per workgroup (more items than compute units, also a count
that is not a multiple of 8), peaky scores that move the running maximum
late, a score jump past the first tiles that makes a step redo its tile, the
log-sum-exp, key/value rows past N that hold NaN (they must read as zeros),
and the largest N with the largest and the smallest stride the kernel takes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-2
# row sums over the bf16-rounded probabilities: within ln(1 + 2^-8) of the
# exact log-sum-exp
LSE_TOL = 4e-3


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_masked_transformer_amd as m
    return m


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def config(B, H, N, W, s, seed=None):
    return dict(dtype="bf16", B=B, Hq=H, Hkv=H, N=N, d=64, dv=64, window=W, stride=s, scale=0.125,
                seed=9100 + N + W % 9973 + H + s % 997 if seed is None else seed)


def run(swa, cfg, q, k, v, with_lse=False, kd=None, vd=None):
    B, H, N, _ = q.shape
    W, s = cfg["window"], cfg["stride"]
    mask = swa.swa_block_mask_build(N, W, s, d=64)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda") if with_lse else None
    out = swa.swa_attn_fwd(bf(q), bf(k) if kd is None else kd, bf(v) if vd is None else vd, W, s,
                           cfg["scale"], mask, lse=lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    return (o, lse.cpu().numpy().astype(np.float64)) if with_lse else o


CASES = [
    # B, H, N, W, stride
    (1, 2, 1, 1, 0),
    (1, 2, 1, 1, 64),
    (1, 2, 64, 64, 64),
    (1, 2, 63, 16, 128),
    (1, 2, 65, 16, 64),
    (1, 2, 200, 1, 64),          # stride keys alone past the diagonal
    (1, 2, 333, 63, 128),
    (1, 2, 333, 65, 64),
    (1, 2, 500, 128, 256),
    (1, 2, 500, 129, 0),
    (1, 4, 1000, 256, 128),
    (1, 2, 777, 1024, 128),      # window longer than the sequence
    (1, 2, 1500, 2 ** 30, 64),   # full causal
    (3, 2, 700, 100, 64),        # pairs of heads within each batch entry
    (3, 1, 900, 70, 128),        # pairs of heads across batch entries
    (1, 2, 4097, 100, 64),       # about 63 gathered keys per item at the end
    (1, 2, 9000, 64, 64),        # three gathered tiles, the last partial
    (1, 2, 3000, 200, 2 ** 18),  # stride past N: key 0 alone
    (1, 2, 5000, 300, 1024),
    # more items than compute units: each workgroup takes several
    (2, 16, 2100, 700, 128),     # 272 items
    (4, 16, 1100, 256, 64),      # 288 items: not a multiple of 8
    (1, 8, 8192, 256, 128),      # 256 items, prefixes of 0 .. 63 keys
]


@pytest.mark.parametrize("B,H,N,W,s", CASES)
def test_str_asm_parity(swa, B, H, N, W, s):
    print(f"[case] str asm B={B} H={H} N={N} W={W} s={s}", flush=True)
    cfg = config(B, H, N, W, s)
    q, k, v = synth.prefill_inputs(cfg)
    got = run(swa, cfg, q, k, v)
    want = oracle.attn_full(q, k, v, W, s, cfg["scale"])
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


@pytest.mark.parametrize("B,H,N,W,s", [(1, 2, 333, 65, 64), (2, 4, 2100, 300, 128), (1, 2, 9000, 64, 64)])
def test_str_asm_lse(swa, B, H, N, W, s):
    print(f"[case] str asm log-sum-exp B={B} H={H} N={N} W={W} s={s}", flush=True)
    cfg = config(B, H, N, W, s)
    q, k, v = synth.prefill_inputs(cfg)
    got, lse = run(swa, cfg, q, k, v, with_lse=True)
    want, want_lse = oracle.attn_full(q, k, v, W, s, cfg["scale"], with_lse=True)
    assert float(np.max(np.abs(got - want))) <= TOL
    assert float(np.max(np.abs(lse - want_lse))) <= LSE_TOL


def test_str_asm_peaky(swa):
    """Queries scaled by 8 and keys ramped along the sequence: the running
    maximum moves late in the band (O and l rescaled)."""
    print("[case] str asm peaky rows", flush=True)
    N, W, s = 3000, 300, 128
    cfg = config(1, 4, N, W, s, seed=6161)
    q, k, v = synth.prefill_inputs(cfg)
    ramp = np.linspace(1.0, 3.0, N, dtype=np.float32)[None, None, :, None]
    q = synth.round_bf16(q * 8.0)
    k = synth.round_bf16(k * ramp)
    got = run(swa, cfg, q, k, v)
    want = oracle.attn_full(q, k, v, W, s, cfg["scale"])
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


def test_str_asm_score_jump_redoes_tile(swa):
    """Keys at two band positions and one stride key score about 100 to 150
    (log2 units) above every other score, in tiles past the first three of
    the items that attend them: the steps there take no row maximum, their
    row-sum check fails, and the tile is computed again with its maximum."""
    print("[case] str asm score jump", flush=True)
    N, W, s = 3000, 300, 128
    cfg = config(1, 2, N, W, s, seed=6262)
    q, k, v = synth.prefill_inputs(cfg)
    q, k = np.abs(q), k.copy()
    for j, val in ((1290, 16.0), (1901, 24.0), (1024, 20.0)):
        k[:, :, j, :] = val
    got = run(swa, cfg, q, k, v)
    want = oracle.attn_full(q, k, v, W, s, cfg["scale"])
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


def test_str_asm_rows_past_n_read_as_zeros(swa):
    """K and V are views at the start of larger buffers whose rows past N
    hold NaN: rows past N must read as zeros (the band's last tile and the
    gathered stride keys past N)."""
    print("[case] str asm NaN past N", flush=True)
    B, H, N, W, s = 1, 2, 1333, 100, 64
    cfg = config(B, H, N, W, s, seed=78)
    q, k, v = synth.prefill_inputs(cfg)
    views = []
    for x in (k, v):
        buf = torch.full((B * H * N + 64, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[:B * H * N] = bf(x).reshape(-1, 64)
        views.append(buf[:B * H * N].view(B, H, N, 64))
    got = run(swa, cfg, q, k, v, kd=views[0], vd=views[1])
    want = oracle.attn_full(q, k, v, W, s, cfg["scale"])
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


def test_str_asm_deterministic(swa):
    print("[case] str asm determinism (chained items)", flush=True)
    cfg = config(2, 16, 2100, 500, 128, seed=92)
    q, k, v = synth.prefill_inputs(cfg)
    a = run(swa, cfg, q, k, v)
    b = run(swa, cfg, q, k, v)
    np.testing.assert_array_equal(a, b)


@pytest.fixture(scope="module")
def long_inputs(swa):
    """One seeded input at N = 2^22 (the largest N the boundary accepts),
    shared by the longest-sequence cases and released with the module."""
    cfg = config(1, 2, swa.SWA_MAX_N, 200, 0, seed=97)
    return synth.prefill_inputs(cfg)


@pytest.mark.parametrize("W,s", [(200, 2 ** 18), (128, 64)])
def test_str_asm_longest_sequence(swa, long_inputs, W, s):
    """N at its maximum (2^22), checked on sampled rows, ends included: with
    s = 2^18 the gathered rows of a prefix tile lie 2^25 bytes apart and
    reach 2^31 bytes past the head's first row (past N: zeros); with s = 64
    the items at the end gather 65,535 stride keys in 1,024 tiles."""
    N = swa.SWA_MAX_N
    print(f"[case] str asm at N={N} W={W} s={s} (sampled rows)", flush=True)
    q, k, v = long_inputs
    cfg = config(1, 2, N, W, s)
    got = run(swa, cfg, q, k, v).reshape(-1, 64)
    must = [h * N + i for h in range(2) for i in (0, 127, 128, 255, N // 2, N - 129, N - 128, N - 1)]
    rows = synth.sample_rows(2 * N, 150, seed=98, must=must)
    want = oracle.attn_rows(q, k, v, W, s, cfg["scale"], rows)
    assert float(np.max(np.abs(got[rows] - want))) <= TOL
    assert np.all(np.isfinite(got[-4096:]))
