"""GPU parity of the differential-attention assembly kernel (the generated
gfx950 kernel that serves bf16, d = 64, dv = 128, window-only differential
attention) against the fp64 oracle.

The kernel works on items of 128 query rows of one query head, the waves of
the first map on one half of the workgroup and those of the second on the
other, a workgroup per compute unit taking items in turn; the cases cover
one-tile bands, ragged sequence ends, windows around the 64-key tile size
and beyond N, grouped-query heads (2 and 4 query heads per key/value head),
chains of several items per workgroup (more items than compute units, also
a count that is not a multiple of 8), several values of lambda, peaky
scores that move one map's running maximum late, and key/value rows past N
that hold NaN (they must read as zeros).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_masked_transformer_amd as m
    return m


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def run(swa, cfg, q1, k1, q2, k2, v, dev_k=None):
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], 0, dtype=torch.bfloat16, d=64, dv=128,
                                    op=swa.SWA_OP_DIFF)
    k1d, k2d, vd = dev_k if dev_k is not None else (bf(k1), bf(k2), bf(v))
    out = swa.diff_attn_fwd(bf(q1), k1d, bf(q2), k2d, vd, cfg["window"], 0, cfg["scale"], cfg["lam"], mask)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def config(B, Hq, Hkv, N, W, lam=0.5, seed=None):
    return dict(dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, N=N, d=64, dv=128, window=W, stride=0, scale=0.125,
                lam=lam, seed=7000 + N + W % 9973 + Hq if seed is None else seed)


CASES = [
    # B, Hq, Hkv, N, W, lambda
    (1, 1, 1, 1, 1, 0.5),
    (1, 2, 2, 64, 64, 0.5),
    (1, 2, 1, 63, 16, 0.5),
    (1, 2, 2, 129, 100, 0.0),
    (1, 2, 2, 200, 1, 0.5),
    (1, 4, 2, 333, 63, 0.5),
    (1, 4, 4, 333, 65, 1.3),
    (1, 2, 2, 500, 128, 0.5),
    (1, 2, 2, 500, 129, -0.4),
    (2, 4, 1, 1000, 256, 0.5),      # four query heads per key/value head
    (1, 3, 3, 777, 1024, 0.5),      # window longer than the sequence
    (1, 2, 2, 1500, 2 ** 30, 0.5),  # full causal
    (1, 2, 2, 3000, 2, 0.5),
    # more items than compute units: each workgroup takes several
    (2, 16, 16, 2100, 700, 0.5),    # 544 items
    (4, 32, 32, 600, 300, 0.8),     # 640 items
    (3, 12, 6, 1000, 100, 0.5),     # 288 items: not a multiple of 8
]


@pytest.mark.parametrize("B,Hq,Hkv,N,W,lam", CASES)
def test_diff_asm_parity(swa, B, Hq, Hkv, N, W, lam):
    print(f"[case] diff asm B={B} Hq={Hq} Hkv={Hkv} N={N} W={W} lambda={lam}", flush=True)
    cfg = config(B, Hq, Hkv, N, W, lam)
    ins = synth.diff_inputs(cfg)
    got = run(swa, cfg, *ins)
    want = oracle.diff_full(*ins, W, 0, cfg["scale"], lam)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


@pytest.mark.parametrize("which", [0, 1])
def test_diff_asm_peaky_map(swa, which):
    """One map's scores spread far beyond the running maximum's slack (its
    maximum moves along the band and O is rescaled); the other map stays
    flat."""
    print(f"[case] diff asm peaky map {which + 1}", flush=True)
    N, W = 1300, 600
    cfg = config(1, 4, 2, N, W, seed=4343 + which)
    q1, k1, q2, k2, v = synth.diff_inputs(cfg)
    ramp = np.linspace(1.0, 3.0, N, dtype=np.float32)[None, None, :, None]
    if which == 0:
        q1 = synth.round_bf16(q1 * 8.0)
        k1 = synth.round_bf16(k1 * ramp)
    else:
        q2 = synth.round_bf16(q2 * 8.0)
        k2 = synth.round_bf16(k2 * ramp)
    got = run(swa, cfg, q1, k1, q2, k2, v)
    want = oracle.diff_full(q1, k1, q2, k2, v, W, 0, cfg["scale"], cfg["lam"])
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


@pytest.mark.parametrize("which", [0, 1])
def test_diff_asm_score_jump_redoes_tile(swa, which):
    """One map's keys at two positions score about 100 and 150 (log2 units)
    above every other score, in tiles past the first three of the items that
    attend them: the steps there take no row maximum, their row-sum check
    fails, and the tile is computed again with its maximum.  Without that,
    p = 2^(score - maximum) of the second key would overflow fp32."""
    print(f"[case] diff asm score jump in map {which + 1}", flush=True)
    N, W = 1300, 600
    cfg = config(1, 4, 2, N, W, seed=5151 + which)
    q1, k1, q2, k2, v = synth.diff_inputs(cfg)
    q1, q2, k1, k2 = np.abs(q1), np.abs(q2), k1.copy(), k2.copy()
    kk = k1 if which == 0 else k2
    for j, val in ((500, 16.0), (901, 24.0)):
        kk[:, :, j, :] = val
    got = run(swa, cfg, q1, k1, q2, k2, v)
    want = oracle.diff_full(q1, k1, q2, k2, v, W, 0, cfg["scale"], cfg["lam"])
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


def test_diff_asm_rows_past_n_read_as_zeros(swa):
    """K1, K2 and V are views at the start of larger buffers whose rows past
    N hold NaN: rows past N must read as zeros."""
    print("[case] diff asm NaN past N", flush=True)
    B, Hq, Hkv, N, W = 1, 2, 2, 333, 100
    cfg = config(B, Hq, Hkv, N, W, seed=77)
    q1, k1, q2, k2, v = synth.diff_inputs(cfg)
    views = []
    for x, w in ((k1, 64), (k2, 64), (v, 128)):
        buf = torch.full((B * Hkv * N + 64, w), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[:B * Hkv * N] = bf(x).reshape(-1, w)
        views.append(buf[:B * Hkv * N].view(B, Hkv, N, w))
    got = run(swa, cfg, q1, k1, q2, k2, v, dev_k=tuple(views))
    want = oracle.diff_full(q1, k1, q2, k2, v, W, 0, cfg["scale"], cfg["lam"])
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


def test_diff_asm_longest_sequence(swa):
    """N at its maximum (2^22), checked on sampled rows, ends included."""
    N = swa.SWA_MAX_N
    print(f"[case] diff asm at N={N} (sampled rows)", flush=True)
    cfg = config(1, 2, 1, N, 200, seed=93)
    ins = synth.diff_inputs(cfg)
    got = run(swa, cfg, *ins).reshape(-1, 128)
    must = [h * N + i for h in range(2) for i in (0, 127, 128, N // 2, N - 129, N - 128, N - 1)]
    rows = synth.sample_rows(2 * N, 160, seed=94, must=must)
    want = oracle.diff_rows(*ins, cfg["window"], 0, cfg["scale"], cfg["lam"], rows)
    assert float(np.max(np.abs(got[rows] - want))) <= TOL
    assert np.all(np.isfinite(got[-4096:]))


def test_diff_asm_deterministic(swa):
    print("[case] diff asm determinism (chained items)", flush=True)
    cfg = config(2, 16, 8, 2100, 500, seed=91)
    ins = synth.diff_inputs(cfg)
    a = run(swa, cfg, *ins)
    b = run(swa, cfg, *ins)
    np.testing.assert_array_equal(a, b)
