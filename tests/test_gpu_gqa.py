"""GPU parity of the grouped-query sliding-window kernel (the generated gfx950
assembly kernel that serves bf16, d = 128, window-only problems with a
multiple of 4 query heads per key/value head) against the fp64 oracle.

The kernel works on items of 64 query rows of 4 query heads of a key/value
head, a workgroup per compute unit taking items in turn; the cases cover
one-tile bands, chains of several items per workgroup, dilated windows
(the variant that walks each residue class of the rows as a plain window),
global tokens (the variant that walks the global columns' tiles ahead of
the band), ragged
sequence ends (rows and keys past N), windows at and around the 64-key tile
size, windows beyond N, several head blocks per key/value head, batches,
peaky scores that move the running maximum late, the log-sum-exp output, and
key/value rows past N that hold NaN (they must read as zeros).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 2e-2
# The kernel's row sums are sums of the bf16-rounded probabilities (the
# values the P V product accumulates), each within a relative 2^-8 of its
# exact value: the log of the sum is within ln(1 + 2^-8) < 4e-3 of the exact
# log-sum-exp.
LSE_TOL = 4e-3


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_masked_transformer_amd as m
    return m


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def run(swa, q, k, v, W, scale, with_lse=True, kd=None, vd=None):
    B, Hq, N, d = q.shape
    mask = swa.swa_block_mask_build(N, W, 0, d=128)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda") if with_lse else None
    out = swa.swa_attn_fwd(bf(q), bf(k) if kd is None else kd, bf(v) if vd is None else vd, W, 0, scale,
                           mask, lse=lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    return (o, lse.cpu().numpy().astype(np.float64)) if with_lse else o


CASES = [
    # B, Hq, Hkv, N, W
    (1, 4, 1, 1, 1),
    (1, 4, 1, 64, 64),
    (1, 4, 1, 63, 16),
    (1, 4, 1, 65, 16),
    (1, 4, 1, 130, 100),
    (1, 4, 1, 200, 1),
    (1, 8, 2, 300, 64),
    (1, 4, 1, 333, 63),
    (1, 4, 1, 333, 65),
    (1, 4, 1, 500, 128),
    (1, 4, 1, 500, 129),
    (2, 8, 1, 1000, 256),       # two head blocks per key/value head
    (1, 12, 3, 777, 1024),      # window longer than the sequence
    (1, 4, 1, 1500, 2 ** 30),   # full causal
    (1, 4, 1, 4097, 1024),
    (2, 16, 2, 2100, 700),
    (1, 4, 1, 3000, 2),
    # more items (row blocks x head blocks) than compute units: a workgroup
    # takes several in turn, each item's first loads overlapping the
    # previous item's last step and output
    (8, 64, 16, 200, 64),       # 512 items, bands of 1 and 2 tiles
    (16, 32, 8, 130, 100),      # 384 items, bands of 1 to 3 tiles
    (4, 64, 16, 700, 300),      # 704 items, bands of 1 to 6 tiles
    (2, 32, 8, 2500, 200),      # 640 items
    (3, 36, 9, 650, 100),       # 297 items: not a multiple of 8
]


@pytest.mark.parametrize("B,Hq,Hkv,N,W", CASES)
def test_gqa_parity(swa, B, Hq, Hkv, N, W):
    print(f"[case] gqa B={B} Hq={Hq} Hkv={Hkv} N={N} W={W}", flush=True)
    cfg = dict(dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, N=N, d=128, dv=128, window=W, stride=0,
               scale=1.0 / math.sqrt(128), seed=1000 + N + W % 9973 + Hq)
    q, k, v = synth.prefill_inputs(cfg)
    got, lse = run(swa, q, k, v, W, cfg["scale"])
    want, want_lse = oracle.attn_full(q, k, v, W, 0, cfg["scale"], with_lse=True)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    lerr = float(np.max(np.abs(lse - want_lse)))
    assert err <= TOL, err
    assert lerr <= LSE_TOL, lerr


DILATED_CASES = [
    # B, Hq, Hkv, N, W, dilation: each residue class of the rows mod the
    # dilation runs as a plain window over every dilation-th row
    (1, 4, 1, 200, 16, 2),
    (1, 4, 1, 333, 40, 3),
    (1, 8, 2, 1000, 100, 2),
    (1, 4, 1, 130, 1, 5),
    (1, 4, 1, 385, 9, 3),          # classes of 129, 128, 128 rows: empty last blocks
    (1, 4, 1, 7, 3, 8),            # N < dilation: one row per class
    (1, 4, 1, 40, 3, 64),          # the largest dilation
    (1, 4, 1, 500, 2 ** 30, 2),    # every earlier key of the class attends
    (1, 4, 1, 4097, 700, 2),
    (2, 8, 2, 2000, 300, 4),
    (4, 16, 4, 2100, 300, 3),      # 528 items
]


@pytest.mark.parametrize("B,Hq,Hkv,N,W,dil", DILATED_CASES)
def test_gqa_dilated_parity(swa, B, Hq, Hkv, N, W, dil):
    print(f"[case] gqa dilated B={B} Hq={Hq} Hkv={Hkv} N={N} W={W} dilation={dil}", flush=True)
    cfg = dict(dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, N=N, d=128, dv=128, window=W, stride=0, dilation=dil,
               scale=1.0 / math.sqrt(128), seed=3000 + N + W % 9973 + dil)
    q, k, v = synth.prefill_inputs(cfg)
    mask = swa.swa_block_mask_build(N, W, 0, d=128, dilation=dil)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    out = swa.swa_attn_fwd(bf(q), bf(k), bf(v), W, 0, cfg["scale"], mask, lse=lse)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want, want_lse = oracle.attn_full(q, k, v, W, 0, cfg["scale"], with_lse=True, dilation=dil)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL
    assert float(np.max(np.abs(lse.cpu().numpy() - want_lse))) <= LSE_TOL


GLOBAL_CASES = [
    # B, Hq, Hkv, N, W, n_global: keys below n_global attend every later row
    # and rows below it attend every earlier key; the variant walks the
    # global columns' tiles ahead of each item's band
    (1, 4, 1, 200, 16, 64),
    (1, 4, 1, 333, 40, 1),
    (1, 4, 1, 333, 40, 65),
    (1, 8, 2, 1000, 100, 130),     # global rows beyond the first item
    (1, 4, 1, 130, 1, 5),
    (1, 4, 1, 64, 64, 64),
    (1, 4, 1, 500, 1000, 64),      # window longer than the sequence
    (1, 4, 1, 700, 50, 300),       # five tiles of global columns
    (2, 8, 2, 1100, 200, 64),
    (1, 4, 1, 257, 3, 200),
    (1, 4, 1, 90, 90, 1000),       # every token global
    (4, 16, 4, 2100, 300, 64),     # 528 items
]


@pytest.mark.parametrize("B,Hq,Hkv,N,W,g", GLOBAL_CASES)
def test_gqa_global_tokens_parity(swa, B, Hq, Hkv, N, W, g):
    print(f"[case] gqa global tokens B={B} Hq={Hq} Hkv={Hkv} N={N} W={W} n_global={g}", flush=True)
    cfg = dict(dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, N=N, d=128, dv=128, window=W, stride=0, n_global=g,
               scale=1.0 / math.sqrt(128), seed=5000 + N + W % 9973 + g)
    q, k, v = synth.prefill_inputs(cfg)
    mask = swa.swa_block_mask_build(N, W, 0, d=128, n_global=g)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    out = swa.swa_attn_fwd(bf(q), bf(k), bf(v), W, 0, cfg["scale"], mask, lse=lse)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want, want_lse = oracle.attn_full(q, k, v, W, 0, cfg["scale"], with_lse=True, n_global=g)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL
    assert float(np.max(np.abs(lse.cpu().numpy() - want_lse))) <= LSE_TOL


@pytest.mark.parametrize("q_scale,W", [(8.0, 300), (16.0, 1024)])
def test_gqa_peaky_scores(swa, q_scale, W):
    """Scores spread far beyond the running maximum's slack: the maximum moves
    after the first tile and O is rescaled mid-band."""
    print(f"[case] gqa peaky q x{q_scale} W={W}", flush=True)
    N = 1300
    cfg = dict(dtype="bf16", B=1, Hq=8, Hkv=2, N=N, d=128, dv=128, window=W, stride=0,
               scale=1.0 / math.sqrt(128), seed=4242)
    q, k, v = synth.prefill_inputs(cfg, q_scale=q_scale)
    # later keys larger: the maximum keeps moving along the band
    k = synth.round_bf16(k * np.linspace(1.0, 3.0, N, dtype=np.float32)[None, None, :, None])
    got, lse = run(swa, q, k, v, W, cfg["scale"])
    want, want_lse = oracle.attn_full(q, k, v, W, 0, cfg["scale"], with_lse=True)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL
    # the log-sum-exp of peaky rows is large: compare relative to its size
    assert float(np.max(np.abs(lse - want_lse) / np.maximum(1.0, np.abs(want_lse)))) <= LSE_TOL


@pytest.mark.parametrize("variant", ["plain", "dilated", "global"])
def test_gqa_score_jump_redoes_tile(swa, variant):
    """Keys whose scores lie 80-130 and 160-270 (log2 units) above every
    other score, in tiles past the first two of the items that attend them:
    the steps there take no row maximum, their row-sum check fails, and the
    tile is computed again with its maximum (the running maximum moves
    twice).  Without that, p = 2^(score - maximum) of the second key would
    overflow fp32."""
    print(f"[case] gqa score jump ({variant})", flush=True)
    N, W = 1300, 600 if variant == "plain" else 300
    dil, g = (2, 0) if variant == "dilated" else ((1, 64) if variant == "global" else (1, 0))
    cfg = dict(dtype="bf16", B=1, Hq=8, Hkv=2, N=N, d=128, dv=128, window=W, stride=0,
               scale=1.0 / math.sqrt(128), seed=4343)
    q, k, v = synth.prefill_inputs(cfg)
    q = np.abs(q)                        # q . k > 0 for the positive rows below
    k = k.copy()
    for j, val in ((400, 8.0), (901, 16.0)):
        k[:, :, j, :] = val
    mask = swa.swa_block_mask_build(N, W, 0, d=128, dilation=dil, n_global=g)
    lse = torch.empty((1, 8, N), dtype=torch.float32, device="cuda")
    out = swa.swa_attn_fwd(bf(q), bf(k), bf(v), W, 0, cfg["scale"], mask, lse=lse)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    want, want_lse = oracle.attn_full(q, k, v, W, 0, cfg["scale"], with_lse=True, dilation=dil, n_global=g)
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert float(np.max(np.abs(got_lse - want_lse) / np.maximum(1.0, np.abs(want_lse)))) <= LSE_TOL


def test_gqa_rows_past_n_read_as_zeros(swa):
    """K and V are views at the start of larger buffers whose rows past N hold
    NaN: the kernel must read rows past N as zeros (masked keys of the last,
    ragged tile), so every output stays finite and equal to the oracle's."""
    print("[case] gqa NaN past N", flush=True)
    B, Hq, Hkv, N, W = 1, 4, 1, 333, 100
    cfg = dict(dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, N=N, d=128, dv=128, window=W, stride=0,
               scale=1.0 / math.sqrt(128), seed=99)
    q, k, v = synth.prefill_inputs(cfg)
    pad = 64
    kb = torch.full((B * Hkv * N + pad, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vb = torch.full((B * Hkv * N + pad, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    kb[:B * Hkv * N] = bf(k).reshape(-1, 128)
    vb[:B * Hkv * N] = bf(v).reshape(-1, 128)
    kd = kb[:B * Hkv * N].view(B, Hkv, N, 128)
    vd = vb[:B * Hkv * N].view(B, Hkv, N, 128)
    got = run(swa, q, k, v, W, cfg["scale"], with_lse=False, kd=kd, vd=vd)
    want = oracle.attn_full(q, k, v, W, 0, cfg["scale"])
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= TOL


def test_gqa_workload_all_rows(swa):
    """The SWA prefill workload (B=1, Hq=32, Hkv=8, N=8192, W=1024), every
    row against the oracle (threaded over rows)."""
    import concurrent.futures
    import os
    print("[case] gqa workload swa_prefill_bf16, all rows", flush=True)
    cfg = synth.workload("swa_prefill_bf16")
    q, k, v = synth.prefill_inputs(cfg)
    got = run(swa, q, k, v, cfg["window"], cfg["scale"], with_lse=False).reshape(-1, 128)
    rows = np.arange(got.shape[0], dtype=np.int64)
    threads = max(1, min(16, os.cpu_count() or 1))
    chunks = np.array_split(rows, threads * 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda r: oracle.attn_rows(q, k, v, cfg["window"], 0, cfg["scale"], r), chunks))
    want = np.concatenate(parts)
    assert float(np.max(np.abs(got - want))) <= TOL


def test_gqa_longest_sequence(swa):
    """N at its maximum (2^22): the largest byte offsets the generated kernel
    forms (row offsets, tile offsets and descriptor ranges up to 1 GiB per
    head), checked on sampled rows of every head, ends included."""
    N = swa.SWA_MAX_N
    print(f"[case] gqa at N={N} (sampled rows)", flush=True)
    cfg = dict(dtype="bf16", B=1, Hq=4, Hkv=1, N=N, d=128, dv=128, window=128, stride=0,
               scale=1.0 / math.sqrt(128), seed=24)
    q, k, v = synth.prefill_inputs(cfg)
    got, lse = run(swa, q, k, v, cfg["window"], cfg["scale"])
    got = got.reshape(-1, 128)
    must = [h * N + i for h in range(4) for i in (0, 63, 64, N // 2, N - 65, N - 64, N - 1)]
    rows = synth.sample_rows(4 * N, 192, seed=25, must=must)
    want, want_lse = oracle.attn_rows(q, k, v, cfg["window"], 0, cfg["scale"], rows, with_lse=True)
    assert float(np.max(np.abs(got[rows] - want))) <= TOL
    assert float(np.max(np.abs(lse.reshape(-1)[rows] - want_lse))) <= LSE_TOL
    assert np.all(np.isfinite(got[-4096:]))


def test_gqa_deterministic(swa):
    cfg = dict(dtype="bf16", B=1, Hq=8, Hkv=2, N=1500, d=128, dv=128, window=300, stride=0,
               scale=1.0 / math.sqrt(128), seed=5)
    print("[case] gqa determinism", flush=True)
    q, k, v = synth.prefill_inputs(cfg)
    a = run(swa, q, k, v, 300, cfg["scale"], with_lse=False)
    b = run(swa, q, k, v, 300, cfg["scale"], with_lse=False)
    np.testing.assert_array_equal(a, b)
