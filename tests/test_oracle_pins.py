"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

Nothing here compares the oracle with itself.  Each test checks it against
one of: a hand-drawn mask from the pages' definitions (tests/golden), a
closed form, a value the pages print, an invariant the pages state, a
special case that reduces to a library routine (PyTorch's
scaled_dot_product_attention in float64 on the CPU), or brute force.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from conftest import parse_mask_golden


# --------------------------------------------------------------------------
# helpers (independent of the oracle)
# --------------------------------------------------------------------------

def band_count(n, w):
    """Closed form of the sliding-window cell count: row i attends min(i+1, w)
    keys, so the total is n(n+1)/2 when w >= n, else n*w - w(w-1)/2."""
    return n * (n + 1) // 2 if w >= n else n * w - w * (w - 1) // 2


def local_stride_row(i, w, s):
    """Keys attended by row i of window w plus stride s (s > 0): the window's
    min(i+1, w) keys, plus the multiples of s below the window start i-w+1,
    which are the multiples of s in [0, i-w]: floor((i-w)/s) + 1 of them."""
    return min(i + 1, w) + ((i - w) // s + 1 if i >= w else 0)


def local_stride_count(n, w, s):
    """Closed form of the total: C(n,w) + T + s*q*(q-1)/2 + r*q with T = n-w,
    q = T // s, r = T % s (valid for w < n, s > 0)."""
    t = n - w
    q, r = divmod(t, s)
    return band_count(n, w) + t + s * q * (q - 1) // 2 + r * q


def sdpa64(q, k, v, scale, mask=None, causal=False):
    """PyTorch's scaled_dot_product_attention in float64 on the CPU, with
    key/value heads shared by contiguous groups of query heads."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))
    g = qt.shape[-3] // kt.shape[-3]
    kt = kt.repeat_interleave(g, dim=-3)
    vt = vt.repeat_interleave(g, dim=-3)
    m = None if mask is None else torch.from_numpy(mask.astype(bool))
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=causal,
                                          scale=scale).numpy()


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


# --------------------------------------------------------------------------
# mask
# --------------------------------------------------------------------------

def test_masks_match_hand_drawn_8x8(golden_dir):
    masks = parse_mask_golden(os.path.join(golden_dir, "masks_8x8.txt"))
    assert set(masks) == {"causal_8", "swa_8_w4", "strided_8_w2_s3", "swa_8_w2"}
    for name, (p, rows) in masks.items():
        got = oracle.mask_dense(p["n"], p["window"], p["stride"])
        np.testing.assert_array_equal(got, np.array(rows, dtype=np.uint8), err_msg=name)
        total, per_row = oracle.count_nonmasked(p["n"], p["window"], p["stride"])
        assert total == sum(map(sum, rows)), name
        np.testing.assert_array_equal(per_row, [sum(r) for r in rows], err_msg=name)


def test_8x8_counts():
    # counts of the four 8x8 examples: 36, 26, 24, 15
    assert oracle.count_nonmasked(8, 8, 0)[0] == 36
    assert oracle.count_nonmasked(8, 4, 0)[0] == 26
    assert oracle.count_nonmasked(8, 2, 3)[0] == 24
    assert oracle.count_nonmasked(8, 2, 0)[0] == 15


@pytest.mark.parametrize("n", [1, 2, 7, 16, 33, 64])
def test_band_count_closed_form(n):
    for w in range(1, n + 3):
        total, rows = oracle.count_nonmasked(n, w, 0)
        assert total == band_count(n, w), (n, w)
        np.testing.assert_array_equal(rows, [min(i + 1, w) for i in range(n)])


def test_window_ge_n_is_causal():
    # "Attention Variants Compared": window >= n gives full causal
    for n in (1, 5, 12):
        causal = np.tril(np.ones((n, n), dtype=np.uint8))
        for w in (n, n + 1, 2 * n):
            np.testing.assert_array_equal(oracle.mask_dense(n, w, 0), causal)


def test_local_stride_closed_form():
    for n in range(1, 41):
        for w in range(1, n + 2):
            for s in range(1, 12):
                total, rows = oracle.count_nonmasked(n, w, s)
                np.testing.assert_array_equal(
                    rows, [local_stride_row(i, w, s) for i in range(n)], err_msg=str((n, w, s)))
                if w < n:
                    assert total == local_stride_count(n, w, s)


def test_stride_one_is_causal():
    for n in (3, 9):
        for w in (1, 2, 5):
            np.testing.assert_array_equal(oracle.mask_dense(n, w, 1),
                                          np.tril(np.ones((n, n), dtype=np.uint8)))


def test_workload_cell_counts():
    # per (b, head) counts of the workloads; all heads share the mask
    assert band_count(256, 64) == 14368
    assert oracle.count_nonmasked(256, 64, 0)[0] == 14368
    assert band_count(8192, 1024) == 7864832
    assert band_count(4096, 1024) == 3670528
    assert local_stride_count(16384, 256, 128) == 5185792


def test_strided_workload_count_by_rows():
    # the full 16384-row local+stride count, row by row in closed form
    n, w, s = 16384, 256, 128
    assert sum(local_stride_row(i, w, s) for i in range(n)) == 5185792


# --------------------------------------------------------------------------
# tile list
# --------------------------------------------------------------------------

def parse_tile_golden(path):
    params, rows = None, []
    for raw in open(path):
        line = raw.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("params"):
            params = {k: int(v) for k, v in (kv.split("=") for kv in line.split()[1:])}
            continue
        body, sk = line.split("|")
        entries = [e.split(":") for e in body.split(":", 1)[1].split()]
        rows.append(([(int(t), {"F": 0, "P": 1, "S": 2}[k], int(c)) for t, k, c in entries],
                     int(sk.split("=")[1])))
    return params, rows


def test_tile_list_hand_worked(golden_dir):
    p, rows = parse_tile_golden(os.path.join(golden_dir, "tile_list_n16_w4_s5_b4.txt"))
    t = oracle.tile_list(p["n"], p["window"], p["stride"], p["bm"], p["bn"])
    assert t["num_q_tiles"] == len(rows)
    for qt, (entries, sk) in enumerate(rows):
        a, b = t["row_ptr"][qt], t["row_ptr"][qt + 1]
        got = list(zip(t["kv_tile"][a:b].tolist(), t["kind"][a:b].tolist(), t["cells"][a:b].tolist()))
        assert got == entries, qt
        assert t["prefix_keys"][qt] == sk


def block_sums(mask, bm, bn):
    n = mask.shape[0]
    nq, nk = -(-n // bm), -(-n // bn)
    pad = np.zeros((nq * bm, nk * bn), dtype=np.int64)
    pad[:n, :n] = mask
    return pad.reshape(nq, bm, nk, bn).sum(axis=(1, 3))


@pytest.mark.parametrize("n,w,s,bm,bn,dil,g", [
    (37, 5, 0, 8, 8, 1, 0), (37, 5, 3, 8, 4, 1, 0), (64, 16, 7, 16, 8, 1, 0), (50, 50, 0, 16, 16, 1, 0),
    (50, 1, 0, 4, 8, 1, 0), (70, 9, 1, 8, 8, 1, 0), (129, 20, 11, 32, 16, 1, 0),
    (100, 300, 6, 16, 32, 1, 0),
    (90, 6, 0, 16, 8, 3, 0), (90, 6, 5, 8, 8, 8, 0), (77, 4, 0, 16, 16, 16, 0),
    (90, 7, 0, 16, 8, 1, 3), (90, 7, 9, 8, 8, 1, 20), (70, 5, 4, 16, 8, 2, 11),
    (40, 3, 0, 8, 8, 1, 40)])
def test_tile_list_against_block_sums(n, w, s, bm, bn, dil, g):
    """Per-tile cell counts equal numpy block sums of the (pinned) dense mask;
    the kinds follow from the band/prefix split of each block; the band tiles
    of a query tile are one contiguous range (for dilation <= bn) with every
    prefix-only tile left of it; prefix_keys counts the multiples of s and
    the global columns below that range."""
    mask = oracle.mask_dense(n, w, s, dil, g)
    ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    band = ((jj <= ii) & (ii - jj <= (w - 1) * dil)).astype(np.int64)
    sums = block_sums(mask, bm, bn)
    bsums = block_sums(band, bm, bn)
    t = oracle.tile_list(n, w, s, bm, bn, dilation=dil, n_global=g)
    nq, nk = sums.shape
    assert t["nnz"] == int((sums > 0).sum())
    assert int(t["cells"].sum()) == int(mask.sum())
    for qt in range(nq):
        a, b = t["row_ptr"][qt], t["row_ptr"][qt + 1]
        tiles = t["kv_tile"][a:b]
        np.testing.assert_array_equal(tiles, np.nonzero(sums[qt])[0])
        rows_in = min(n, (qt + 1) * bm) - qt * bm
        for e in range(a, b):
            kt = t["kv_tile"][e]
            cols_in = min(n, (kt + 1) * bn) - kt * bn
            assert t["cells"][e] == sums[qt, kt]
            want = 2 if bsums[qt, kt] == 0 else (0 if sums[qt, kt] == rows_in * cols_in else 1)
            assert t["kind"][e] == want
        kinds = t["kind"][a:b]
        band_idx = np.nonzero(kinds != 2)[0]
        assert len(band_idx) > 0
        assert np.all(np.diff(tiles[band_idx]) == 1)
        assert np.all(kinds[: band_idx[0]] == 2) and np.all(kinds[band_idx[0]:] != 2)
        assert t["band_begin"][qt] == a + band_idx[0]
        lo_key = tiles[band_idx[0]] * bn
        want_pk = len([j for j in range(lo_key) if j < g or (s > 0 and j % s == 0)])
        assert t["prefix_keys"][qt] == want_pk


def test_stride_only_tiles_attended_by_every_row():
    # a stride-only tile's stride columns are open in every row of its query tile
    n, w, s, bm, bn = 96, 10, 7, 16, 8
    mask = oracle.mask_dense(n, w, s)
    t = oracle.tile_list(n, w, s, bm, bn)
    for qt in range(t["num_q_tiles"]):
        for e in range(t["row_ptr"][qt], t["row_ptr"][qt + 1]):
            if t["kind"][e] != 2:
                continue
            kt = t["kv_tile"][e]
            cols = [j for j in range(kt * bn, min(n, (kt + 1) * bn)) if j % s == 0]
            rows = range(qt * bm, min(n, (qt + 1) * bm))
            assert all(mask[i, j] for i in rows for j in cols)


def test_workload_tile_lists():
    # 8192 x 8192 window 1024 at 128 x 64 tiles: 840 full + 240 partial tiles per head
    t = oracle.tile_list(2048, 1024, 0, 128, 64)
    assert int(t["cells"].sum()) == band_count(2048, 1024)
    big = oracle.tile_list(8192, 1024, 0, 128, 64)
    assert int((big["kind"] == 0).sum()) == 840 and int((big["kind"] == 1).sum()) == 240
    assert int(big["cells"].sum()) == 7864832


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B,Hq,Hkv,N,d,dv,w,s", [
    (1, 2, 2, 40, 8, 8, 7, 0), (2, 4, 2, 33, 16, 8, 5, 4), (1, 8, 2, 64, 32, 48, 64, 0),
    (1, 3, 1, 29, 4, 4, 1, 0), (2, 2, 1, 50, 8, 8, 3, 1), (1, 4, 4, 45, 8, 16, 100, 9)])
def test_attention_matches_sdpa_with_pinned_mask(B, Hq, Hkv, N, d, dv, w, s):
    q, k, v = rand((B, Hq, N, d), 1), rand((B, Hkv, N, d), 2), rand((B, Hkv, N, dv), 3)
    scale = 1.0 / math.sqrt(d) * 1.3
    got, lse = oracle.attn_full(q, k, v, w, s, scale, with_lse=True)
    want = sdpa64(q, k, v, scale, mask=oracle.mask_dense(N, w, s))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # log-sum-exp of the scaled scores over the attended keys
    kk = np.repeat(k.astype(np.float64), Hq // Hkv, axis=1)
    sc = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), kk) * scale
    sc = np.where(oracle.mask_dense(N, w, s)[None, None].astype(bool), sc, -np.inf)
    mx = sc.max(-1, keepdims=True)
    np.testing.assert_allclose(lse, (mx + np.log(np.exp(sc - mx).sum(-1, keepdims=True)))[..., 0],
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N,w", [(17, 17), (24, 100)])
def test_window_ge_n_reduces_to_causal_sdpa(N, w):
    q, k, v = rand((1, 4, N, 8), 4), rand((1, 2, N, 8), 5), rand((1, 2, N, 8), 6)
    got = oracle.attn_full(q, k, v, w, 0, 0.35)
    np.testing.assert_allclose(got, sdpa64(q, k, v, 0.35, causal=True), rtol=1e-12, atol=1e-12)


def test_peaky_scores_need_max_subtraction():
    # scores around +-1000: exp without subtracting the row max overflows
    q, k, v = rand((1, 2, 30, 16), 7) * 40, rand((1, 2, 30, 16), 8), rand((1, 2, 30, 16), 9)
    got = oracle.attn_full(q, k, v, 6, 4, 1.0)
    want = sdpa64(q, k, v, 1.0, mask=oracle.mask_dense(30, 6, 4))
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_window_one_returns_own_value():
    q, k, v = rand((2, 4, 21, 8), 10), rand((2, 2, 21, 8), 11), rand((2, 2, 21, 12), 12)
    got = oracle.attn_full(q, k, v, 1, 0, 0.5)
    np.testing.assert_array_equal(got, np.repeat(v.astype(np.float64), 2, axis=1))


def test_zero_keys_give_mean_of_attended_values():
    N, w, s = 40, 6, 5
    q, v = rand((1, 2, N, 8), 13), rand((1, 2, N, 8), 14)
    got = oracle.attn_full(q, np.zeros((1, 2, N, 8), np.float32), v, w, s, 0.7)
    mask = oracle.mask_dense(N, w, s).astype(np.float64)
    want = np.einsum("ij,bhjc->bhic", mask / mask.sum(1, keepdims=True), v.astype(np.float64))
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_first_row_is_first_value():
    q, k, v = rand((1, 2, 9, 4), 15), rand((1, 2, 9, 4), 16), rand((1, 2, 9, 4), 17)
    got = oracle.attn_full(q, k, v, 5, 2, 1.0)
    np.testing.assert_array_equal(got[:, :, 0, :], v[:, :, 0, :].astype(np.float64))


def test_attention_row_weights_sum_to_one():
    # "Attention Variants Compared" glossary: rows sum to 1
    rng = np.random.default_rng(18)
    n, d = 25, 6
    q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    mask = oracle.mask_dense(n, 4, 3)[n - 1]
    out, w, lse = oracle.attention_row(q, K, V, mask, 0.9)
    assert abs(w.sum() - 1.0) < 1e-14
    assert np.all(w[mask == 0] == 0) and np.all(w[mask == 1] > 0)
    np.testing.assert_allclose(out, w @ V.astype(np.float32).astype(np.float64), rtol=1e-13)


@pytest.mark.parametrize("n,tile", [(16, 4), (17, 4), (5, 1), (30, 7), (12, 12), (9, 50)])
def test_tiled_softmax_equals_direct(n, tile):
    rng = np.random.default_rng(19 + n)
    q = rng.standard_normal(8) * 3
    K, V = rng.standard_normal((n, 8)), rng.standard_normal((n, 5))
    direct, _, _ = oracle.attention_row(q, K, V, np.ones(n, np.uint8), 0.6)
    tiled = oracle.tiled_softmax_dot(q, K, V, 0.6, tile=tile)
    np.testing.assert_allclose(tiled, direct, rtol=1e-12, atol=1e-13)
    q32, K32, V32 = (x.astype(np.float32) for x in (q, K, V))
    want = sdpa64(q32[None, None, None], K32[None, None], V32[None, None], 0.6)[0, 0, 0]
    np.testing.assert_allclose(tiled, want, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# differential attention
# --------------------------------------------------------------------------

def test_diff_matches_two_sdpa_maps():
    B, H, N, d, dv, w = 1, 4, 37, 8, 16, 9
    q1, k1, q2, k2 = (rand((B, H, N, d), 20 + i) for i in range(4))
    v = rand((B, H, N, dv), 24)
    got = oracle.diff_full(q1, k1, q2, k2, v, w, 0, 0.125, 0.5)
    mask = oracle.mask_dense(N, w, 0)
    want = sdpa64(q1, k1, v, 0.125, mask) - 0.5 * sdpa64(q2, k2, v, 0.125, mask)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_diff_special_cases():
    B, H, N, d, dv, w = 1, 2, 20, 8, 8, 5
    q1, k1, q2, k2 = (rand((B, H, N, d), 30 + i) for i in range(4))
    v = rand((B, H, N, dv), 34)
    single = oracle.attn_full(q1, k1, v, w, 0, 0.3)
    np.testing.assert_allclose(oracle.diff_full(q1, k1, q2, k2, v, w, 0, 0.3, 0.0), single,
                               rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(oracle.diff_full(q1, k1, q1, k1, v, w, 0, 0.3, 0.5), 0.5 * single,
                               rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# Longformer: dilated window and global tokens
# --------------------------------------------------------------------------

def test_dilated_row_counts_closed_form():
    # "Learn: Sparse & Sliding-Window Attention" §3b: every dil-th key, the
    # same budget of w keys: row i attends min(w, floor(i/dil) + 1) keys
    for n in (1, 7, 40):
        for w in (1, 3, 8):
            for dil in (1, 2, 3, 7):
                total, rows = oracle.count_nonmasked(n, w, 0, dil, 0)
                want = [min(w, i // dil + 1) for i in range(n)]
                np.testing.assert_array_equal(rows, want, err_msg=str((n, w, dil)))
                assert total == sum(want)


@pytest.mark.parametrize("N,w,dil", [(30, 4, 3), (41, 6, 2), (25, 30, 4), (33, 1, 5)])
def test_dilated_window_is_plain_window_on_residue_classes(N, w, dil):
    # rows i = r (mod dil) attend keys of the same residue class only, the w
    # nearest: a plain window of w on the subsequence r, r+dil, r+2dil, ...
    q, k, v = rand((1, 4, N, 8), 80), rand((1, 2, N, 8), 81), rand((1, 2, N, 8), 82)
    got = oracle.attn_full(q, k, v, w, 0, 0.4, dilation=dil)
    for r in range(dil):
        qs, ks, vs = q[:, :, r::dil], k[:, :, r::dil], v[:, :, r::dil]
        n = qs.shape[2]
        band = np.tril(np.ones((n, n), dtype=np.uint8)) - np.tril(np.ones((n, n), dtype=np.uint8), -w)
        want = sdpa64(qs, ks, vs, 0.4, mask=band)
        np.testing.assert_allclose(got[:, :, r::dil], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("N,w,g,s", [(30, 5, 3, 0), (30, 5, 9, 0), (40, 6, 2, 7), (20, 3, 20, 0),
                                     (26, 4, 1, 0)])
def test_global_tokens_by_key_gather(N, w, g, s):
    # §3b global tokens under the causal order: row i < g attends every j <= i;
    # every other row attends the global keys j < g, its window, and (with a
    # stride) the multiples of s -- checked row by row against SDPA over the
    # explicitly gathered key set
    B, Hq, Hkv, d = 1, 2, 1, 8
    q, k, v = rand((B, Hq, N, d), 83), rand((B, Hkv, N, d), 84), rand((B, Hkv, N, d), 85)
    got = oracle.attn_full(q, k, v, w, s, 0.3, n_global=g)
    for i in range(N):
        if i < g:
            keep = list(range(i + 1))
        else:
            keep = sorted(set(range(g)) | set(range(max(0, i - w + 1), i + 1)) |
                          (set(range(0, i + 1, s)) if s else set()))
        want = sdpa64(q[:, :, i:i + 1], k[:, :, keep], v[:, :, keep], 0.3)[:, :, 0]
        np.testing.assert_allclose(got[:, :, i], want, rtol=1e-12, atol=1e-12)


def test_global_count_closed_form():
    # g <= w: the global rows lie inside their own windows, and key j < g adds
    # the rows i >= j + w that the window does not reach: N - j - w of them
    for n in (5, 20, 64):
        for w in (1, 4, 9):
            for g in range(0, w + 1):
                total, _ = oracle.count_nonmasked(n, w, 0, 1, g)
                want = band_count(n, w) + sum(max(0, n - j - w) for j in range(g))
                assert total == want, (n, w, g)
    # g >= n: the full causal triangle
    assert oracle.count_nonmasked(12, 2, 0, 1, 12)[0] == 12 * 13 // 2


@pytest.mark.parametrize("L,W,S", [(40, 8, 4), (9, 8, 4), (30, 16, 2)])
def test_global_prefill_row_is_sink_decode(L, W, S):
    # the newest row of a prefill with S global tokens attends the same keys
    # as a decode step with S sink slots and a ring of W ("Learn: Sparse &
    # Sliding-Window Attention" §4): two separate paths of the oracle
    B, Hq, Hkv, d = 1, 4, 2, 8
    kseq, vseq = rand((B, Hkv, L, d), 86), rand((B, Hkv, L, d), 87)
    qseq = rand((B, Hq, L, d), 88)
    rows = [(b * Hq + h) * L + L - 1 for b in range(B) for h in range(Hq)]
    pre = oracle.attn_rows(qseq, kseq, vseq, W, 0, 0.4, rows, n_global=S)
    kr, vr = ring_from_sequence(kseq, vseq, L, W)
    got = oracle.decode(qseq[:, :, L - 1], kr, vr, [L], 0.4, k_sink=kseq[:, :, :S].copy(),
                        v_sink=vseq[:, :, :S].copy())
    np.testing.assert_allclose(got.reshape(-1, d), pre, rtol=1e-12, atol=1e-12)


def test_prefix_only_tiles_attended_by_every_row():
    # stride and global columns in a prefix-only tile are open in every row
    n, w, s, g, dil, bm, bn = 120, 6, 13, 5, 2, 16, 8
    mask = oracle.mask_dense(n, w, s, dil, g)
    t = oracle.tile_list(n, w, s, bm, bn, dilation=dil, n_global=g)
    for qt in range(t["num_q_tiles"]):
        for e in range(t["row_ptr"][qt], t["row_ptr"][qt + 1]):
            if t["kind"][e] != 2:
                continue
            kt = t["kv_tile"][e]
            cols = [j for j in range(kt * bn, min(n, (kt + 1) * bn)) if j < g or j % s == 0]
            rows = range(qt * bm, min(n, (qt + 1) * bm))
            assert cols and all(mask[i, j] for i in rows for j in cols)


# --------------------------------------------------------------------------
# decode over a rolling window
# --------------------------------------------------------------------------

def ring_from_sequence(kseq, vseq, L, W):
    """Place positions max(0, L-W) .. L-1 of [B, Hkv, L, d] sequences into a
    ring of W slots at slot p mod W (slots never written stay random)."""
    B, Hkv, _, d = kseq.shape
    kr = rand((B, Hkv, W, d), 99)
    vr = rand((B, Hkv, W, vseq.shape[3]), 98)
    for p in range(max(0, L - W), L):
        kr[:, :, p % W] = kseq[:, :, p]
        vr[:, :, p % W] = vseq[:, :, p]
    return kr, vr


@pytest.mark.parametrize("L,W", [(1, 8), (5, 8), (8, 8), (13, 8), (30, 8), (64, 16)])
def test_decode_is_last_row_of_window_attention(L, W):
    B, Hq, Hkv, d = 2, 4, 2, 8
    kseq, vseq = rand((B, Hkv, L, d), 40), rand((B, Hkv, L, d), 41)
    qlast = rand((B, Hq, d), 42)
    kr, vr = ring_from_sequence(kseq, vseq, L, W)
    got = oracle.decode(qlast, kr, vr, np.full(B, L), 0.4)
    lo = max(0, L - W)
    want = sdpa64(qlast[:, :, None], kseq[:, :, lo:L], vseq[:, :, lo:L], 0.4)[:, :, 0]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # the same row of a prefill over the whole sequence
    qseq = rand((B, Hq, L, d), 43)
    qseq[:, :, L - 1] = qlast
    pre = oracle.attn_rows(qseq, kseq, vseq, W, 0, 0.4,
                           [(b * Hq + h) * L + L - 1 for b in range(B) for h in range(Hq)])
    np.testing.assert_allclose(got.reshape(-1, d), pre, rtol=1e-12, atol=1e-12)


def test_decode_ring_rotation_invariance():
    # same window contents, stored at two different rotations of the ring
    B, Hq, Hkv, d, W = 1, 2, 1, 8, 8
    kseq, vseq = rand((B, Hkv, 40, d), 44), rand((B, Hkv, 40, d), 45)
    q = rand((B, Hq, d), 46)
    a = oracle.decode(q, *ring_from_sequence(kseq[:, :, 3:], vseq[:, :, 3:], 20, W), [20], 0.5)
    b = oracle.decode(q, *ring_from_sequence(kseq[:, :, :], vseq[:, :, :], 23, W), [23], 0.5)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("L,W,S", [(3, 8, 4), (12, 8, 4), (40, 8, 4), (40, 8, 0), (20, 16, 4)])
def test_decode_with_sinks(L, W, S):
    # "Learn: Sparse & Sliding-Window Attention" §4: first S tokens + last W
    B, Hq, Hkv, d = 1, 4, 2, 8
    kseq, vseq = rand((B, Hkv, L, d), 47), rand((B, Hkv, L, d), 48)
    q = rand((B, Hq, d), 49)
    kr, vr = ring_from_sequence(kseq, vseq, L, W)
    ks = vs = None
    if S:
        # sink slot p holds position p; slots at or beyond L stay random
        ks, vs = rand((B, Hkv, S, d), 97), rand((B, Hkv, S, d), 96)
        ks[:, :, :min(S, L)] = kseq[:, :, :min(S, L)]
        vs[:, :, :min(S, L)] = vseq[:, :, :min(S, L)]
    got = oracle.decode(q, kr, vr, [L], 0.4, k_sink=ks, v_sink=vs)
    keep = sorted(set(range(min(S, L))) | set(range(max(0, L - W), L)))
    want = sdpa64(q[:, :, None], kseq[:, :, keep], vseq[:, :, keep], 0.4)[:, :, 0]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("L,W", [(1, 8), (6, 8), (8, 8), (29, 8), (40, 16)])
def test_diff_decode_is_last_row_of_diff_prefill(L, W):
    # decode of the newest token equals the last row of the masked two-map
    # prefill over the whole sequence (window of that row = the ring)
    B, H, d, dv = 2, 3, 8, 12
    k1seq, k2seq = rand((B, H, L, d), 60), rand((B, H, L, d), 61)
    vseq = rand((B, H, L, dv), 62)
    q1seq, q2seq = rand((B, H, L, d), 63), rand((B, H, L, d), 64)
    k1r, vr = ring_from_sequence(k1seq, vseq, L, W)
    k2r, _ = ring_from_sequence(k2seq, vseq, L, W)
    got = oracle.diff_decode(q1seq[:, :, L - 1], k1r, q2seq[:, :, L - 1], k2r, vr, np.full(B, L),
                             0.3, 0.7)
    rows = [(b * H + h) * L + L - 1 for b in range(B) for h in range(H)]
    want = oracle.diff_rows(q1seq, k1seq, q2seq, k2seq, vseq, W, 0, 0.3, 0.7, rows)
    np.testing.assert_allclose(got.reshape(-1, dv), want, rtol=1e-12, atol=1e-12)


def test_diff_decode_special_cases():
    B, Hq, Hkv, W, d, dv = 2, 4, 2, 8, 8, 8
    q1, q2 = rand((B, Hq, d), 65), rand((B, Hq, d), 66)
    k1, k2 = rand((B, Hkv, W, d), 67), rand((B, Hkv, W, d), 68)
    v = rand((B, Hkv, W, dv), 69)
    L = np.array([5, 20])
    # the same map twice: (1 - lambda) times one map, by brute force over the
    # attended slots (slots 0..4 of sequence 0, every slot of sequence 1)
    got = oracle.diff_decode(q1, k1, q1, k1, v, L, 0.5, 0.25)
    for b, n in ((0, 5), (1, W)):
        G = Hq // Hkv
        for h in range(Hq):
            kk, vv = k1[b, h // G, :n].astype(np.float64), v[b, h // G, :n].astype(np.float64)
            s = kk @ q1[b, h].astype(np.float64) * 0.5
            p = np.exp(s - s.max())
            want = 0.75 * (p / p.sum()) @ vv
            np.testing.assert_allclose(got[b, h], want, rtol=1e-12, atol=1e-12)
    # lambda = 0: the first map alone; a sequence with no tokens gives zeros
    L0 = np.array([0, 20])
    z = oracle.diff_decode(q1, k1, q2, k2, v, L0, 0.5, 0.0)
    assert np.all(z[0] == 0)
    np.testing.assert_allclose(z[1], oracle.decode(q1, k1, v, L0, 0.5)[1], rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# counting helpers and inputs
# --------------------------------------------------------------------------

def test_nsa_key_count_printed_value():
    # "Attention Variants Compared": 32 + 128 + 128 = 288 keys at 1024 tokens,
    # l 32, k 4, w 128, "3.5x fewer"
    assert oracle.count_nsa(1024, 32, 4, 128) == 288
    assert 1024 / oracle.count_nsa(1024, 32, 4, 128) >= 3.5


def test_kv_cache_bytes_worked_example():
    """The 128K-token example of "Exploring Attention Variants" (80 layers, 8
    KV heads, head dimension 128, 131,072 positions, 2-byte elements): K and
    V at 80 x 8 x 128 = 81,920 elements per position each, 2 bytes per
    element, 131,072 = 2^17 positions -- 81,920 x 4 x 2^17 bytes = 40 GiB
    exactly; a 4,096-token window keeps 4096/131072 = 1/32 of it, 1.25 GiB.
    (The page's own printed figures, about 17 GB and 2.8 GB and "up to 6x",
    cannot both hold under the linear window scaling the same page states:
    2.8/17 is not 4096/131072.  They are left unpinned.)"""
    full = oracle.kv_cache_bytes(131072, 80, 8, 128)
    assert full == 40 * 2 ** 30
    assert oracle.kv_cache_bytes(4096, 80, 8, 128) == 5 * 2 ** 28
    assert abs(2.8 / 17 - 4096 / 131072) > 0.1


def test_kv_cache_bytes_rolling_window_and_sinks():
    """Learn: Sparse & Sliding-Window Attention, §6 "FLOPs & memory": dense
    decode keeps every past position (the cache grows with s), a rolling
    window keeps the last w whatever s is, StreamingLLM keeps k sinks plus
    the last w.  Bytes are additive over positions and proportional to the
    element size; a single element of K and one of V is 2 x dtype bytes."""
    L, H, d = 2, 3, 5
    assert oracle.kv_cache_bytes(1, 1, 1, 1, dtype=1) == 2
    assert oracle.kv_cache_bytes(1, 1, 1, 1, dtype=4) == 8
    one = oracle.kv_cache_bytes(1, L, H, d)
    for s_, w, k in ((10, 4, 2), (100, 16, 4), (3, 8, 1)):
        # dense: every one of the s positions; grows by one position per token
        assert oracle.kv_cache_bytes(s_, L, H, d) == s_ * one
        assert oracle.kv_cache_bytes(s_ + 1, L, H, d) - oracle.kv_cache_bytes(s_, L, H, d) == one
        # rolling window: min(s, w) positions, the same for every s >= w
        held = [oracle.kv_cache_bytes(min(t, w), L, H, d) for t in range(w, w + 50)]
        assert len(set(held)) == 1 and held[0] == w * one
        # sinks plus window: k + w positions
        assert oracle.kv_cache_bytes(k + w, L, H, d) == (k + w) * one
    # the elements of one position: a key and a value vector per layer and head
    assert oracle.kv_cache_bytes(1, L, H, d, dtype=1) == 2 * L * H * d


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(50).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0]  # ties to even
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(synth.round_bf16(x), want)


def test_workload_inputs_are_seeded():
    cfg = synth.workload("tiny_swa_f32")
    a = synth.prefill_inputs(cfg)
    b = synth.prefill_inputs(cfg)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert a[0].shape == (1, 2, 256, 32) and a[0].dtype == np.float32
