"""GPU test of swa_attn_decode_noalloc, the decode entry point that allocates
nothing: its split partials live in the library's static per-GPU scratch
instead of a caller's workspace.  Its output must equal swa_attn_decode's
(same kernels, same inputs) bit for bit, on two calls in a row, the second
smaller, so a stale partial left by the first call would show.  Both calls
split the ring across workgroups, so the scratch is really used.
"""
import math

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_masked_transformer_amd as m
    return m


def _inputs(B, Hq, Hkv, W, seq_len, seed, dtype):
    cfg = dict(dtype="bf16" if dtype == torch.bfloat16 else "f32", B=B, Hq=Hq, Hkv=Hkv, window=W, d=128,
               dv=128, position=0, n_sink=0, scale=1.0 / math.sqrt(128), seed=seed)
    ins = synth.decode_inputs(cfg, seq_len=seq_len)
    dev = lambda x: torch.from_numpy(x).to(dtype).cuda()
    sl = torch.from_numpy(ins["seq_len"].astype(np.int32)).cuda()
    return dev(ins["q"]), dev(ins["k_ring"]), dev(ins["v_ring"]), sl, cfg["scale"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_equals_workspace_decode(swa, dtype):
    # (B, Hq, Hkv, window, lengths): a full ring past its wrap, a ring still
    # filling and an empty sequence; then a smaller call with fewer splits
    cases = [(3, 8, 2, 4096, [5000, 1500, 0], 31), (1, 4, 1, 1000, [700], 32)]
    for B, Hq, Hkv, W, lens, seed in cases:
        need = swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, 128, W)
        assert 0 < need <= swa.SWA_DECODE_SCRATCH_BYTES
        q, k, v, sl, scale = _inputs(B, Hq, Hkv, W, lens, seed, dtype)
        want = swa.swa_attn_decode(q, k, v, sl, scale)
        got = torch.full_like(q, float("nan"))
        swa.swa_attn_decode_noalloc(q, k, v, sl, scale, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"B={B} Hq={Hq} Hkv={Hkv} W={W}: max diff " \
                                       f"{(got.float() - want.float()).abs().max().item()}"


def test_noalloc_without_split(swa):
    """A call that needs no scratch (one split per sequence) also matches."""
    B, Hq, Hkv, W = 64, 32, 8, 4096
    assert swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, 128, W) == 0
    q, k, v, sl, scale = _inputs(B, Hq, Hkv, W, [W + 3] * B, 33, torch.bfloat16)
    want = swa.swa_attn_decode(q, k, v, sl, scale)
    got = torch.empty_like(q)
    swa.swa_attn_decode_noalloc(q, k, v, sl, scale, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_noalloc_rejects_beyond_scratch(swa):
    B, Hq, Hkv, W = 1, 1024, 1, 4096
    assert swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, 128, W) > swa.SWA_DECODE_SCRATCH_BYTES
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, W, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(swa.SwaError) as e:
        swa.swa_attn_decode_noalloc(q, k, k, None, 0.1, torch.empty_like(q), N=10)
    assert e.value.status == swa.SWA_ERR_SCRATCH
