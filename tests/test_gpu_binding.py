"""The Python binding rejects tensors whose shape, dtype or device disagree
with the sizes it passes to the C ABI (the kernels would otherwise read or
write out of bounds); every rejected call raises before anything is launched.
A valid call after the rejections still runs."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_masked_transformer_amd as m
    return m


def t(*shape, dtype=torch.bfloat16):
    return torch.randn(*shape, device="cuda").to(dtype)


def test_fwd_rejects_mismatched_tensors(swa):
    B, Hq, Hkv, N, d, W = 1, 4, 2, 200, 64, 32
    q, k, v = t(B, Hq, N, d), t(B, Hkv, N, d), t(B, Hkv, N, d)
    mask = swa.swa_block_mask_build(N, W, 0, d=d)
    fwd = lambda **kw: swa.swa_attn_fwd(**{**dict(q=q, k=k, v=v, window=W, stride=0, scale=0.125,
                                                 mask=mask), **kw})
    with pytest.raises(ValueError):
        fwd(v=t(B, Hkv, N - 1, d))                   # one key row short
    with pytest.raises(ValueError):
        fwd(k=t(B, Hq, N, d))                        # head count differs from v
    with pytest.raises(TypeError):
        fwd(k=t(B, Hkv, N, d, dtype=torch.float32))  # another dtype
    with pytest.raises(ValueError):
        fwd(out=t(B, Hq, N, d // 2))
    with pytest.raises(TypeError):
        fwd(lse=torch.empty(B, Hq, N, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fwd(lse=torch.empty(B, Hq, N - 1, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fwd(q=t(Hq, N, d))                           # 3-D query
    with pytest.raises(ValueError):
        fwd(k=t(B, Hkv, d, N).transpose(2, 3))       # not contiguous
    with pytest.raises(ValueError):
        fwd(v=v.cpu())
    out = fwd()
    assert out.shape == q.shape and torch.isfinite(out.float()).all()


def test_diff_fwd_rejects_mismatched_tensors(swa):
    B, H, N, d, dv, W = 1, 2, 150, 64, 128, 40
    q1, k1, q2, k2, v = t(B, H, N, d), t(B, H, N, d), t(B, H, N, d), t(B, H, N, d), t(B, H, N, dv)
    mask = swa.swa_block_mask_build(N, W, 0, d=d, dv=dv, op=swa.SWA_OP_DIFF)
    call = lambda **kw: swa.diff_attn_fwd(**{**dict(q1=q1, k1=k1, q2=q2, k2=k2, v=v, window=W,
                                                    stride=0, scale=0.125, lam=0.5, mask=mask),
                                             **kw})
    with pytest.raises(ValueError):
        call(q2=t(B, H, N + 1, d))
    with pytest.raises(ValueError):
        call(k2=t(B, H, N, d // 2))
    with pytest.raises(ValueError):
        call(v=t(B, H, N - 5, dv))
    with pytest.raises(ValueError):
        call(out=t(B, H, N, d))                      # out has dv columns
    out = call()
    assert out.shape == (B, H, N, dv) and torch.isfinite(out.float()).all()


def test_decode_rejects_mismatched_tensors(swa):
    B, Hq, Hkv, W, d = 3, 8, 2, 96, 64
    q, kr, vr = t(B, Hq, d), t(B, Hkv, W, d), t(B, Hkv, W, d)
    sl = torch.tensor([5, 96, 500], dtype=torch.int32, device="cuda")
    call = lambda **kw: swa.swa_attn_decode(**{**dict(q=q, k_ring=kr, v_ring=vr, seq_len=sl,
                                                      scale=0.125), **kw})
    with pytest.raises(ValueError):
        call(v_ring=t(B, Hkv, W - 1, d))
    with pytest.raises(ValueError):
        call(k_ring=t(B + 1, Hkv, W, d))
    with pytest.raises(TypeError):
        call(seq_len=sl.to(torch.int64))
    with pytest.raises(ValueError):
        call(seq_len=sl[:2].contiguous())
    with pytest.raises(ValueError):
        call(out=t(B, Hq, d + 32))
    out = call()
    assert out.shape == q.shape and torch.isfinite(out.float()).all()


def test_decode_sinks_and_diff_decode_reject_mismatched_tensors(swa):
    B, Hq, Hkv, W, d, S = 2, 4, 2, 64, 64, 4
    q, kr, vr = t(B, Hq, d), t(B, Hkv, W, d), t(B, Hkv, W, d)
    ks, vs = t(B, Hkv, S, d), t(B, Hkv, S, d)
    sl = torch.tensor([10, 300], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        swa.swa_attn_decode_sinks(q, ks, t(B, Hkv, S - 1, d), kr, vr, sl, 0.125)
    with pytest.raises(ValueError):
        swa.swa_attn_decode_sinks(q, ks, vs, kr, t(B, Hkv, W, d // 2), sl, 0.125)
    out = swa.swa_attn_decode_sinks(q, ks, vs, kr, vr, sl, 0.125)
    assert torch.isfinite(out.float()).all()

    dv = 128
    q2, k2, v = t(B, Hq, d), t(B, Hkv, W, d), t(B, Hkv, W, dv)
    with pytest.raises(ValueError):
        swa.diff_attn_decode(q, kr, q2, t(B, Hkv, W, d // 2), v, sl, 0.125, 0.5)
    with pytest.raises(ValueError):
        swa.diff_attn_decode(q, kr, t(B, Hq + 1, d), k2, v, sl, 0.125, 0.5)
    with pytest.raises(ValueError):
        swa.diff_attn_decode(q, kr, q2, k2, v, sl, 0.125, 0.5, out=t(B, Hq, d))
    out = swa.diff_attn_decode(q, kr, q2, k2, v, sl, 0.125, 0.5)
    assert out.shape == (B, Hq, dv) and torch.isfinite(out.float()).all()
