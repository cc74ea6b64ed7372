"""The library holds no mutable state between calls, so calls on different
streams may overlap as long as their outputs differ.  Here prefill,
differential attention and decode run concurrently on two streams (default
priority), issued in interleaved order and from two host threads, and each
result is checked against the fp64 oracle."""
import math
import threading

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def swa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_masked_transformer_amd as m
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def problems(swa):
    """Four independent problems, inputs on the device, each with its oracle:
    a strided prefill (the HIP kernel), a grouped-query window prefill and a
    differential prefill (the generated persistent kernels), a decode."""
    pcfg = dict(dtype="bf16", B=1, Hq=8, Hkv=2, N=1500, d=128, dv=128, window=200, stride=37,
                scale=1.0 / math.sqrt(128), seed=301)
    q, k, v = synth.prefill_inputs(pcfg)
    pmask = swa.swa_block_mask_build(pcfg["N"], pcfg["window"], pcfg["stride"], d=128)
    pin = (dev(q), dev(k), dev(v))
    pwant = oracle.attn_full(q, k, v, pcfg["window"], pcfg["stride"], pcfg["scale"])

    gcfg = dict(dtype="bf16", B=2, Hq=16, Hkv=4, N=2100, d=128, dv=128, window=300, stride=0,
                scale=1.0 / math.sqrt(128), seed=304)
    gq, gk, gv = synth.prefill_inputs(gcfg)
    gmask = swa.swa_block_mask_build(gcfg["N"], gcfg["window"], 0, d=128)
    gin = (dev(gq), dev(gk), dev(gv))
    gwant = oracle.attn_full(gq, gk, gv, gcfg["window"], 0, gcfg["scale"])

    fcfg = dict(dtype="bf16", B=1, Hq=4, Hkv=4, N=900, d=64, dv=128, window=150, stride=0,
                scale=0.125, lam=0.5, seed=302)
    fins = synth.diff_inputs(fcfg)
    fmask = swa.swa_block_mask_build(fcfg["N"], fcfg["window"], 0, d=64, dv=128, op=swa.SWA_OP_DIFF)
    fin = tuple(dev(x) for x in fins)
    fwant = oracle.diff_full(*fins, fcfg["window"], 0, fcfg["scale"], fcfg["lam"])

    dcfg = dict(dtype="bf16", B=8, Hq=16, Hkv=4, window=700, d=128, dv=128, position=0, n_sink=0,
                scale=1.0 / math.sqrt(128), seed=303)
    dins = synth.decode_inputs(dcfg, seq_len=[1, 50, 699, 700, 701, 1400, 3000, 333])
    din = (dev(dins["q"]), dev(dins["k_ring"]), dev(dins["v_ring"]),
           torch.from_numpy(dins["seq_len"].astype(np.int32)).cuda())
    dwant = oracle.decode(dins["q"], dins["k_ring"], dins["v_ring"], dins["seq_len"], dcfg["scale"])

    calls = {
        "prefill": (lambda: swa.swa_attn_fwd(*pin, pcfg["window"], pcfg["stride"], pcfg["scale"], pmask),
                    pwant),
        "gqa": (lambda: swa.swa_attn_fwd(*gin, gcfg["window"], 0, gcfg["scale"], gmask), gwant),
        "diff": (lambda: swa.diff_attn_fwd(*fin, fcfg["window"], 0, fcfg["scale"], fcfg["lam"], fmask),
                 fwant),
        "decode": (lambda: swa.swa_attn_decode(*din, dcfg["scale"]), dwant),
    }
    return calls


def check(outs, calls):
    for name, out in outs.items():
        err = float(np.max(np.abs(host(out) - calls[name][1])))
        assert err <= 2e-2, f"{name}: max-abs error {err}"


def test_two_streams_interleaved(swa):
    print("[case] prefill, grouped-query prefill, diff, decode on two streams, interleaved", flush=True)
    calls = problems(swa)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {}
    for rep in range(3):   # several rounds, so the streams' work overlaps
        with torch.cuda.stream(s1):
            outs["prefill"] = calls["prefill"][0]()
        with torch.cuda.stream(s2):
            outs["decode"] = calls["decode"][0]()
        with torch.cuda.stream(s1):
            outs["diff"] = calls["diff"][0]()
        with torch.cuda.stream(s2):
            outs["gqa"] = calls["gqa"][0]()
    torch.cuda.synchronize()
    check(outs, calls)


def test_two_host_threads(swa):
    print("[case] prefill, grouped-query prefill, diff and decode from four host threads", flush=True)
    calls = problems(swa)
    torch.cuda.synchronize()
    outs, errors = {}, []

    def run(name):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(3):
                    outs[name] = calls[name][0]()
            stream.synchronize()
        except Exception as e:   # reported below, on the main thread
            errors.append(f"{name}: {e!r}")

    threads = [threading.Thread(target=run, args=(n,)) for n in ("prefill", "decode", "diff", "gqa")]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    check(outs, calls)
