"""Benchmark of the masked-attention hot path on one MI355X.

Prints ONE JSON line.  The timed step is one masked-attention forward of the
sliding-window prefill workload (B=1, Hq=32, Hkv=8, N=8192, d=128, W=1024,
bf16) with the block mask built once beforehand, as the method builds it
once per shape.  `value` is unmasked TFLOP/s: 4*d FLOPs per attended cell
(2d for Q K^T, 2d for P V), counted over attended cells only.

The same run also measures, each on its own seeded synthetic inputs:
  decode     rolling-window decode, 64 sequences x ring 4096, Hq=32, Hkv=8,
             d=128 (GB/s over the algorithmic bytes: the K and V window, q and
             out, each once; two independent ring sets alternate so no
             iteration finds the previous one's data in cache)
  sink_decode  the same plus 4 sink slots per (sequence, key/value head)
  diff_decode  differential decode, 32 sequences x ring 4096, H=16, d=64 per
             map, dv=128 (both K rings and the one V ring, each read once)
  strided    local+strided prefill, B=2, H=16, N=16384, d=64, W=256, s=128
  global     the prefill workload plus 64 global tokens (Longformer)
  dilated    the prefill workload with 512 window keys at dilation 2
  diff       differential attention, B=1, H=16, N=4096, d=64/dv=128, W=1024
  tiny_f32   the small fp32 window problem (latency only)
  mask_build block-mask build for the prefill workload
and times the fp64 CPU oracle on a bounded sample of prefill rows
(cpu_baseline), which also yields a parity check of those rows.

Kernel times come from HIP events recorded on the stream the kernels run on.
Each workload is warmed up for at least --warm-seconds (default 0.5 s) and --warmup calls
before its timed calls, so the GPU clock has settled.
"""
import argparse
import concurrent.futures
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "unmasked TFLOP/s, SWA prefill N=8K W=1K bf16 (+ decode KV GB/s) on 1 GPU"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def band_cells(n, w):
    return n * (n + 1) // 2 if w >= n else n * w - w * (w - 1) // 2


def cells_of(cfg):
    """Attended cells per (batch, head) from the closed forms of the mask."""
    n, w, s = cfg["N"], cfg["window"], cfg["stride"]
    dil, g = cfg.get("dilation", 1), cfg.get("n_global", 0)
    if dil > 1 or g > 0:
        # per row: the (dilated) window holds min(w, i // dil + 1) keys; the
        # global columns add the keys j < g left of the window span
        if s:
            raise ValueError("no closed form here for a stride with dilation or global tokens")
        i = np.arange(n, dtype=np.int64)
        span = (w - 1) * dil
        c = np.minimum(w, i // dil + 1)
        if g > 0:
            if dil > 1:
                raise ValueError("no closed form here for dilation with global tokens")
            c = c + np.maximum(0, np.minimum(g, i - span))
        return int(c.sum())
    c = band_cells(n, w)
    if s > 0 and w < n:
        t = n - w
        q, r = divmod(t, s)
        c += t + s * q * (q - 1) // 2 + r * q
    return c


WARM_S = 0.5


def timed(fn, steps, warmup, torch, min_warm_s=None):
    """Run fn `warmup` times and, if that took less than min_warm_s seconds,
    keep warming until it has (clocks settle under sustained load), then time
    `steps` calls; return (ms per call by wall clock, ms per call by HIP events
    on the current stream)."""
    if min_warm_s is None:
        min_warm_s = WARM_S
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(10):
            fn(0)
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        fn(i)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps


def dev(x, torch, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def kernel_build_sha(kernel_src):
    """Hash of a kernel's source together with the build script (its compiler
    flags), the key under which its measured traffic is stored."""
    h = hashlib.sha256()
    for f in (kernel_src, os.path.join(ROOT, "sparse_masked_transformer_amd", "build.py")):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_record(kernel_src, key):
    """HBM traffic per launch measured with rocprofv3 counters, if neither the
    kernel source nor the build flags have changed since (null otherwise)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(key)
    if not rec:
        return None
    return rec["bytes_per_launch"] if rec.get("kernel_sha256") == kernel_build_sha(kernel_src) else None


def cpu_baseline(q, k, v, cfg, out_gpu, budget_s, threads):
    """Time the oracle on a seeded sample of rows; compare those rows too."""
    import oracle
    B, Hq, N, d = q.shape
    rng = np.random.default_rng(99)
    total = B * Hq * N
    # per-row cost probe on one thread
    probe = rng.choice(total, size=16, replace=False)
    t0 = time.perf_counter()
    oracle.attn_rows(q, k, v, cfg["window"], cfg["stride"], cfg["scale"], probe)
    per_row = (time.perf_counter() - t0) / len(probe)
    n_rows = int(max(64, min(total, budget_s * threads / max(per_row, 1e-6))))
    rows = np.sort(rng.choice(total, size=n_rows, replace=False))
    chunks = np.array_split(rows, threads * 4)
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda r: oracle.attn_rows(q, k, v, cfg["window"], cfg["stride"],
                                                       cfg["scale"], r), chunks))
    dt = time.perf_counter() - t0
    want = np.concatenate(parts)
    i = rows % N
    w = cfg["window"]
    keys = np.minimum(i + 1, w)  # no stride pattern in this workload
    flops = float(np.sum(4.0 * d * keys))
    err = float(np.max(np.abs(out_gpu.reshape(-1, d)[rows] - want)))
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{n_rows} of {total} rows of the same workload (seeded uniform), "
                       f"fp64 C oracle, {dt:.1f} s on {threads} threads",
                seconds=round(dt, 3), max_abs_err_vs_gpu=err)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="minimum warm-up time per workload (0 for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "sink_decode", "diff_decode", "strided",
                                       "global", "dilated", "diff", "tiny", "copy"], default=None,
                    help="time one workload only (for profiler runs); `copy` times a plain "
                         "1 GiB device-to-device copy, the reference for HBM byte counters")
    args = ap.parse_args()
    global WARM_S
    WARM_S = args.warm_seconds
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU design is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not os.path.exists(os.path.join(ROOT, "sparse_masked_transformer_amd", "libswa.so")):
        subprocess.run([sys.executable, os.path.join(ROOT, "sparse_masked_transformer_amd", "build.py")],
                       check=True)
    import sparse_masked_transformer_amd as swa
    import synth

    torch.cuda.set_device(0)
    bf16 = torch.bfloat16
    res = {}
    K, W = args.steps, args.warmup

    if args.only == "copy":
        src = torch.empty(1 << 29, dtype=bf16, device="cuda").normal_()
        dst = torch.empty_like(src)
        wall_ms, ev_ms = timed(lambda i: dst.copy_(src), K, W, torch)
        nbytes = 2 * src.numel() * 2
        print(json.dumps({"only": "copy", "bytes_read": src.numel() * 2, "bytes_written": src.numel() * 2,
                          "us": round(ev_ms * 1e3, 2), "gbs": round(nbytes / (ev_ms * 1e-3) / 1e9, 1)}))
        return

    # ---- SWA prefill (the metric) --------------------------------------------
    cfg = synth.workload("swa_prefill_bf16")
    q, k, v = synth.prefill_inputs(cfg)
    qd, kd, vd = dev(q, torch, bf16), dev(k, torch, bf16), dev(v, torch, bf16)
    out = torch.empty_like(qd)
    torch.cuda.synchronize()
    mask = swa.swa_block_mask_build(cfg["N"], cfg["window"], cfg["stride"])
    mb_ms = timed(lambda i: swa.swa_block_mask_build(cfg["N"], cfg["window"], cfg["stride"], into=mask),
                  5, 2, torch)[1]
    cells = cells_of(cfg) * cfg["B"] * cfg["Hq"]
    flops = 4.0 * cfg["d"] * cells
    pf = lambda i: swa.swa_attn_fwd(qd, kd, vd, cfg["window"], cfg["stride"], cfg["scale"], mask, out=out)
    if args.only in (None, "prefill"):
        log(f"prefill: {K} steps after {W} warmup")
        wall_ms, ev_ms = timed(pf, K, W, torch)
        res["prefill"] = dict(wall_ms=wall_ms, event_ms=ev_ms, tflops=flops / (ev_ms * 1e-3) / 1e12)
        log(f"prefill: {ev_ms * 1e3:.1f} us/launch, {res['prefill']['tflops']:.1f} TFLOP/s")

    # ---- decode: window, window + sinks, differential ------------------------
    def time_decode(name, make_inputs, call, alg_bytes):
        """Two seeded input sets alternate, so no step reads a cache that the
        previous step left in L2/MALL."""
        sets = [make_inputs(s) for s in range(2)]
        fn = lambda i: call(sets[i & 1])
        log(f"{name}: {K} steps after {W} warmup")
        wall_ms, ev_ms = timed(fn, K, W, torch)
        gbs = alg_bytes / (ev_ms * 1e-3) / 1e9
        log(f"{name}: {ev_ms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
        del sets
        return dict(wall_ms=wall_ms, event_ms=ev_ms, alg_bytes=alg_bytes, gbs=gbs)

    def i32(x):
        return torch.from_numpy(x.astype(np.int32)).cuda()

    if args.only in (None, "decode"):
        dcfg = synth.workload("window_decode_bf16")
        B, Hq, Hkv, d, Wr = dcfg["B"], dcfg["Hq"], dcfg["Hkv"], dcfg["d"], dcfg["window"]

        def mk(s):
            ins = synth.decode_inputs(dict(dcfg, seed=dcfg["seed"] + 10 * s))
            return dict(q=dev(ins["q"], torch, bf16), k=dev(ins["k_ring"], torch, bf16),
                        v=dev(ins["v_ring"], torch, bf16), sl=i32(ins["seq_len"]))
        ws = torch.empty(max(1, swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, Wr)),
                         dtype=torch.uint8, device="cuda")
        dout = torch.empty((B, Hq, d), dtype=bf16, device="cuda")
        kv_bytes = 2 * B * Hkv * Wr * d * 2
        res["decode"] = time_decode(
            "decode", mk, lambda t: swa.swa_attn_decode(t["q"], t["k"], t["v"], t["sl"], dcfg["scale"],
                                                        workspace=ws, out=dout),
            kv_bytes + 2 * B * Hq * d * 2)
        res["decode"]["kv_gbs"] = kv_bytes / (res["decode"]["event_ms"] * 1e-3) / 1e9

    if args.only in (None, "sink_decode"):
        scfg_ = synth.workload("sink_decode_bf16")
        B, Hq, Hkv, d, Wr, S = (scfg_[x] for x in ("B", "Hq", "Hkv", "d", "window", "n_sink"))

        def mk(s):
            ins = synth.decode_inputs(dict(scfg_, seed=scfg_["seed"] + 10 * s))
            return {x: dev(ins[x], torch, bf16) for x in ("q", "k_sink", "v_sink", "k_ring", "v_ring")} | \
                dict(sl=i32(ins["seq_len"]))
        ws = torch.empty(max(1, swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, Wr, S)),
                         dtype=torch.uint8, device="cuda")
        dout = torch.empty((B, Hq, d), dtype=bf16, device="cuda")
        res["sink_decode"] = time_decode(
            "sink decode", mk,
            lambda t: swa.swa_attn_decode_sinks(t["q"], t["k_sink"], t["v_sink"], t["k_ring"], t["v_ring"],
                                                t["sl"], scfg_["scale"], workspace=ws, out=dout),
            2 * B * Hkv * (Wr + S) * d * 2 + 2 * B * Hq * d * 2)

    if args.only in (None, "diff_decode"):
        gcfg = synth.workload("diff_decode_bf16")
        B, Hq, Hkv, d, dv, Wr = (gcfg[x] for x in ("B", "Hq", "Hkv", "d", "dv", "window"))

        def mk(s):
            ins = synth.diff_decode_inputs(dict(gcfg, seed=gcfg["seed"] + 10 * s))
            return {x: dev(ins[x], torch, bf16) for x in ("q1", "k1_ring", "q2", "k2_ring", "v_ring")} | \
                dict(sl=i32(ins["seq_len"]))
        ws = torch.empty(max(1, swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, dv, Wr, 0, swa.SWA_OP_DIFF)),
                         dtype=torch.uint8, device="cuda")
        dout = torch.empty((B, Hq, dv), dtype=bf16, device="cuda")
        res["diff_decode"] = time_decode(
            "diff decode", mk,
            lambda t: swa.diff_attn_decode(t["q1"], t["k1_ring"], t["q2"], t["k2_ring"], t["v_ring"], t["sl"],
                                           gcfg["scale"], gcfg["lam"], workspace=ws, out=dout),
            B * Hkv * Wr * (2 * d + dv) * 2 + B * Hq * (2 * d + dv) * 2)

    # ---- local + strided prefill ----------------------------------------------
    if args.only in (None, "strided"):
        scfg = synth.workload("local_strided_bf16")
        sq, sk, sv = synth.prefill_inputs(scfg)
        sqd, skd, svd = dev(sq, torch, bf16), dev(sk, torch, bf16), dev(sv, torch, bf16)
        smask = swa.swa_block_mask_build(scfg["N"], scfg["window"], scfg["stride"], d=scfg["d"])
        sout = torch.empty_like(sqd)
        fn = lambda i: swa.swa_attn_fwd(sqd, skd, svd, scfg["window"], scfg["stride"], scfg["scale"],
                                        smask, out=sout)
        log("strided prefill")
        wall_ms, ev_ms = timed(fn, K, W, torch)
        sflops = 4.0 * scfg["d"] * cells_of(scfg) * scfg["B"] * scfg["Hq"]
        sbytes = 4 * sq.size * 2
        res["strided"] = dict(event_ms=ev_ms, tflops=sflops / (ev_ms * 1e-3) / 1e12,
                              gbs=sbytes / (ev_ms * 1e-3) / 1e9, alg_flops=sflops, alg_bytes=sbytes)
        del sqd, skd, svd, sout

    # ---- Longformer patterns: global tokens, dilated window ----------------------
    for key, wl in (("global", "global_prefill_bf16"), ("dilated", "dilated_prefill_bf16")):
        if args.only not in (None, key):
            continue
        xcfg = synth.workload(wl)
        xq, xk, xv = synth.prefill_inputs(xcfg)
        xqd, xkd, xvd = dev(xq, torch, bf16), dev(xk, torch, bf16), dev(xv, torch, bf16)
        del xq, xk, xv
        xmask = swa.swa_block_mask_build(xcfg["N"], xcfg["window"], 0, d=xcfg["d"],
                                         dilation=xcfg.get("dilation", 1),
                                         n_global=xcfg.get("n_global", 0))
        xout = torch.empty_like(xqd)
        fn = lambda i: swa.swa_attn_fwd(xqd, xkd, xvd, xcfg["window"], 0, xcfg["scale"], xmask, out=xout)
        log(f"{wl}")
        wall_ms, ev_ms = timed(fn, K, W, torch)
        xcells = cells_of(xcfg) * xcfg["B"] * xcfg["Hq"]
        res[key] = dict(event_ms=ev_ms, tflops=4.0 * xcfg["d"] * xcells / (ev_ms * 1e-3) / 1e12,
                        workload=wl)
        del xqd, xkd, xvd, xout

    # ---- differential attention ------------------------------------------------
    if args.only in (None, "diff"):
        fcfg = synth.workload("diff_bf16")
        fins = [dev(x, torch, bf16) for x in synth.diff_inputs(fcfg)]
        fmask = swa.swa_block_mask_build(fcfg["N"], fcfg["window"], 0, d=fcfg["d"], dv=fcfg["dv"],
                                         op=swa.SWA_OP_DIFF)
        fout = torch.empty((fcfg["B"], fcfg["Hq"], fcfg["N"], fcfg["dv"]), dtype=bf16, device="cuda")
        fn = lambda i: swa.diff_attn_fwd(*fins, fcfg["window"], 0, fcfg["scale"], fcfg["lam"], fmask,
                                         out=fout)
        log("differential attention")
        wall_ms, ev_ms = timed(fn, K, W, torch)
        fcells = cells_of(fcfg) * fcfg["B"] * fcfg["Hq"]
        per_cell = 2 * (2 * fcfg["d"] + 2 * fcfg["dv"])   # two maps, each QK^T and PV
        res["diff"] = dict(event_ms=ev_ms, tflops=per_cell * fcells / (ev_ms * 1e-3) / 1e12,
                           tflops_formula=(2 * 2 * fcfg["d"] + 2 * fcfg["dv"]) * fcells / (ev_ms * 1e-3) / 1e12)
        del fins, fout

    # ---- tiny fp32 --------------------------------------------------------------
    if args.only in (None, "tiny"):
        tcfg = synth.workload("tiny_swa_f32")
        tq, tk, tv = (dev(x, torch, torch.float32) for x in synth.prefill_inputs(tcfg))
        tmask = swa.swa_block_mask_build(tcfg["N"], tcfg["window"], 0, dtype=torch.float32, d=tcfg["d"])
        tout = torch.empty_like(tq)
        fn = lambda i: swa.swa_attn_fwd(tq, tk, tv, tcfg["window"], 0, tcfg["scale"], tmask, out=tout)
        res["tiny_f32"] = dict(event_ms=timed(fn, K, W, torch)[1])

    if "prefill" not in res:
        print(json.dumps({"only": args.only, "results": res}))
        return

    # ---- CPU baseline (oracle) + parity of the sampled rows ------------------------
    cpu = None
    if not args.no_cpu_baseline:
        threads = max(1, min(16, os.cpu_count() or 1))
        log(f"cpu baseline: ~{args.cpu_seconds:.0f} s of oracle work on {threads} threads")
        out_host = out.float().cpu().numpy()
        cpu = cpu_baseline(q, k, v, cfg, out_host, args.cpu_seconds, threads)

    p = res["prefill"]
    src = os.path.join(ROOT, "sparse_masked_transformer_amd", "csrc", "fwd_bf16.hip")
    line = {
        "metric": METRIC,
        "value": round(p["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(p["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "swa_prefill_bf16", "B": cfg["B"], "Hq": cfg["Hq"], "Hkv": cfg["Hkv"],
                   "N": cfg["N"], "d": cfg["d"], "window": cfg["window"], "stride": cfg["stride"],
                   "attended_cells": cells, "gflop_per_step": round(flops / 1e9, 3)},
        "roofline": {"bound": "mfma", "kernel": "fwd_bf16_kernel<128,128,0>",
                     "achieved": round(p["tflops"], 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(p["tflops"] / PEAK_BF16_TFLOPS, 4),
                     "avg_launch_us": round(p["event_ms"] * 1e3, 2),
                     "traffic": traffic_record(src, "fwd_bf16_swa_prefill")},
        "cpu_baseline": cpu,
        "mask_build_us": round(mb_ms * 1e3, 2),
    }
    if "decode" in res:
        dd = res["decode"]
        dsrc = os.path.join(ROOT, "sparse_masked_transformer_amd", "csrc", "decode_bf16.hip")
        line["decode"] = {"workload": "window_decode_bf16", "value": round(dd["gbs"], 1), "unit": "GB/s",
                          "kv_gbs": round(dd["kv_gbs"], 1), "us_per_step": round(dd["event_ms"] * 1e3, 2),
                          "roofline": {"bound": "hbm", "kernel": "decode_kernel<128,128,1,true,false>",
                                       "achieved": round(dd["gbs"], 1),
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": round(dd["gbs"] / PEAK_HBM_GBS, 4),
                                       "traffic": traffic_record(dsrc, "decode_bf16_window")}}
    for key, wl in (("sink_decode", "sink_decode_bf16"), ("diff_decode", "diff_decode_bf16")):
        if key in res:
            dd = res[key]
            line[key] = {"workload": wl, "value": round(dd["gbs"], 1), "unit": "GB/s",
                         "us_per_step": round(dd["event_ms"] * 1e3, 2),
                         "roofline": {"bound": "hbm", "achieved": round(dd["gbs"], 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(dd["gbs"] / PEAK_HBM_GBS, 4)}}
    if "strided" in res:
        s = res["strided"]
        t_hbm = s["alg_bytes"] / (PEAK_HBM_GBS * 1e9)
        t_mfma = s["alg_flops"] / (PEAK_BF16_TFLOPS * 1e12)
        line["strided"] = {"workload": "local_strided_bf16", "tflops": round(s["tflops"], 2),
                           "gbs": round(s["gbs"], 1), "us": round(s["event_ms"] * 1e3, 2),
                           "roofline_frac": round(max(t_hbm, t_mfma) / (s["event_ms"] * 1e-3), 4),
                           "bound": "hbm" if t_hbm > t_mfma else "mfma"}
    for key in ("global", "dilated"):
        if key in res:
            x = res[key]
            line[key] = {"workload": x["workload"], "tflops": round(x["tflops"], 2),
                         "us": round(x["event_ms"] * 1e3, 2), "bound": "mfma",
                         "roofline_frac": round(x["tflops"] / PEAK_BF16_TFLOPS, 4)}
    if "diff" in res:
        f = res["diff"]
        line["diff"] = {"workload": "diff_bf16", "tflops": round(f["tflops"], 2),
                        "tflops_512_per_cell": round(f["tflops_formula"], 2),
                        "us": round(f["event_ms"] * 1e3, 2),
                        "roofline_frac": round(f["tflops"] / PEAK_BF16_TFLOPS, 4)}
    if "tiny_f32" in res:
        line["tiny_f32_us"] = round(res["tiny_f32"]["event_ms"] * 1e3, 2)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
