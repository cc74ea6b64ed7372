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
  peaks      the sustained dense bf16 MFMA rate and HBM read rate of this GPU
             (include/swa_probe.h), and the vendor library's bf16 GEMM rate
             on random data, reported beside the published peaks (measured
             last: at full power they would lower the clock of what follows)
and times the fp64 CPU oracle on every configuration -- all rows of the tiny
problem and all 64 decode sequences, a seeded sample of rows of the prefill,
local+strided and differential workloads -- which also checks those outputs
against the GPU's (cpu_baseline).

Kernel times come from HIP events recorded on the stream the kernels run on:
a pair around the K back-to-back timed calls gives the per-call time that
the throughput figures use (K = 100 by default; the decode legs time at most
50), and a pair around each of K more calls gives the median isolated
latency, reported beside it.  ms_per_step is the wall clock over the K timed
prefill steps, bracketed by device synchronizations.
Each workload is warmed up for at least --warm-seconds (default 0.5 s) and
--warmup calls before its timed calls, so the GPU clock has settled.
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
    keep warming until it has (clocks settle under sustained load); then
      1. time `steps` calls back to back between two HIP events on the
         current stream (the stream the library launches on), bracketed by
         device synchronizations -- the throughput figure;
      2. time `steps` more calls one by one, each between its own event pair
         -- the median isolated latency (each call then also pays its own
         ramp-up and drain, which back-to-back calls overlap).
    Returns (ms per call by wall clock over 1., ms per call by the events of
    1., median ms per call of 2.)."""
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
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        fn(i)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return ((t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps,
            float(np.median([a.elapsed_time(b) for a, b in ev])))


def host_cpus():
    """Logical CPUs, the ones this process may run on, and the physical cores
    and sockets lscpu reports (None where it is unavailable)."""
    info = dict(logical_cpus=os.cpu_count(), affinity_cpus=len(os.sched_getaffinity(0)),
                physical_cores=None, sockets=None)
    try:
        out = subprocess.run(["lscpu", "-p=CORE,SOCKET"], capture_output=True, text=True, timeout=10).stdout
        pairs = {tuple(l.split(",")) for l in out.splitlines() if l and not l.startswith("#")}
        info["physical_cores"] = len(pairs)
        info["sockets"] = len({p[1] for p in pairs})
    except (OSError, subprocess.SubprocessError):
        pass
    return info


def dev(x, torch, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def kernel_build_sha(kernel_src):
    """Hash of a kernel's source (one path, or a list of the files it is
    generated from) together with the build script (its compiler flags),
    the key under which its measured traffic is stored."""
    h = hashlib.sha256()
    srcs = [kernel_src] if isinstance(kernel_src, str) else list(kernel_src)
    for f in srcs + [os.path.join(ROOT, "sparse_masked_transformer_amd", "build.py")]:
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


def decode_alg_bytes(cfg, n_sink=0):
    """Bytes one decode step must move: the K and V of the window (and of the
    sink slots) of every (sequence, key/value head) read once, q read and
    the output written once (2-byte elements)."""
    B, Hq, Hkv, W, d, dv = (cfg[x] for x in ("B", "Hq", "Hkv", "window", "d", "dv"))
    return B * Hkv * (W + n_sink) * (d + dv) * 2 + B * Hq * (d + dv) * 2


def diff_decode_alg_bytes(cfg):
    """Bytes one differential decode step must move: the two key windows and
    the one value window read once, q1, q2 read and the output written once."""
    B, Hq, Hkv, W, d, dv = (cfg[x] for x in ("B", "Hq", "Hkv", "window", "d", "dv"))
    return B * Hkv * W * (2 * d + dv) * 2 + B * Hq * (2 * d + dv) * 2


def row_keys(i, w, s):
    """Attended keys of query row i: the window's min(i + 1, w) plus the
    stride keys j <= i - w with j mod s == 0 (the mask's closed form)."""
    k = np.minimum(i + 1, w)
    if s:
        k = k + np.where(i >= w, (i - w) // s + 1, 0)
    return k


def oracle_rows(fn, rows, budget_s, threads, per_row_flop, out_gpu, d_out, seed):
    """Time fn(rows) (the fp64 oracle on a set of flat row indices) on a
    seeded sample of `rows` sized to about budget_s seconds on `threads`
    threads, and compare the sampled rows with the GPU's output."""
    rng = np.random.default_rng(seed)
    total = len(rows)
    probe = rng.choice(total, size=min(total, 16), replace=False)
    t0 = time.perf_counter()
    fn(rows[probe])
    per_row = (time.perf_counter() - t0) / len(probe)
    n = int(max(min(total, 64), min(total, budget_s * threads / max(per_row, 1e-9))))
    pick = np.sort(rng.choice(total, size=n, replace=False)) if n < total else np.arange(total)
    sel = rows[pick]
    chunks = [c for c in np.array_split(sel, threads * 4) if len(c)]
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(fn, chunks))
    dt = time.perf_counter() - t0
    want = np.concatenate(parts)
    err = float(np.max(np.abs(out_gpu.reshape(-1, d_out)[sel] - want)))
    return dict(rows=int(n), of=int(total), seconds=round(dt, 3), flop=float(np.sum(per_row_flop(sel))),
                max_abs_err_vs_gpu=err)


def measure_peaks(swa, torch):
    """Sustained dense bf16 MFMA rate and HBM read rate of this GPU (the
    probes of include/swa_probe.h), each the median of 10 calls."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    ops = torch.randn((512, 8), generator=gen, device="cuda").to(torch.bfloat16)
    wg, iters = 256, 4096
    out = torch.empty(wg * 512, dtype=torch.float32, device="cuda")
    _, _, ms = timed(lambda i: swa.swa_probe_mfma_bf16(ops, out, wg, iters), 10, 2, torch)
    flop = wg * 8 * iters * 32 * 32768
    buf = torch.randint(0, 1 << 30, (1 << 28,), dtype=torch.int32, device="cuda")   # 1 GiB
    swg = 1024
    sout = torch.empty(swg * 256, dtype=torch.int32, device="cuda")
    _, _, ms2 = timed(lambda i: swa.swa_probe_stream_read(buf, sout, swg), 10, 2, torch)
    nbytes = buf.numel() * 4
    del buf
    # the vendor library's dense bf16 GEMM on random data, for reference
    n = 8192
    a = torch.randn((n, n), generator=gen, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=gen, device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    _, _, ms3 = timed(lambda i: torch.matmul(a, b, out=c), 10, 2, torch)
    del a, b, c
    return dict(mfma_bf16_tflops=round(flop / (ms * 1e-3) / 1e12, 1),
                hbm_read_gbs=round(nbytes / (ms2 * 1e-3) / 1e9, 1),
                gemm_bf16_tflops=round(2 * n ** 3 / (ms3 * 1e-3) / 1e12, 1),
                gemm="torch.matmul (hipBLASLt) 8192 x 8192 x 8192 bf16, random inputs",
                mfma_probe=f"{wg} workgroups (one per CU) x 8 waves x {iters} x 32 v_mfma_f32_32x32x16_bf16, "
                           "random bf16 operands rotating between products",
                read_probe=f"1 GiB read once with 16-byte non-temporal loads, {swg} workgroups x 256 threads")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="about how long the oracle runs over all configurations")
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="minimum warm-up time per workload (0 for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "sink_decode", "diff_decode", "strided",
                                       "global", "dilated", "diff", "tiny", "copy", "peaks"], default=None,
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
    keep = {}              # host copies of inputs and GPU outputs for the oracle
    K, W = args.steps, args.warmup
    KD = max(1, min(K, 50))
    full = args.only is None

    if args.only == "copy":
        src = torch.empty(1 << 29, dtype=bf16, device="cuda").normal_()
        dst = torch.empty_like(src)
        wall_ms, ev_ms, med_ms = timed(lambda i: dst.copy_(src), K, W, torch)
        nbytes = 2 * src.numel() * 2
        print(json.dumps({"only": "copy", "bytes_read": src.numel() * 2, "bytes_written": src.numel() * 2,
                          "us": round(ev_ms * 1e3, 2), "gbs": round(nbytes / (ev_ms * 1e-3) / 1e9, 1)}))
        return

    peaks = None

    def run_peaks():
        log("peak probes: dense bf16 MFMA loop, 1 GiB streaming read, bf16 GEMM")
        pk = measure_peaks(swa, torch)
        log(f"peaks: {pk['mfma_bf16_tflops']} TFLOP/s bf16 MFMA loop, {pk['hbm_read_gbs']} GB/s HBM read, "
            f"{pk['gemm_bf16_tflops']} TFLOP/s bf16 GEMM")
        return pk
    if args.only == "peaks":
        print(json.dumps({"only": "peaks", "peaks": run_peaks()}))
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
        wall_ms, ev_ms, med_ms = timed(pf, K, W, torch)
        res["prefill"] = dict(wall_ms=wall_ms, event_ms=ev_ms, median_ms=med_ms,
                              tflops=flops / (ev_ms * 1e-3) / 1e12)
        log(f"prefill: {ev_ms * 1e3:.1f} us/launch (isolated median {med_ms * 1e3:.1f}), "
            f"{res['prefill']['tflops']:.1f} TFLOP/s")
        keep["swa_prefill_bf16"] = (cfg, (q, k, v), out.float().cpu().numpy())
    del qd, kd, vd

    # ---- decode: window, window + sinks, differential ------------------------
    def time_decode(name, make_inputs, call, alg_bytes, keep_name=None):
        """Two seeded input sets alternate, so no step reads a cache that the
        previous step left in L2/MALL; the output of set 0 is kept for the
        oracle."""
        made = [make_inputs(s) for s in range(2)]
        sets = [m[0] for m in made]
        fn = lambda i: call(sets[i & 1])
        log(f"{name}: {KD} steps after {W} warmup")
        wall_ms, ev_ms, med_ms = timed(fn, KD, W, torch)
        gbs = alg_bytes / (ev_ms * 1e-3) / 1e9
        log(f"{name}: {ev_ms * 1e3:.1f} us/step (isolated median {med_ms * 1e3:.1f}), {gbs:.0f} GB/s")
        if keep_name and full:
            o = call(sets[0])
            torch.cuda.synchronize()
            keep[keep_name] = (made[0][1], o.float().cpu().numpy())
        del sets, made
        return dict(wall_ms=wall_ms, event_ms=ev_ms, median_ms=med_ms, alg_bytes=alg_bytes, gbs=gbs)

    def i32(x):
        return torch.from_numpy(x.astype(np.int32)).cuda()

    if args.only in (None, "decode"):
        dcfg = synth.workload("window_decode_bf16")
        B, Hq, Hkv, d, Wr = dcfg["B"], dcfg["Hq"], dcfg["Hkv"], dcfg["d"], dcfg["window"]

        def mk(s):
            ins = synth.decode_inputs(dict(dcfg, seed=dcfg["seed"] + 10 * s))
            return (dict(q=dev(ins["q"], torch, bf16), k=dev(ins["k_ring"], torch, bf16),
                         v=dev(ins["v_ring"], torch, bf16), sl=i32(ins["seq_len"])),
                    ins if s == 0 else None)
        ws = torch.empty(max(1, swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, Wr)),
                         dtype=torch.uint8, device="cuda")
        dout = torch.empty((B, Hq, d), dtype=bf16, device="cuda")
        kv_bytes = decode_alg_bytes(dcfg) - B * Hq * 2 * d * 2
        res["decode"] = time_decode(
            "decode", mk, lambda t: swa.swa_attn_decode(t["q"], t["k"], t["v"], t["sl"], dcfg["scale"],
                                                        workspace=ws, out=dout),
            decode_alg_bytes(dcfg), keep_name="window_decode_bf16")
        res["decode"]["kv_gbs"] = kv_bytes / (res["decode"]["event_ms"] * 1e-3) / 1e9

    if args.only in (None, "sink_decode"):
        scfg_ = synth.workload("sink_decode_bf16")
        B, Hq, Hkv, d, Wr, S = (scfg_[x] for x in ("B", "Hq", "Hkv", "d", "window", "n_sink"))

        def mk(s):
            ins = synth.decode_inputs(dict(scfg_, seed=scfg_["seed"] + 10 * s))
            return ({x: dev(ins[x], torch, bf16) for x in ("q", "k_sink", "v_sink", "k_ring", "v_ring")} |
                    dict(sl=i32(ins["seq_len"])), None)
        ws = torch.empty(max(1, swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, d, Wr, S)),
                         dtype=torch.uint8, device="cuda")
        dout = torch.empty((B, Hq, d), dtype=bf16, device="cuda")
        res["sink_decode"] = time_decode(
            "sink decode", mk,
            lambda t: swa.swa_attn_decode_sinks(t["q"], t["k_sink"], t["v_sink"], t["k_ring"], t["v_ring"],
                                                t["sl"], scfg_["scale"], workspace=ws, out=dout),
            decode_alg_bytes(scfg_, S))

    if args.only in (None, "diff_decode"):
        gcfg = synth.workload("diff_decode_bf16")
        B, Hq, Hkv, d, dv, Wr = (gcfg[x] for x in ("B", "Hq", "Hkv", "d", "dv", "window"))

        def mk(s):
            ins = synth.diff_decode_inputs(dict(gcfg, seed=gcfg["seed"] + 10 * s))
            return ({x: dev(ins[x], torch, bf16) for x in ("q1", "k1_ring", "q2", "k2_ring", "v_ring")} |
                    dict(sl=i32(ins["seq_len"])), None)
        ws = torch.empty(max(1, swa.swa_attn_decode_workspace_bytes(B, Hq, Hkv, dv, Wr, 0, swa.SWA_OP_DIFF)),
                         dtype=torch.uint8, device="cuda")
        dout = torch.empty((B, Hq, dv), dtype=bf16, device="cuda")
        res["diff_decode"] = time_decode(
            "diff decode", mk,
            lambda t: swa.diff_attn_decode(t["q1"], t["k1_ring"], t["q2"], t["k2_ring"], t["v_ring"], t["sl"],
                                           gcfg["scale"], gcfg["lam"], workspace=ws, out=dout),
            diff_decode_alg_bytes(gcfg))

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
        wall_ms, ev_ms, med_ms = timed(fn, K, W, torch)
        sflops = 4.0 * scfg["d"] * cells_of(scfg) * scfg["B"] * scfg["Hq"]
        sbytes = 4 * sq.size * 2
        res["strided"] = dict(event_ms=ev_ms, median_ms=med_ms, tflops=sflops / (ev_ms * 1e-3) / 1e12,
                              gbs=sbytes / (ev_ms * 1e-3) / 1e9, alg_flops=sflops, alg_bytes=sbytes)
        if full:
            keep["local_strided_bf16"] = (scfg, (sq, sk, sv), sout.float().cpu().numpy())
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
        wall_ms, ev_ms, med_ms = timed(fn, K, W, torch)
        xcells = cells_of(xcfg) * xcfg["B"] * xcfg["Hq"]
        res[key] = dict(event_ms=ev_ms, median_ms=med_ms,
                        tflops=4.0 * xcfg["d"] * xcells / (ev_ms * 1e-3) / 1e12, workload=wl)
        del xqd, xkd, xvd, xout

    # ---- differential attention ------------------------------------------------
    if args.only in (None, "diff"):
        fcfg = synth.workload("diff_bf16")
        fhost = synth.diff_inputs(fcfg)
        fins = [dev(x, torch, bf16) for x in fhost]
        fmask = swa.swa_block_mask_build(fcfg["N"], fcfg["window"], 0, d=fcfg["d"], dv=fcfg["dv"],
                                         op=swa.SWA_OP_DIFF)
        fout = torch.empty((fcfg["B"], fcfg["Hq"], fcfg["N"], fcfg["dv"]), dtype=bf16, device="cuda")
        fn = lambda i: swa.diff_attn_fwd(*fins, fcfg["window"], 0, fcfg["scale"], fcfg["lam"], fmask,
                                         out=fout)
        log("differential attention")
        wall_ms, ev_ms, med_ms = timed(fn, K, W, torch)
        fcells = cells_of(fcfg) * fcfg["B"] * fcfg["Hq"]
        per_cell = 2 * (2 * fcfg["d"] + 2 * fcfg["dv"])   # two maps, each QK^T and PV
        res["diff"] = dict(event_ms=ev_ms, median_ms=med_ms, tflops=per_cell * fcells / (ev_ms * 1e-3) / 1e12,
                           tflops_formula=(2 * 2 * fcfg["d"] + 2 * fcfg["dv"]) * fcells / (ev_ms * 1e-3) / 1e12)
        if full:
            keep["diff_bf16"] = (fcfg, fhost, fout.float().cpu().numpy())
        del fins, fout

    # ---- tiny fp32 --------------------------------------------------------------
    if args.only in (None, "tiny"):
        tcfg = synth.workload("tiny_swa_f32")
        thost = synth.prefill_inputs(tcfg)
        tq, tk, tv = (dev(x, torch, torch.float32) for x in thost)
        tmask = swa.swa_block_mask_build(tcfg["N"], tcfg["window"], 0, dtype=torch.float32, d=tcfg["d"])
        tout = torch.empty_like(tq)
        fn = lambda i: swa.swa_attn_fwd(tq, tk, tv, tcfg["window"], 0, tcfg["scale"], tmask, out=tout)
        res["tiny_f32"] = dict(event_ms=timed(fn, K, W, torch)[1])
        if full:
            keep["tiny_swa_f32"] = (tcfg, thost, tout.float().cpu().numpy())

    if "prefill" not in res:
        print(json.dumps({"only": args.only, "results": res}))
        return
    # (after the workloads: the probes run the GPU at full power, which would
    # lower the clock of whatever ran next)
    if full:
        peaks = run_peaks()

    # ---- CPU baseline (oracle on every configuration) + parity of its rows ----------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baselines(keep, args.cpu_seconds)

    p = res["prefill"]
    src = os.path.join(ROOT, "sparse_masked_transformer_amd", "csrc", "gen_fwd_gqa.py")
    roof = {"bound": "mfma", "kernel": "swa_fwd_gqa_d128",
            "achieved": round(p["tflops"], 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(p["tflops"] / PEAK_BF16_TFLOPS, 4),
            "avg_launch_us": round(p["event_ms"] * 1e3, 2),
            "isolated_median_launch_us": round(p["median_ms"] * 1e3, 2),
            "traffic": traffic_record(src, "fwd_gqa_swa_prefill")}
    if peaks:
        roof["peak_measured"] = peaks["mfma_bf16_tflops"]
        roof["frac_measured"] = round(p["tflops"] / peaks["mfma_bf16_tflops"], 4)
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
        "roofline": roof,
        "cpu_baseline": cpu,
        "peaks_measured": peaks,
        "mask_build_us": round(mb_ms * 1e3, 2),
    }

    def hbm_roof(gbs, extra):
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(gbs / PEAK_HBM_GBS, 4)} | extra
        if peaks:
            r["peak_measured"] = peaks["hbm_read_gbs"]
            r["frac_measured"] = round(gbs / peaks["hbm_read_gbs"], 4)
        return r
    if "decode" in res:
        dd = res["decode"]
        dsrc = os.path.join(ROOT, "sparse_masked_transformer_amd", "csrc", "decode_bf16.hip")
        line["decode"] = {"workload": "window_decode_bf16", "value": round(dd["gbs"], 1), "unit": "GB/s",
                          "kv_gbs": round(dd["kv_gbs"], 1), "us_per_step": round(dd["event_ms"] * 1e3, 2),
                          "isolated_median_us": round(dd["median_ms"] * 1e3, 2),
                          "roofline": hbm_roof(dd["gbs"], {"kernel": "decode_kernel<128,128,1,true,false>",
                                                           "traffic": traffic_record(dsrc, "decode_bf16_window")})}
    for key, wl in (("sink_decode", "sink_decode_bf16"), ("diff_decode", "diff_decode_bf16")):
        if key in res:
            dd = res[key]
            line[key] = {"workload": wl, "value": round(dd["gbs"], 1), "unit": "GB/s",
                         "us_per_step": round(dd["event_ms"] * 1e3, 2),
                         "isolated_median_us": round(dd["median_ms"] * 1e3, 2),
                         "roofline": hbm_roof(dd["gbs"], {})}
    if "strided" in res:
        s = res["strided"]
        t_hbm = s["alg_bytes"] / (PEAK_HBM_GBS * 1e9)
        t_mfma = s["alg_flops"] / (PEAK_BF16_TFLOPS * 1e12)
        ssrc = os.path.join(ROOT, "sparse_masked_transformer_amd", "csrc", "gen_fwd_str.py")
        line["strided"] = {"workload": "local_strided_bf16", "kernel": "swa_fwd_mha_d64_str",
                           "tflops": round(s["tflops"], 2),
                           "gbs": round(s["gbs"], 1), "us": round(s["event_ms"] * 1e3, 2),
                           "isolated_median_us": round(s["median_ms"] * 1e3, 2),
                           "roofline_frac": round(max(t_hbm, t_mfma) / (s["event_ms"] * 1e-3), 4),
                           "bound": "hbm" if t_hbm > t_mfma else "mfma",
                           "traffic": traffic_record([ssrc, os.path.join(os.path.dirname(ssrc), "gen_fwd_gqa.py")],
                                                     "fwd_str_local_strided")}
    for key in ("global", "dilated"):
        if key in res:
            x = res[key]
            line[key] = {"workload": x["workload"], "tflops": round(x["tflops"], 2),
                         "us": round(x["event_ms"] * 1e3, 2), "bound": "mfma",
                         "roofline_frac": round(x["tflops"] / PEAK_BF16_TFLOPS, 4)}
    if "diff" in res:
        f = res["diff"]
        line["diff"] = {"workload": "diff_bf16", "kernel": "diff_fwd_d64_dv128", "tflops": round(f["tflops"], 2),
                        "tflops_512_per_cell": round(f["tflops_formula"], 2),
                        "us": round(f["event_ms"] * 1e3, 2),
                        "roofline_frac": round(f["tflops"] / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_record([os.path.join(ROOT, "sparse_masked_transformer_amd", "csrc", x)
                                                   for x in ("gen_fwd_diff.py", "gen_fwd_gqa.py")], "diff_bf16")}
        if peaks:
            line["diff"]["frac_measured"] = round(f["tflops"] / peaks["mfma_bf16_tflops"], 4)
    if "tiny_f32" in res:
        line["tiny_f32_us"] = round(res["tiny_f32"]["event_ms"] * 1e3, 2)
    print(json.dumps(line), flush=True)


def cpu_baselines(keep, budget_s):
    """The fp64 oracle on every configuration the run kept (its share of
    budget_s each), with the GPU's outputs compared on the same rows."""
    import oracle
    host = host_cpus()
    # the GPU machine gives one GPU's process a share of 16 host CPUs
    threads = max(1, min(16, host["affinity_cpus"]))
    log(f"cpu baseline: ~{budget_s:.0f} s of oracle work on {threads} threads")
    per = {}
    share = {"swa_prefill_bf16": 0.4, "local_strided_bf16": 0.2, "diff_bf16": 0.2, "tiny_swa_f32": 0.05}
    for name, kept in keep.items():
        if name == "window_decode_bf16":
            continue
        cfg, ins, gout = kept
        t0 = time.perf_counter()
        B, Hq, N = cfg["B"], cfg["Hq"], cfg["N"]
        w, s, sc = cfg["window"], cfg.get("stride", 0), cfg["scale"]
        rows = np.arange(B * Hq * N, dtype=np.int64)
        if name == "diff_bf16":
            q1, k1, q2, k2, v = ins
            fn = lambda r: oracle.diff_rows(q1, k1, q2, k2, v, w, 0, sc, cfg["lam"], r)
            flop = lambda r: 2.0 * (2 * cfg["d"] + 2 * cfg["dv"]) * row_keys(r % N, w, 0)
        else:
            q, k, v = ins
            fn = lambda r: oracle.attn_rows(q, k, v, w, s, sc, r)
            flop = lambda r: 4.0 * cfg["d"] * row_keys(r % N, w, s)
        r = oracle_rows(fn, rows, budget_s * share.get(name, 0.1), threads, flop, gout, cfg["dv"], 99)
        r["value"] = round(r["flop"] / r["seconds"] / 1e12, 5)
        r["unit"] = "TFLOP/s"
        per[name] = r
        log(f"oracle {name}: {r['rows']} of {r['of']} rows in {r['seconds']} s, max |gpu - oracle| "
            f"{r['max_abs_err_vs_gpu']:.3g} ({time.perf_counter() - t0:.1f} s)")
    if "window_decode_bf16" in keep:
        import synth
        scale = synth.workload("window_decode_bf16")["scale"]
        ins, gout = keep["window_decode_bf16"]
        B = ins["q"].shape[0]
        parts = np.array_split(np.arange(B), min(threads, B))
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
            outs = list(ex.map(lambda b: oracle.decode(ins["q"][b], ins["k_ring"][b], ins["v_ring"][b],
                                                       ins["seq_len"][b], scale), parts))
        dt = time.perf_counter() - t0
        want = np.concatenate(outs)
        _, Hq, d = ins["q"].shape
        Hkv, Wr = ins["k_ring"].shape[1], ins["k_ring"].shape[2]
        nbytes = decode_alg_bytes(synth.workload("window_decode_bf16"))
        per["window_decode_bf16"] = dict(rows=int(B * Hq), of=int(B * Hq), sequences=int(B), seconds=round(dt, 3),
                                         value=round(nbytes / dt / 1e9, 3), unit="GB/s",
                                         max_abs_err_vs_gpu=float(np.max(np.abs(gout - want))))
        log(f"oracle window_decode_bf16: all {B} sequences in {dt:.2f} s")
    head = per.get("swa_prefill_bf16")
    if head is None:
        return None
    return dict(value=head["value"], unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{head['rows']} of {head['of']} rows of the same workload (seeded uniform), fp64 C "
                       f"oracle, {head['seconds']} s on {threads} threads",
                seconds=head["seconds"], max_abs_err_vs_gpu=head["max_abs_err_vs_gpu"],
                host=host | {"threads_used": threads,
                             "note": "threads: the process's CPUs, at most the 16 a one-GPU job is given"},
                per_config=per)


if __name__ == "__main__":
    main()
