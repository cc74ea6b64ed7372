"""The benchmark's accounting.  FLOPs: the attended-cell counts bench.py uses
(closed forms) equal the oracle's brute-force count of the mask, for every
prefill-type workload it times; FLOPs are 4·d per attended cell (Learn:
Sparse & Sliding-Window Attention, §6 "FLOPs & memory": multiply-add = 2
FLOPs, core cost proportional to the allowed entries).  Bytes: each decode
step's algorithmic bytes are the oracle's KV-cache bytes of the window (and
sink slots) per sequence, for one layer, plus q and the output ("Attention
Variants Compared", task table, kv_cache_bytes; same §6: a rolling window
keeps the last w positions, sinks add k)."""
import pytest

import bench
import oracle
import synth


@pytest.mark.parametrize("name", ["tiny_swa_f32", "swa_prefill_bf16", "local_strided_bf16",
                                  "diff_bf16", "global_prefill_bf16", "dilated_prefill_bf16"])
def test_bench_cell_counts_match_brute_force(name):
    cfg = synth.workload(name)
    want, _ = oracle.count_nonmasked(cfg["N"], cfg["window"], cfg["stride"],
                                     cfg.get("dilation", 1), cfg.get("n_global", 0))
    assert bench.cells_of(cfg) == want


def test_headline_flops():
    cfg = synth.workload("swa_prefill_bf16")
    flops = 4 * cfg["d"] * bench.cells_of(cfg) * cfg["B"] * cfg["Hq"]
    assert flops == 128_857_407_488   # 251,674,624 attended cells x 512


def test_decode_bytes_are_kv_cache_bytes():
    for name in ("window_decode_bf16", "sink_decode_bf16"):
        cfg = synth.workload(name)
        S = cfg.get("n_sink", 0)
        qo = cfg["B"] * cfg["Hq"] * (cfg["d"] + cfg["dv"]) * 2
        kv = cfg["B"] * oracle.kv_cache_bytes(cfg["window"] + S, 1, cfg["Hkv"], cfg["d"])
        assert cfg["d"] == cfg["dv"]
        assert bench.decode_alg_bytes(cfg, S) == kv + qo
    # 64 sequences x 8 heads x 4096 positions x 2 x 128 x 2 bytes = 1 GiB, plus q and out
    cfg = synth.workload("window_decode_bf16")
    assert bench.decode_alg_bytes(cfg) == 2 ** 30 + 64 * 32 * 256 * 2


def test_diff_decode_bytes():
    cfg = synth.workload("diff_decode_bf16")
    B, Hq, Hkv, W, d, dv = (cfg[x] for x in ("B", "Hq", "Hkv", "window", "d", "dv"))
    # the two key windows are one K and one V of width d in kv_cache_bytes'
    # terms; the value window adds half of a (K, V) pair of width dv
    kv = B * (oracle.kv_cache_bytes(W, 1, Hkv, d) + oracle.kv_cache_bytes(W, 1, Hkv, dv) // 2)
    assert bench.diff_decode_alg_bytes(cfg) == kv + B * Hq * (2 * d + dv) * 2
