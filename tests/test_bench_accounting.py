"""The benchmark's FLOP accounting: the attended-cell counts bench.py uses
(closed forms) equal the oracle's brute-force count of the mask, for every
prefill-type workload it times.  FLOPs are 4·d per attended cell
(Attention Variants Compared, §6 cost table: multiply-add = 2 FLOPs, cost
proportional to the attended entries)."""
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
