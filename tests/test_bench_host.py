"""Host-side pieces of bench.py that need no GPU: its own closed-form MAC
count (the TFLOP/s numerator) must equal the oracle's count for every
workload, and reproduce the pages' printed Gflops for DiT-XL/2 (118.6 at
256x256 and 524.6 at 512x512, itwiki "확산 트랜스포머", ImageNet results
table)."""
import pytest

import bench
import dit_inputs
from oracle import flops as oflops


@pytest.mark.parametrize("name", sorted(dit_inputs.WORKLOADS))
def test_bench_mac_count_matches_oracle(name):
    cfg = dit_inputs.workload(name)
    assert bench.gmac_per_row(cfg) == pytest.approx(oflops.gmac_for(cfg), rel=1e-12)


def test_bench_mac_count_reproduces_the_pages():
    assert round(bench.gmac_per_row(dit_inputs.workload("dit_xl2_256_cfg")), 1) == 118.6
    assert abs(bench.gmac_per_row(dit_inputs.workload("dit_xl2_512_cfg")) / 524.6 - 1) < 2.5e-3


def test_rocminfo_parse(monkeypatch):
    text = ("Agent 1\n  Name: AMD EPYC\n  Compute Unit: 128\n"
            "Agent 2\n  Name: gfx950\n  Compute Unit:            256\n"
            "  Max Clock Freq. (MHz):   2400\n")

    class R:
        stdout = text

    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: R())
    cus, mhz, tf = bench.rocminfo_peak()
    assert (cus, mhz) == (256, 2400) and tf == pytest.approx(2516.6, abs=0.1)
