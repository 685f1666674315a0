"""CPU-only: the benchmark's accounting of algorithmic bytes and FLOPs against
the decode sweep table printed on "[Cute,Fwd,Sm100] Support q_stage=1 for
inference" (section Benchmarks), stored in tests/golden/."""
from __future__ import annotations

import csv
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_split_sweep_sm100.csv")


def rows():
    with open(GOLDEN) as f:
        lines = [ln for ln in f if not ln.startswith("#")]
    return list(csv.DictReader(lines))


def test_golden_table_loaded():
    assert len(rows()) == 8


@pytest.mark.parametrize("row", rows(), ids=lambda r: f"splits{r['num_splits']}")
def test_decode_accounting_matches_page_table(row):
    w = bench._spec("g", "bf16", [int(row["Q"])] * int(row["B"]), [int(row["K"])] * int(row["B"]),
                    int(row["H"]), int(row["H"]), int(row["D"]), int(row["D"]))
    nb, nf = bench.alg_bytes(w), bench.alg_flops(w)
    assert abs(nf / nb - float(row["arithmetic_intensity"])) < 1e-14
    t_ms = float(row["avg_time"])
    assert abs(nf / t_ms / 1e9 - float(row["tflops"])) < 1e-9
    assert abs(nb / t_ms / 1e9 - float(row["bw"])) < 1e-9


def test_headline_workload_is_the_table_shape():
    w = bench.workloads()["long_decode"]
    assert (w["lens_q"], w["lens_k"], w["hq"], w["dqk"]) == ([1], [131072], 32, 128)
    assert bench.alg_bytes(w) == 2_147_500_032 and bench.alg_flops(w) == 2_147_483_648


def test_causal_pairs_closed_form():
    for s in (1, 7, 2048):
        assert bench.attended_pairs(s, s, True, (-1, -1)) == s * (s + 1) // 2
    assert bench.attended_pairs(70, 16384, False, (-1, -1)) == 70 * 16384
    assert bench.attended_pairs(5, 3, True, (-1, -1)) == 0 + 0 + 1 + 2 + 3
    assert bench.attended_pairs(10, 10, False, (2, 0)) == 1 + 2 + 3 * 8


def test_multi_gpu_request_exits(tmp_path):
    import subprocess
    import sys
    res = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                         text=True)
    assert res.returncode != 0 and "one GPU" in res.stderr


def test_kernel_family_names():
    """kernel_id = dtype * 1000 + instance id; instance ranges name the family."""
    assert bench.kernel_name(2 * 1000 + 101) == "fmha_decode_kernel"
    assert bench.kernel_name(1 * 1000 + 201) == "fmha_prefill_kernel"
    assert bench.kernel_name(3 * 1000 + 211) == "fmha_prefill8_kernel"
    assert bench.kernel_name(0 * 1000 + 7) == "fmha_fwd_kernel"
    for name, files in bench.KERNEL_SOURCES.items():
        assert len(bench.kernel_source_hash(name)) == 16 and files
