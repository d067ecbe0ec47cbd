"""Host-side checks of bench.py (no GPU needed).

* More than one GPU is refused with a message, before anything touches a GPU.
* The kernel source hash ignores comments and blank lines but sees code and
  build flags, so HBM traffic from profiles/traffic.json is reported only for
  the kernel version that was profiled.
* The algorithmic byte count of the headline workload.
* Every benchmark workload has a plan.
"""
import json
import os
import subprocess
import sys

import bench
from software_pipelined_tiled_loop_amd import binding as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for args, env in (([" --gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + [a.strip() for a in args],
                           capture_output=True, text=True, env=dict(os.environ, **env), timeout=120)
        assert r.returncode == 2, r.stderr
        assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_code_only_ignores_comments_and_layout():
    a = "int x = 1; // one\n/* block\n comment */\n\n  int   y = 2;\n"
    b = "int x = 1;\nint y = 2;"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(b.replace("2", "3"))


def test_source_hash_is_stable_and_covers_build_flags(monkeypatch):
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) == 16
    from software_pipelined_tiled_loop_amd import build
    monkeypatch.setattr(build, "HIPCC_FLAGS", build.HIPCC_FLAGS + ["-O0"])
    assert bench.kernel_source_hash() != h


def test_source_hash_does_not_depend_on_the_checkout_location(monkeypatch):
    h = bench.kernel_source_hash()
    from software_pipelined_tiled_loop_amd import build
    moved = [("-I/elsewhere/include" if f.startswith("-I") else f) for f in build.HIPCC_FLAGS]
    assert moved != build.HIPCC_FLAGS
    monkeypatch.setattr(build, "HIPCC_FLAGS", moved)
    assert bench.kernel_source_hash() == h


def test_traffic_only_for_the_profiled_sources():
    d = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    entries = {k: v for k, v in d.items() if not k.startswith("_")}
    assert entries
    for key, e in entries.items():
        assert bench.load_traffic(key, e["kernel_source_hash"]) == e["bytes_per_launch"]
        assert bench.load_traffic(key, "0" * 16) is None
        assert abs(e["bytes_per_launch"] - e["read_bytes"] - e["write_bytes"]) <= 1  # each rounded down
    assert bench.load_traffic("no_such_kernel", bench.kernel_source_hash()) is None


def test_headline_algorithmic_bytes():
    # A and B read once, C read (beta != 0) and written once, fp32
    assert bench.algorithmic_bytes("f32", 4096, 4096, 4096, 0.5) == 4 * 4096 * 4096 * 4
    assert bench.algorithmic_bytes("bf16", 4096, 4096, 4096, 0.0) == 2 * 4096 * 4096 * 2 + 4096 * 4096 * 4


def test_every_workload_has_a_plan():
    from software_pipelined_tiled_loop_amd import inputs
    for name, w in bench.WORKLOADS.items():
        dt, M, N, K = w["dtype"], w["M"], w["N"], w["K"]
        lda, ldb = w.get("lda", K), w.get("ldb", N)
        aligned = int(all(x * inputs.ELEM_BYTES[dt] % 16 == 0 for x in (lda, ldb, K, N)))
        assert bench.plan_of(lib, dt, M, N, K, aligned=aligned) is not None, name


def test_pages_context_ratios():
    """The report's context block: the pages' figures verbatim, and the same
    ratios from the measured points (vendor share; int8 2-stage gain)."""
    rep = {"f32_4096_page_tile": {"128x64x16 s1 direct": 120.0, "128x64x16 s2 direct": 135.0, "auto": 145.0,
                                  "vendor_blas": 150.0},
           "i8_4096": {"variants": {"256x256x128 s1 direct": 1500.0, "256x256x128 s2 direct": 2100.0}}}
    c = bench.pages_context(rep)
    assert c["sgemm_pct_of_vendor_blas"]["pages"]["1 stage"] == 81.9
    assert c["sgemm_pct_of_vendor_blas"]["pages"]["2 stages"] == 89.2
    assert c["sgemm_pct_of_vendor_blas"]["here"]["128x64x16 s1"] == 80.0
    assert c["sgemm_pct_of_vendor_blas"]["here"]["128x64x16 s2"] == 90.0
    assert c["int8_4096_pipelining_gain_pct"]["pages"]["async-copy pipeline over none"] == 35
    assert c["int8_4096_pipelining_gain_pct"]["here"]["256x256x128 s2 over s1"] == 40.0
    # the int8 labels are the ones the variant sweep produces
    labels = {bench.plan_label(lib.pgemm_variant_info(i)) for i in range(lib.pgemm_num_variants())
              if lib.pgemm_variant_info(i)["dtype"] == "i8"}
    assert {"256x256x128 s1 direct", "256x256x128 s2 direct"} <= labels
