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
    for name, w in bench.WORKLOADS.items():
        dt, M, N, K = w["dtype"], w["M"], w["N"], w["K"]
        assert bench.plan_of(lib, dt, M, N, K, aligned=bench.is_aligned(name)) is not None, name
    # the ragged workload: K = 4001 breaks A's chunk rule only, so both
    # operands keep LDS-DMA and A's K tail is completed by element loads
    assert bench.is_aligned("ragged") == lib.ALIGNED_B
    p = bench.plan_of(lib, "bf16", 4000, 3968, 4001, aligned=lib.ALIGNED_B)
    assert p["producer"] == "direct"


def test_pages_context_ratios():
    """The report's context block: the pages' figures verbatim, and the same
    ratios from the measured points (2-stage over 1-stage gains)."""
    rep = {"f32_4096_page_tile": {"128x64x16 s1 direct": 120.0, "128x64x16 s2 direct": 135.0, "auto": 145.0},
           "i8_4096": {"variants": {"256x256x128 s1 direct": 1500.0, "256x256x128 s2 direct": 2100.0}}}
    c = bench.pages_context(rep)
    assert c["sgemm_2stage_gain_pct"]["pages"]["kernel 11 over kernel 10"] == 8.9
    assert c["sgemm_2stage_gain_pct"]["pages"]["share of vendor library"] == {"1 stage": 81.9, "2 stages": 89.2}
    assert c["sgemm_2stage_gain_pct"]["here"]["128x64x16 s2 over s1"] == 12.5
    assert c["int8_4096_pipelining_gain_pct"]["pages"]["async-copy pipeline over none"] == 35
    assert c["int8_4096_pipelining_gain_pct"]["here"]["256x256x128 s2 over s1"] == 40.0
    # the int8 labels are the ones the variant sweep produces
    labels = {p["key"] for p in bench.report_points(lib) if p["section"] == "i8_4096"}
    assert {"256x256x128 s1 direct", "256x256x128 s2 direct"} <= labels


def test_report_points_cover_every_timed_variant():
    """The report times the planner's plan and every compiled vector-producer
    variant at 4096^3 for int8, bf16 and fp16, the pages' fp32 tile at 1 and 2
    stages, and the K-sweep at every depth: the list the full-size parity
    tests walk holds all of them, each on a workload with a plan."""
    pts = bench.report_points(lib)
    for dt, sec in (("i8", "i8_4096"), ("bf16", "bf16_4096"), ("f16", "f16_4096")):
        want = {bench.plan_label(v) for v in (lib.pgemm_variant_info(i) for i in range(lib.pgemm_num_variants()))
                if v["dtype"] == dt and v["producer"] != "generic"}
        assert {p["key"] for p in pts if p["section"] == sec} == want | {"auto"}
    for K in bench.K_SWEEP:
        assert {p["key"] for p in pts if p["workload"] == "bf16_k%d" % K} == {"K%d s%d" % (K, s) for s in
                                                                             (1, 2, 3, 4)} | {"K%d auto" % K}
    assert any(p["workload"] == "ragged" for p in pts)
    for p in pts:
        w = bench.WORKLOADS[p["workload"]]
        plan = bench.plan_of(lib, w["dtype"], w["M"], w["N"], w["K"], p["stages"], p["producer"], p["tile"],
                             aligned=bench.is_aligned(p["workload"]))
        assert plan is not None, p
