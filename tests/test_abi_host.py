"""Host-only checks of the C ABI (no GPU needed).

* libpgemm.so loads and exports every function include/pgemm.h declares;
* argument errors come back before anything is launched;
* planner invariants: LDS ring within 160 KiB, effective depth clipped to the
  number of K tiles, explicit depths honoured or refused, misaligned data
  routed to the generic producer;
* the planner's models reproduce the figures the pages print
  (tests/golden/page_models.json).
"""
import json
import os
import re
import subprocess
import sys

import pytest

from software_pipelined_tiled_loop_amd import binding as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pgemm.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_models.json")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(pgemm_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("pgemm_gemm", "pgemm_gemm_ex", "pgemm_plan", "pgemm_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], stdout=subprocess.PIPE, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\s[TW]\s(\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib._lib, n)
    assert set(lib.EXPORTED) <= set(names)


FAKE = 1 << 20  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("args,code", [
    (dict(dtype=7), -2),
    (dict(stages=5), -3),
    (dict(stages=-1), -3),
    (dict(M=-1), -1),
    (dict(lda=7), -1),
    (dict(ldb=3), -1),
    (dict(ldc=3), -1),
    (dict(dtype="i8", alpha=0.5), -5),
    (dict(dtype="i8", beta=float("nan")), -5),
    (dict(dtype="i8", alpha=2.0 ** 40), -5),
    (dict(A=None), -1),
    (dict(C=None), -1),
    (dict(lda=1 << 26, dtype="f32"), -7),
    (dict(M=2 ** 31 - 255), -7),           # a tile origin plus one tile would overflow 32 bits
    (dict(N=2 ** 31 - 255, ldb=2 ** 31 - 255, ldc=2 ** 31 - 255), -7),
    (dict(K=2 ** 31 - 255, lda=2 ** 31 - 255), -7),
    (dict(A=FAKE + 1, dtype="f32"), -1),   # not element aligned
])
def test_argument_errors_before_any_launch(args, code):
    a = dict(M=8, N=8, K=8, alpha=1.0, A=FAKE, lda=8, B=FAKE, ldb=8, beta=0.0, C=FAKE, ldc=8, dtype="bf16",
             stages=0)
    a.update(args)
    r = lib._lib.pgemm_gemm(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"], a["ldb"], a["beta"],
                            a["C"], a["ldc"], lib.DTYPE_CODE.get(a["dtype"], a["dtype"]), a["stages"], None)
    assert r == code, (args, r, lib.pgemm_strerror(r))


@pytest.mark.parametrize("opts", [dict(skew=65), dict(skew=-1), dict(workgroups=-8)])
def test_option_errors_before_any_launch(opts):
    o = lib._opts(tile=(128, 128, 64), skew=opts.get("skew", 0), workgroups=opts.get("workgroups", 0))
    r = lib.pgemm_gemm_ex(8, 8, 8, 1.0, FAKE, 8, FAKE, 8, 0.0, FAKE, 8, "bf16", 0, o, 0)
    assert r == -1, lib.pgemm_strerror(r)
    o = lib._opts(tile=(128, 128, 64))
    o.reserved[0] = 3
    assert lib.pgemm_gemm_ex(8, 8, 8, 1.0, FAKE, 8, FAKE, 8, 0.0, FAKE, 8, "bf16", 0, o, 0) == -1


@pytest.mark.parametrize("alpha,beta,code", [
    (-2.0 ** 31, 0.0, 0), (2.0 ** 31 - 1, -2.0 ** 31, 0),          # the ends of int32 are accepted
    (-2.0 ** 31 - 1, 0.0, -5), (2.0 ** 31, 0.0, -5), (1.0, 2.0 ** 31, -5), (float("inf"), 0.0, -5),
])
def test_int8_scalars_must_be_int32_integers(alpha, beta, code):
    # M = 0: the scalars are checked, then the call is a no-op, so nothing is launched
    r = lib._lib.pgemm_gemm(0, 8, 8, alpha, FAKE, 8, FAKE, 8, beta, FAKE, 8, lib.DTYPE_CODE["i8"], 0, None)
    assert r == code, (alpha, beta, r)


def test_ldc_beyond_32_bit_tile_addressing_is_rejected():
    r = lib._lib.pgemm_gemm(8, 8, 8, 1.0, FAKE, 8, FAKE, 8, 0.0, FAKE, 1 << 21, 2, 0, None)
    assert r == -7


def test_grid_is_a_multiple_of_8_and_persistent_workgroups_are_capped():
    # one workgroup per tile, rounded up to a multiple of 8
    r, p = lib.pgemm_plan(4096, 4096, 4096, "bf16", 0, 1, {"tile": (256, 256, 64)})
    assert r == 0 and p["grid"] == 256
    r, p = lib.pgemm_plan(300, 300, 64, "bf16", 0, 1, {"tile": (128, 128, 64)})
    assert r == 0 and p["grid"] == 16          # 9 tiles -> 16 workgroups, 7 find no tile
    # persistent: the requested count, rounded up to 8, never more than the default grid
    for want, got in ((1, 8), (8, 8), (20, 24), (256, 256), (100000, 1024)):
        r, p = lib.pgemm_plan(4096, 4096, 256, "bf16", 0, 1, {"tile": (128, 128, 64), "workgroups": want})
        assert r == 0 and p["grid"] == got, (want, p["grid"])


def test_waves_option_selects_the_wave_layout():
    r, p = lib.pgemm_plan(4096, 4096, 4096, "bf16", 0, 1, {"tile": (128, 128, 64), "waves": 4})
    assert r == 0 and p["waves_m"] * p["waves_n"] == 4
    r, _ = lib.pgemm_plan(4096, 4096, 4096, "bf16", 0, 1, {"tile": (128, 128, 64), "waves": 8})
    assert r == -4
    o = lib._opts(tile=(128, 128, 64), waves=-1)
    assert lib.pgemm_gemm_ex(8, 8, 8, 1.0, FAKE, 8, FAKE, 8, 0.0, FAKE, 8, "bf16", 0, o, 0) == -1


def test_binding_leaves_one_hip_runtime_in_the_process():
    """torch bundles HIP and HSA runtimes under the sonames the library links
    against; importing the binding before anything else must still leave one
    copy of each (two copies made the library's runtime find no device)."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from software_pipelined_tiled_loop_amd import binding\n"
            "import torch\n"
            "libs = set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l or 'libhsa-runtime64' in l)\n"
            "print(len([x for x in libs if 'amdhip64' in x]), len([x for x in libs if 'hsa-runtime64' in x]))\n" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], stdout=subprocess.PIPE, text=True, check=True).stdout.split()
    assert out == ["1", "1"], out


def test_empty_problems_are_noops():
    assert lib._lib.pgemm_gemm(0, 8, 8, 1.0, None, 8, None, 8, 0.0, None, 8, 2, 0, None) == 0
    assert lib._lib.pgemm_gemm(8, 0, 8, 1.0, None, 8, None, 8, 0.0, None, 8, 2, 0, None) == 0


HAZARD_OK = dict(X=FAKE, rows=32, cols=512, ldx=512, row_sums=FAKE, reuse_wait=1, delay_wave=-1, delay_cycles=0,
                 trace=None, trace_len=0, trace_wg=0)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=15), -1), (dict(rows=-16), -1), (dict(cols=255), -1), (dict(cols=-256), -1),
    (dict(ldx=508), -1), (dict(ldx=514), -1), (dict(reuse_wait=2), -1), (dict(reuse_wait=-1), -1),
    (dict(delay_wave=4), -1), (dict(delay_wave=-2), -1), (dict(delay_cycles=-1), -1),
    (dict(delay_cycles=10000001), -1), (dict(X=FAKE + 4), -1), (dict(X=None), -1), (dict(row_sums=None), -1),
    (dict(trace=FAKE, trace_len=47), -1), (dict(trace=FAKE, trace_len=48, trace_wg=2), -1),
    (dict(trace=FAKE, trace_len=48, trace_wg=-1), -1), (dict(trace=FAKE + 4, trace_len=48), -1),
    (dict(cols=256 * (2 ** 31 // 24 + 1), ldx=256 * (2 ** 31 // 24 + 1)), -7),
])
def test_hazard_argument_errors_before_any_launch(kw, code):
    args = dict(HAZARD_OK, **kw)
    assert lib.pgemm_hazard_copy_reduce(**args, stream=0) == code


def test_hazard_without_rows_is_a_noop():
    assert lib.pgemm_hazard_copy_reduce(**dict(HAZARD_OK, rows=0, X=None, row_sums=None), stream=0) == 0


def _planner_check():
    return json.load(open(os.path.join(ROOT, "profiles", "planner_check.json")))["shapes"]


# Shapes where the cost model is known to miss by more than 3 %, with the
# bound it keeps: fp32 at K <= 64, where the 128x64x16 tile at one stage (four
# co-resident workgroups per CU) hides its epilogue better than the fixed
# costs fitted at K >= 128 predict.
KNOWN_MISSES = {"f32 4096x4096x32": 1.15, "f32 8192x8192x64": 1.08}


@pytest.mark.parametrize("key", sorted(_planner_check()))
def test_planner_pick_is_within_3_percent_of_the_best_measured_class(key):
    """A regression check of the planner's cost model against measurement,
    not a correctness property: profiles/planner_check.json holds, for each
    shape, every compiled DIRECT variant (tile class and ring depth) timed
    on MI355X (bench.py --planner-check); the variant the planner picks now
    must have measured within 3 % of the fastest one (KNOWN_MISSES: within
    the stated bound)."""
    v = _planner_check()[key]
    dt, shape = key.split()
    M, N, K = (int(x) for x in shape.split("x"))
    r, p = lib.pgemm_plan(M, N, K, dt, 0, 1)
    assert r == 0
    pick = "%dx%dx%d s%d direct" % (p["tile_m"], p["tile_n"], p["tile_k"], p["stages"])
    assert pick in v["classes"], (key, pick, v["classes"])
    got = v["classes"][pick]
    assert v["best_tflops"] <= KNOWN_MISSES.get(key, 1.03) * got, (key, pick, got, v["best"], v["best_tflops"])


def test_torch_wrapper_rejects_tensors_that_are_not_row_major():
    """binding.gemm refuses, before anything reaches the library, tensors
    whose columns are not contiguous or that are not 2-D."""
    import torch
    A, B, C = torch.zeros(8, 8), torch.zeros(8, 8), torch.zeros(8, 8)
    with pytest.raises(ValueError):
        lib.gemm(A.t(), B, C)
    with pytest.raises(ValueError):
        lib.gemm(A, B[:, ::2], C)
    with pytest.raises(ValueError):
        lib.gemm(A, B, C[None])


def test_torch_wrapper_validates_before_any_launch():
    """Each bad call raises ValueError before the library is reached: these
    tensors are on the CPU, so a call that got through would hand host
    addresses to a kernel.  The dtype and size checks come first, so each
    fault is named even with CPU tensors; well-formed CPU tensors then fail
    the device check."""
    import torch
    f32, bf = torch.float32, torch.bfloat16
    A, B, C = torch.zeros(8, 16, dtype=bf), torch.zeros(16, 12, dtype=bf), torch.zeros(8, 12)
    bad = [
        (A, B.to(torch.float16), C),                                # B dtype differs from A
        (A, B, C.to(bf)),                                           # C not fp32
        (A.to(torch.int8), B.to(torch.int8), C),                    # int8 needs int32 C
        (A.to(torch.float64), B.to(torch.float64), C),              # unsupported input dtype
        (A, B[:12], C),                                             # B has fewer than K rows
        (A, B, C[:7]),                                              # C has fewer than M rows
        (A, B, C[:, :11]),                                          # C has fewer than N columns
        (A, B, C),                                                  # well-formed, but on the CPU
    ]
    for args in bad:
        with pytest.raises(ValueError):
            lib.gemm(*args)
    with pytest.raises(ValueError):
        lib.gemm(A, B, C, M=9)                                      # M beyond A's rows
    with pytest.raises(ValueError):
        lib.gemm(A.to(f32), B.to(f32), C, K=17)                     # K beyond A's columns


def test_torch_wrapper_refuses_output_overlapping_an_input():
    """C must not share memory with A or B (the kernels read A and B while
    C is written); the overlap check comes before the device check, so CPU
    tensors show it without reaching the library."""
    import torch
    buf = torch.zeros(64, 64)
    with pytest.raises(ValueError, match="overlaps A"):
        lib.gemm(buf[:16, :16], torch.zeros(16, 16), buf[8:24, :16])
    with pytest.raises(ValueError, match="overlaps B"):
        lib.gemm(torch.zeros(16, 16), buf[:16, 32:48], buf[15:31, 47:63])
    # side by side in one allocation, no shared element: only the device check remains
    with pytest.raises(ValueError, match="GPU tensors"):
        lib.gemm(buf[:16, :16], buf[:16, 16:32], buf[:16, 32:48])


def test_diagnostics_refuse_bad_arguments_before_any_launch():
    """The diagnostics validate everything on the host: dtype, counts, output
    buffers, sizes, alignment and the compiled classes and ladder steps.
    The pointers are never dereferenced."""
    assert lib.pgemm_diag_mfma_ceiling(7, 0, 16, 256, 1, FAKE, stream=0)[0] == -2
    assert lib.pgemm_diag_mfma_ceiling("bf16", 2, 16, 256, 1, FAKE, stream=0)[0] == -1
    assert lib.pgemm_diag_mfma_ceiling("bf16", 0, -1, 256, 1, FAKE, stream=0)[0] == -1
    assert lib.pgemm_diag_mfma_ceiling("bf16", 0, 16, 0, 1, FAKE, stream=0)[0] == -1
    assert lib.pgemm_diag_mfma_ceiling("bf16", 0, 16, 256, 1, 0, stream=0)[0] == -1
    assert lib.pgemm_diag_mfma_ceiling("bf16", 0, 16, 256, 1, FAKE + 2, stream=0)[0] == -1
    assert lib.pgemm_diag_mfma_ceiling("bf16", 0, 16, 256, 1, FAKE, stream=0, waves_per_simd=3)[0] == -1
    assert lib.pgemm_diag_mfma_ceiling("bf16", 0, 16, 256, 1, FAKE, stream=0, waves_per_simd=0)[0] == -1
    assert lib.pgemm_diag_mfma_ceiling("bf16", 0, 16, 256, 1, FAKE, stream=0, block=8)[0] == -1
    assert lib.pgemm_diag_mfma_ceiling("f32", 0, 16, 256, 1, FAKE, stream=0, block=32)[0] == -1
    ok = dict(M=4096, N=4096, K=4096, A=FAKE, lda=4096, B=FAKE, ldb=4096, dtype="bf16", tile=(256, 256, 64), stages=2)

    def stream(**kw):
        a = dict(ok, **kw)
        return lib.pgemm_diag_lds_stream(a["M"], a["N"], a["K"], a["A"], a["lda"], a["B"], a["ldb"], a["dtype"],
                                         a["tile"], a["stages"], stream=0)[0]
    assert stream(dtype=9) == -2
    assert stream(K=0) == -1 and stream(lda=4095) == -1 and stream(A=FAKE + 2) == -1 and stream(N=4092) == -1
    assert stream(tile=(128, 128, 64)) == -4 and stream(stages=3) == -4
    assert stream(lda=1 << 24) == -7
    assert lib.pgemm_diag_mfma_ceiling("bf16", 0, 16, 256, 1, FAKE, clock=FAKE + 4, stream=0)[0] == -1

    def parts(**kw):
        a = dict(dict(ok, C=FAKE, ldc=4096, parts=lib.PART_ALL, clock=FAKE, clock_len=256 * 4), **kw)
        return lib.pgemm_diag_parts(a["M"], a["N"], a["K"], a["A"], a["lda"], a["B"], a["ldb"], a["C"], a["ldc"],
                                    a["dtype"], a["tile"], a["stages"], a["parts"], a["clock"], a["clock_len"],
                                    stream=0)
    assert parts(dtype=9) == -2
    assert parts(K=0) == -1 and parts(ldc=4095) == -1 and parts(C=FAKE + 2) == -1 and parts(clock=0) == -1
    assert parts(clock=FAKE + 4) == -1 and parts(parts=16) == -1 and parts(parts=-1) == -1
    assert parts(clock_len=256 * 4 - 1) == -1                   # one word short of grid * 4
    assert parts(parts=lib.PART_DMA) == -4                       # not a compiled ladder step
    assert parts(tile=(256, 256, 32)) == -4 and parts(stages=3) == -4
    assert parts(lda=1 << 24) == -7


def test_strerror_covers_every_status():
    for code in range(0, -8, -1):
        assert lib.pgemm_strerror(code) != "unknown status"
    assert lib.pgemm_strerror(-99) == "unknown status"


def all_variants():
    return [lib.pgemm_variant_info(i) for i in range(lib.pgemm_num_variants())]


def test_variant_table_invariants():
    es = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}
    vs = all_variants()
    assert len(vs) >= 40
    for v in vs:
        assert v["lds_bytes"] <= 163840
        assert v["lds_bytes"] == lib.pgemm_model_lds_bytes(v["tile_m"], v["tile_n"], v["tile_k"], v["stages"],
                                                           es[v["dtype"]], 0)
        assert 1 <= v["stages"] <= 4
        assert v["threads"] == 64 * v["waves_m"] * v["waves_n"]
    # every dtype offers 1..4 stages and both vector producers somewhere
    for dt in es:
        mine = [v for v in vs if v["dtype"] == dt]
        assert {v["stages"] for v in mine} == {1, 2, 3, 4}
        assert {"direct", "register", "generic"} <= {v["producer"] for v in mine}
    # the pages' SGEMM tile class exists with 1 and 2 stages
    page = [v for v in vs if v["dtype"] == "f32" and (v["tile_m"], v["tile_n"], v["tile_k"]) == (128, 64, 16)]
    assert {1, 2} <= {v["stages"] for v in page}


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_planner_clips_depth_to_k_tiles(dtype):
    for K in (1, 16, 32, 64, 100, 256, 4096, 16384):
        r, p = lib.pgemm_plan(4096, 4096, K, dtype, 0, 1)
        assert r == 0
        assert p["stages"] <= max(p["num_k_tiles"], 1)
        assert p["stages_eff"] == min(p["stages"], max(p["num_k_tiles"], 1))
        assert p["lds_bytes"] <= 163840


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_planner_honours_explicit_depth(dtype):
    for S in (1, 2, 3, 4):
        r, p = lib.pgemm_plan(1024, 1024, 2048, dtype, S, 1)
        assert r == 0 and p["stages"] == S
    r, _ = lib.pgemm_plan(1024, 1024, 2048, dtype, 0, 0, {"producer": "direct"})
    assert r == -4  # the direct producer needs B's chunk rule
    r, p = lib.pgemm_plan(1024, 1024, 2047, dtype, 0, 0)
    assert r == 0 and p["producer"] == "generic"
    r, _ = lib.pgemm_plan(1024, 1024, 2048, dtype, 0, 1, {"tile": (8, 8, 8)})
    assert r == -4


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_planner_keeps_the_direct_copy_for_the_aligned_operand(dtype):
    """Per-operand producers: each forced producer is admitted exactly for the
    chunk-rule classes it can serve (DIRECT needs B's rule and completes A's
    K tail by element loads; REGISTER needs both; each staged producer the
    rule of the operand it keeps on LDS-DMA); with only B whole the planner
    keeps DIRECT, with only A whole it picks among GENERIC and STAGED_B;
    unknown classes are argument errors."""
    need = {"direct": {lib.ALIGNED_BOTH, lib.ALIGNED_B}, "register": {lib.ALIGNED_BOTH},
            "staged_a": {lib.ALIGNED_BOTH, lib.ALIGNED_B}, "staged_b": {lib.ALIGNED_BOTH, lib.ALIGNED_A},
            "generic": {lib.ALIGNED_NONE, lib.ALIGNED_BOTH, lib.ALIGNED_A, lib.ALIGNED_B}}
    for prod, ok in need.items():
        for cls in (lib.ALIGNED_NONE, lib.ALIGNED_BOTH, lib.ALIGNED_A, lib.ALIGNED_B):
            r, p = lib.pgemm_plan(4096, 4096, 4096, dtype, 0, cls, {"producer": prod})
            assert (r == 0) == (cls in ok), (prod, cls, r)
            if r == 0:
                assert p["producer"] == prod
    for cls, allowed in ((lib.ALIGNED_A, {"generic", "staged_b"}), (lib.ALIGNED_B, {"direct"}),
                         (lib.ALIGNED_NONE, {"generic"})):
        r, p = lib.pgemm_plan(4000, 3968, 4001, dtype, 0, cls)
        assert r == 0 and p["producer"] in allowed, (cls, p)
    for bad in (-1, 4, 7):
        assert lib.pgemm_plan(64, 64, 64, dtype, 0, bad)[0] == -1


def test_planner_prefers_big_tiles_for_big_problems_and_small_for_small():
    r, big = lib.pgemm_plan(4096, 4096, 4096, "bf16", 0, 1)
    r2, small = lib.pgemm_plan(512, 512, 4096, "bf16", 0, 1)
    assert r == 0 and r2 == 0
    assert big["tile_m"] * big["tile_n"] >= small["tile_m"] * small["tile_n"]
    assert small["grid"] >= 16


def test_page_models_golden():
    g = json.load(open(GOLDEN))
    u = g["uncovered_cycles_two_stages"]
    assert lib.pgemm_model_uncovered_cycles(u["latency"], u["compute_per_tile"], u["stages"]) == u["expected"]
    # deeper rings cover more of the same latency; a single buffer covers none of it
    assert lib.pgemm_model_uncovered_cycles(500, 220, 4) == 0
    assert lib.pgemm_model_uncovered_cycles(500, 220, 1) == 500
    q = g["global_loads_per_output_128x64_K4096"]
    assert lib.pgemm_model_global_loads_per_output(q["bm"], q["bn"], q["K"]) == q["expected"]
    for key in ("page_kernel_lds_bytes", "page_kernel_single_buffer_lds_bytes"):
        s = g[key]
        assert lib.pgemm_model_lds_bytes(s["bm"], s["bn"], s["bk"], s["stages"], s["elem_bytes"],
                                         s["a_pad_elems_per_k"]) == s["expected"]
    c = g["compute_load_ratio_page_kernel_tile"]
    got = lib.pgemm_model_compute_load_ratio(c["bm"], c["bn"], c["bk"], c["elem_bytes"])
    assert abs(got - c["expected_num"] / c["expected_den"]) < 1e-12
    # square tiles: 2*B*B*BK / (2*B*BK*s) = B/s, independent of BK
    for b, bk, es in ((256, 32, 2), (256, 64, 2), (256, 128, 1), (128, 64, 4)):
        assert lib.pgemm_model_compute_load_ratio(b, b, bk, es) == b / es
    assert lib.pgemm_model_compute_load_ratio(0, 64, 16, 4) == 0


def test_planner_tables_cover_every_compiled_variant():
    """planner_tables.json (written by bench.py --retune, compiled in by
    build.py) has a class-model row for every DIRECT variant (tile class
    and ring depth) and a
    measured efficiency for every register-staged variant, so no compiled
    variant falls back to the planner's heuristic; values are fractions of
    peak and partial-round costs in [0, 1]; the compiled include matches the
    JSON."""
    from software_pipelined_tiled_loop_amd import build
    t = build.load_tables()
    cls = {(r["dtype"], tuple(r["tile"]), r["stages"]) for r in t["class_model"]}
    stg = {(r["dtype"], tuple(r["tile"]), r["stages"], r["producer"]) for r in t["staged_efficiency"]}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        tile = (v["tile_m"], v["tile_n"], v["tile_k"])
        if v["producer"] == "direct":
            assert (v["dtype"], tile, v["stages"]) in cls, v
        else:
            assert (v["dtype"], tile, v["stages"], v["producer"]) in stg, v
    for r in t["class_model"]:
        assert 0.05 < r["eff"] <= 1.0 and 0.0 <= r["lam"] <= 1.0, r
    for r in t["staged_efficiency"]:
        assert 0.02 < r["eff"] <= 1.0, r
    assert t["load_latency_cycles"] > 0 and t["prologue_cycles"] > 0
    for r in t["class_model"]:
        assert r["round_cycles"] >= 0 and r["first_round_cycles"] >= 0, r
    inc = open(os.path.join(build.GEN_DIR, "planner_tables.inc")).read()
    assert inc == build.tables_include(t)


def test_planner_tables_were_measured_on_these_kernel_sources():
    """planner_tables.json records the kernel source hash (kernel code,
    comments stripped, and the code-generation flags) it was measured on;
    after any kernel change the tables must be measured again (bench.py
    --retune) before they are trusted, as page "Double Buffering: Software
    Pipelining the K-Loop", section "What Could Be Improved", asks of the
    tile search."""
    import bench
    from software_pipelined_tiled_loop_amd import build
    assert build.load_tables()["kernel_source_hash"] == bench.kernel_source_hash()


def test_overlap_check_against_brute_force():
    """binding._regions_overlap against the sets of bytes two slices of one
    buffer touch: exact for equal row strides, never a missed overlap
    otherwise."""
    import random

    import torch
    rng = random.Random(5)
    for _ in range(3000):
        w1, w2 = rng.choice([(16, 16), (16, 24), (24, 16)])
        buf1, buf2 = torch.zeros(48 * w1), torch.zeros(48 * w2)
        X = buf1.view(48, w1)
        Y = (buf1.view(48, w1) if rng.random() < 0.7 else buf2.view(48, w2)) if w1 == w2 else buf1.view(-1, w2)
        xr, xc, yr, yc = rng.randint(0, 6), rng.randint(0, 8), rng.randint(0, 6), rng.randint(0, 8)
        xi, xj = rng.randint(0, 40), rng.randint(0, 8)
        yi, yj = rng.randint(0, 40), rng.randint(0, 8)
        Xs, Ys = X[xi:xi + xr, xj:xj + xc], Y[yi:yi + yr, yj:yj + yc]
        xr, xc, yr, yc = Xs.shape[0], Xs.shape[1], Ys.shape[0], Ys.shape[1]

        def cells(t, r, c):
            return {t.data_ptr() + (i * t.stride(0) + j) * 4 + b for i in range(r) for j in range(c) for b in range(4)}

        truth = bool(cells(Xs, xr, xc) & cells(Ys, yr, yc))
        got = lib._regions_overlap(Xs, xr, xc, Ys, yr, yc)
        if Xs.stride(0) == Ys.stride(0):
            assert got == truth, (xi, xj, xr, xc, yi, yj, yr, yc)
        else:
            assert got or not truth
