"""Benchmark of the software-pipelined GEMM on one MI355X.

One JSON line on stdout.  A "step" is one call of the whole hot path
(pgemm_gemm: plan, prologue, pipelined K loop, fused alpha/beta epilogue) on
the headline workload, fp32 SGEMM M = N = K = 4096, alpha = 1, beta = 0.5,
with inputs resident in HBM.  Untimed calls for --settle-ms (clock settling)
and W untimed warm-up steps, then K timed steps between HIP events on the
stream the kernels are launched on.

Also reported (same JSON line, key "reports"): int8 / bf16 / fp16 at 4096^3,
the stage-count sweep (1 vs 2 vs 3-4 stages) and producer comparison, and
the bf16 K-sweep with the ragged 4000 x 3968 x 4001 shape.  The oracle is
timed on a bounded sample of the headline workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 40] [--settle-ms 300] [--quick] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6, "i8": 5033.2}  # dense TFLOP/s (TOP/s), MI355X
HBM_PEAK_GBS = 8000.0
CLOCK_GHZ = 2.4  # the clock the dense peaks are quoted at
PAGE_SGEMM_GFLOPS = 32107.5  # 2-stage SGEMM 4096^3 on the first page's (unnamed NVIDIA) GPU


WORKLOADS = {
    "f32": dict(name="fp32 SGEMM M=N=K=4096 row-major alpha=1 beta=0.5", dtype="f32", M=4096, N=4096, K=4096,
                alpha=1.0, beta=0.5, seed="fp32_4096", data="seeded uniform[-1,1) fp32"),
    "i8": dict(name="int8 IGEMM M=N=K=4096 int32 out", dtype="i8", M=4096, N=4096, K=4096, alpha=1, beta=0,
               seed="int8_4096", data="seeded uniform int8 [-128,127]"),
    "bf16": dict(name="bf16 GEMM M=N=K=4096 fp32 out", dtype="bf16", M=4096, N=4096, K=4096, alpha=1.0,
                 beta=0.0, seed="half_4096", data="seeded normal(0,1) rounded to bf16"),
    "f16": dict(name="fp16 GEMM M=N=K=4096 fp32 out", dtype="f16", M=4096, N=4096, K=4096, alpha=1.0,
                beta=0.0, seed="half_4096", seed_variant=1, data="seeded normal(0,1) rounded to fp16"),
    "ragged": dict(name="bf16 GEMM M=4000 N=3968 K=4001 lda=4001 ldb=ldc=3968 fp32 out", dtype="bf16", M=4000,
                   N=3968, K=4001, lda=4001, ldb=3968, ldc=3968, alpha=1.0, beta=0.0, seed="bf16_k_sweep", seed_variant=9,
                   data="seeded normal(0,1) rounded to bf16"),
    "f32_256": dict(name="fp32 SGEMM M=N=K=256 alpha=1 beta=0", dtype="f32", M=256, N=256, K=256, alpha=1.0,
                    beta=0.0, seed="fp32_256", data="seeded uniform[-1,1) fp32"),
}
K_SWEEP = (32, 64, 256, 1024, 4096, 16384)
for _k in K_SWEEP:
    WORKLOADS["bf16_k%d" % _k] = dict(name="bf16 GEMM M=N=4096 K=%d fp32 out" % _k, dtype="bf16", M=4096, N=4096, K=_k,
                                      alpha=1.0, beta=0.0, seed="bf16_k_sweep", seed_variant=_k % 97,
                                      data="seeded normal(0,1) rounded to bf16")


def _code_only(text: str) -> str:
    """C++ source without comments and blank runs: what the compiler sees."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())


KERNEL_FILES = ("pgemm_kernel.hpp", "kern_f32.hip", "kern_f16.hip", "kern_bf16.hip", "kern_i8.hip")


def kernel_source_hash() -> str:
    """Hash of the code (comments stripped) of the files that define the
    kernels and their compiled variants, and of the hipcc flags they are built
    with -- not the host launcher or planner: HBM traffic measured on one
    version stays valid while only comments or host code change."""
    from software_pipelined_tiled_loop_amd import build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "software_pipelined_tiled_loop_amd", "csrc")
    for f in KERNEL_FILES:
        h.update(_code_only(open(os.path.join(csrc, f)).read()).encode())
    # code-generation flags only: include paths name this checkout's location
    h.update(" ".join(f for f in build.HIPCC_FLAGS if not f.startswith("-I")).encode())
    return h.hexdigest()[:16]


def make_device_operands(dtype, M, N, K, seed, alpha, beta, lda=None, ldb=None, ldc=None):
    from software_pipelined_tiled_loop_amd import inputs
    op = inputs.make_operands(dtype, M, N, K, seed=seed, alpha=alpha, beta=beta, lda=lda, ldb=ldb, ldc=ldc)
    return op, op.A.cuda(), op.B.cuda(), op.C.cuda()


def workload_operands(name):
    """Seeded host operands of a named workload (the tests build the same ones)."""
    from software_pipelined_tiled_loop_amd import inputs
    w = WORKLOADS[name]
    return inputs.make_operands(w["dtype"], w["M"], w["N"], w["K"],
                                seed=inputs.seed_for(w["seed"], w.get("seed_variant", 0)), alpha=w["alpha"],
                                beta=w["beta"], lda=w.get("lda"), ldb=w.get("ldb"), ldc=w.get("ldc"))


def is_aligned(name):
    """The pgemm_aligned class of a workload: which operands hold whole 16-byte
    chunks per row (A: K elements, B: N elements) -- 1 both, 2 A only, 3 B
    only, 0 none.  Row starts may have any element alignment."""
    from software_pipelined_tiled_loop_amd import inputs
    w = WORKLOADS[name]
    K, N, es = w["K"], w["N"], inputs.ELEM_BYTES[w["dtype"]]
    a = K == 0 or K * es % 16 == 0
    b = K == 0 or N * es % 16 == 0
    return 1 if a and b else 2 if a else 3 if b else 0


WARMUP_MS = 150.0
TRIAL_MS = 5.0


def time_calls(call, reps=None, warmup=None, trials=5):
    """ms per call of `call` (which launches on the current stream): the
    median over `trials` of the average over `reps` back-to-back calls (HIP
    events on that stream), `reps` chosen so that a trial lasts about
    TRIAL_MS (at least 20 calls).  The median keeps a disturbed trial (clock
    ramp, a profiler's buffer flush) out of the reported sweep points; with
    20-launch trials, kernels of ~15 us varied by 10 % between identical
    runs.  Warm-up runs the call for about WARMUP_MS first: after the GPU has
    idled (while the host draws the next operands) its clock takes on the
    order of 100 ms of load to settle, and with a 20 ms warm-up the first of
    several successive timings of one kernel read 10-13 % low."""
    import torch
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if warmup is None:
        call()
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        per = max(e0.elapsed_time(e1), 1e-3)
        warmup = max(3, min(20000, int(WARMUP_MS / per)))
        if reps is None:
            reps = max(20, min(2000, int(TRIAL_MS / per)))
    if reps is None:
        reps = 20
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(trials):
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    return sorted(times)[len(times) // 2]


def time_gemm(lib, op, A, B, C, stages=0, producer=None, tile=None, reps=None, warmup=None, trials=5):
    """ms per pgemm call (see time_calls)."""
    import torch
    stream = torch.cuda.current_stream()
    opts = lib._opts(producer, tile)

    def call():
        r = lib.pgemm_gemm_ex(op.M, op.N, op.K, op.alpha, A, op.lda, B, op.ldb, op.beta, C, op.ldc, op.dtype,
                              stages, opts, stream)
        if r != 0:
            raise lib.PgemmError(r)

    return time_calls(call, reps=reps, warmup=warmup, trials=trials)


def tflops(M, N, K, ms):
    return 2.0 * M * N * K / (ms * 1e-3) / 1e12


def algorithmic_bytes(dtype, M, N, K, beta):
    from software_pipelined_tiled_loop_amd import inputs
    s = inputs.ELEM_BYTES[dtype]
    return M * K * s + K * N * s + M * N * 4 * (2 if beta != 0 else 1)


def plan_of(lib, dtype, M, N, K, stages=0, producer=None, tile=None, aligned=1):
    r, p = lib.pgemm_plan(M, N, K, dtype, stages, aligned, lib._opts(producer, tile))
    return p if r == 0 else None


def cpu_baseline(target_s=12.0):
    """The oracle on a bounded sample of the headline workload: the first R
    rows of the fp32 4096^3 GEMM (R chosen for ~target_s of CPU work)."""
    import oracle
    from software_pipelined_tiled_loop_amd import inputs
    M = N = K = 4096
    op = inputs.make_operands("f32", M, N, K, seed=inputs.seed_for("fp32_4096"), alpha=1.0, beta=0.5)
    A, B, C0 = op.numpy_views()
    threads = oracle.num_threads()
    rows = 16
    t0 = time.perf_counter()
    oracle.gemm("f32", rows, N, K, 1.0, A[:rows], B, 0.5, C0[:rows])
    t = time.perf_counter() - t0
    rows = int(min(M, max(16, rows * target_s / max(t, 1e-3))))
    t0 = time.perf_counter()
    oracle.gemm("f32", rows, N, K, 1.0, A[:rows], B, 0.5, C0[:rows])
    t = time.perf_counter() - t0
    return {"value": round(tflops(rows, N, K, t * 1e3), 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(t, 3),
            "sample": "first %d of 4096 rows of the fp32 4096^3 GEMM (alpha=1, beta=0.5), fp64 accumulation"
                      % rows}


def planner_tables_current(src_hash):
    """Whether the planner's measured tables were taken on these kernel
    sources (False: re-run bench.py --retune)."""
    from software_pipelined_tiled_loop_amd import build
    return build.load_tables().get("kernel_source_hash") == src_hash


def load_traffic(kernel_key, src_hash):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None
    when missing or taken on another version of the kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(p))
    except Exception:
        return None
    e = d.get(kernel_key)
    if not e or e.get("kernel_source_hash") != src_hash:
        return None
    return e.get("bytes_per_launch")


# ---- the re-run tile and depth search (planner_tables.json) ------------------------

# Shapes the planner's picks are checked on: the benchmark's, squares, tall,
# wide and short-K problems per dtype.
CHECK_SHAPES = (
    ("f32", 4096, 4096, 4096), ("f16", 4096, 4096, 4096), ("bf16", 4096, 4096, 4096), ("i8", 4096, 4096, 4096),
    ("bf16", 3000, 3000, 3000), ("bf16", 6144, 6144, 6144), ("bf16", 5120, 5120, 5120), ("bf16", 2048, 2048, 2048),
    ("f32", 1024, 1024, 1024), ("f32", 2048, 2048, 2048), ("f16", 4096, 4096, 256), ("i8", 2560, 2560, 2560),
    ("f32", 8192, 8192, 1024), ("f32", 4096, 4096, 512), ("f32", 8192, 4096, 4096), ("f32", 8192, 8192, 64),
    ("f32", 4096, 4096, 32), ("bf16", 4096, 4096, 32), ("bf16", 4096, 4096, 256), ("bf16", 4096, 4096, 1024),
    ("i8", 8192, 8192, 1024), ("f16", 1024, 8192, 4096),
)


def _tflops_of(lib, op, A, B, C, stages=0, producer=None, tile=None):
    return tflops(op.M, op.N, op.K, time_gemm(lib, op, A, B, C, stages=stages, producer=producer, tile=tile))


def _device(op):
    return op.A.cuda(), op.B.cuda(), op.C.cuda()


def _variants_of(lib, dt):
    return [v for v in (lib.pgemm_variant_info(i) for i in range(lib.pgemm_num_variants())) if v["dtype"] == dt]


def _misaligned_problem(dt, which):
    """The problem register-staged producers are measured on: the ragged
    4000 x 3968 x 4001 shape with A misaligned (lda = K = 4001) for GENERIC
    and STAGED_A, or 4000 x 3969 x 4000 with B misaligned (ldb = N = 3969)
    for STAGED_B."""
    from software_pipelined_tiled_loop_amd import inputs
    if which == "a":
        return inputs.make_operands(dt, 4000, 3968, 4001, seed=inputs.seed_for("bf16_k_sweep", 9), lda=4001, ldb=3968)
    return inputs.make_operands(dt, 4000, 3969, 4000, seed=inputs.seed_for("bf16_k_sweep", 11), lda=4000, ldb=3969)


def rounds_units(lib, dt, o, tile, S):
    """Rounds of co-resident workgroups and workgroup-units on the busiest CU
    for problem o with DIRECT tile class `tile` at depth S."""
    p = plan_of(lib, dt, o.M, o.N, o.K, S, "direct", tile)
    n = -(-(-(-o.M // tile[0]) * -(-o.N // tile[1])) // 256)   # tiles on the busiest CU
    occ = p["wg_per_cu"]
    return -(-n // occ), (n // occ) * occ + n % occ


def retune(lib, torch, out_path):
    """Time every compiled variant on the problems behind each planner
    constant and write planner_tables.json to out_path (copy it into the
    package and rebuild)."""
    from software_pipelined_tiled_loop_amd import build as bld
    from software_pipelined_tiled_loop_amd import inputs
    old = bld.load_tables()
    log = {}
    # Per DIRECT tile class: the fixed cost of the first round of workgroups
    # (prologue with cold first loads, epilogue and C store) and of each later
    # round (whose start overlaps the previous round's tail), fitted at the
    # class's fastest depth from three problems -- 4096 x 4096 outputs at
    # K = 4096 and K = 256, 8192 x 8192 at K = 128; per ring depth of the
    # class, the cost of a K tile from that depth's 4096^3 time; the model is
    #   cycles = first_round + (rounds - 1) * round + units * (2*BM*BN*K) / (eff * dense flops per CU-clock)
    # (the partial-round cost lam from one workgroup per CU against a full
    # round of co-resident ones, at that depth, when two or more fit).
    classes = []
    for dt in ("f32", "f16", "bf16", "i8"):
        by_class = {}
        op = workload_operands(dt)
        A, B, C = _device(op)
        for v in _variants_of(lib, dt):
            if v["producer"] != "direct":
                continue
            tile = (v["tile_m"], v["tile_n"], v["tile_k"])
            by_class.setdefault(tile, {})[v["stages"]] = _tflops_of(lib, op, A, B, C, v["stages"], "direct", tile)
        del A, B, C
        short = inputs.make_operands(dt, 4096, 4096, 256, seed=inputs.seed_for("bf16_k_sweep", 5))
        wide = inputs.make_operands(dt, 8192, 8192, 128, seed=inputs.seed_for("bf16_k_sweep", 6))
        probs = [(o,) + _device(o) for o in (op, short, wide)]
        import numpy as np
        fpc = {"f32": 64.0, "i8": 2048.0}.get(dt, 1024.0)

        def fit_points(tile, S):
            pts = []
            for o, a, b, c in probs:
                ms = time_gemm(lib, o, a, b, c, stages=S, producer="direct", tile=tile)
                pts.append((o.K, ms * 1e-3 * 2.4e9) + rounds_units(lib, dt, o, tile, S))
            return pts

        for tile, by_s in sorted(by_class.items()):
            # fixed costs from the depth that runs 4096^3 fastest: three
            # problems, t = units * K * c + first + (rounds - 1) * later
            s_ref = max(by_s, key=lambda S: by_s[S])
            pts = fit_points(tile, s_ref)
            mat = np.array([[u * k, 1.0, r - 1.0] for k, t, r, u in pts])
            rhs = np.array([t for k, t, r, u in pts])
            c_k, first, later = np.linalg.solve(mat, rhs)
            first, round_cycles = max(0.0, float(first)), max(0.0, float(later))
            for S in sorted(by_s):
                # each depth's K-tile cost from its own 4096^3 time, with the
                # class's fixed costs
                r4, u4 = rounds_units(lib, dt, op, tile, S)
                t4 = 2.0 * op.M * op.N * op.K / (by_s[S] * 1e12) * 2.4e9
                c_s = (t4 - first - (r4 - 1) * round_cycles) / (u4 * op.K)
                eff = 2.0 * tile[0] * tile[1] / (max(c_s, 1e-9) * 4.0 * fpc)
                # partial last round: one workgroup per CU against a full
                # round of co-resident ones at this depth
                r, p1 = lib.pgemm_plan(16 * tile[0], 16 * tile[1], 4096, dt, S, 1, {"tile": tile, "producer": "direct"})
                occ, lam = p1["wg_per_cu"], 0.0
                if occ >= 2:
                    t = {}
                    for rows in (16 * tile[0], 16 * tile[0] * occ):
                        o = inputs.make_operands(dt, rows, 16 * tile[1], 4096, seed=77)
                        a, b, c = _device(o)
                        t[rows] = time_gemm(lib, o, a, b, c, stages=S, producer="direct", tile=tile)
                        del a, b, c
                    lam = min(1.0, max(0.0, (occ * t[16 * tile[0]] / t[16 * tile[0] * occ] - 1.0) / (occ - 1)))
                classes.append({"dtype": dt, "tile": list(tile), "stages": S, "eff": round(min(max(eff, 0.06), 1.0), 4),
                                "lam": round(lam, 3), "first_round_cycles": round(first, 0),
                                "round_cycles": round(round_cycles, 0)})
                log["%s %dx%dx%d s%d" % (dt, *tile, S)] = {"tflops_4096": round(by_s[S], 1),
                                                          "partial_round_workgroups_per_cu": occ}
            log["%s %dx%dx%d" % (dt, *tile)] = {"fit_depth": s_ref,
                                               "fit_points_K_cycles_rounds_units": [[k, round(t), r, u] for k, t, r, u in pts]}
        del probs
    # register-staged variants
    staged = []
    for dt in ("f32", "f16", "bf16", "i8"):
        vs = [v for v in _variants_of(lib, dt) if v["producer"] != "direct"]
        groups = {"register": workload_operands(dt), "a": _misaligned_problem(dt, "a"), "b": _misaligned_problem(dt, "b")}
        for key, op in groups.items():
            A, B, C = _device(op)
            for v in vs:
                want = {"register": ("register",), "a": ("generic", "staged_a"), "b": ("staged_b",)}[key]
                if v["producer"] not in want:
                    continue
                tile = (v["tile_m"], v["tile_n"], v["tile_k"])
                t = _tflops_of(lib, op, A, B, C, v["stages"], v["producer"], tile)
                staged.append({"dtype": dt, "tile": list(tile), "stages": v["stages"], "producer": v["producer"],
                               "eff": round(t / PEAK[dt], 4)})
            del A, B, C
    # load latency: the single-buffer kernels' vmcnt wait per K tile
    prof = wait_profile(lib, torch, runs=10)
    latency = max(v["vmcnt_cycles_per_edge"] for k, v in prof.items() if k.endswith(" s1") and "256x256" in k)
    tables = {"_about": old["_about"], "kernel_source_hash": kernel_source_hash(),
              "load_latency_cycles": round(float(latency), 1), "prologue_cycles": old["prologue_cycles"],
              "tie_margin": old["tie_margin"],
              "class_model": classes, "staged_efficiency": staged}
    bld.dump_tables(tables, out_path)
    log["load_latency_from"] = {k: v["vmcnt_cycles_per_edge"] for k, v in prof.items() if k.endswith(" s1")}
    return log


def planner_check(lib, torch):
    """For each check shape: the planner's plan against every compiled DIRECT
    variant (every tile class at every ring depth), best measured over the
    planner's pick."""
    from software_pipelined_tiled_loop_amd import inputs
    out = {}
    for dt, M, N, K in CHECK_SHAPES:
        op = inputs.make_operands(dt, M, N, K, seed=1000 + M % 997 + K % 89)
        A, B, C = _device(op)
        auto = _tflops_of(lib, op, A, B, C)
        plan = plan_label(plan_of(lib, dt, M, N, K))
        best, best_label = 0.0, None
        variants = sorted({((v["tile_m"], v["tile_n"], v["tile_k"]), v["stages"]) for v in _variants_of(lib, dt)
                           if v["producer"] == "direct"})
        per = {}
        for tile, S in variants:
            lab = plan_label(plan_of(lib, dt, M, N, K, S, "direct", tile))
            if lab in per:
                continue  # a depth beyond the number of K tiles runs as a shallower one
            t = _tflops_of(lib, op, A, B, C, S, "direct", tile)
            per[lab] = round(t, 1)
            if t > best:
                best, best_label = t, lab
        out["%s %dx%dx%d" % (dt, M, N, K)] = {"planner": plan, "planner_tflops": round(auto, 1), "best": best_label,
                                              "best_tflops": round(best, 1), "best_over_planner": round(best / auto, 3),
                                              "classes": per}
        del A, B, C
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="f32", choices=sorted(WORKLOADS),
                    help="timed workload (default: the fp32 4096^3 headline); others are for profiling")
    ap.add_argument("--stages", type=int, default=0, help="ring depth (0 = planner)")
    ap.add_argument("--producer", default=None, choices=[None, "direct", "register", "generic", "staged_a", "staged_b"])
    ap.add_argument("--tile", default=None, help="BMxBNxBK, e.g. 256x256x32")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed calls before the warm-up, for this long, so the clock has settled (0 = off)")
    ap.add_argument("--retune", action="store_true",
                    help="re-run the tile/depth search and write the planner's tables (--retune-out)")
    ap.add_argument("--retune-out", default=os.path.join(os.getcwd(), "planner_tables.retuned.json"))
    ap.add_argument("--planner-check", action="store_true",
                    help="time every tile class on the check shapes against the planner's pick")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (scales HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library runs each GEMM on a single MI355X and has no "
              "multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from software_pipelined_tiled_loop_amd import binding as lib
    from software_pipelined_tiled_loop_amd import inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    src_hash = kernel_source_hash()
    if args.retune or args.planner_check:
        rep = {}
        if args.retune:
            os.makedirs(os.path.dirname(os.path.abspath(args.retune_out)), exist_ok=True)
            rep["retune"] = retune(lib, torch, args.retune_out)
            rep["retune"]["written"] = args.retune_out
        if args.planner_check:
            rep["planner_check"] = planner_check(lib, torch)
        print(json.dumps(rep))
        return

    # ---- timed workload (default: fp32 SGEMM 4096^3, alpha=1, beta=0.5) ----
    w = WORKLOADS[args.workload]
    dt, M, N, K, alpha, beta = w["dtype"], w["M"], w["N"], w["K"], w["alpha"], w["beta"]
    tile = tuple(int(x) for x in args.tile.split("x")) if args.tile else None
    lda, ldb, ldc = w.get("lda", K), w.get("ldb", N), w.get("ldc", N)
    aligned = is_aligned(args.workload)
    op, A, B, C = make_device_operands(dt, M, N, K, inputs.seed_for(w["seed"], w.get("seed_variant", 0)), alpha, beta,
                                       lda, ldb, ldc)
    plan = plan_of(lib, dt, M, N, K, args.stages, args.producer, tile, aligned=aligned)
    if plan is None:
        print("no compiled variant for these options", file=sys.stderr)
        sys.exit(1)
    # the compute/load ratio of the plan's tile, reported as a diagnostic (the
    # page's thresholds for it are not used to choose)
    plan["compute_load_ratio"] = round(lib.pgemm_model_compute_load_ratio(
        plan["tile_m"], plan["tile_n"], plan["tile_k"], inputs.ELEM_BYTES[dt]), 2)
    stream = torch.cuda.current_stream()
    opts = lib._opts(args.producer, tile)

    def step():
        r = lib.pgemm_gemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dt, args.stages, opts, stream)
        if r != 0:
            raise lib.PgemmError(r)

    if args.copy_calibration:
        # a plain copy of 512 MiB: reads and writes exactly 512 MiB of HBM
        src = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Clock settling before the W warm-up steps: from an idle GPU the shader
    # clock needs on the order of 100 ms of load to reach its steady value
    # (the first dispatches of the headline kernel ran 15-20 % long), so a
    # short warm-up would leave the ramp inside the timed window.  These calls
    # are untimed, like the warm-up; the timed region holds exactly K steps.
    settle_calls = 0
    if args.settle_ms > 0:
        t_end = time.perf_counter() + args.settle_ms / 1e3
        while time.perf_counter() < t_end:
            for _ in range(8):
                step()
            settle_calls += 8
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    value = tflops(M, N, K, ms)
    kernel_key = "%s_%dx%dx%d_s%d_%s" % (dt, plan["tile_m"], plan["tile_n"], plan["tile_k"], plan["stages"],
                                         plan["producer"])
    traffic = load_traffic(kernel_key, src_hash)
    roofline = {"bound": "mfma", "achieved": round(value, 3), "peak": PEAK[dt], "unit": "TFLOP/s",
                "frac": round(value / PEAK[dt], 4), "traffic": traffic,
                "kernel": kernel_key, "algorithmic_flops_per_launch": 2 * M * N * K,
                "algorithmic_bytes_per_launch": algorithmic_bytes(dt, M, N, K, beta)}
    del A, B, C

    reports = {}
    if not args.quick:
        reports = run_reports(lib, torch)

    out = {
        "metric": "GEMM TFLOP/s (int8 TOP/s) at 4096^3 and % of MI355X dtype peak; K-sweep by stages",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": round(value * 1000.0 / PAGE_SGEMM_GFLOPS, 4) if args.workload == "f32" else None,
        "dtype": dt, "data": "synthetic (%s)" % w["data"],
        "config": {"workload": w["name"], "M": M, "N": N, "K": K,
                   "pct_of_peak": round(100.0 * value / PEAK[dt], 2), "plan": plan,
                   "wall_s_timed_region": round(t_wall, 4), "clock_settle_calls": settle_calls,
                   "kernel_source_hash": src_hash, "planner_tables_current": planner_tables_current(src_hash)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline and args.workload == "f32":
        out["cpu_baseline"] = cpu_baseline()
    if reports:
        out["reports"] = reports
    print(json.dumps(out))


def plan_label(p):
    return "%dx%dx%d s%d %s" % (p["tile_m"], p["tile_n"], p["tile_k"], p["stages"], p["producer"])


def report_points(lib):
    """Every GEMM launch the report times, as dicts with the report section,
    the point's label, the workload it runs on and the launch options.  The
    full-size parity tests walk this same list, so every timed variant is also
    compared with the oracle on its full output.

      * i8_4096, bf16_4096, f16_4096: the planner's plan and every compiled
        vector-producer variant (tile x depth x producer);
      * f32_4096_page_tile: the pages' 128 x 64 x 16 tile at 1 and 2 stages
        and the planner's plan on the headline workload;
      * f32_256_pages_tile: the same tile at 1 and 2 stages on fp32 256^3;
      * bf16_k_sweep: per K, the planner's plan at each ring depth 1..4 and
        with the depth left to it; then the ragged shape."""
    pts = []
    for sec, name in (("i8_4096", "i8"), ("bf16_4096", "bf16"), ("f16_4096", "f16")):
        dt = WORKLOADS[name]["dtype"]
        pts.append(dict(section=sec, key="auto", workload=name, stages=0, producer=None, tile=None))
        for i in range(lib.pgemm_num_variants()):
            v = lib.pgemm_variant_info(i)
            if v["dtype"] != dt or v["producer"] == "generic":
                continue
            pts.append(dict(section=sec, key=plan_label(v), workload=name, stages=v["stages"],
                            producer=v["producer"], tile=(v["tile_m"], v["tile_n"], v["tile_k"])))
    for s in (1, 2):
        pts.append(dict(section="f32_4096_page_tile", key="128x64x16 s%d direct" % s, workload="f32", stages=s,
                        producer="direct", tile=(128, 64, 16)))
    pts.append(dict(section="f32_4096_page_tile", key="auto", workload="f32", stages=0, producer=None, tile=None))
    for s in (1, 2):
        pts.append(dict(section="f32_256_pages_tile", key="128x64x16 s%d direct" % s, workload="f32_256", stages=s,
                        producer="direct", tile=(128, 64, 16)))
    for K in K_SWEEP:
        for s in (1, 2, 3, 4):
            pts.append(dict(section="bf16_k_sweep", key="K%d s%d" % (K, s), workload="bf16_k%d" % K, stages=s,
                            producer=None, tile=None))
        pts.append(dict(section="bf16_k_sweep", key="K%d auto" % K, workload="bf16_k%d" % K, stages=0,
                        producer=None, tile=None))
    pts.append(dict(section="bf16_k_sweep", key="ragged auto", workload="ragged", stages=0, producer=None, tile=None))
    return pts


def pages_context(rep):
    """The pages' own figures, measured on other hardware (context only),
    beside the same ratios measured here: the first page's gain from its
    2-stage SGEMM over its 1-stage one (kernel 11 over kernel 10 on its
    128 x 64 x 16 tile, 4.660 -> 4.281 ms on its unnamed NVIDIA GPU, where the
    two ran at 81.9 % and 89.2 % of the vendor library), against the same
    tile class at 2 stages over 1 here; and the German page's gain from
    asynchronous-copy pipelining on a 4096^3 int8 GEMM on GA104, against the
    int8 256 x 256 x 128 tile here at 2 stages over 1."""
    f = rep["f32_4096_page_tile"]
    v8 = rep["i8_4096"]["variants"]
    s1, s2 = v8.get("256x256x128 s1 direct"), v8.get("256x256x128 s2 direct")
    f1, f2 = f.get("128x64x16 s1 direct"), f.get("128x64x16 s2 direct")
    return {
        "sgemm_2stage_gain_pct": {
            "pages": {"kernel 11 over kernel 10": round(100 * (4.660 / 4.281 - 1), 1),
                      "share of vendor library": {"1 stage": 81.9, "2 stages": 89.2},
                      "hardware": "first page's NVIDIA GPU (model not named)"},
            "here": {"128x64x16 s2 over s1": round(100 * (f2 / f1 - 1), 1) if f1 and f2 else None,
                     "hardware": "MI355X"}},
        "int8_4096_pipelining_gain_pct": {
            "pages": {"async-copy pipeline over none": 35, "hardware": "GA104"},
            "here": {"256x256x128 s2 over s1": round(100 * (s2 / s1 - 1), 1) if s1 and s2 else None,
                     "hardware": "MI355X"}},
    }


def _graph_us(lib, torch, op, A, B, C, p):
    """Per-call time of 50 calls replayed from a HIP graph (launch overhead
    out of the way on the small, launch-bound problem)."""
    opts = lib._opts(p["producer"], p["tile"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(50):
            lib.pgemm_gemm_ex(op.M, op.N, op.K, op.alpha, A, op.lda, B, op.ldb, op.beta, C, op.ldc, op.dtype,
                              p["stages"], opts, None)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        g.replay()
    e1.record()
    e1.synchronize()
    del g
    return e0.elapsed_time(e1) / 250 * 1e3


CEILING_ITERS = {"f32": 1024, "f16": 8192, "bf16": 8192, "i8": 8192}
# (workload, tile, stages): the tile classes of the 4096^3 plans, and the bf16
# 256 x 256 x 32 class at each ring depth
STREAM_POINTS = (("bf16", (256, 256, 64), 2), ("f16", (256, 256, 64), 2), ("i8", (256, 256, 128), 2),
                 ("f32", (128, 64, 16), 2), ("f32", (256, 256, 32), 2), ("bf16", (256, 256, 32), 2),
                 ("bf16", (256, 256, 32), 3), ("bf16", (256, 256, 32), 4))


def ceilings(lib, torch):
    """The two diagnostics that bound the GEMM (pgemm_diag_*): the matrix
    cores alone on random and on zero operands (% of dense peak; also with
    one wave per SIMD and with 32x32 blocks), and the
    producer alone -- the LDS-DMA pieces of a tile class on the 4096^3
    workload with no arithmetic -- as LDS bytes per second and as the GEMM
    rate it could feed (2MNK over its time)."""
    out = {"mfma_only": {}, "lds_stream": {}}
    grid = 256
    buf = torch.zeros(grid * 8, dtype=torch.float32, device="cuda")
    clock = torch.zeros(grid * 4, dtype=torch.int64, device="cuda")
    for dt in ("f32", "f16", "bf16", "i8"):
        row = {}
        for zero in (0, 1):
            box = {}

            def call():
                r, box["flops"] = lib.pgemm_diag_mfma_ceiling(dt, zero, CEILING_ITERS[dt], grid, 12345, buf,
                                                              clock=clock)
                if r != 0:
                    raise lib.PgemmError(r)

            ms = time_calls(call)
            t = box["flops"] / (ms * 1e-3) / 1e12
            row["zero" if zero else "random"] = {"tflops": round(t, 1), "pct_peak": round(100 * t / PEAK[dt], 1),
                                                 "clock_ghz": clock_ghz(clock, grid)}
        out["mfma_only"][dt] = row
    # one wave per SIMD against two, 16x16 blocks against 32x32 ones: what a
    # single issuing wave keeps busy, and what each block shape costs in clock
    out["mfma_issue"] = {}
    for dt in ("f16", "bf16", "i8"):
        row = {}
        for waves, blk in ((2, 16), (1, 16), (2, 32), (1, 32)):
            for zero in (0, 1):
                box = {}

                def call():
                    r, box["flops"] = lib.pgemm_diag_mfma_ceiling(dt, zero, CEILING_ITERS[dt], grid, 12345, buf,
                                                                  clock=clock, waves_per_simd=waves, block=blk)
                    if r != 0:
                        raise lib.PgemmError(r)

                ms = time_calls(call)
                t = box["flops"] / (ms * 1e-3) / 1e12
                row["%dx%d %d wave%s/SIMD %s" % (blk, blk, waves, "s" if waves > 1 else "", "zero" if zero else "random")] = {
                    "tflops": round(t, 1), "pct_peak": round(100 * t / PEAK[dt], 1), "clock_ghz": clock_ghz(clock, grid)}
        out["mfma_issue"][dt] = row
    for wl, tile, S in STREAM_POINTS:
        op = workload_operands(wl)
        A, B = op.A.cuda(), op.B.cuda()
        box = {}

        def call():
            r, box["bytes"] = lib.pgemm_diag_lds_stream(op.M, op.N, op.K, A, op.lda, B, op.ldb, op.dtype, tile, S)
            if r != 0:
                raise lib.PgemmError(r)

        ms = time_calls(call)
        t = tflops(op.M, op.N, op.K, ms)
        out["lds_stream"]["%s %dx%dx%d s%d" % (op.dtype, tile[0], tile[1], tile[2], S)] = {
            "us": round(ms * 1e3, 2), "TBs": round(box["bytes"] / (ms * 1e-3) / 1e12, 2),
            "gemm_tflops_fed": round(t, 1), "pct_peak_fed": round(100 * t / PEAK[op.dtype], 1)}
        del A, B
    return out


def clock_ghz(clock, n):
    """Mean shader clock (GHz) over the first n workgroups of a diagnostic's
    clock stamps: shader-clock span over the 100 MHz span of each."""
    c = clock.view(-1, 4)[:n].cpu().double()
    return round(float(((c[:, 2] - c[:, 0]) / ((c[:, 3] - c[:, 1]) / 100e6)).mean()) / 1e9, 3)


# The parts ladder (pgemm_diag_parts): the steps, each adding one part of the
# K loop's steady state, and the planner's 4096^3 class of each dtype at two
# stages.
PARTS_LADDER = (("mfma only", 0), ("+ A reads", 4), ("B reads only", 8), ("+ A and B reads", 12),
                ("+ barrier", 14), ("+ LDS-DMA (the GEMM)", 15))
PARTS_POINTS = (("bf16", (256, 256, 64)), ("f16", (256, 256, 64)), ("i8", (256, 256, 128)), ("f32", (128, 64, 16)))


def parts_ladder(lib, torch):
    """The GEMM kernel of each 4096^3 class built with parts of its K loop
    left out (pgemm_diag_parts), from the MFMAs alone to the whole loop: the
    rate of each step, the shader clock it ran at (stamped by the kernel),
    and its MFMA share at that clock (rate over the dense peak scaled to the
    clock).  What each part costs, in rate and in clock."""
    out = {}
    for wl, tile in PARTS_POINTS:
        op = workload_operands(wl)
        A, B, C = op.A.cuda(), op.B.cuda(), op.C.cuda()
        tiles = -(-op.M // tile[0]) * -(-op.N // tile[1])
        grid = -(-tiles // 8) * 8
        clock = torch.zeros(grid * 4, dtype=torch.int64, device="cuda")
        row = {}
        for label, parts in PARTS_LADDER:
            def call():
                r = lib.pgemm_diag_parts(op.M, op.N, op.K, A, op.lda, B, op.ldb, C, op.ldc, op.dtype, tile, 2, parts,
                                         clock, clock.numel())
                if r != 0:
                    raise lib.PgemmError(r)
            ms = time_calls(call)
            t = tflops(op.M, op.N, op.K, ms)
            ghz = clock_ghz(clock, tiles)
            row[label] = {"us": round(ms * 1e3, 2), "tflops": round(t, 1), "pct_peak": round(100 * t / PEAK[wl], 1),
                          "clock_ghz": ghz, "mfma_share_at_clock": round(t / (PEAK[wl] * ghz / CLOCK_GHZ), 3)}
        out["%s %dx%dx%d s2" % (op.dtype, tile[0], tile[1], tile[2])] = row
        del A, B, C, clock
    return out


# (workload, tile): the planner's 4096^3 classes, profiled at one and two stages
PROFILE_POINTS = (("bf16", (256, 256, 64)), ("f16", (256, 256, 64)), ("i8", (256, 256, 128)), ("f32", (128, 64, 16)),
                  ("f32", (256, 256, 32)))


def _warm_then_run(call, torch, runs):
    """Run `call` for about WARMUP_MS (the clock settles under load), then
    `runs` more times; the output of the last one is what is read."""
    t_end = time.perf_counter() + WARMUP_MS / 1e3
    while time.perf_counter() < t_end:
        for _ in range(10):
            call()
        torch.cuda.synchronize()
    for _ in range(runs):
        call()
    torch.cuda.synchronize()


def wait_profile(lib, torch, runs=20):
    """Where the waves of a ready edge wait (pgemm_diag_wait_profile: the
    GEMM kernel built with clock stamps around its waits), at one and two
    stages of each 4096^3 class: the share of the K loop's wave-cycles spent
    in the vmcnt wait for the K tile's loads, and in the workgroup barrier
    after it.  The last of `runs` back-to-back launches after the warm-up
    is read (clock settled)."""
    out = {}
    for wl, tile in PROFILE_POINTS:
        op = workload_operands(wl)
        A, B, C = op.A.cuda(), op.B.cuda(), op.C.cuda()
        tiles = -(-op.M // tile[0]) * -(-op.N // tile[1])
        grid = -(-tiles // 8) * 8
        nw = 8 if tile[0] * tile[1] >= 256 * 256 else 4
        buf = torch.zeros(grid * nw * 8, dtype=torch.int64, device="cuda")
        for S in (1, 2):
            def call():
                r = lib.pgemm_diag_wait_profile(op.M, op.N, op.K, A, op.lda, B, op.ldb, C, op.ldc, op.dtype, tile, S,
                                                buf, buf.numel())
                if r != 0:
                    raise lib.PgemmError(r)
            _warm_then_run(call, torch, runs)
            v = buf.view(grid, nw, 8)[:tiles].cpu().double()
            vm, bar, n, loop = (float(v[..., i].sum()) for i in range(4))
            out["%s %dx%dx%d s%d" % (op.dtype, tile[0], tile[1], tile[2], S)] = {
                "vmcnt_wait_share": round(vm / loop, 4), "barrier_wait_share": round(bar / loop, 4),
                "ready_edges_per_wave": round(n / (tiles * nw), 2),
                "vmcnt_cycles_per_edge": round(vm / max(n, 1), 1), "barrier_cycles_per_edge": round(bar / max(n, 1), 1),
                "loop_cycles_per_edge": round(loop / max(n, 1), 1)}
        del A, B, C, buf
    return out


# (label, workload, tile, stages): the short-K point with the plan the
# planner picks and the designs with more, smaller tiles per CU
TIMELINE_POINTS = (("256x256x64 s2 (planner)", "bf16_k1024", (256, 256, 64), 2),
                   ("128x128x64 s2", "bf16_k1024", (128, 128, 64), 2),
                   ("128x128x64 s3", "bf16_k1024", (128, 128, 64), 3),
                   ("256x256x64 s2 at K=4096", "bf16", (256, 256, 64), 2))


def timeline(lib, torch, runs=20):
    """Per-workgroup timeline of a launch on the GPU's 100 MHz clock (the
    wait-profile build): for each workgroup its start, the end of its
    prologue (first ready edge), the end of its K loop and the completion of
    its C stores (wave 0 of each workgroup).  Reported as the launch's span
    and the median / extreme phase times over workgroups, in microseconds:
    where a short-K launch spends its time (page "Software pipelines and
    asynchronous copies", section "Worked example": prologue and epilogue
    occupy a large fraction at short K)."""
    import numpy as np
    out = {}
    for label, wl, tile, S in TIMELINE_POINTS:
        op = workload_operands(wl)
        A, B, C = op.A.cuda(), op.B.cuda(), op.C.cuda()
        tiles = -(-op.M // tile[0]) * -(-op.N // tile[1])
        grid = -(-tiles // 8) * 8
        nw = 8 if tile[0] * tile[1] >= 256 * 256 else 4
        buf = torch.zeros(grid * nw * 8, dtype=torch.int64, device="cuda")
        def call():
            r = lib.pgemm_diag_wait_profile(op.M, op.N, op.K, A, op.lda, B, op.ldb, C, op.ldc, op.dtype, tile, S,
                                            buf, buf.numel())
            if r != 0:
                raise lib.PgemmError(r)
        _warm_then_run(call, torch, runs)
        raw = buf.view(grid, nw, 8)[:tiles, 0].cpu().numpy().astype(np.float64)
        v = raw / 100.0  # 100 MHz ticks -> us
        start, loop_end, store_end, ready0 = v[:, 4], v[:, 5], v[:, 6], v[:, 7]
        t0 = start.min()
        med = lambda x: round(float(np.median(x)), 2)
        out[label] = {"M": op.M, "N": op.N, "K": op.K, "workgroups": tiles,
                      "span_us": round(float(store_end.max() - t0), 2),
                      "median_prologue_us": med(ready0 - start), "median_k_loop_us": med(loop_end - ready0),
                      "median_store_us": med(store_end - loop_end),
                      "start_us": [round(float(start.min() - t0), 2), round(float(start.max() - t0), 2)],
                      "k_loop_end_us": [round(float(loop_end.min() - t0), 2), round(float(loop_end.max() - t0), 2)],
                      "store_end_us": [round(float(store_end.min() - t0), 2), round(float(store_end.max() - t0), 2)]}
        if tiles % 8 == 0:
            # workgroup b runs on XCD b % 8: the same phases per XCD, and the
            # shader clock over the K loop (shader cycles of the loop over its
            # 100 MHz span, which starts at the wave's start)
            ghz = raw[:, 3] / ((raw[:, 5] - raw[:, 4]) / 100e6) / 1e9
            xcd = np.arange(tiles) % 8
            out[label]["per_xcd"] = [
                {"xcd": x, "median_prologue_us": med((ready0 - start)[xcd == x]),
                 "median_k_loop_us": med((loop_end - ready0)[xcd == x]),
                 "median_store_us": med((store_end - loop_end)[xcd == x]),
                 "last_store_end_us": round(float(store_end[xcd == x].max() - t0), 2),
                 "clock_ghz": round(float(np.mean(ghz[xcd == x])), 3)} for x in range(8)]
        del A, B, C, buf
    return out


def run_reports(lib, torch):
    pts = report_points(lib)
    rep = {}
    ops = {}

    def operands(name):
        if name not in ops:
            ops.clear()  # one workload resident at a time
            op = workload_operands(name)
            ops[name] = (op, op.A.cuda(), op.B.cuda(), op.C.cuda())
        return ops[name]

    for p in pts:
        op, A, B, C = operands(p["workload"])
        M, N, K = op.M, op.N, op.K
        if p["section"] == "f32_256_pages_tile":
            ms = time_gemm(lib, op, A, B, C, stages=p["stages"], producer=p["producer"], tile=p["tile"], reps=50)
            rep.setdefault(p["section"], {})[p["key"]] = {
                "eager_us": round(ms * 1e3, 2), "graph_us": round(_graph_us(lib, torch, op, A, B, C, p), 2)}
            continue
        ms = time_gemm(lib, op, A, B, C, stages=p["stages"], producer=p["producer"], tile=p["tile"])
        t = round(tflops(M, N, K, ms), 2)
        aligned = is_aligned(p["workload"])
        plan = plan_of(lib, op.dtype, M, N, K, p["stages"], p["producer"], p["tile"], aligned=aligned)
        if p["section"] in ("i8_4096", "bf16_4096", "f16_4096"):
            d = rep.setdefault(p["section"], {"variants": {}})
            if p["key"] == "auto":
                d.update(auto=t, pct_peak=round(100 * t / PEAK[op.dtype], 2), plan=plan_label(plan))
            else:
                d["variants"][p["key"]] = t
        elif p["section"] == "f32_4096_page_tile":
            rep.setdefault(p["section"], {"compute_load_ratio": round(
                lib.pgemm_model_compute_load_ratio(128, 64, 16, 4), 2)})[p["key"]] = t
        else:  # bf16_k_sweep
            sweep = rep.setdefault("bf16_k_sweep", {})
            if p["workload"] == "ragged":
                sweep["ragged_4000x3968x4001"] = {"tflops": t, "pct_peak": round(100 * t / PEAK["bf16"], 2),
                                                  "plan": plan_label(plan)}
                continue
            row = sweep.setdefault("K%d" % K, {})
            tag = p["key"].split()[1]
            row[tag] = {"tflops": t, "plan": plan_label(plan)}
            if tag == "auto":
                byts = algorithmic_bytes("bf16", M, N, K, 0.0)
                roof = min(PEAK["bf16"], 2.0 * M * N * K / byts * HBM_PEAK_GBS / 1e3)
                row["auto"].update(pct_of_roof=round(100 * t / roof, 1), roof="hbm" if roof < PEAK["bf16"] else "mfma",
                                   GBs=round(byts / (ms * 1e-3) / 1e9, 0))
                best = max(("s1", "s2", "s3", "s4"), key=lambda k: row[k]["tflops"])
                row["best_measured"] = {"stages": best, "plan": row[best]["plan"], "tflops": row[best]["tflops"],
                                        "auto_vs_best": round(t / row[best]["tflops"], 3)}
    ops.clear()
    rep["pages_context"] = pages_context(rep)
    rep["ceilings"] = ceilings(lib, torch)
    rep["parts_ladder"] = parts_ladder(lib, torch)
    rep["wait_profile"] = wait_profile(lib, torch)
    rep["timeline"] = timeline(lib, torch)
    return rep


if __name__ == "__main__":
    main()
