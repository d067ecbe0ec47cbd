"""Full-size parity: every launch the benchmark times, on its own workload,
against the oracle over all M x N outputs.

The workloads are the benchmark's: fp32 4096^3 with beta = 0.5; int8, bf16
and fp16 4096^3; the bf16 K-sweep (M = N = 4096, K in {32, 64, 256, 1024,
4096, 16384}); the ragged 4000 x 3968 x 4001 problem with lda = 4001.  For
each, the oracle's result is computed once, and every point of
bench.report_points on that workload (the planner's plan, every compiled
tile x depth x producer variant the report times, each ring depth of the
K-sweep) runs through the C ABI and is compared element by element:

  int8 -> int32   bit-exact
  fp32            max|C - C_ref| <= 1e-5 * sqrt(K) * max|C_ref|
  fp16 / bf16     max|C - C_ref| <= 2e-3 * sqrt(K) * max|C_ref|

Pipelining changes no arithmetic (page "GPU-Kernel pipelinen", step 5, which
also asks for the test at the target size), so a dropped, duplicated or stale
K tile anywhere in the 4096 x 4096 output shows up here.  Before each launch C
is reset (to NaN when beta = 0, to C0 otherwise), so every output element
must have been written by that launch.  The difference is reduced on the
GPU; only its maximum comes back.
"""
import math

import numpy as np
import pytest
import torch

import bench
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
WORKLOADS = ["f32", "i8", "bf16", "f16", "ragged"] + ["bf16_k%d" % K for K in bench.K_SWEEP]


@pytest.fixture(scope="module")
def lib():
    from software_pipelined_tiled_loop_amd import binding
    return binding


def say(*a):
    print("[case]", *a, flush=True)


def oracle_result(op):
    A, B, C0 = op.numpy_views()
    return oracle.gemm(op.dtype, op.M, op.N, op.K, op.alpha, A, B, op.beta, C0 if op.beta != 0 else None)


@pytest.mark.parametrize("name", WORKLOADS)
def test_every_timed_launch_matches_the_oracle_at_full_size(lib, name):
    pts = [p for p in bench.report_points(lib) if p["workload"] == name]
    if name in ("f32", "i8", "bf16", "f16", "ragged"):
        pts.append(dict(section="headline", key="planner", workload=name, stages=0, producer=None, tile=None))
    assert pts
    op = bench.workload_operands(name)
    say(name, "oracle", (op.M, op.N, op.K), "points", len(pts))
    ref = oracle_result(op)
    dev = torch.device("cuda:0")
    A, B = op.A.to(dev), op.B.to(dev)
    C0 = op.C.to(dev)
    C = torch.empty_like(C0)
    N = op.N
    if op.dtype == "i8":
        ref_d = torch.from_numpy(ref).to(dev)
        bound = 0.0
    else:
        ref_d = torch.from_numpy(ref).to(dev)
        bound = TOL[op.dtype] * math.sqrt(max(op.K, 1)) * float(np.max(np.abs(ref)))
    for p in pts:
        say(name, p["section"], p["key"])
        C.copy_(C0)
        r = lib.pgemm_gemm_ex(op.M, op.N, op.K, op.alpha, A, op.lda, B, op.ldb, op.beta, C, op.ldc, op.dtype,
                              p["stages"], lib._opts(p["producer"], p["tile"]), None)
        assert r == 0, (p["key"], lib.pgemm_strerror(r))
        torch.cuda.synchronize()
        got = C[:, :N]
        if op.dtype == "i8":
            bad = int((got != ref_d).sum().item())
            assert bad == 0, "%s: %d of %d int8 outputs differ" % (p["key"], bad, op.M * N)
        else:
            finite = bool(torch.isfinite(got).all().item())
            assert finite, "%s: non-finite output" % p["key"]
            err = float((got.double() - ref_d).abs().max().item())
            assert err <= bound, "%s: max err %g > bound %g" % (p["key"], err, bound)
        if op.ldc > N:
            pad_same = bool(torch.equal(C[:, N:].view(torch.int32), C0[:, N:].view(torch.int32)))
            assert pad_same, "%s: columns past N were written" % p["key"]
    del A, B, C, C0, ref_d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,M,N,K", [
    ("bf16", 8192, 8192, 1024),   # 1024 tiles of 256 x 256: four workgroups in turn on every CU
    ("i8", 8192, 8192, 1024),
    ("f32", 8192, 8192, 64),      # short K, the planner's co-resident small tiles
    ("f16", 1024, 8192, 4096),    # a wide, short output
])
def test_planner_check_shapes_beyond_the_workloads(lib, dtype, M, N, K):
    """Shapes of the planner check that are larger than the benchmark's
    workloads (several rounds of workgroups per CU), with the planner's own
    plan, against the oracle over all M x N outputs."""
    from software_pipelined_tiled_loop_amd import inputs
    say("beyond", dtype, (M, N, K))
    op = inputs.make_operands(dtype, M, N, K, seed=inputs.seed_for("bf16_k_sweep", 60 + K % 37))
    ref = oracle_result(op)
    dev = torch.device("cuda:0")
    A, B, C = op.A.to(dev), op.B.to(dev), op.C.to(dev)
    r = lib.pgemm_gemm(M, N, K, op.alpha, A, op.lda, B, op.ldb, op.beta, C, op.ldc, dtype, 0)
    assert r == 0, lib.pgemm_strerror(r)
    torch.cuda.synchronize()
    ref_d = torch.from_numpy(ref).to(dev)
    if dtype == "i8":
        assert int((C != ref_d).sum().item()) == 0
    else:
        assert bool(torch.isfinite(C).all().item())
        err = float((C.double() - ref_d).abs().max().item())
        bound = TOL[dtype] * math.sqrt(K) * float(np.max(np.abs(ref)))
        assert err <= bound, (err, bound)
    del A, B, C, ref_d
    torch.cuda.empty_cache()
