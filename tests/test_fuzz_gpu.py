"""Seeded random parity sweep: shapes, leading dimensions, scalars and launch
options drawn at random, each GPU result checked against the oracle.

The directed tests pin the edges one by one; this sweep draws combinations
none of them lists: every compiled variant (tile class, ring depth, producer)
of every dtype, forced or left to the planner, on shapes that cut tiles and K
tiles at random places, with padded or odd leading dimensions, nonzero beta,
and sometimes persistent workgroups.  Tolerances are the benchmark's (see
test_parity_gpu).  A forced producer the operands' chunk rule (rows of whole
16-byte chunks) does not admit must be refused before launch with PGEMM_ERR_INFEASIBLE_PLAN, and the
planner (pgemm_plan, same options and alignment class) must agree with the
launch about every refusal.  Every case prints its parameters before it runs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_loop_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
N_CASES = 400
INFEASIBLE = -4


@pytest.fixture(scope="module")
def lib():
    from software_pipelined_tiled_loop_amd import binding
    return binding


def aligned_class(lib, dtype, K, N, lda, ldb):
    """The pgemm_aligned class: which operands hold whole 16-byte chunks per
    row (A: K elements, B: N elements); leading dimensions do not matter."""
    es = inputs.ELEM_BYTES[dtype]
    a = K == 0 or K * es % 16 == 0
    b = K == 0 or N * es % 16 == 0
    return lib.ALIGNED_BOTH if a and b else lib.ALIGNED_A if a else lib.ALIGNED_B if b else lib.ALIGNED_NONE


def admitted(lib, producer, cls):
    a = cls in (lib.ALIGNED_BOTH, lib.ALIGNED_A)
    b = cls in (lib.ALIGNED_BOTH, lib.ALIGNED_B)
    return {"direct": b, "register": a and b, "staged_a": b, "staged_b": a, "generic": True}[producer]


def draw_dim(rng, hi):
    """Small sizes often (below and around one tile), the rest uniform."""
    r = rng.random()
    if r < 0.25:
        return int(rng.integers(1, 20))
    if r < 0.5:
        return int(rng.choice([15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]))
    return int(rng.integers(1, hi + 1))


def check(op, got):
    A, B, C0 = op.numpy_views()
    ref = oracle.gemm(op.dtype, op.M, op.N, op.K, op.alpha, A, B, op.beta, C0 if op.beta != 0 else None)
    g = got[:, :op.N]
    if op.dtype == "i8":
        bad = np.nonzero(g.numpy() != ref)
        assert bad[0].size == 0, "int8 mismatch at %s" % (list(zip(bad[0][:5], bad[1][:5])),)
        return
    gd = g.to(torch.float64).numpy()
    assert np.all(np.isfinite(gd)), "non-finite output"
    err = float(np.max(np.abs(gd - ref))) if ref.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = TOL[op.dtype] * math.sqrt(max(op.K, 1)) * scale
    assert err <= bound, "max err %g > bound %g" % (err, bound)


def test_random_shapes_layouts_and_options(lib):
    rng = np.random.default_rng(20261202)
    variants = {}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        variants.setdefault(v["dtype"], []).append(v)
    dev = torch.device("cuda:0")
    ran = refused = 0
    for case in range(N_CASES):
        dtype = str(rng.choice(["f32", "f16", "bf16", "i8"]))
        epc = 16 // inputs.ELEM_BYTES[dtype]
        M, N = draw_dim(rng, 520), draw_dim(rng, 520)
        K = 0 if rng.random() < 0.04 else draw_dim(rng, 600)
        pads = [0, 0, 0, 1, epc, int(rng.integers(0, 10))]
        lda = K + int(rng.choice(pads))
        ldb = N + int(rng.choice(pads))
        ldc = N + int(rng.choice(pads))
        if dtype == "i8":
            alpha, beta = int(rng.integers(-3, 4)), int(rng.choice([0, 0, 1, -2]))
        else:
            alpha, beta = float(rng.choice([1.0, 1.0, 0.5, -1.25])), float(rng.choice([0.0, 0.0, 0.5, -1.0]))
        cls = aligned_class(lib, dtype, K, N, lda, ldb)
        forced = rng.random() < 0.7
        # mostly a variant the layout admits; sometimes any, to see refusals
        pool = [w for w in variants[dtype] if admitted(lib, w["producer"], cls)]
        if not pool or rng.random() < 0.15:
            pool = variants[dtype]
        v = pool[int(rng.integers(len(pool)))] if forced else None
        producer = v["producer"] if forced else None
        tile = (v["tile_m"], v["tile_n"], v["tile_k"]) if forced else None
        stages = v["stages"] if forced else 0
        workgroups = int(rng.choice([8, 16, 64])) if forced and stages > 1 and rng.random() < 0.15 else 0
        desc = dict(case=case, dtype=dtype, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc, alpha=alpha, beta=beta,
                    producer=producer, tile=tile, stages=stages, workgroups=workgroups)
        print("[case] fuzz", desc, flush=True)
        op = inputs.make_operands(dtype, M, N, K, seed=1000 + case, alpha=alpha, beta=beta, lda=lda, ldb=ldb,
                                  ldc=ldc)
        opts = lib._opts(producer, tile, workgroups=workgroups)
        rp, _ = lib.pgemm_plan(M, N, K, dtype, stages, cls, opts)
        A, B, C = op.A.to(dev), op.B.to(dev), op.C.to(dev)
        r = lib.pgemm_gemm_ex(M, N, K, alpha, A if K else 0, max(lda, 1), B if K else 0, max(ldb, 1), beta, C,
                              ldc, dtype, stages, opts, None)
        assert r == rp, (desc, r, rp)  # the launch and the planner agree
        if forced and not admitted(lib, producer, cls):
            assert r == INFEASIBLE, (desc, r)
        if r == INFEASIBLE:
            refused += 1
            continue
        assert r == 0, (desc, lib.pgemm_strerror(r))
        torch.cuda.synchronize()
        got = C.cpu()
        check(op, got)
        if ldc > N:  # columns past N are the caller's memory: untouched
            pad, ref = got[:, N:], op.C[:, N:]
            if dtype == "i8":
                assert torch.equal(pad, ref), desc
            else:
                assert torch.equal(torch.isnan(pad), torch.isnan(ref)), desc
        ran += 1
        del A, B, C
    print("[fuzz] ran %d cases, %d refused before launch" % (ran, refused), flush=True)
    assert ran >= N_CASES // 2 and refused > 0
