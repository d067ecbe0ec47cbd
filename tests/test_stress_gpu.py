"""Stress of the stage protocol on the GPU (correct protocol only).

Page "Software pipelines and asynchronous copies" (section "Practice") asks
for many repeated runs with randomised input and an artificial delay in one
consumer, with failure counts.  Here the library's stress hook skews one wave
of every workgroup per K tile (rotating) by ~8k cycles after the ready
barrier, so the other waves reach the next barrier, and issue the next
tile's loads into the freed stage, far ahead of it.  Every launch must give
exactly the same int8 result, equal to the oracle: 6 variants x 1000 runs.
The GEMM has no build with a wait removed.  The reuse edge's removal is shown
by the host model checker (tests/test_schedule_model.py) and, on the GPU, by
the two-stage copy-and-reduce demonstrator (tests/test_hazard_gpu.py), whose
variant without the reuse barrier fails every delayed run.
"""
import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_loop_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("producer,stages,tile", [
    ("direct", 2, (256, 256, 128)), ("direct", 3, (256, 256, 64)), ("direct", 4, (256, 256, 64)),
    ("register", 2, (256, 256, 64)), ("direct", 1, (256, 256, 64)), ("register", 1, (256, 256, 64)),
])
def test_skewed_waves_many_runs_bit_exact(producer, stages, tile):
    from software_pipelined_tiled_loop_amd import binding as lib
    M, N, K = 1024, 1024, 768
    runs = 1000
    print("[case] stress", producer, stages, tile, "runs", runs, flush=True)
    op = inputs.make_operands("i8", M, N, K, seed=4321 + stages, alpha=1, beta=0)
    A, B = op.A.cuda(), op.B.cuda()
    ref = oracle.gemm("i8", M, N, K, 1, *op.numpy_views()[:2])
    first = None
    failures = 0
    for r in range(runs):
        C = torch.full((M, N), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
        skew = 1 + (r % 2)
        st = lib.pgemm_gemm_ex(M, N, K, 1, A, K, B, N, 0, C, N, "i8", stages,
                               lib._opts(producer, tile, skew), None)
        assert st == 0, lib.pgemm_strerror(st)
        if first is None:
            torch.cuda.synchronize()
            first = C.clone()
            assert np.array_equal(first.cpu().numpy(), ref)
        elif not torch.equal(C, first):
            failures += 1
    torch.cuda.synchronize()
    assert failures == 0, "%d of %d skewed runs differed" % (failures, runs)
    # the hook really skews: each K tile waits at its barrier for the sleeping
    # wave, less the work the other waves do meanwhile.  The visible delay
    # depends on that overlap and on the clock (one run measured 18.3 us for
    # 6 K tiles with a sleep of 2 x 8128 cycles each), so the bar is a quarter
    # of the nominal sleep time at 2.5 GHz: far above run-to-run noise, far
    # below the delay.
    def timed(skew):
        C = torch.empty((M, N), dtype=torch.int32, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        r = lib.pgemm_gemm_ex(M, N, K, 1, A, K, B, N, 0, C, N, "i8", stages, lib._opts(producer, tile, skew), None)
        assert r == 0, lib.pgemm_strerror(r)
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3  # us
    base = min(timed(0) for _ in range(3))
    skewed = min(timed(2) for _ in range(3))
    nk = (K + tile[2] - 1) // tile[2]
    assert skewed - base > 0.25 * nk * 2 * 8128 / 2.5e3, (base, skewed)
