"""HIP graph capture of the C ABI.

A call enqueues one kernel on the caller's stream, allocates nothing and
never synchronises, so it can be recorded in a HIP graph (here through
torch's graph capture, which records the caller's stream).  The graph is
replayed several times with eager work and synchronisations between the
replays, and every replay must equal the eager call bit for bit (same kernel,
same inputs).  With beta != 0 the old C is restored eagerly before each
replay.
"""
import pytest
import torch

import oracle
from software_pipelined_tiled_loop_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,M,N,K,beta,stages", [
    ("f32", 256, 256, 256, 0.0, 2),      # the fp32 256^3 configuration
    ("f32", 256, 256, 256, 0.0, 1),
    ("bf16", 512, 384, 640, 0.0, 0),
    ("f32", 300, 200, 100, 0.5, 3),
    ("i8", 640, 520, 384, 2, 2),
])
def test_graph_replay_matches_eager(dtype, M, N, K, beta, stages):
    from software_pipelined_tiled_loop_amd import binding as lib
    print("[case] graph", dtype, (M, N, K), "beta", beta, "stages", stages, flush=True)
    alpha = 1 if dtype == "i8" else 1.0
    op = inputs.make_operands(dtype, M, N, K, seed=M + K, alpha=alpha, beta=beta)
    A, B, C0 = op.A.cuda(), op.B.cuda(), op.C.cuda()
    C_eager = C0.clone()
    r = lib.pgemm_gemm(M, N, K, alpha, A, K, B, N, beta, C_eager, N, dtype, stages)
    assert r == 0, lib.pgemm_strerror(r)
    torch.cuda.synchronize()

    C_graph = C0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        status = lib.pgemm_gemm(M, N, K, alpha, A, K, B, N, beta, C_graph, N, dtype, stages)
    assert status == 0
    x = torch.ones(1 << 20, device="cuda")
    for rep in range(4):
        C_graph.copy_(C0)            # eager work between replays
        x.mul_(1.5).add_(rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(C_graph.view(torch.int32), C_eager.view(torch.int32)))
        assert same, rep
    # and the eager result is the oracle's (to the dtype's rule)
    a, b, c0 = op.numpy_views()
    ref = oracle.gemm(dtype, M, N, K, alpha, a, b, beta, c0 if beta != 0 else None)
    got = C_eager[:, :N].cpu()
    if dtype == "i8":
        assert (got.numpy() == ref).all()
    else:
        import math
        import numpy as np
        err = float(np.max(np.abs(got.double().numpy() - ref)))
        tol = 1e-5 if dtype == "f32" else 2e-3
        assert err <= tol * math.sqrt(K) * float(np.max(np.abs(ref)))
