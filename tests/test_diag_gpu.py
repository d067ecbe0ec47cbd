"""The ceiling diagnostics (pgemm_diag_*) on the GPU: they run, and the MFMA
kernel's accumulators hold what its operands make them.

These kernels are measurement tools, not part of the GEMM path; the bench's
"ceilings" report times them.  Zero operands must leave every accumulator at
zero; random operands give finite sums (bf16/fp16/fp32, values in [-1, 1))
that differ between seeds.  The LDS stream moves exactly the bytes it reports
and reads only inside the operands (it runs on the 4096^3 workload and on a
ragged-free small one).  The parts ladder's whole build computes exactly what
the GEMM computes, and every step of the ladder runs and stamps its clocks."""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    from software_pipelined_tiled_loop_amd import binding
    return binding


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_mfma_ceiling_runs_and_keeps_its_accumulators(lib, dtype):
    print("[case] mfma ceiling", dtype, flush=True)
    grid = 256
    out = torch.full((grid * 8,), float("nan"), dtype=torch.float32, device="cuda")
    r, flops = lib.pgemm_diag_mfma_ceiling(dtype, 1, 64, grid, 7, out)
    assert r == 0
    torch.cuda.synchronize()
    zeros = bool((out == 0).all().item())
    assert zeros
    per_block = {"f32": 8192, "f16": 16384, "bf16": 16384, "i8": 32768}[dtype]
    assert flops == grid * 8 * 64 * 16 * per_block
    sums = []
    for seed in (7, 8):
        r, _ = lib.pgemm_diag_mfma_ceiling(dtype, 0, 64, grid, seed, out)
        assert r == 0
        torch.cuda.synchronize()
        sums.append(out.cpu())
    assert bool(torch.isfinite(sums[0]).all())
    assert not torch.equal(sums[0], sums[1])
    clock = torch.zeros(grid * 4, dtype=torch.int64, device="cuda")
    r, _ = lib.pgemm_diag_mfma_ceiling(dtype, 0, 4096, grid, 7, out, clock=clock)
    assert r == 0
    torch.cuda.synchronize()
    c = clock.view(grid, 4).cpu().double()
    ghz = (c[:, 2] - c[:, 0]) / ((c[:, 3] - c[:, 1]) / 100e6) / 1e9
    assert bool((c[:, 3] > c[:, 1]).all()) and 0.3 < float(ghz.mean()) < 3.0


@pytest.mark.parametrize("dtype", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("waves,block", [(1, 16), (2, 32), (1, 32)])
def test_mfma_ceiling_variants_run_with_the_same_flops(lib, dtype, waves, block):
    print("[case] mfma ceiling variant", dtype, waves, block, flush=True)
    grid = 256
    nw = grid * 4 * waves
    out = torch.full((grid * 8,), float("nan"), dtype=torch.float32, device="cuda")
    r, flops = lib.pgemm_diag_mfma_ceiling(dtype, 1, 64, grid, 7, out, waves_per_simd=waves, block=block)
    assert r == 0
    torch.cuda.synchronize()
    host = out.cpu()
    assert bool((host[:nw] == 0).all()) and bool(torch.isnan(host[nw:]).all())
    per_block = {"f16": 16384, "bf16": 16384, "i8": 32768}[dtype]
    assert flops == nw * 64 * 16 * per_block
    sums = []
    for seed in (7, 8):
        r, _ = lib.pgemm_diag_mfma_ceiling(dtype, 0, 64, grid, seed, out, waves_per_simd=waves, block=block)
        assert r == 0
        torch.cuda.synchronize()
        sums.append(out[:nw].cpu())
    assert bool(torch.isfinite(sums[0]).all())
    assert not torch.equal(sums[0], sums[1])


@pytest.mark.parametrize("dtype,tile,stages", [("bf16", (256, 256, 64), 2), ("bf16", (256, 256, 32), 4),
                                               ("i8", (256, 256, 128), 2), ("f32", (128, 64, 16), 2)])
def test_lds_stream_runs_and_counts_its_bytes(lib, dtype, tile, stages):
    M, N, K = 1024, 768, 640
    print("[case] lds stream", dtype, tile, stages, flush=True)
    es = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}[dtype]
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}[dtype]
    A = torch.zeros(M, K, dtype=dt, device="cuda")
    B = torch.zeros(K, N, dtype=dt, device="cuda")
    r, nbytes = lib.pgemm_diag_lds_stream(M, N, K, A, K, B, N, dtype, tile, stages)
    assert r == 0, lib.pgemm_strerror(r)
    torch.cuda.synchronize()
    tiles = math.ceil(M / tile[0]) * math.ceil(N / tile[1])
    assert nbytes == tiles * math.ceil(K / tile[2]) * (tile[0] + tile[1]) * tile[2] * es


@pytest.mark.parametrize("dtype,tile,stages", [("bf16", (256, 256, 64), 1), ("bf16", (256, 256, 64), 2),
                                               ("bf16", (256, 256, 32), 4), ("i8", (256, 256, 128), 2),
                                               ("f32", (128, 64, 16), 2), ("f16", (256, 256, 64), 1),
                                               ("bf16", (128, 128, 64), 3)])
def test_wait_profile_is_the_gemm_with_clock_stamps(lib, dtype, tile, stages):
    """The wait-profile build computes exactly what the GEMM's own DIRECT
    variant computes (same bits), and its totals are consistent: every wave
    passes one ready edge per K tile (plus the prologue's at two or more
    stages), and its waits fit inside its K loop."""
    from software_pipelined_tiled_loop_amd import inputs
    M, N, K = 3 * tile[0] + 5, 2 * tile[1] + 16, 5 * tile[2]
    print("[case] wait profile", dtype, tile, stages, (M, N, K), flush=True)
    op = inputs.make_operands(dtype, M, N, K, seed=321, alpha=1.0, beta=0.0)
    A, B = op.A.cuda(), op.B.cuda()
    C1, C2 = op.C.cuda(), op.C.cuda()
    tiles = math.ceil(M / tile[0]) * math.ceil(N / tile[1])
    grid = math.ceil(tiles / 8) * 8
    nw = 8 if tile[0] * tile[1] >= 256 * 256 else 4
    buf = torch.full((grid * nw * 8,), -1, dtype=torch.int64, device="cuda")
    assert lib.pgemm_diag_wait_profile(M, N, K, A, op.lda, B, op.ldb, C1, op.ldc, dtype, tile, stages, buf,
                                       buf.numel() - 1) == -1        # out too short: refused
    r = lib.pgemm_diag_wait_profile(M, N, K, A, op.lda, B, op.ldb, C1, op.ldc, dtype, tile, stages, buf, buf.numel())
    assert r == 0, lib.pgemm_strerror(r)
    r = lib.pgemm_gemm_ex(M, N, K, 1.0, A, op.lda, B, op.ldb, 0.0, C2, op.ldc, dtype, stages,
                          lib._opts("direct", tile), None)
    assert r == 0
    torch.cuda.synchronize()
    same = bool(torch.equal(C1.view(torch.int32), C2.view(torch.int32)))
    assert same
    v = buf.view(grid, nw, 8)[:tiles].cpu()
    nK = math.ceil(K / tile[2])
    assert bool((v[..., 2] == (nK if stages == 1 else nK + 1)).all())
    assert bool((v[..., 0] >= 0).all()) and bool((v[..., 1] > 0).all())
    assert bool((v[..., 0] + v[..., 1] < v[..., 3]).all())
    # timeline on the 100 MHz clock: start <= first ready edge <= K loop end <= stores complete
    assert bool((v[..., 4] <= v[..., 7]).all()) and bool((v[..., 7] <= v[..., 5]).all())
    assert bool((v[..., 5] <= v[..., 6]).all()) and bool((v[..., 4] > 0).all())
    assert bool((buf.view(grid, nw, 8)[tiles:] == -1).all())         # idle workgroups write nothing


LADDER = [0, 4, 8, 12, 14, 15]  # MFMA only, + A reads, B reads only, + both, + barrier, + LDS-DMA (the GEMM)


@pytest.mark.parametrize("dtype,tile", [("bf16", (256, 256, 64)), ("f16", (256, 256, 64)), ("i8", (256, 256, 128)),
                                        ("f32", (128, 64, 16))])
def test_parts_ladder_whole_build_is_the_gemm_and_every_step_runs(lib, dtype, tile):
    """The parts-ladder build with every part in computes exactly what the
    GEMM's own DIRECT variant computes (same bits, on a shape with edge tiles
    and several K tiles); every other step runs to completion on the same
    operands and stamps a start and an end clock for each workgroup."""
    from software_pipelined_tiled_loop_amd import inputs
    M, N, K = 3 * tile[0] + 5, 2 * tile[1] + 16, 6 * tile[2]
    print("[case] parts ladder", dtype, tile, (M, N, K), flush=True)
    op = inputs.make_operands(dtype, M, N, K, seed=322, alpha=1.0, beta=0.0)
    A, B = op.A.cuda(), op.B.cuda()
    C1, C2 = op.C.cuda(), op.C.cuda()
    tiles = math.ceil(M / tile[0]) * math.ceil(N / tile[1])
    grid = math.ceil(tiles / 8) * 8
    clock = torch.full((grid * 4,), -1, dtype=torch.int64, device="cuda")
    r = lib.pgemm_gemm_ex(M, N, K, 1.0, A, op.lda, B, op.ldb, 0.0, C2, op.ldc, dtype, 2, lib._opts("direct", tile),
                          None)
    assert r == 0
    for parts in LADDER:
        print("[case] parts", parts, flush=True)
        clock.fill_(-1)
        r = lib.pgemm_diag_parts(M, N, K, A, op.lda, B, op.ldb, C1, op.ldc, dtype, tile, 2, parts, clock,
                                 clock.numel())
        assert r == 0, lib.pgemm_strerror(r)
        torch.cuda.synchronize()
        c = clock.view(grid, 4).cpu()
        assert bool((c[:tiles, 2] > c[:tiles, 0]).all()) and bool((c[:tiles, 3] >= c[:tiles, 1]).all())
        assert bool((c[tiles:] == -1).all())                         # idle workgroups write nothing
        if parts == lib.PART_ALL:
            same = bool(torch.equal(C1.view(torch.int32), C2.view(torch.int32)))
            assert same
