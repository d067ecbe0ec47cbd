"""GPU parity: the HIP library against the oracle, through the C ABI.

Rules (the benchmark's stated tolerances):
  int8 -> int32   bit-exact
  fp32            max|C - C_ref| <= 1e-5 * sqrt(K) * max|C_ref|
  fp16 / bf16     max|C - C_ref| <= 2e-3 * sqrt(K) * max|C_ref|
The oracle sees exactly the rounded inputs the GPU sees, so input rounding is
not error.  Pipelining changes no arithmetic (page "GPU-Kernel pipelinen",
step 5): within one tile class the output must also be bit-identical across
ring depths and producers, which catches a stale, duplicated or missing K tile
even in float.  Every case prints its parameters before it runs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_loop_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


@pytest.fixture(scope="module")
def lib():
    from software_pipelined_tiled_loop_amd import binding
    return binding


def say(*a):
    print("[case]", *a, flush=True)


def run_gpu(lib, op, stages=0, producer=None, tile=None, expect=0, workgroups=0):
    dev = torch.device("cuda:0")
    A = op.A.to(dev)
    B = op.B.to(dev)
    C = op.C.to(dev)
    o = lib._opts(producer, tile, workgroups=workgroups)
    r = lib.pgemm_gemm_ex(op.M, op.N, op.K, op.alpha, A if op.M and op.K else 0, max(op.lda, 1),
                          B if op.K and op.N else 0, max(op.ldb, 1), op.beta, C if op.M else 0, max(op.ldc, 1),
                          op.dtype, stages, o, None)
    assert r == expect, lib.pgemm_strerror(r)
    torch.cuda.synchronize()
    return C.cpu()


def reference(op, rows=None):
    A, B, C0 = op.numpy_views()
    return oracle.gemm(op.dtype, op.M, op.N, op.K, op.alpha, A, B, op.beta, C0 if op.beta != 0 else None,
                       rows=rows)


def check(op, got, rows=None):
    ref = reference(op, rows)
    g = got[:, :op.N] if rows is None else got[rows, :op.N]
    if op.dtype == "i8":
        diff = np.nonzero(g.numpy() != ref)
        assert diff[0].size == 0, "int8 mismatch at %s: got %s want %s" % (
            list(zip(diff[0][:5], diff[1][:5])), g.numpy()[diff][:5], ref[diff][:5])
        return 0.0
    gd = g.to(torch.float64).numpy()
    assert np.all(np.isfinite(gd)), "non-finite output"
    err = np.max(np.abs(gd - ref)) if ref.size else 0.0
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    bound = TOL[op.dtype] * math.sqrt(max(op.K, 1)) * scale
    assert err <= bound, "max err %g > bound %g (scale %g)" % (err, bound, scale)
    return err


def padding_untouched(op, got):
    """Columns n >= N of C are the caller's memory beyond the matrix: unchanged."""
    if op.ldc > op.N and op.M:
        pad = got[:, op.N:]
        ref = op.C[:, op.N:]
        if op.dtype == "i8":
            assert torch.equal(pad, ref)
        else:
            assert torch.equal(torch.isnan(pad), torch.isnan(ref))


# ------------------------------------------------------------------ torch wrapper

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_torch_wrapper_on_column_slices(lib, dtype):
    """binding.gemm takes the sizes from the tensor shapes, the leading
    dimensions from the row strides and the dtype from A.  Here A, B and C are
    column slices of wider tensors, so lda, ldb and ldc exceed K and N; the
    columns of C beyond the slice must stay untouched."""
    M, N, K = 200, 136, 300
    alpha = 2 if dtype == "i8" else 1.5
    say("torch wrapper", dtype, (M, N, K))
    op = inputs.make_operands(dtype, M, N, K, seed=inputs.seed_for("half_4096", 40), alpha=alpha, beta=0.0,
                              lda=K + 8, ldb=N + 24, ldc=N + 8)
    A, B, C = op.A.cuda(), op.B.cuda(), op.C.cuda()
    lib.gemm(A[:, :K], B[:, :N], C[:, :N], alpha=alpha)
    torch.cuda.synchronize()
    got = C.cpu()
    check(op, got)
    padding_untouched(op, got)


# ------------------------------------------------------------------ small workloads

@pytest.mark.parametrize("stages", [1, 2])
def test_fp32_256_pages_tile_single_vs_double_buffer(lib, stages):
    say("fp32 256^3 stages", stages, "tile 128x64x16")
    op = inputs.make_operands("f32", 256, 256, 256, seed=inputs.seed_for("fp32_256"), alpha=1.0, beta=0.0)
    got = run_gpu(lib, op, stages=stages, tile=(128, 64, 16))
    check(op, got)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
@pytest.mark.parametrize("stages", [1, 2, 3, 4])
def test_all_dtypes_all_stages_small(lib, dtype, stages):
    # several tiles in M and N plus ragged tails; K spans several K tiles + tail
    M, N, K = 300, 280, 16 * 37  # K multiple of 16 keeps every dtype on the vector path
    say("small", dtype, "stages", stages, (M, N, K))
    op = inputs.make_operands(dtype, M, N, K, seed=inputs.seed_for("half_4096", stages), alpha=1.0, beta=0.0)
    got = run_gpu(lib, op, stages=stages)
    check(op, got)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_alpha_beta_and_padded_leading_dims(lib, dtype):
    M, N, K = 200, 136, 272
    alpha, beta = (2, -3) if dtype == "i8" else (1.5, -0.5)
    say("alpha/beta + ld padding", dtype)
    op = inputs.make_operands(dtype, M, N, K, seed=77, alpha=alpha, beta=beta, lda=K + 16, ldb=N + 16,
                              ldc=N + 5)
    got = run_gpu(lib, op, stages=2)
    check(op, got)
    padding_untouched(op, got)


# ------------------------------------------------------------------ invariance pins

def tile_classes(lib, dtype):
    seen = {}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        if v["dtype"] != dtype or v["producer"] == "generic":
            continue
        key = (v["tile_m"], v["tile_n"], v["tile_k"])
        seen.setdefault(key, []).append((v["stages"], v["producer"]))
    return seen


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_bit_identical_across_stages_and_producers(lib, dtype):
    """One tile class = one MFMA schedule: every ring depth and producer must
    give the same bits (a stale, duplicated or skipped K tile would not).
    384 x 320 holds both whole output tiles and edge tiles for every class:
    with the DIRECT producer the whole ones load all but their last K tiles
    without per-lane range selects, the edge ones take the general path, and
    the register producers never take the select-free path, so this also
    pins that path against the general one bit for bit."""
    M, N, K = 384, 320, 16 * 40
    op = inputs.make_operands(dtype, M, N, K, seed=4242, alpha=1.0, beta=0.0)
    for tile, variants in tile_classes(lib, dtype).items():
        outs = []
        for stages, producer in sorted(variants):
            say("invariance", dtype, tile, stages, producer)
            outs.append(((stages, producer), run_gpu(lib, op, stages=stages, producer=producer, tile=tile)))
        check(op, outs[0][1])
        for key, o in outs[1:]:
            assert torch.equal(o.view(torch.int32), outs[0][1].view(torch.int32)), (tile, key, outs[0][0])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_whole_tile_load_path_boundaries(lib, dtype):
    """With the DIRECT producer an output tile that lies wholly inside C loads
    its slots t + S < K / BK without per-lane range selects and the rest on
    the general path.  For every DIRECT tile class, K is swept over 2..6 K
    tiles, whole and with a tail, so that the number of select-free slots runs
    through -1..4 for each ring depth; M = 520 adds edge tiles beside whole
    ones.  Each depth must match the oracle and give the same bits as every
    other depth of its class, the single-buffer loop included."""
    es = inputs.ELEM_BYTES[dtype]
    epc = 16 // es
    classes = {}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        if v["dtype"] == dtype and v["producer"] == "direct":
            classes.setdefault((v["tile_m"], v["tile_n"], v["tile_k"]), []).append(v["stages"])
    for bk in sorted({t[2] for t in classes}):
        for n in range(2, 7):
            for K in (bk * n, bk * n + epc):
                M = 520 if n % 2 else 512
                op = inputs.make_operands(dtype, M, 512, K, seed=inputs.seed_for("half_4096", 50 + n), alpha=1.0,
                                          beta=0.0)
                for tile, depths in sorted(classes.items()):
                    if tile[2] != bk:
                        continue
                    outs = []
                    for stages in sorted(depths):
                        say("whole-tile path", dtype, tile, "K", K, "M", M, "stages", stages)
                        outs.append((stages, run_gpu(lib, op, stages=stages, producer="direct", tile=tile)))
                    check(op, outs[0][1])
                    for stages, o in outs[1:]:
                        assert torch.equal(o.view(torch.int32), outs[0][1].view(torch.int32)), (tile, K, stages)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_persistent_workgroups_bit_identical(lib, dtype):
    """Persistent workgroups stream the K tiles of several output tiles through
    one ring (the next tile's loads overlap this tile's last K tiles and its
    C store).  Each output tile's arithmetic is unchanged, so C must be
    bit-identical to one workgroup per tile: every tile class, depth and
    producer, ragged edges, beta != 0, and grids that leave workgroups idle."""
    alpha, beta = (2, -3) if dtype == "i8" else (1.5, -0.5)
    classes = {}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        if v["dtype"] == dtype:
            classes.setdefault((v["tile_m"], v["tile_n"], v["tile_k"]), []).append((v["stages"], v["producer"]))
    for tile, variants in sorted(classes.items()):
        M, N, K = 3 * tile[0] - 37, 2 * tile[1] + 32, 2 * tile[2] + 16  # 16-byte rows: every producer
        op = inputs.make_operands(dtype, M, N, K, seed=606, alpha=alpha, beta=beta)
        for stages, producer in sorted(variants):
            say("persistent", dtype, tile, stages, producer, (M, N, K))
            ref = run_gpu(lib, op, stages=stages, producer=producer, tile=tile)
            for wg in (8, 16):
                got = run_gpu(lib, op, stages=stages, producer=producer, tile=tile, workgroups=wg)
                assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (tile, stages, producer, wg)
        check(op, ref)
        padding_untouched(op, ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "i8"])
def test_persistent_workgroups_short_k_and_k0(lib, dtype):
    """Fewer K tiles than stages, one K tile, and K = 0 (C = beta*C) with
    several output tiles per workgroup."""
    bk = {"f32": 32, "bf16": 64, "i8": 128}[dtype]
    alpha, beta = (1, 2) if dtype == "i8" else (1.0, 0.25)
    for K in (0, 1, bk, bk + 16, 3 * bk):
        for stages in (1, 2, 4):
            say("persistent short K", dtype, K, "stages", stages)
            op = inputs.make_operands(dtype, 520, 390, K, seed=K + 7, alpha=alpha, beta=beta)
            ref = run_gpu(lib, op, stages=stages)
            got = run_gpu(lib, op, stages=stages, workgroups=8)
            assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (K, stages)
            check(op, got)


@pytest.mark.parametrize("stages", [1, 2, 3, 4])
def test_k_slice_fingerprint_int8(lib, stages):
    """A = 1; B[k, j] = ((k // 64) + j) % 7 + 1: the exact column sums reveal a
    dropped, duplicated or stale K tile (page "GPU-Kernel pipelinen", common
    pitfalls: a forgotten epilogue tile silently drops the last BK columns)."""
    M, N = 256, 256
    for K in (64, 128, 192, 64 * stages, 64 * stages + 64, 64 * 9):
        say("fingerprint stages", stages, "K", K)
        op = inputs.make_operands("i8", M, N, K, seed=1, alpha=1, beta=0)
        op.A[:, :K] = 1
        kk = torch.arange(K).unsqueeze(1)
        jj = torch.arange(N).unsqueeze(0)
        op.B[:, :N] = (((kk // 64) + jj) % 7 + 1).to(torch.int8)
        got = run_gpu(lib, op, stages=stages, tile=(256, 256, 64))
        check(op, got)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_alpha_and_beta_scaling_are_exact(lib, dtype):
    """Exact identities of the fused epilogue, on a shape that cuts tiles:
    alpha = 2 gives twice the alpha = 1 output (a power of two scales
    exactly), and C = A*B + 1*C1 with C1 = A*B gives 2*C1 (x + x = 2x
    exactly), which also pins where old C is read from."""
    say("alpha/beta identities", dtype)
    op = inputs.make_operands(dtype, 300, 272, 520, seed=8, alpha=1.0, beta=0.0, ldc=280)
    c1 = run_gpu(lib, op, stages=2)
    op.alpha = 2.0
    c2 = run_gpu(lib, op, stages=2)
    assert torch.equal(c2[:, :272], c1[:, :272] * 2)
    op.alpha, op.beta = 1.0, 1.0
    op.C = c1.clone()
    c3 = run_gpu(lib, op, stages=2)
    assert torch.equal(c3[:, :272], c1[:, :272] * 2)
    assert torch.equal(c3[:, 272:], c1[:, 272:]) if dtype == "i8" else torch.equal(
        torch.isnan(c3[:, 272:]), torch.isnan(c1[:, 272:]))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_closed_forms_without_the_oracle(lib, dtype):
    """Closed forms checked on the GPU directly: all-ones A and B give
    C = alpha*K + beta*C0 rounded once to fp32 (alpha*K and the sums over K
    are exact for these K); int8 A = B = -128 gives
    16384*K and A = 1, B = -1 gives -K.  Shapes cut the output tiles and K
    tiles; every ring depth of the planner's tile."""
    M, N = 270, 260
    for K in (1, 77, 640, 1029):
        for stages in (1, 2, 3, 4):
            say("closed form", dtype, K, "stages", stages)
            alpha, beta = (3, -2) if dtype == "i8" else (0.5, 2.0)
            op = inputs.make_operands(dtype, M, N, K, seed=K + stages, alpha=alpha, beta=beta)
            op.A[:, :K] = 1
            op.B[:, :N] = 1
            got = run_gpu(lib, op, stages=stages)
            # alpha*K and beta*C0 are exact, so is their sum in fp64; rounding it once to
            # the output type is the fused epilogue's result
            want = (alpha * K + beta * op.C[:, :N].to(torch.float64)).to(got.dtype)
            assert torch.equal(got[:, :N], want), (K, stages)
            if dtype == "i8":
                for a, b, per_k in ((-128, -128, 16384), (1, -1, -1)):
                    op = inputs.make_operands("i8", M, N, K, seed=K, alpha=1, beta=0)
                    op.A[:, :K] = a
                    op.B[:, :N] = b
                    got = run_gpu(lib, op, stages=stages)
                    assert bool((got[:, :N] == per_k * K).all()), (a, b, K, stages)


@pytest.mark.parametrize("alpha,beta", [(-2 ** 31, 2 ** 31 - 1), (2 ** 31 - 1, -2 ** 31), (-3, -2 ** 31)])
def test_int8_scalars_at_the_ends_of_int32(lib, alpha, beta):
    """alpha and beta anywhere in int32: alpha*acc + beta*C0 wraps modulo
    2^32 on both sides, so the result is still bit-exact."""
    say("int8 scalars", alpha, beta)
    op = inputs.make_operands("i8", 300, 272, 200, seed=12, alpha=float(alpha), beta=float(beta))
    got = run_gpu(lib, op)
    check(op, got)
    assert oracle.gemm.last_overflow[0] > 0  # the exact result left int32: the wrap was exercised


@pytest.mark.parametrize("K", [2 ** 17 + 2 ** 12, 2 ** 17 + 2 ** 12 - 56])
def test_int8_accumulator_wraps_modulo_2_32(lib, K):
    """K beyond 2^17 lets the int32 accumulators of a long int8 dot product
    leave int32: rows of A = -128 against B of -128 (every seventh row -127)
    sum to about 16384 * K > 2^31 - 1, rows of A = 127 to about -16250 * K <
    -2^31, so every output's exact sum is outside int32.  The GPU's int32
    accumulation wraps modulo 2^32 like the oracle's exact sum reduced to
    int32 (no saturation), with a K tail that is not whole 16-byte chunks in
    the second case."""
    say("int8 accumulator wrap", K)
    op = inputs.make_operands("i8", 40, 48, K, seed=21)
    op.A[:, :K] = -128
    op.A[1::3, :K] = 127
    op.B[:, :48] = -128
    op.B[5::7, :48] = -127   # every seventh row of B one step smaller
    got = run_gpu(lib, op)
    check(op, got)
    assert oracle.gemm.last_overflow[1] > 0  # raw sums left int32 on the oracle's side too


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_subnormal_inputs_and_results_are_kept(lib, dtype):
    """Subnormal operands (and, for fp32 and bf16, subnormal fp32 results)
    are not flushed to zero: powers of two whose sums are exact, so the GPU
    must equal the oracle exactly."""
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    sub, big = {"f16": (2.0 ** -20, 2.0 ** 10), "bf16": (2.0 ** -130, 2.0 ** 20), "f32": (2.0 ** -140, 2.0 ** 30)}[dtype]
    M, N, K = 64, 80, 256
    for aval, bval in ((sub, big), (big, sub), (sub, 1.0)):
        say("subnormal", dtype, aval, bval)
        op = inputs.make_operands(dtype, M, N, K, seed=3)
        op.A[:, :K] = torch.tensor(aval, dtype=tdt)
        op.B[:, :N] = torch.tensor(bval, dtype=tdt)
        assert float(op.A[0, 0]) == aval and float(op.B[0, 0]) == bval  # representable as given
        got = run_gpu(lib, op)
        ref = reference(op)
        assert ref[0, 0] != 0.0
        assert np.array_equal(got[:, :N].double().numpy(), ref), (aval, bval)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_nan_and_inf_in_operands_propagate(lib, dtype):
    """IEEE propagation through the pipeline: a NaN in row 3 of A makes row 3
    of C NaN, a +Inf in row 7 (against a positive B) makes row 7 +Inf, a NaN
    in column 11 of B makes column 11 NaN; every other output is finite and
    within tolerance.  Padding past K stays NaN in the caller's memory and
    must not leak in (the tile's zeros there keep every other output finite)."""
    M, N, K = 130, 140, 300
    say("nan/inf", dtype)
    op = inputs.make_operands(dtype, M, N, K, seed=31, lda=K + 8, ldb=N + 8)
    op.B[:, :N] = op.B[:, :N].abs() + 0.5
    op.A[3, 17] = float("nan")
    op.A[7, 250] = float("inf")
    op.B[120, 11] = float("nan")
    got = run_gpu(lib, op)
    ref = reference(op)
    g = got[:, :N].double().numpy()
    assert np.all(np.isnan(g[3])) and np.all(np.isnan(g[:, 11]))
    assert np.all(np.isposinf(np.delete(g[7], 11)))
    assert np.array_equal(np.isnan(g), np.isnan(ref)) and np.array_equal(np.isinf(g), np.isinf(ref))
    rest = np.ones((M, N), bool)
    rest[[3, 7], :] = False
    rest[:, 11] = False
    err = np.max(np.abs(g[rest] - ref[rest]))
    bound = TOL[dtype] * math.sqrt(K) * np.max(np.abs(ref[rest]))
    assert err <= bound, (err, bound)


def test_calls_on_a_side_stream_follow_stream_order(lib):
    """Page "Software pipelines and asynchronous copies", section "Common
    errors": issuing is not completing.  On a side stream (default priority),
    a torch kernel writes A, a first GEMM reads it into C1, a second GEMM reads
    C1 as its A; only the side stream is synchronised at the end.  Each GEMM
    must see its predecessor's finished output: the second result equals the
    oracle applied to the first GPU result."""
    M = N = K = 1536
    say("side stream chain", (M, N, K))
    op1 = inputs.make_operands("f32", M, N, K, seed=41)
    op2 = inputs.make_operands("f32", M, N, N, seed=43)
    dev = torch.device("cuda:0")
    A_half = (op1.A * 0.5).to(dev)
    B1, B2 = op1.B.to(dev), op2.B.to(dev)
    C1 = torch.full((M, N), float("nan"), device=dev)
    C2 = torch.full((M, N), float("nan"), device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        A = A_half * 2.0                       # written on the side stream
        for _ in range(3):                     # and again, so the first GEMM would race a late write
            A.mul_(1.0)
        assert lib.pgemm_gemm(M, N, K, 1.0, A, K, B1, N, 0.0, C1, N, "f32", 0, side) == 0
        assert lib.pgemm_gemm(M, N, N, 1.0, C1, N, B2, N, 0.0, C2, N, "f32", 0, side) == 0
    side.synchronize()
    c1 = C1.cpu()
    a, b1, _ = op1.numpy_views()
    ref1 = oracle.gemm("f32", M, N, K, 1.0, a, b1)
    assert np.max(np.abs(c1.double().numpy() - ref1)) <= TOL["f32"] * math.sqrt(K) * np.max(np.abs(ref1))
    _, b2, _ = op2.numpy_views()
    ref2 = oracle.gemm("f32", M, N, N, 1.0, c1.numpy(), b2)
    g2 = C2.cpu().double().numpy()
    assert np.max(np.abs(g2 - ref2)) <= TOL["f32"] * math.sqrt(N) * np.max(np.abs(ref2))


def test_concurrent_calls_on_two_streams(lib):
    """The library keeps no state between calls: GEMMs of different dtypes
    and plans issued alternately on two streams (default priority) that run
    concurrently each match the oracle."""
    say("two streams")
    dev = torch.device("cuda:0")
    cases = [("bf16", 1024, 768, 1024), ("i8", 768, 1024, 512), ("f32", 512, 640, 384), ("f16", 640, 512, 700)]
    ops = [inputs.make_operands(dt, M, N, K, seed=50 + i, alpha=(2 if dt == "i8" else 1.5),
                                beta=(1 if dt == "i8" else 0.5)) for i, (dt, M, N, K) in enumerate(cases)]
    bufs = [(o.A.to(dev), o.B.to(dev), o.C.to(dev)) for o in ops]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for i, (o, (A, B, C)) in enumerate(zip(ops, bufs)):
            s = streams[i % 2]
            with torch.cuda.stream(s):
                C.copy_(o.C.to(dev))  # the same C0 for every repetition, in stream order
                r = lib.pgemm_gemm(o.M, o.N, o.K, o.alpha, A, o.lda, B, o.ldb, o.beta, C, o.ldc, o.dtype, 0, s)
                assert r == 0, lib.pgemm_strerror(r)
        for s in streams:
            s.synchronize()
        for o, (A, B, C) in zip(ops, bufs):
            check(o, C.cpu())


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_k_around_whole_rings_of_k_tiles(lib, dtype):
    """Prologue and drain at every compiled DIRECT tile class and ring depth
    S: K = nK * BK - 1, nK * BK and nK * BK + 1 for nK in {1, S - 1, S, S + 1}
    (page "Software pipelines and asynchronous copies", section "Prologue,
    steady state, and epilogue": fewer K tiles than stages; page "GPU-Kernel
    pipelinen", pitfalls: a forgotten epilogue tile and K tails).  One
    workgroup's tile is cut in M and N as well (150 x 144 outputs)."""
    classes = {}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        if v["dtype"] == dtype and v["producer"] == "direct":
            classes.setdefault((v["tile_m"], v["tile_n"], v["tile_k"]), []).append(v["stages"])
    M, N = 150, 144
    ran = 0
    for tile, depths in sorted(classes.items()):
        bk = tile[2]
        for S in sorted(depths):
            for nk in sorted({max(1, S - 1), S, S + 1, 1}):
                for delta in (-1, 0, 1):
                    K = nk * bk + delta
                    if K < 1:
                        continue
                    say("ring edges", dtype, tile, "S", S, "K", K)
                    op = inputs.make_operands(dtype, M, N, K, seed=7000 + K, alpha=1.0, beta=0.0)
                    got = run_gpu(lib, op, stages=S, producer="direct", tile=tile)
                    check(op, got)
                    ran += 1
    assert ran >= 60


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_edge_sizes(lib, dtype):
    """M, N around 16 and the tile edge; K around the K tile and the ring
    depth, including fewer K tiles than stages and K = 0."""
    es = inputs.ELEM_BYTES[dtype]
    epc = 16 // es
    bk = {"f32": 32, "f16": 64, "bf16": 64, "i8": 128}[dtype]
    for (M, N) in [(1, 1), (15, 17), (16, 16), (127, 129), (128, 128), (129, 1)]:
        for K in (0, 1, 3, epc, bk - epc, bk, bk + epc, 3 * bk, 4 * bk + 1):
            for stages in (1, 4):
                say("edge", dtype, (M, N, K), "stages", stages)
                op = inputs.make_operands(dtype, M, N, K, seed=M * 1000 + N * 10 + K, alpha=1.0, beta=0.0)
                got = run_gpu(lib, op, stages=stages)
                check(op, got)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_generic_producer_misaligned(lib, dtype):
    """Odd K, N and leading dimensions select the generic producer.  Its
    16-byte reads cross the end of a row (into NaN/0x7F padding when the
    leading dimension is padded, into the next row when it is tight).  Past K
    every element must be zero; past N the elements only feed columns that are
    never stored.  The last K tile reads chunk by chunk, element-wise at the
    very end of the matrix.  The narrow shapes put ldb below and just above 16
    bytes over many K tiles: below, every K tile takes the chunk-by-chunk path;
    above, whole reads spill into the next row of B."""
    for (M, N, K, pa, pb, pc) in [(130, 77, 203, 1, 2, 3), (129, 131, 97, 0, 0, 0), (64, 5, 3, 0, 1, 0),
                                  (200, 255, 1001, 3, 0, 1), (300, 272, 400, 1, 1, 0), (260, 400, 272, 1, 0, 0),
                                  (70, 3, 300, 0, 0, 0), (70, 6, 300, 1, 1, 0), (33, 17, 500, 0, 0, 1)]:
        for stages in (1, 2, 3, 4):
            say("misaligned", dtype, (M, N, K), "ld pads", (pa, pb, pc), "stages", stages)
            op = inputs.make_operands(dtype, M, N, K, seed=5 + K, alpha=1.0, beta=0.0, lda=K + pa, ldb=N + pb,
                                      ldc=N + pc)
            got = run_gpu(lib, op, stages=stages)
            check(op, got)
            padding_untouched(op, got)


def staged_classes(lib, dtype):
    out = {}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        if v["dtype"] == dtype and v["producer"] in ("staged_a", "staged_b"):
            out.setdefault(v["producer"], []).append((v["tile_m"], v["tile_n"], v["tile_k"]))
    return out


def _device_copy(t, dev, offset_elems=0):
    """t on the GPU; with offset_elems > 0 the returned view starts that many
    elements into a slightly larger buffer (element-aligned, not 16-byte
    aligned), holding the same rows with the same leading dimension."""
    if not offset_elems:
        return t.to(dev), None
    flat = torch.zeros(t.numel() + offset_elems, dtype=t.dtype, device=dev)
    flat[offset_elems:] = t.reshape(-1).to(dev)
    return flat[offset_elems:].view(t.shape), flat


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_one_operand_misaligned(lib, dtype):
    """One producer per operand.  STAGED_A keeps LDS-DMA for B and stages A
    through registers, STAGED_B the reverse; each is forced on layouts where
    the staged operand is awkward (an odd leading dimension, rows that are not
    whole 16-byte chunks, a pointer off 16-byte alignment), and the planner's
    own pick (DIRECT when B's rows are whole chunks) runs beside it.  Each
    result is checked against the oracle, and the forced one -- since both
    producers of an operand fill the LDS stage with the same bytes -- must be
    bit-identical, in every stored column, to the DIRECT producer on a
    zero-padded aligned copy (K and N rounded up to whole chunks), with the
    same tile class."""
    es = inputs.ELEM_BYTES[dtype]
    epc = 16 // es
    dev = torch.device("cuda:0")
    classes = staged_classes(lib, dtype)
    assert set(classes) == {"staged_a", "staged_b"}
    for prod, tiles in sorted(classes.items()):
        for tile in tiles:
            BM, BN, BK = tile
            if prod == "staged_a":   # A breaks the rules, B keeps them
                cases = [dict(M=2 * BM + 3, N=BN + 2 * epc, K=3 * BK + 5, lda=3 * BK + 6, ldb=BN + 2 * epc, off=0),
                         dict(M=BM + 7, N=2 * BN, K=2 * BK + 1, lda=2 * BK + 1, ldb=2 * BN + epc, off=0),
                         dict(M=BM + 1, N=BN + epc, K=4 * BK, lda=4 * BK + epc, ldb=BN + epc, off=1)]
            else:                    # B breaks the rules, A keeps them
                cases = [dict(M=2 * BM + 3, N=BN + 5, K=3 * BK + epc, lda=3 * BK + epc, ldb=BN + 6, off=0),
                         dict(M=BM + 7, N=2 * BN + 3, K=2 * BK, lda=2 * BK + epc, ldb=2 * BN + 3, off=0),
                         dict(M=BM + 1, N=BN + epc, K=4 * BK, lda=4 * BK, ldb=BN + epc, off=1)]
            for c in cases:
                M, N, K = c["M"], c["N"], c["K"]
                say("one operand misaligned", dtype, prod, tile, c)
                op = inputs.make_operands(dtype, M, N, K, seed=M + N + K, alpha=1.0, beta=0.0, lda=c["lda"],
                                          ldb=c["ldb"])
                # device operands, the misaligned one possibly one element off 16-byte alignment
                A, keep_a = _device_copy(op.A, dev, c["off"] if prod == "staged_a" else 0)
                B, keep_b = _device_copy(op.B, dev, c["off"] if prod == "staged_b" else 0)
                cls = lib.ALIGNED_B if prod == "staged_a" else lib.ALIGNED_A
                r, plan = lib.pgemm_plan(M, N, K, dtype, 0, cls, None)
                assert r == 0 and plan["producer"] in ("direct", prod, "generic"), plan
                outs = {}
                for key, stages, producer, t in (("auto", 0, None, None), ("forced", 2, prod, tile)):
                    C = op.C.to(dev)
                    rr = lib.pgemm_gemm_ex(M, N, K, 1.0, A, op.lda, B, op.ldb, 0.0, C, op.ldc, dtype, stages,
                                           lib._opts(producer, t), None)
                    assert rr == 0, lib.pgemm_strerror(rr)
                    torch.cuda.synchronize()
                    outs[key] = C.cpu()
                check(op, outs["auto"])
                check(op, outs["forced"])
                # the DIRECT producer on a zero-padded aligned copy, same tile class
                Kp, Np = -(-K // epc) * epc, -(-N // epc) * epc
                pad = inputs.make_operands(dtype, M, Np, Kp, seed=1, alpha=1.0, beta=0.0)
                pad.A.zero_()
                pad.B.zero_()
                pad.A[:, :K] = op.A[:, :K]
                pad.B[:K, :N] = op.B[:, :N]
                ref = run_gpu(lib, pad, stages=2, producer="direct", tile=tile)[:, :N].contiguous()
                got = outs["forced"][:, :N].contiguous()
                assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (prod, tile, c)
                del A, B, keep_a, keep_b


def direct_classes(lib, dtype):
    out = {}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        if v["dtype"] == dtype and v["producer"] == "direct":
            out.setdefault((v["tile_m"], v["tile_n"], v["tile_k"]), []).append(v["stages"])
    return out


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_direct_unaligned_rows_and_k_tail(lib, dtype):
    """DIRECT on rows that start anywhere (odd lda and ldb, pointers one
    element off 16-byte alignment) and on a K that is not whole 16-byte
    chunks: LDS-DMA takes the element-aligned rows as they are, and in the K
    tile that holds the end of K the chunk of each row that straddles K is
    loaded element by element, zero past K (in the loop, or in the prologue
    when the ring holds every K tile).  Every compiled DIRECT variant, and
    persistent workgroups, against the oracle and bit-identical to DIRECT on
    a zero-padded aligned copy (K rounded up to whole chunks), same tile
    class and depth: the stage holds the same bytes either way."""
    es = inputs.ELEM_BYTES[dtype]
    epc = 16 // es
    dev = torch.device("cuda:0")
    for tile, depths in sorted(direct_classes(lib, dtype).items()):
        BM, BN, BK = tile
        for S in sorted(depths):
            cases = [dict(M=BM + 5, N=2 * BN - epc, K=3 * BK + 1, lda=3 * BK + 1, ldb=2 * BN - epc + 1, off=1, wg=0),
                     dict(M=2 * BM + 3, N=BN + 2 * epc, K=S * BK - 3, lda=S * BK + 2, ldb=BN + 2 * epc, off=0, wg=0),
                     dict(M=BM - 7, N=BN, K=BK // 2 + 1, lda=BK // 2 + 1, ldb=BN + 3, off=1, wg=0),
                     dict(M=3 * BM + 1, N=2 * BN, K=4 * BK + epc - 1, lda=4 * BK + epc + 5, ldb=2 * BN, off=1,
                          wg=8 if S > 1 else 0)]
            for c in cases:
                M, N, K = c["M"], c["N"], c["K"]
                say("direct unaligned", dtype, tile, "S", S, c)
                op = inputs.make_operands(dtype, M, N, K, seed=M + 3 * N + K, alpha=1.0, beta=0.0, lda=c["lda"],
                                          ldb=c["ldb"])
                A, keep_a = _device_copy(op.A, dev, c["off"])
                B, keep_b = _device_copy(op.B, dev, c["off"])
                C = op.C.to(dev)
                rr = lib.pgemm_gemm_ex(M, N, K, 1.0, A, op.lda, B, op.ldb, 0.0, C, op.ldc, dtype, S,
                                       lib._opts("direct", tile, workgroups=c["wg"]), None)
                assert rr == 0, lib.pgemm_strerror(rr)
                torch.cuda.synchronize()
                got = C.cpu()
                check(op, got)
                padding_untouched(op, got)
                Kp = -(-K // epc) * epc
                pad = inputs.make_operands(dtype, M, N, Kp, seed=1, alpha=1.0, beta=0.0)
                pad.A.zero_()
                pad.B.zero_()
                pad.A[:, :K] = op.A[:, :K]
                pad.B[:K, :N] = op.B[:, :N]
                ref = run_gpu(lib, pad, stages=S, producer="direct", tile=tile)[:, :N].contiguous()
                assert torch.equal(got[:, :N].contiguous().view(torch.int32), ref.view(torch.int32)), (tile, S, c)
                del A, B, C, keep_a, keep_b


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "i8"])
def test_generic_matches_direct_on_zero_padded_copy(lib, dtype):
    """The generic producer on an odd-sized problem fills each LDS stage, in
    every column below N, with exactly the bytes the direct producer copies
    from a zero-padded, aligned copy of the same matrices (K and N rounded up
    to 16 bytes), so within one tile class the stored C is bit-identical, for
    every tile class and depth the generic producer is compiled for."""
    epc = 16 // inputs.ELEM_BYTES[dtype]
    classes = {}
    for i in range(lib.pgemm_num_variants()):
        v = lib.pgemm_variant_info(i)
        if v["dtype"] == dtype and v["producer"] == "generic":
            classes.setdefault((v["tile_m"], v["tile_n"], v["tile_k"]), []).append(v["stages"])
    assert classes
    for tile, depths in sorted(classes.items()):
        M, N, K = 2 * tile[0] + 3, tile[1] + 5, 3 * tile[2] + 5
        Kp, Np = -(-K // epc) * epc, -(-N // epc) * epc
        op = inputs.make_operands(dtype, M, N, K, seed=99, alpha=1.0, beta=0.0, lda=K + 1, ldb=N)
        pad = inputs.make_operands(dtype, M, Np, Kp, seed=99, alpha=1.0, beta=0.0)
        pad.A.zero_()
        pad.B.zero_()
        pad.A[:, :K] = op.A[:, :K]
        pad.B[:K, :N] = op.B[:, :N]
        say("generic vs direct", dtype, tile, (M, N, K), "padded", (Kp, Np))
        ref = run_gpu(lib, pad, stages=1, producer="direct", tile=tile)[:, :N]
        for stages in sorted(depths):
            say("generic", dtype, tile, "stages", stages)
            got = run_gpu(lib, op, stages=stages, producer="generic", tile=tile)[:, :N]
            assert torch.equal(got.contiguous().view(torch.int32), ref.contiguous().view(torch.int32)), (tile, stages)
        check(op, run_gpu(lib, op, stages=min(depths), producer="generic", tile=tile))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_leading_dimensions_at_the_addressing_limit(lib, dtype):
    """lda, ldb and ldc just below the 32-bit tile addressing limits the ABI
    enforces (lda*s*256, ldb*s*128, ldc*4*256 < 2^31): the per-tile byte
    offsets reach their largest values.  The matrices live in a few GiB of
    device memory; padding is NaN.  One element more is refused."""
    es = inputs.ELEM_BYTES[dtype]
    M, N, K = 300, 136, 96
    lda = (1 << 31) // (es * 256) - 16
    ldb = (1 << 31) // (es * 128) - 16
    ldc = (1 << 31) // (4 * 256) - 16
    say("addressing limit", dtype, (M, N, K), "ld", (lda, ldb, ldc))
    op = inputs.make_operands(dtype, M, N, K, seed=17, alpha=1.0, beta=0.5)
    dev = torch.device("cuda:0")
    A = torch.full((M, lda), float("nan"), dtype=op.A.dtype, device=dev)
    B = torch.full((K, ldb), float("nan"), dtype=op.B.dtype, device=dev)
    C = torch.full((M, ldc), float("nan"), dtype=torch.float32, device=dev)
    A[:, :K] = op.A[:, :K].to(dev)
    B[:, :N] = op.B[:, :N].to(dev)
    C[:, :N] = op.C[:, :N].to(dev)
    r = lib.pgemm_gemm(M, N, K, 1.0, A, lda, B, ldb, 0.5, C, ldc, dtype, 0)
    assert r == 0, lib.pgemm_strerror(r)
    torch.cuda.synchronize()
    got = C[:, :N].cpu()
    untouched = bool(torch.isnan(C[:, N:N + 64]).all())
    assert untouched                                # the caller's memory past N is untouched
    del A, B, C
    torch.cuda.empty_cache()
    check(op, got)
    big = (1 << 31) // (4 * 256)
    assert lib.pgemm_gemm(M, N, K, 1.0, 1 << 20, lda, 1 << 20, ldb, 0.5, 1 << 20, big, dtype, 0) == -7


def test_beta_zero_ignores_nan_in_C_and_K0(lib):
    op = inputs.make_operands("f32", 64, 64, 0, seed=2, alpha=1.0, beta=0.0)
    got = run_gpu(lib, op)
    assert torch.equal(got[:, :64], torch.zeros(64, 64))
    op = inputs.make_operands("f32", 64, 64, 0, seed=2, alpha=1.0, beta=0.5)
    got = run_gpu(lib, op)
    assert torch.equal(got[:, :64], 0.5 * op.C[:, :64])


def test_argument_errors_before_launch(lib):
    op = inputs.make_operands("bf16", 8, 8, 8, seed=1)
    say("errors")
    A = op.A.cuda()
    C = op.C.cuda()
    a, c = A.data_ptr(), C.data_ptr()  # plain addresses: a failing assert never prints a device tensor
    assert lib.pgemm_gemm(8, 8, 8, 1.0, a, 4, a, 8, 0.0, c, 8, "bf16", 0) == -1  # lda < K
    assert lib.pgemm_gemm(8, 8, 8, 1.0, a, 8, a, 8, 0.0, c, 8, 7, 0) == -2
    assert lib.pgemm_gemm(8, 8, 8, 1.0, a, 8, a, 8, 0.0, c, 8, "bf16", 5) == -3
    assert lib.pgemm_gemm(8, 8, 8, 0.5, a, 8, a, 8, 0.0, c, 8, "i8", 0) == -5
    assert lib.pgemm_gemm(0, 8, 8, 1.0, 0, 8, 0, 8, 0.0, 0, 8, "bf16", 0) == 0


# ------------------------------------------------------------------ full-size workloads
# (the benchmark workloads themselves: tests/test_fullsize_gpu.py)

def test_persistent_workgroups_full_size(lib):
    """8192 x 4096 outputs (512 tiles of 256 x 256) on one round of 256
    persistent workgroups, two tiles each: every output against the oracle,
    and bit-identical to one workgroup per tile."""
    M, N, K = 8192, 4096, 1024
    say("persistent full size", (M, N, K))
    op = inputs.make_operands("bf16", M, N, K, seed=4321, alpha=1.0, beta=0.0)
    ref = run_gpu(lib, op)
    got = run_gpu(lib, op, workgroups=256)
    check(op, got)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


def test_identity_B_full_size_is_exact(lib):
    """B = I gives C = A exactly (one nonzero product per sum), over every tile
    of a 4096 x 4096 problem."""
    say("identity 4096")
    N = 4096
    A = inputs.draw("bf16", 4096, N, seed=31).cuda()
    B = torch.eye(N, dtype=torch.bfloat16).cuda()
    C = torch.empty(4096, N, dtype=torch.float32).cuda()
    r = lib.pgemm_gemm(4096, N, N, 1.0, A, N, B, N, 0.0, C, N, "bf16", 0)
    assert r == 0, lib.pgemm_strerror(r)
    torch.cuda.synchronize()
    same = bool(torch.equal(C, A.float()))
    assert same
