"""Consume-before-reuse hazard demonstrator on the GPU (page "Software pipelines
and asynchronous copies", sections "Producer-consumer synchronization" and
"Practice").

pgemm_hazard_copy_reduce reduces a 4096 x 4096 int32 array to row sums through
two LDS stages, with the correct protocol (reuse barrier, then the rewrite of
stage t%2 with tile t+2, then the readiness barrier) or with only the reuse
barrier removed.  Row sums are exact integers, so every run is compared with
the oracle bit for bit:

* edge shapes (one and two column tiles, padded rows, no columns) and the full
  array, correct protocol: equal to the oracle;
* stress iterations on eight randomized inputs with one consumer wave delayed
  (each wave in turn, varying delays): the correct protocol never fails in
  5000; without the reuse barrier the runs (1000) fail, and the
  wrong rows are the delayed wave's;
* without the reuse barrier and without a delay the failures are intermittent
  (counted, not asserted); a sweep of the delay shows where failures begin:
  once the delayed wave lags by more than the other waves need to load tile
  t+2 and rewrite the stage;
* the timeline of one workgroup (shader-clock stamps per wave and tile) shows
  the ordering edge: with the reuse barrier no wave rewrites stage t%2 before
  the delayed wave has finished reading tile t from it; without it the other
  waves rewrite the stage before the delayed wave starts reading.

All inputs stay in device memory; the oracle's sums are computed once per
input on the host.
"""
import numpy as np
import pytest
import torch

import oracle
from software_pipelined_tiled_loop_amd import inputs

pytestmark = pytest.mark.gpu

ROWS = COLS = 4096
RB, TC, NWAVE, EV = 16, 256, 4, 6
N_INPUTS = 8
ITERS = 1000
ITERS_CORRECT = 5000  # correct protocol: more runs, since it must never fail
SLEEP = 8128  # shader clocks of one long s_sleep


def say(*a):
    print("[hazard]", *a, flush=True)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from software_pipelined_tiled_loop_amd import binding
    return binding


@pytest.fixture(scope="module")
def arrays(lib):
    """Eight randomized 4096 x 4096 inputs on the device and the oracle's sums of each."""
    xs, refs = [], []
    for i in range(N_INPUTS):
        X = inputs.make_hazard_input(ROWS, COLS, seed=inputs.seed_for("hazard", i))
        refs.append(torch.from_numpy(oracle.row_sums(X.numpy(), ROWS, COLS)).cuda())
        xs.append(X.cuda())
    return xs, refs


def run(lib, X, rows, cols, ldx, reuse_wait, delay_wave=-1, delay_cycles=0, trace=None, trace_wg=0):
    sums = torch.full((max(rows, 1),), inputs.POISON_I32, dtype=torch.int32, device="cuda")
    r = lib.pgemm_hazard_copy_reduce(X, rows, cols, ldx, sums, reuse_wait, delay_wave, delay_cycles, trace,
                                     0 if trace is None else trace.numel(), trace_wg)
    assert r == 0, lib.pgemm_strerror(r)
    return sums[:rows]


@pytest.mark.parametrize("rows,cols,ldx", [(16, 256, 256), (16, 512, 512), (48, 768, 780), (32, 1280, 1284),
                                           (64, 0, 4)])
def test_correct_protocol_matches_oracle_on_edge_shapes(lib, rows, cols, ldx):
    say("edge", rows, cols, ldx)
    X = inputs.make_hazard_input(rows, cols, seed=inputs.seed_for("hazard", 100 + cols), ldx=ldx)
    ref = oracle.row_sums(X.numpy(), rows, cols, ldx)
    Xd = X.cuda()
    for delay_wave in (-1, 0, 3):
        got = run(lib, Xd, rows, cols, ldx, 1, delay_wave, 2 * SLEEP if delay_wave >= 0 else 0).cpu().numpy()
        assert np.array_equal(got, ref), (rows, cols, ldx, delay_wave)


def test_correct_protocol_matches_oracle_on_the_full_array(lib, arrays):
    xs, refs = arrays
    for i in range(N_INPUTS):
        say("full array, input", i)
        assert torch.equal(run(lib, xs[i], ROWS, COLS, COLS, 1), refs[i])


def stress(lib, arrays, reuse_wait, with_delay, iters=ITERS):
    """Failing runs, wrong rows, and the wrong rows that belong to the delayed wave."""
    xs, refs = arrays
    failing_runs = wrong_rows = wrong_rows_of_delayed = 0
    for i in range(iters):
        d = i % NWAVE if with_delay else -1
        cycles = (1 + i % 4) * SLEEP if with_delay else 0
        got = run(lib, xs[i % N_INPUTS], ROWS, COLS, COLS, reuse_wait, d, cycles)
        bad = (got != refs[i % N_INPUTS]).nonzero().flatten()
        if bad.numel():
            failing_runs += 1
            wrong_rows += bad.numel()
            if d >= 0:
                wrong_rows_of_delayed += int(((bad % RB) // (RB // NWAVE) == d).sum())
    return failing_runs, wrong_rows, wrong_rows_of_delayed


def test_stress_correct_protocol_never_fails(lib, arrays):
    say("stress: reuse barrier, delayed wave,", ITERS_CORRECT, "iterations")
    runs, rows, _ = stress(lib, arrays, 1, True, ITERS_CORRECT)
    say("  failing runs", runs, "of", ITERS_CORRECT, "wrong rows", rows)
    assert runs == 0


def test_stress_without_reuse_barrier_fails_on_the_delayed_wave(lib, arrays):
    say("stress: reuse barrier removed, delayed wave,", ITERS, "iterations")
    runs, rows, of_delayed = stress(lib, arrays, 0, True)
    say("  failing runs", runs, "of", ITERS, "wrong rows", rows, "of which the delayed wave's", of_delayed)
    assert runs > 0
    assert of_delayed > 0


def test_stress_without_reuse_barrier_and_without_delay_is_counted(lib, arrays):
    say("stress: reuse barrier removed, no delay,", ITERS, "iterations")
    runs, rows, _ = stress(lib, arrays, 0, False)
    say("  failing runs", runs, "of", ITERS, "wrong rows", rows)


def timeline(lib, arrays, reuse_wait, delay_wave, cycles):
    xs, refs = arrays
    nT = COLS // TC
    trace = torch.zeros(NWAVE * nT * EV, dtype=torch.int64, device="cuda")
    run(lib, xs[0], ROWS, COLS, COLS, reuse_wait, delay_wave, cycles, trace=trace, trace_wg=5)
    T = trace.cpu().numpy().reshape(NWAVE, nT, EV)
    return T - T[:, 0, 0].min()


EVENTS = ("top", "read start", "read end", "past reuse", "rewritten", "past ready")


def test_timeline_shows_the_reuse_edge(lib, arrays):
    d, cycles = 1, 2 * SLEEP
    nT = COLS // TC
    for reuse_wait in (1, 0):
        T = timeline(lib, arrays, reuse_wait, d, cycles)
        say("timeline, workgroup 5, wave %d delayed by %d cycles, reuse barrier %s (cycles from the first stamp)"
            % (d, cycles, "kept" if reuse_wait else "removed"))
        for t in range(3):
            for w in range(NWAVE):
                say("  tile %d wave %d: " % (t, w) + ", ".join("%s %d" % (n, v) for n, v in zip(EVENTS, T[w, t])))
        assert (np.diff(T.reshape(NWAVE, -1), axis=1) >= 0).all()  # each wave's stamps in program order
        others = [w for w in range(NWAVE) if w != d]
        refills = range(nT - 2)  # tiles whose stage is rewritten
        if reuse_wait:
            for t in refills:
                for w in others:
                    assert T[w, t, 4] >= T[d, t, 2], (t, w)
        else:
            early = sum(1 for t in refills for w in others if T[w, t, 4] < T[d, t, 1])
            say("  rewrites of stage t%%2 before the delayed wave started reading tile t: %d of %d"
                % (early, len(refills) * len(others)))
            assert early > 0


def test_failures_begin_when_the_delay_exceeds_the_rewrite_time(lib, arrays):
    """Without the reuse barrier, the share of failing runs against the delay of
    one consumer wave (200 runs per delay, the delayed wave rotating).  The
    other waves rewrite the stage about as long after the top of the iteration
    as their loads of tile t+2 take, so short delays leave the race unseen."""
    xs, refs = arrays
    rows_out = []
    for cycles in (0, 256, 512, 768, 1024, 1536, 2048, 3072, 4096, 8192, 16384):
        fails = 0
        for i in range(200):
            got = run(lib, xs[i % N_INPUTS], ROWS, COLS, COLS, 0, i % NWAVE, cycles)
            fails += int(not torch.equal(got, refs[i % N_INPUTS]))
        rows_out.append((cycles, fails))
        say("  delay %5d cycles: %3d of 200 runs failed" % (cycles, fails))
    assert rows_out[-1][1] == 200 and rows_out[-2][1] == 200
