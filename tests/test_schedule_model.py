"""Model check of the LDS stage protocol (host only).

Page "Software pipelines and asynchronous copies" (section "Producer-consumer
synchronization") gives each stage two transitions: after the producer
finishes writing it, consumers may read it (ready); after every consumer
finishes reading it, the producer may overwrite it (reuse).  Section
"Prologue, steady state, and epilogue" adds that the prologue must not run
past K and the epilogue must not consume a stage whose load was not waited
for.

This test replays the event sequence of the kernel's K loop (pertile_loop /
stream_loop / tile_body / single_buffer_loop of pgemm_kernel.hpp) for every
producer, ring depth S = 1..4, K steps per tile NKS = 1..2, number of K tiles
nK = 0..12 and 1..3 output tiles per workgroup (a persistent workgroup streams
the K tiles of all its output tiles through one ring), and checks, for a
workgroup of waves that all run the same program and meet only at barriers:

  ready   every read of a stage sees the slot the step expects; that slot's
          load was waited for (vector loads retire in issue order, so a wait
          with P pending groups completes all but the last P) or written by
          ds_write, and a barrier lies between that and the read;
  reuse   between any read of a stage and a later load into it there is a
          barrier (our barriers drain LDS reads first), and the stage's
          previous load had completed (no two loads race into one stage);
  order   every K tile of every output tile is multiplied exactly once, its
          steps in order, from fragments read after its ready edge; each
          output tile is stored once, after its last MFMA and before the next
          tile's first; no real load targets a slot past the workgroup's
          work; nothing is in flight when the workgroup ends.
"""
import itertools

import pytest


class Trace:
    """Events of one wave's program.  Each K tile has an A half and a B half
    in its stage; a load group moves one or both halves, by LDS-DMA (into the
    stage) or into registers (written to the stage later by ds_write)."""

    def __init__(self, nK):
        self.nK = nK
        self.ev = []          # (kind, ...) in program order

    def issue(self, tile, stage, direct, halves="AB"):
        # direct: an LDS-DMA group into the stage; else a register load (no LDS effect)
        self.ev.append(("issue", tile, stage if direct else None, tile < self.nK, halves))

    def write(self, tile, stage, halves="AB"):
        self.ev.append(("write", tile, stage, tile < self.nK, halves))

    def wait(self, pending):
        self.ev.append(("wait", pending))

    def barrier(self):
        self.ev.append(("barrier",))

    def read(self, stage, tile, ks):
        self.ev.append(("read", stage, tile, ks))

    def mfma(self, tile, ks):
        self.ev.append(("mfma", tile, ks))

    def store(self, out_tile):
        self.ev.append(("store", out_tile))

    def waitall(self):
        self.ev.append(("wait", 0))


# ---- the kernel's control flow, event by event -------------------------------
# A "slot" is one K tile of one output tile: slot s = tile s // nK, K tile s % nK.
# mode: "direct" (both halves by LDS-DMA), "register" (both through registers)
# or "mixed" (one producer per operand: A through registers, B by LDS-DMA; the
# other assignment has the same event order).  Before a ds_write of staged
# registers the compiler waits for their load; with no later register load of
# its own in flight that is vmcnt(0), modelled as wait(0).

def _halves(mode):
    return {"direct": ("AB", ""), "register": ("", "AB"), "mixed": ("B", "A")}[mode]


def stream_loop(S, NKS, nK, ntiles, mode):
    dma_h, reg_h = _halves(mode)
    total = ntiles * nK
    tr = Trace(total)
    for p in range(S - 1):                       # prologue slots 0..S-2
        if reg_h:
            tr.issue(p, None, False, reg_h)
        if dma_h:
            tr.issue(p, p, True, dma_h)
        if reg_h:
            tr.wait(0)
            tr.write(p, p, reg_h)
    if reg_h:
        tr.issue(S - 1, None, False, reg_h)      # slot S-1 into registers
    sync_ring(tr, S, mode)                       # B_0
    if reg_h:                                    # stage S-1 never used before
        tr.wait(0)
        tr.write(S - 1, S - 1, reg_h)
    if dma_h:
        tr.issue(S - 1, S - 1, True, dma_h)
    if reg_h:
        tr.issue(S, None, False, reg_h)
    tr.read(0, 0, 0)
    cur = 0
    for s in range(total):
        nstage = (cur + 1) % S
        for ks in range(NKS):
            if ks + 1 < NKS:
                tr.read(cur, s, ks + 1)
            else:
                sync_ring(tr, S, mode)           # B_{s+1}
                if reg_h:
                    tr.wait(0)
                    tr.write(s + S, cur, reg_h)
                if dma_h:
                    tr.issue(s + S, cur, True, dma_h)
                if reg_h:
                    tr.issue(s + S + 1, None, False, reg_h)
                tr.read(nstage, s + 1, 0)
            tr.mfma(s, ks)
        cur = nstage
        if (s + 1) % nK == 0:                    # last K tile of an output tile: its epilogue
            tr.store(s // nK)
    tr.waitall()
    return tr


def sync_ring(tr, S, mode):
    if mode == "direct":
        tr.wait(S - 2)
    elif mode == "mixed":
        tr.wait(1)                               # the register loads issued after the pieces
    tr.barrier()


def single_buffer_tile(tr, base, NKS, nK, direct):
    """One output tile with one LDS buffer; slots base .. base+nK-1."""
    if direct:
        for t in range(nK):
            tr.issue(base + t, 0, True)
            tr.wait(0)
            tr.barrier()
            for ks in range(NKS):
                tr.read(0, base + t, ks)
                tr.mfma(base + t, ks)
            tr.barrier()
    else:
        if nK > 0:
            tr.issue(base, None, False)
            tr.wait(0)
            tr.write(base, 0)
        for t in range(nK):
            tr.barrier()
            more = t + 1 < nK
            if more:
                tr.issue(base + t + 1, None, False)
            for ks in range(NKS):
                tr.read(0, base + t, ks)
                tr.mfma(base + t, ks)
            tr.barrier()
            if more:
                tr.wait(0)
                tr.write(base + t + 1, 0)


def kernel_trace(S, NKS, nK, mode, ntiles=1):
    if mode is True or mode is False:
        mode = "direct" if mode else "register"
    if nK > 0 and S > 1:
        tr = stream_loop(S, NKS, nK, ntiles, mode)
    else:
        assert mode != "mixed", "one producer per operand runs a two-stage ring"
        tr = Trace(ntiles * nK)                  # tile by tile (S = 1, or K = 0)
        for j in range(ntiles):
            if S == 1:
                single_buffer_tile(tr, j * nK, NKS, nK, mode == "direct")
            tr.store(j)
        tr.waitall()
    tr.k_tiles, tr.ntiles = nK, ntiles
    return tr


# ---- the checker ----------------------------------------------------------------

def check(tr, S, NKS):
    ev = tr.ev
    loads = []               # (position, tile, stage or None, halves) of every load group, in issue order
    completed = {}           # index into loads -> position of the wait that completed it (vmcnt counts
    #                          every load, DMA or register, in issue order)
    content = {}             # (stage, half) -> (tile, position of the load/write, kind)
    reads_since = {}         # (stage, half) -> positions of reads of its current content
    last_barrier = -1
    read_ok = {}             # (tile, ks) -> position of a valid read
    consumed = []
    stores = []

    def load_index(pos):
        return [k for k, d in enumerate(loads) if d[0] == pos][0]

    for pos, e in enumerate(ev):
        kind = e[0]
        if kind == "barrier":
            last_barrier = pos
        elif kind == "wait":
            pending = e[1]
            for i in range(len(loads) - pending):
                completed.setdefault(i, pos)
        elif kind in ("issue", "write"):
            tile, stage, real, halves = e[1], e[2], e[3], e[4]
            if kind == "issue":
                loads.append((pos, tile, stage, halves))
                if stage is None:
                    continue                      # register load: no LDS effect yet
            else:
                # the registers written must hold this tile's completed load
                src = [k for k, d in enumerate(loads) if d[2] is None and d[1] == tile and d[3] == halves]
                assert src and src[-1] in completed, "tile %d written from registers before its load" % tile
            for h in halves:
                key = (stage, h)
                # reuse edge: every read of the half's current content precedes a barrier before us
                for rp in reads_since.get(key, []):
                    assert rp < last_barrier, "stage %d overwritten at %d while read at %d" % (stage, pos, rp)
                prev = content.get(key)
                if prev is not None and prev[2] == "issue":
                    assert load_index(prev[1]) in completed, \
                        "stage %d re-filled before its previous load completed" % stage
                content[key] = (tile, pos, kind)
                reads_since[key] = []
        elif kind == "read":
            stage, tile, ks = e[1], e[2], e[3]
            if tile >= tr.nK:
                continue                          # look-ahead read past the last tile: never multiplied
            for h in "AB":
                c = content.get((stage, h))
                assert c is not None and c[0] == tile, \
                    "read of stage %d half %s expects tile %d, holds %s" % (stage, h, tile, c)
                # ready edge
                if c[2] == "issue":
                    i = load_index(c[1])
                    assert i in completed, "tile %d read before its load was waited for" % tile
                    # every wave waits for its own pieces, then the barrier makes all of them visible
                    assert completed[i] < last_barrier, "tile %d: no barrier after the wait for its load" % tile
                assert last_barrier > c[1], "tile %d read without a barrier after its load/write" % tile
                reads_since.setdefault((stage, h), []).append(pos)
            read_ok[(tile, ks)] = pos
        elif kind == "mfma":
            tile, ks = e[1], e[2]
            assert (tile, ks) in read_ok and read_ok[(tile, ks)] < pos, "MFMA on unread fragments %s" % ((tile, ks),)
            consumed.append((tile, ks))
        elif kind == "store":
            # output tile e[1] is complete: every MFMA of its slots done, none of a later tile's
            j = e[1]
            mine = [(j * tr.k_tiles + t, k) for t in range(tr.k_tiles) for k in range(NKS)]
            assert all(m in consumed for m in mine), "output tile %d stored before its last MFMA" % j
            assert all(c[0] < (j + 1) * tr.k_tiles for c in consumed), "output tile %d stored late" % j
            stores.append(j)
    # order: each slot once, steps in order; each output tile stored once, in order
    assert consumed == [(t, k) for t in range(tr.nK) for k in range(NKS)]
    assert stores == list(range(tr.ntiles))
    # nothing in flight at the end
    assert len(completed) == len(loads)
    # no real load targets a tile >= nK
    for e in ev:
        if e[0] in ("issue", "write"):
            assert e[3] == (e[1] < tr.nK)


@pytest.mark.parametrize("NKS", [1, 2])
@pytest.mark.parametrize("ntiles", [1, 2, 3])
def test_stage_protocol_one_producer_per_operand(NKS, ntiles):
    """The two-stage ring of STAGED_A / STAGED_B: one half of each stage by
    LDS-DMA, the other from registers; the barrier waits for all but the
    register loads issued after the pieces."""
    for nK in range(0, 13):
        check(kernel_trace(2 if nK else 1, NKS, nK, "mixed" if nK else "direct", ntiles), 2, NKS)


def test_checker_catches_a_mixed_ring_that_waits_for_too_few_loads():
    """Sensitivity: with one producer per operand, letting the LDS-DMA pieces
    stay in flight across the barrier (waiting as if they were the register
    loads issued after them) breaks the ready edge."""
    tr = kernel_trace(2, 1, 6, "mixed")
    tr.ev = [("wait", 2) if e == ("wait", 1) else e for e in tr.ev]
    with pytest.raises(AssertionError):
        check(tr, 2, 1)


def test_checker_catches_register_loads_issued_before_the_pieces():
    """Sensitivity: if the register loads of slot s+3 were issued before the
    pieces of slot s+2, the barrier's wait for all but the last group would
    leave those pieces in flight."""
    tr = kernel_trace(2, 1, 6, "mixed")
    ev = tr.ev
    for i in range(len(ev) - 1):
        a, b = ev[i], ev[i + 1]
        if a[0] == "issue" and a[2] is not None and b[0] == "issue" and b[2] is None:
            ev[i], ev[i + 1] = b, a
    with pytest.raises(AssertionError):
        check(tr, 2, 1)


@pytest.mark.parametrize("direct", [True, False], ids=["direct", "register"])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("NKS", [1, 2])
@pytest.mark.parametrize("ntiles", [1, 2, 3])
def test_stage_protocol(direct, S, NKS, ntiles):
    for nK in range(0, 13):
        check(kernel_trace(S, NKS, nK, direct, ntiles), S, NKS)


def test_checker_catches_a_missing_reuse_barrier():
    """Sensitivity: drop the barrier before the producer's issue (the reuse
    edge of the practice exercise on the second page) and the model fails."""
    tr = kernel_trace(2, 1, 6, True)
    ev = tr.ev
    # remove the second barrier B_1 (ready of tile 1 and reuse of stage 0)
    idx = [i for i, e in enumerate(ev) if e[0] == "barrier"][1]
    del ev[idx]
    with pytest.raises(AssertionError):
        check(tr, 2, 1)


def test_checker_catches_a_short_wait():
    """Sensitivity: waiting for one group fewer than needed breaks the ready edge."""
    tr = kernel_trace(3, 1, 8, True)
    tr.ev = [("wait", e[1] + 1) if e[0] == "wait" and e[1] > 0 else e for e in tr.ev]
    with pytest.raises(AssertionError):
        check(tr, 3, 1)


def test_checker_catches_a_forgotten_epilogue_tile():
    """Sensitivity: skipping the last tile's MFMAs (page "GPU-Kernel
    pipelinen", common pitfalls) is caught by the order check."""
    tr = kernel_trace(2, 2, 5, True)
    tr.ev = [e for e in tr.ev if not (e[0] == "mfma" and e[1] == 4)]
    with pytest.raises(AssertionError):
        check(tr, 2, 2)


def test_checker_catches_a_store_before_the_last_k_tile():
    """Sensitivity: storing an output tile one slot early (the last K tile
    not yet multiplied) is caught."""
    tr = kernel_trace(2, 1, 4, True, ntiles=2)
    ev = tr.ev
    st = [i for i, e in enumerate(ev) if e[0] == "store"][0]
    last_mfma = max(i for i, e in enumerate(ev) if e[0] == "mfma" and e[1] == 3)
    ev.insert(last_mfma, ev.pop(st))
    with pytest.raises(AssertionError):
        check(tr, 2, 1)


def test_checker_catches_a_ring_that_restarts_per_tile_without_a_wait():
    """Sensitivity: a streamed ring whose next tile's first slot is read
    before its load's wait (the cross-tile prologue overlap done wrong)."""
    tr = kernel_trace(3, 1, 2, True, ntiles=2)
    tr.ev = [("wait", e[1] + 1) if e[0] == "wait" and e[1] > 0 else e for e in tr.ev]
    with pytest.raises(AssertionError):
        check(tr, 3, 1)
