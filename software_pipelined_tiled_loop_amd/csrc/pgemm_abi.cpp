// pgemm_abi.cpp -- the C ABI: argument validation, the planner and the launch.
//
// The planner picks (tile, stages, producer) for a problem:
//   * producer: DIRECT whenever both operands meet the 16-byte vector rules;
//     otherwise the register-staged variants the alignment admits (GENERIC,
//     and STAGED_A / STAGED_B when B / A alone keeps the rules), chosen with
//     tile and depth by their measured efficiencies (REGISTER only on
//     request);
//   * tile: the compiled tile class with the smallest estimated time of the
//     busiest CU (its tiles in rounds of co-resident workgroups, a partial
//     last round at its measured cost, a prologue per round), each class
//     estimated at the ring depth it would run with; for fp16, bf16 and
//     int8 near-equal estimates go to the larger tile (tie_margin);
//   * stages (DIRECT): the smallest ring depth whose lookahead covers the load latency,
//     using the uncovered-latency estimate max(0, L - (S-1)*C) of page
//     "Software pipelines and asynchronous copies" (section "Worked example:
//     Choosing between two and four stages"), with C the MFMA time of one K
//     tile on a SIMD shared by the workgroups actually resident on the CU.
//     The depth is clipped to the number of K tiles (section "Prologue,
//     steady state, and epilogue": fewer K tiles than stages).
//   * register-staged producers take tile and depth together from measured
//     per-variant efficiencies (register pressure decides their depth).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "../../include/pgemm.h"
#include "variants.hpp"

using namespace pgemm;

namespace {

constexpr int kNumCU = 256;
constexpr int kLdsPerCU = 163840;
// Effective global->LDS latency the ring has to cover, in SIMD clocks.  Set
// from measurement on MI355X at 4096^3: one K tile of a 256 x 256 tile
// (>= 1024 MFMA cycles) covers it, and deeper rings measured slower there
// (more loads in flight, same L2 bandwidth), so the model asks for S = 2.
constexpr double kLoadLatencyCycles = 1000.0;
// Exposed start of a round of workgroups (launch, first K tile in flight), in
// SIMD clocks; the choice of tile is insensitive to it between 1000 and 4000.
constexpr double kPrologueCycles = 2000.0;
// Estimates within this factor of the best count as equal, and the larger
// tile wins: it pulls fewer bytes from L2 per flop, and when it leaves CUs
// idle the busy ones run at a higher clock (bf16 6144^3: 256 x 256 measured
// 11 % faster than 128 x 128, whose estimate was 1 % lower).  That holds for
// the dtypes whose clock falls with data movement (fp16, bf16, int8).  fp32
// keeps its clock, and there the small tile's co-resident workgroups hide
// each other's epilogues: 128 x 64 x 16 measured faster than 256 x 256 x 32
// on every fp32 shape timed (4096^3 +0.9 %, 8192^2 x 1024 +7.3 %, 4096^2 x
// 512 +7.0 %), so fp32 takes the cheapest estimate as it is.
double tie_margin(int dtype) { return dtype == PGEMM_F32 ? 1.0 : 1.10; }

struct Table {
    const VariantDesc* v;
    int n;
};

Table table_for(int dtype) {
    Table t{nullptr, 0};
    switch (dtype) {
        case PGEMM_F32: t.v = variants_f32(&t.n); break;
        case PGEMM_F16: t.v = variants_f16(&t.n); break;
        case PGEMM_BF16: t.v = variants_bf16(&t.n); break;
        case PGEMM_I8: t.v = variants_i8(&t.n); break;
        default: break;
    }
    return t;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int elem_bytes(int dtype) { return dtype == PGEMM_F32 ? 4 : dtype == PGEMM_I8 ? 1 : 2; }

// Dense MFMA rate per SIMD per clock for the dtype (MI355X: 256 CUs x 4 SIMDs at 2.4 GHz).
double flops_per_simd_clk(int dtype) {
    switch (dtype) {
        case PGEMM_F32: return 64.0;
        case PGEMM_I8: return 2048.0;
        default: return 1024.0;
    }
}

// Register estimate of a variant (accumulators + two fragment sets + staging
// + addressing) -> waves per SIMD.  Used only to estimate residency.
int est_vgprs(const VariantDesc& d) {
    const int nw = d.wgm * d.wgn;
    const int wm = d.bm / d.wgm, wn = d.bn / d.wgn;
    const int fm = wm / 16, fn = wn / 16;
    const int es = elem_bytes(d.dtype);
    const int acc = fm * fn * 4;
    const int frags = 2 * (fm + fn) * 4;
    const int staging = d.producer == PROD_DIRECT ? 0 : (d.bm * d.bk + d.bk * d.bn) * es / (64 * nw) / 4;
    return acc + frags + staging + 40;
}

int wg_per_cu(const VariantDesc& d) {
    const int nw = d.wgm * d.wgn;
    int v = est_vgprs(d);
    v = (v + 7) / 8 * 8;
    int waves_per_simd = 512 / (v < 512 ? v : 512);
    if (waves_per_simd > 8) waves_per_simd = 8;
    int by_regs = waves_per_simd * 4 / nw;
    int by_lds = kLdsPerCU / d.lds_bytes;
    int r = by_regs < by_lds ? by_regs : by_lds;
    return r < 1 ? 1 : r;
}

// MFMA cycles of one K tile on one SIMD, with `share` workgroups per CU.
double tile_compute_cycles(const VariantDesc& d, int share) {
    const double flops = 2.0 * d.bm * d.bn * d.bk;
    return flops / (4.0 * flops_per_simd_clk(d.dtype)) * share;
}

// Measured behaviour of a tile class on MI355X (seeded inputs), the re-run
// tile search that follows any change to the pipelined kernel:
//   eff  fraction of dense peak at 4096^3 with the class's best ring depth;
//   lam  cost of a partial last round: r < occ co-resident workgroups take
//        r + lam*(occ - r) workgroup-times.  0 would be perfect sharing; 1
//        would make a lone workgroup take as long as a full round.
//        Measured: bf16 128 x 128 0.37 (a workgroup alone on a CU finishes
//        in 0.68 of the time two co-resident ones take), fp32 128 x 64 x 16
//        0.11.
// Classes not listed fall back to an operand-traffic estimate.
struct ClassModel {
    double eff, lam;
};

ClassModel class_model(const VariantDesc& d) {
    struct E { int dt, bm, bn, bk; double e, lam; };
    static const E table[] = {
        {PGEMM_BF16, 256, 256, 64, 0.541, 0.0}, {PGEMM_BF16, 256, 256, 32, 0.510, 0.0},
        {PGEMM_BF16, 128, 128, 64, 0.392, 0.37}, {PGEMM_F16, 256, 256, 64, 0.516, 0.0},
        {PGEMM_F16, 256, 256, 32, 0.477, 0.0},  {PGEMM_F16, 128, 128, 64, 0.375, 0.37},
        {PGEMM_I8, 256, 256, 128, 0.473, 0.0},  {PGEMM_I8, 256, 256, 64, 0.447, 0.0},
        {PGEMM_I8, 128, 128, 128, 0.351, 0.37}, {PGEMM_F32, 256, 256, 32, 0.948, 0.0},
        {PGEMM_F32, 128, 64, 16, 0.956, 0.11},  {PGEMM_F32, 128, 128, 32, 0.867, 0.3},
    };
    for (const E& x : table)
        if (x.dt == d.dtype && x.bm == d.bm && x.bn == d.bn && x.bk == d.bk) return {x.e, x.lam};
    const double per = (double)(d.bm + d.bn) / (2.0 * d.bm * d.bn);
    const double ref = 512.0 / (2.0 * 256 * 256);
    const double e = ref / per;
    return {0.4 * (e > 1.0 ? 1.0 : std::pow(e, 0.5)), 0.3};
}

double tile_efficiency(const VariantDesc& d) { return class_model(d).eff; }

// Output tiles on the busiest CU: the dispatcher spreads workgroups over all
// CUs before it stacks them.
int64_t tiles_per_cu(const VariantDesc& d, int64_t M, int64_t N) {
    return ceil_div(ceil_div(M, d.bm) * ceil_div(N, d.bn), kNumCU);
}

// Estimated SIMD clocks of the busiest CU for variant d at efficiency eff:
// its tiles run in rounds of up to wg_per_cu co-resident workgroups, a
// partial last round costs as the class model says, and every round pays the
// prologue once.
double est_cycles(const VariantDesc& d, int64_t M, int64_t N, int64_t K, double eff) {
    const int64_t occ = wg_per_cu(d);
    const int64_t n = tiles_per_cu(d, M, N);
    const int64_t full = n / occ, r = n % occ;
    const double units = (double)(full * occ) + (r ? (double)r + class_model(d).lam * (double)(occ - r) : 0.0);
    const double kp = (double)(ceil_div(K, d.bk) * d.bk);
    const double per_tile = 2.0 * d.bm * d.bn * kp / (eff * 4.0 * flops_per_simd_clk(d.dtype));
    return units * per_tile + (double)ceil_div(n, occ) * kPrologueCycles;
}

// MFMA cycles of one K tile on one SIMD with the workgroups that actually
// share the CU: at most wg_per_cu, and no more than the CU has tiles.
double shared_tile_cycles(const VariantDesc& d, int64_t M, int64_t N) {
    const int64_t n = tiles_per_cu(d, M, N);
    const int occ = wg_per_cu(d);
    return tile_compute_cycles(d, (int)(n < occ ? (n < 1 ? 1 : n) : occ));
}

// Register-staged producers (REGISTER, GENERIC): measured efficiency of each
// (tile class, ring depth) pair, MI355X, seeded inputs (GENERIC on the ragged
// 4000 x 3968 x 4001 problem with lda = 4001; REGISTER at 4096^3).  For these
// producers the best depth depends on register pressure as much as on
// latency (staging registers next to the doubled fragment set, at the 256
// registers a wave of a two-waves-per-SIMD workgroup may hold), so the
// planner picks the (tile, depth) pair directly from this table.
double staged_efficiency(const VariantDesc& d) {
    struct E { int dt, bm, bn, bk, s, p; double e; };
    static const E table[] = {
        {PGEMM_BF16, 256, 256, 32, 1, PROD_GENERIC, 0.343}, {PGEMM_BF16, 256, 256, 32, 2, PROD_GENERIC, 0.376},
        {PGEMM_BF16, 128, 128, 64, 1, PROD_GENERIC, 0.280}, {PGEMM_BF16, 128, 128, 64, 2, PROD_GENERIC, 0.265},
        {PGEMM_BF16, 128, 128, 64, 3, PROD_GENERIC, 0.166}, {PGEMM_BF16, 128, 128, 64, 4, PROD_GENERIC, 0.171},
        {PGEMM_F16, 256, 256, 32, 1, PROD_GENERIC, 0.336},  {PGEMM_F16, 256, 256, 32, 2, PROD_GENERIC, 0.369},
        {PGEMM_F16, 128, 128, 64, 1, PROD_GENERIC, 0.271},  {PGEMM_F16, 128, 128, 64, 2, PROD_GENERIC, 0.258},
        {PGEMM_F16, 128, 128, 64, 3, PROD_GENERIC, 0.166},  {PGEMM_F16, 128, 128, 64, 4, PROD_GENERIC, 0.171},
        {PGEMM_I8, 256, 256, 64, 1, PROD_GENERIC, 0.285},   {PGEMM_I8, 256, 256, 64, 2, PROD_GENERIC, 0.324},
        {PGEMM_I8, 128, 128, 128, 1, PROD_GENERIC, 0.153},  {PGEMM_I8, 128, 128, 128, 2, PROD_GENERIC, 0.219},
        {PGEMM_I8, 128, 128, 128, 3, PROD_GENERIC, 0.142},  {PGEMM_I8, 128, 128, 128, 4, PROD_GENERIC, 0.140},
        {PGEMM_F32, 256, 256, 32, 1, PROD_GENERIC, 0.807},  {PGEMM_F32, 256, 256, 32, 2, PROD_GENERIC, 0.807},
        {PGEMM_F32, 128, 64, 16, 1, PROD_GENERIC, 0.788},   {PGEMM_F32, 128, 64, 16, 2, PROD_GENERIC, 0.712},
        {PGEMM_F32, 128, 128, 32, 1, PROD_GENERIC, 0.788},  {PGEMM_F32, 128, 128, 32, 2, PROD_GENERIC, 0.699},
        {PGEMM_F32, 128, 128, 32, 3, PROD_GENERIC, 0.572},  {PGEMM_F32, 128, 128, 32, 4, PROD_GENERIC, 0.566},
        {PGEMM_BF16, 256, 256, 32, 1, PROD_REGISTER, 0.400}, {PGEMM_BF16, 256, 256, 32, 2, PROD_REGISTER, 0.414},
        {PGEMM_BF16, 256, 256, 32, 3, PROD_REGISTER, 0.409}, {PGEMM_BF16, 256, 256, 32, 4, PROD_REGISTER, 0.410},
        {PGEMM_BF16, 128, 128, 64, 2, PROD_REGISTER, 0.300},
        {PGEMM_F16, 256, 256, 32, 1, PROD_REGISTER, 0.385},  {PGEMM_F16, 256, 256, 32, 2, PROD_REGISTER, 0.400},
        {PGEMM_F16, 256, 256, 32, 3, PROD_REGISTER, 0.396},  {PGEMM_F16, 256, 256, 32, 4, PROD_REGISTER, 0.395},
        {PGEMM_F16, 128, 128, 64, 2, PROD_REGISTER, 0.293},
        {PGEMM_I8, 256, 256, 64, 1, PROD_REGISTER, 0.326},   {PGEMM_I8, 256, 256, 64, 2, PROD_REGISTER, 0.341},
        {PGEMM_I8, 256, 256, 64, 3, PROD_REGISTER, 0.338},   {PGEMM_I8, 256, 256, 64, 4, PROD_REGISTER, 0.346},
        {PGEMM_F32, 128, 64, 16, 1, PROD_REGISTER, 0.858},   {PGEMM_F32, 128, 64, 16, 2, PROD_REGISTER, 0.787},
        {PGEMM_BF16, 256, 256, 32, 2, PROD_STAGED_A, 0.470}, {PGEMM_BF16, 256, 256, 32, 2, PROD_STAGED_B, 0.470},
        {PGEMM_F16, 256, 256, 32, 2, PROD_STAGED_A, 0.450},  {PGEMM_F16, 256, 256, 32, 2, PROD_STAGED_B, 0.450},
        {PGEMM_I8, 256, 256, 64, 2, PROD_STAGED_A, 0.420},   {PGEMM_I8, 256, 256, 64, 2, PROD_STAGED_B, 0.420},
        {PGEMM_F32, 128, 64, 16, 2, PROD_STAGED_A, 0.900},   {PGEMM_F32, 128, 64, 16, 2, PROD_STAGED_B, 0.900},
        {PGEMM_F32, 256, 256, 32, 2, PROD_STAGED_A, 0.900},  {PGEMM_F32, 256, 256, 32, 2, PROD_STAGED_B, 0.900},
    };
    for (const E& x : table)
        if (x.dt == d.dtype && x.bm == d.bm && x.bn == d.bn && x.bk == d.bk && x.s == d.stages && x.p == d.producer)
            return x.e;
    return 0.5 * tile_efficiency(d);
}


// Workgroups to launch: one per output tile (default), or, on request
// (pgemm_opts.workgroups), fewer persistent ones that loop over the tiles
// with one K-tile ring across tile boundaries.  Always a multiple of 8 (the
// kernel splits the tiles into one contiguous range per XCD); surplus
// workgroups find no tile and exit.
//
// Persistence is not the default.  Measured on MI355X (bf16): 2-7 % faster
// on 128 x 128 tiles at 4096^2 with K <= 1024 and 4 % at 8192^2 x 1024, but
// 9 % slower at 8192^2 x 4096.  The C stores count in the same vmcnt as the
// ring's loads, so a persistent workgroup's next ready barrier also waits for
// its own stores; with one workgroup per tile a retiring workgroup's stores
// drain while a fresh one (with its own counters) starts on the CU.  A
// persistent grid must also match residency exactly: the dispatcher packs
// workgroups onto CUs, so a smaller grid leaves CUs idle.
int launch_grid(int64_t M, int64_t N, const VariantDesc& d, const pgemm_opts* opts) {
    const int64_t tiles = ceil_div(M, d.bm) * ceil_div(N, d.bn);
    int64_t grid = ceil_div(tiles, 8) * 8;
    if (opts && opts->workgroups > 0) {
        const int64_t want = ceil_div(opts->workgroups, 8) * 8;
        if (want < grid) grid = want;
    }
    return grid < 8 ? 8 : (int)grid;
}

bool producer_matches(const VariantDesc& d, int want) { return d.producer == want; }

// Whether a producer can run on operands of the given pgemm_aligned class:
// LDS-DMA and the REGISTER producer's unchecked 16-byte loads need the
// 16-byte rules for every operand they move.
bool admissible(int producer, int aligned) {
    const bool a = aligned == PGEMM_ALIGNED_BOTH || aligned == PGEMM_ALIGNED_A;
    const bool b = aligned == PGEMM_ALIGNED_BOTH || aligned == PGEMM_ALIGNED_B;
    switch (producer) {
        case PROD_DIRECT:
        case PROD_REGISTER: return a && b;
        case PROD_STAGED_A: return b;
        case PROD_STAGED_B: return a;
        case PROD_GENERIC: return true;
        default: return false;
    }
}

struct Choice {
    int index = -1;
    int stages_req = 0;
    double uncovered = 0.0;
};

int plan_impl(int64_t M, int64_t N, int64_t K, int dtype, int stages, int aligned, const pgemm_opts* opts,
              Choice& out) {
    Table t = table_for(dtype);
    if (!t.v) return PGEMM_ERR_UNSUPPORTED_DTYPE;
    if (stages < 0 || stages > 4) return PGEMM_ERR_BAD_STAGES;
    if (aligned < PGEMM_ALIGNED_NONE || aligned > PGEMM_ALIGNED_B) return PGEMM_ERR_INVALID_ARG;
    // 0: the planner chooses among the producers the alignment admits
    int want_prod = aligned == PGEMM_ALIGNED_BOTH ? PROD_DIRECT : 0;
    if (opts && opts->producer != PGEMM_PRODUCER_AUTO) {
        if (opts->producer < PGEMM_PRODUCER_DIRECT || opts->producer > PGEMM_PRODUCER_STAGED_B)
            return PGEMM_ERR_INVALID_ARG;
        if (!admissible(opts->producer, aligned)) return PGEMM_ERR_INFEASIBLE_PLAN;
        want_prod = opts->producer;
    }
    const bool force_tile = opts && (opts->tile_m || opts->tile_n || opts->tile_k);
    if (opts && (opts->skew < 0 || opts->skew > 64 || opts->workgroups < 0 || opts->waves < 0 ||
                 opts->reserved[0] != 0))
        return PGEMM_ERR_INVALID_ARG;
    const int force_waves = opts ? opts->waves : 0;

    // Register-staged producers: the (producer, tile, depth) with the best
    // estimated time at its measured efficiency, among the forced producer or
    // every one the alignment admits; an explicit depth restricts the choice
    // to variants of that depth.
    if (want_prod != PROD_DIRECT) {
        double best_time = 0.0;
        int best = -1;
        for (int i = 0; i < t.n; ++i) {
            const VariantDesc& d = t.v[i];
            if (want_prod ? !producer_matches(d, want_prod)
                          : (d.producer == PROD_DIRECT || d.producer == PROD_REGISTER || !admissible(d.producer, aligned)))
                continue;
            if (force_tile && (d.bm != opts->tile_m || d.bn != opts->tile_n || d.bk != opts->tile_k)) continue;
            if (force_waves && d.wgm * d.wgn != force_waves) continue;
            if (stages != 0 && d.stages != stages) continue;
            const double time = est_cycles(d, M, N, K, staged_efficiency(d));
            if (best < 0 || time < best_time * 0.999) {
                best = i;
                best_time = time;
            }
        }
        if (best < 0) return PGEMM_ERR_INFEASIBLE_PLAN;
        const VariantDesc& d = t.v[best];
        out.index = best;
        out.stages_req = d.stages;
        out.uncovered = pgemm_model_uncovered_cycles(kLoadLatencyCycles, shared_tile_cycles(d, M, N), d.stages);
        return PGEMM_OK;
    }

    // DIRECT: every tile class is estimated at the ring depth it would run
    // with, and the cheapest wins (for fp16/bf16/int8 the larger tile among
    // near-equal ones).
    auto same_class = [](const VariantDesc& a, const VariantDesc& b) {
        return a.bm == b.bm && a.bn == b.bn && a.bk == b.bk && a.wgm == b.wgm && a.wgn == b.wgn;
    };
    // The variant of class `c` with ring depth S, or the deepest one below it
    // (an explicit depth is never downgraded); -1 when there is none.
    auto variant_at = [&](const VariantDesc& c, int S, bool exact) {
        for (int s = S; s >= 1; --s) {
            for (int i = 0; i < t.n; ++i)
                if (same_class(t.v[i], c) && producer_matches(t.v[i], want_prod) && t.v[i].stages == s) return i;
            if (exact) break;
        }
        return -1;
    };
    // Ring depth: the smallest S in 2..4 whose lookahead covers the load
    // latency, max(0, L - (S-1)*C) = 0, with C the MFMA time of one K tile on a
    // SIMD shared by the workgroups that really share the CU; clipped to the
    // number of K tiles.
    auto depth_for = [&](const VariantDesc& c) {
        if (stages != 0) return variant_at(c, stages, true);
        int S = 4;
        for (int s = 2; s <= 4; ++s) {
            const int i = variant_at(c, s, true);
            if (i >= 0 && pgemm_model_uncovered_cycles(kLoadLatencyCycles, shared_tile_cycles(t.v[i], M, N), s) <= 0.0) {
                S = s;
                break;
            }
        }
        const int nK = (int)ceil_div(K, c.bk);
        if (S > nK) S = nK < 1 ? 1 : nK;
        return variant_at(c, S, false);
    };
    struct Cand {
        int index;
        double time;
    };
    Cand cands[64];
    int nc = 0;
    for (int i = 0; i < t.n && nc < 64; ++i) {
        const VariantDesc& d = t.v[i];
        if (!producer_matches(d, want_prod)) continue;
        if (force_tile && (d.bm != opts->tile_m || d.bn != opts->tile_n || d.bk != opts->tile_k)) continue;
        if (force_waves && d.wgm * d.wgn != force_waves) continue;
        bool seen = false;  // one candidate per tile class
        for (int j = 0; j < nc; ++j) seen = seen || same_class(t.v[cands[j].index], d);
        if (seen) continue;
        const int pick = depth_for(d);
        if (pick < 0) continue;
        cands[nc++] = {pick, est_cycles(t.v[pick], M, N, K, tile_efficiency(t.v[pick]))};
    }
    if (nc == 0) return PGEMM_ERR_INFEASIBLE_PLAN;
    double best_time = cands[0].time;
    for (int j = 1; j < nc; ++j) best_time = cands[j].time < best_time ? cands[j].time : best_time;
    int pick = -1;
    for (int j = 0; j < nc; ++j) {
        if (cands[j].time > best_time * tie_margin(dtype)) continue;
        const VariantDesc& d = t.v[cands[j].index];
        if (pick < 0) {
            pick = cands[j].index;
            continue;
        }
        const VariantDesc& p = t.v[pick];
        const int64_t area = (int64_t)d.bm * d.bn, parea = (int64_t)p.bm * p.bn;
        if (area > parea || (area == parea && cands[j].time < est_cycles(p, M, N, K, tile_efficiency(p))))
            pick = cands[j].index;
    }
    out.index = pick;
    out.stages_req = t.v[pick].stages;
    out.uncovered = pgemm_model_uncovered_cycles(kLoadLatencyCycles, shared_tile_cycles(t.v[pick], M, N),
                                                 t.v[pick].stages);
    return PGEMM_OK;
}

void fill_info(int dtype, const VariantDesc& d, int idx, int64_t M, int64_t N, int64_t K, double uncovered,
               const pgemm_opts* opts, pgemm_plan_info* info) {
    std::memset(info, 0, sizeof(*info));
    info->tile_m = d.bm;
    info->tile_n = d.bn;
    info->tile_k = d.bk;
    info->stages = d.stages;
    info->num_k_tiles = (int)ceil_div(K, d.bk);
    const int nk1 = info->num_k_tiles < 1 ? 1 : info->num_k_tiles;
    info->stages_eff = d.stages < nk1 ? d.stages : nk1;
    info->producer = d.producer;
    info->threads = d.threads;
    info->waves_m = d.wgm;
    info->waves_n = d.wgn;
    info->lds_bytes = d.lds_bytes;
    info->wg_per_cu = wg_per_cu(d);
    info->grid = launch_grid(M, N, d, opts);
    int base = 0;  // global index: variants of lower dtypes come first
    for (int t = 0; t < dtype; ++t) base += table_for(t).n;
    info->variant = base + idx;
    info->est_uncovered_cycles = uncovered;
}

bool is_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

double pgemm_model_uncovered_cycles(double latency, double compute_per_tile, int stages) {
    if (stages <= 1) return latency;
    const double u = latency - (stages - 1) * compute_per_tile;
    return u > 0.0 ? u : 0.0;
}

int64_t pgemm_model_lds_bytes(int bm, int bn, int bk, int stages, int elem_bytes, int a_pad_elems_per_k) {
    // stages * (A tile + B tile) elements, plus any padding of the A rows
    return (int64_t)stages * ((int64_t)bm * bk + (int64_t)bk * bn + (int64_t)bk * a_pad_elems_per_k) * elem_bytes;
}

double pgemm_model_global_loads_per_output(int bm, int bn, int64_t K) {
    // A workgroup loads BM*K elements of A and K*BN of B for BM*BN outputs:
    // K/BN + K/BM global loads per output element.
    return (double)K / bn + (double)K / bm;
}

double pgemm_model_compute_load_ratio(int bm, int bn, int bk, int elem_bytes) {
    if (bm <= 0 || bn <= 0 || bk <= 0 || elem_bytes <= 0) return 0.0;
    // two flops per multiply-add of the K tile, over the A and B bytes it loads
    const double flops = 2.0 * bm * bn * bk;
    const double bytes = ((double)bm * bk + (double)bk * bn) * elem_bytes;
    return flops / bytes;
}

const char* pgemm_strerror(int status) {
    switch (status) {
        case PGEMM_OK: return "ok";
        case PGEMM_ERR_INVALID_ARG: return "invalid argument (size, leading dimension or null pointer)";
        case PGEMM_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
        case PGEMM_ERR_BAD_STAGES: return "stages must be 0 (auto) or 1..4";
        case PGEMM_ERR_INFEASIBLE_PLAN: return "no compiled variant satisfies the requested options";
        case PGEMM_ERR_NONINTEGRAL_SCALAR: return "int8 GEMM needs integer alpha and beta in int32 range";
        case PGEMM_ERR_HIP: return "HIP runtime error at launch";
        case PGEMM_ERR_TOO_LARGE: return "problem exceeds 32-bit tile addressing";
        default: return "unknown status";
    }
}

int pgemm_version(void) { return 10000; }

int pgemm_num_variants(void) {
    int n = 0;
    for (int d = 0; d < 4; ++d) n += table_for(d).n;
    return n;
}

int pgemm_variant_info(int index, pgemm_plan_info* out, int* dtype) {
    if (!out || index < 0) return PGEMM_ERR_INVALID_ARG;
    for (int d = 0; d < 4; ++d) {
        Table t = table_for(d);
        if (index < t.n) {
            fill_info(d, t.v[index], index, t.v[index].bm, t.v[index].bn, t.v[index].bk, 0.0, nullptr, out);
            if (dtype) *dtype = d;
            return PGEMM_OK;
        }
        index -= t.n;
    }
    return PGEMM_ERR_INVALID_ARG;
}

int pgemm_plan(int64_t M, int64_t N, int64_t K, int dtype, int stages, int aligned, const pgemm_opts* opts,
               pgemm_plan_info* out) {
    if (!out) return PGEMM_ERR_INVALID_ARG;
    if (dtype < 0 || dtype > 3) return PGEMM_ERR_UNSUPPORTED_DTYPE;
    if (M < 0 || N < 0 || K < 0) return PGEMM_ERR_INVALID_ARG;
    Choice c;
    int r = plan_impl(M, N, K, dtype, stages, aligned, opts, c);
    if (r != PGEMM_OK) return r;
    Table t = table_for(dtype);
    fill_info(dtype, t.v[c.index], c.index, M, N, K, c.uncovered, opts, out);
    return PGEMM_OK;
}

int pgemm_gemm_ex(int64_t M, int64_t N, int64_t K, double alpha, const void* A, int64_t lda, const void* B,
                  int64_t ldb, double beta, void* C, int64_t ldc, int dtype, int stages, const pgemm_opts* opts,
                  void* stream) {
    // ---- argument checks: all before anything touches the GPU ----
    if (dtype < 0 || dtype > 3) return PGEMM_ERR_UNSUPPORTED_DTYPE;
    if (stages < 0 || stages > 4) return PGEMM_ERR_BAD_STAGES;
    if (M < 0 || N < 0 || K < 0) return PGEMM_ERR_INVALID_ARG;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1)) return PGEMM_ERR_INVALID_ARG;
    if (dtype == PGEMM_I8) {
        if (!(std::isfinite(alpha) && std::isfinite(beta)) || alpha != std::floor(alpha) ||
            beta != std::floor(beta) || std::fabs(alpha) > 2147483647.0 || std::fabs(beta) > 2147483647.0)
            return PGEMM_ERR_NONINTEGRAL_SCALAR;
    }
    if (M == 0 || N == 0) return PGEMM_OK;
    if (!C) return PGEMM_ERR_INVALID_ARG;
    if (K > 0 && (!A || !B)) return PGEMM_ERR_INVALID_ARG;
    const int es = elem_bytes(dtype);
    const int epc = 16 / es;
    // 32-bit tile addressing: byte offsets inside one tile must stay below 2^31,
    // and a tile origin plus one tile extent (at most 256) must fit a 32-bit int.
    if (M > 0x7fffff00 || N > 0x7fffff00 || K > 0x7fffff00) return PGEMM_ERR_TOO_LARGE;
    if ((double)lda * es * 256.0 >= 2147483648.0 || (double)ldb * es * 128.0 >= 2147483648.0 ||
        (double)ldc * 4.0 * 256.0 >= 2147483648.0)
        return PGEMM_ERR_TOO_LARGE;
    if (ceil_div(M, 128) * ceil_div(N, 64) > 0x7ffffff0) return PGEMM_ERR_TOO_LARGE;
    // Element alignment is required; 16-byte alignment selects the vector producers.
    if (((uintptr_t)A % es) || ((uintptr_t)B % es) || ((uintptr_t)C % 4)) return PGEMM_ERR_INVALID_ARG;
    // The 16-byte rules per operand: a chunk of 16 bytes never straddles the
    // end of A's K columns (A) or of B's N columns (B), and every row starts
    // 16-byte aligned.
    const bool a_ok = K == 0 || (is_aligned16(A) && (lda * es) % 16 == 0 && K % epc == 0);
    const bool b_ok = K == 0 || (is_aligned16(B) && (ldb * es) % 16 == 0 && N % epc == 0);
    const int aligned = a_ok && b_ok ? PGEMM_ALIGNED_BOTH
                        : a_ok       ? PGEMM_ALIGNED_A
                        : b_ok       ? PGEMM_ALIGNED_B
                                     : PGEMM_ALIGNED_NONE;

    Choice c;
    int r = plan_impl(M, N, K, dtype, stages, aligned, opts, c);
    if (r != PGEMM_OK) return r;
    const VariantDesc& d = table_for(dtype).v[c.index];

    KernelArgs a;
    std::memset(&a, 0, sizeof(a));
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.tiles_m = (int)ceil_div(M, d.bm);
    a.tiles_n = (int)ceil_div(N, d.bn);
    a.group_m = 4;
    a.alpha = (float)alpha;
    a.beta = (float)beta;
    a.ialpha = dtype == PGEMM_I8 ? (int)(int64_t)alpha : 0;
    a.ibeta = dtype == PGEMM_I8 ? (int)(int64_t)beta : 0;
    a.beta_nonzero = beta != 0.0;
    a.dbg_sleep = opts ? opts->skew : 0;
    const int grid = launch_grid(M, N, d, opts);
    const bool persistent = grid < ceil_div((int64_t)a.tiles_m * a.tiles_n, 8) * 8;
    hipError_t e = (persistent ? d.launch_persistent : d.launch)(a, grid, (hipStream_t)stream);
    if (e != hipSuccess) {
        // The status code alone cannot say which runtime error it was.
        std::fprintf(stderr, "pgemm: launch of %s %dx%dx%d S=%d (grid %d) failed: %s (%d)\n",
                     dtype == PGEMM_F32 ? "f32" : dtype == PGEMM_F16 ? "f16" : dtype == PGEMM_BF16 ? "bf16" : "i8",
                     d.bm, d.bn, d.bk, d.stages, grid, hipGetErrorString(e), (int)e);
        return PGEMM_ERR_HIP;
    }
    return PGEMM_OK;
}

int pgemm_gemm(int64_t M, int64_t N, int64_t K, double alpha, const void* A, int64_t lda, const void* B, int64_t ldb,
               double beta, void* C, int64_t ldc, int dtype, int stages, void* stream) {
    return pgemm_gemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, dtype, stages, nullptr, stream);
}

}  // extern "C"
