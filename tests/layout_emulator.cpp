// Host emulation of the kernel's data path (no GPU): producer placement into
// the LDS stage, fragment reads (ds_read_b128, the transposing ds_read_b64_tr
// reads, ds_read_b32) and the MFMA lane layouts, using the kernel's own index
// functions from pgemm_kernel.hpp.  For every tile class it checks that
//   * the producer writes every byte of the stage exactly once,
//   * every fragment read stays inside its region,
//   * the emulated MFMA results equal a naive GEMM of the tile.
// Lane semantics of the gfx950 instructions were probed in-bounds on the GPU:
//   ds_read_b64_tr_b16: lane i (of a 16-lane block) element e <- element i%4
//                       of the piece addressed by lane 4e + i/4
//   ds_read_b64_tr_b8:  lane i byte e <- byte i%8 of lane 2e + i/8
//   MFMA 16x16xK: A lane l holds row l%16, B lane l column l%16, K in lane
//   groups l/16; D lane l holds rows 4*(l/16)+r, column l%16.
// Prints "OK <n>" on success; exits non-zero on the first mismatch.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <vector>

#include "../software_pipelined_tiled_loop_amd/csrc/hazard_demo.hpp"
#include "../software_pipelined_tiled_loop_amd/csrc/pgemm_kernel.hpp"

using namespace pgemm;

static uint32_t rng_state = 12345;
static int small_int() {
    rng_state = rng_state * 1664525u + 1013904223u;
    return (int)((rng_state >> 24) % 7) - 3;
}

template <int D>
static void encode(int v, uint8_t* dst) {
    if constexpr (D == DT_F32) {
        float f = (float)v;
        memcpy(dst, &f, 4);
    } else if constexpr (D == DT_BF16) {
        float f = (float)v;
        uint32_t u;
        memcpy(&u, &f, 4);
        uint16_t h = (uint16_t)(u >> 16);
        memcpy(dst, &h, 2);
    } else if constexpr (D == DT_F16) {
        _Float16 h = (_Float16)v;
        memcpy(dst, &h, 2);
    } else {
        int8_t b = (int8_t)v;
        memcpy(dst, &b, 1);
    }
}
template <int D>
static int decode(const uint8_t* src) {
    if constexpr (D == DT_F32) {
        float f;
        memcpy(&f, src, 4);
        return (int)f;
    } else if constexpr (D == DT_BF16) {
        uint16_t h;
        memcpy(&h, src, 2);
        uint32_t u = (uint32_t)h << 16;
        float f;
        memcpy(&f, &u, 4);
        return (int)f;
    } else if constexpr (D == DT_F16) {
        _Float16 h;
        memcpy(&h, src, 2);
        return (int)(float)h;
    } else {
        return (int)(int8_t)src[0];
    }
}

#define FAIL(...)                                  \
    do {                                           \
        printf("FAIL %s: ", name);                 \
        printf(__VA_ARGS__);                       \
        printf("\n");                              \
        exit(1);                                   \
    } while (0)

template <class C>
static void emulate(const char* name) {
    constexpr int D = C::Dt, ES = C::ES, EPC = C::EPC;
    std::vector<int> A(C::BM * C::BK), B(C::BK * C::BN);
    for (int& v : A) v = small_int();
    for (int& v : B) v = small_int();
    std::vector<uint8_t> lds(C::STAGE_BYTES, 0);
    std::vector<int> hits(C::STAGE_BYTES / 16, 0);
    // producer placement
    for (int w = 0; w < C::NW; ++w)
        for (int l = 0; l < 64; ++l) {
            for (int q = 0; q < C::A_INSTR; ++q) {
                int row, kel;
                a_chunk<C>(w, l, q, row, kel);
                const int off = (w * C::A_INSTR + q) * 1024 + l * 16;
                if (row < 0 || row >= C::BM || kel < 0 || kel + EPC > C::BK) FAIL("A chunk out of tile");
                for (int e = 0; e < EPC; ++e) encode<D>(A[row * C::BK + kel + e], &lds[off + e * ES]);
                hits[off / 16]++;
            }
            for (int q = 0; q < C::B_INSTR; ++q) {
                int krow, nel;
                b_chunk<C>(w, l, q, krow, nel);
                const int off = C::A_BYTES + (w * C::B_INSTR + q) * 1024 + l * 16;
                if (krow < 0 || krow >= C::BK || nel < 0 || nel + EPC > C::BN) FAIL("B chunk out of tile");
                for (int e = 0; e < EPC; ++e) encode<D>(B[krow * C::BN + nel + e], &lds[off + e * ES]);
                hits[off / 16]++;
            }
        }
    for (size_t i = 0; i < hits.size(); ++i)
        if (hits[i] != 1) FAIL("LDS chunk %zu written %d times", i, hits[i]);
    // consumer
    std::vector<long> out(C::BM * C::BN, 0);
    for (int w = 0; w < C::NW; ++w) {
        const int wm0 = (w / C::WGN) * C::WM, wn0 = (w % C::WGN) * C::WN;
        for (int ks = 0; ks < C::BK / C::KSTEP; ++ks)
            for (int i = 0; i < C::FM; ++i)
                for (int j = 0; j < C::FN; ++j) {
                    // A fragment: EPC elements per lane
                    int af[64][16], bf[64][16];
                    for (int l = 0; l < 64; ++l) {
                        const int off = a_frag_off<C>(ks, i, wm0, l);
                        if (off < 0 || off + 16 > C::A_BYTES) FAIL("A read out of region");
                        for (int e = 0; e < EPC; ++e) af[l][e] = decode<D>(&lds[off + e * ES]);
                    }
                    if constexpr (D == DT_F16 || D == DT_BF16) {
                        for (int h = 0; h < 2; ++h) {
                            int R[64][4];
                            for (int l = 0; l < 64; ++l) {
                                const int off = b_frag_off<C>(ks, j, wn0, l, h);
                                if (off < 0 || off + 8 > C::B_BYTES) FAIL("B read out of region");
                                for (int e = 0; e < 4; ++e) R[l][e] = decode<D>(&lds[C::A_BYTES + off + e * 2]);
                            }
                            for (int l = 0; l < 64; ++l)
                                for (int e = 0; e < 4; ++e) {
                                    const int i16 = l & 15, blk = l & ~15;
                                    bf[l][4 * h + e] = R[blk + 4 * e + i16 / 4][i16 % 4];
                                }
                        }
                    } else if constexpr (D == DT_I8) {
                        for (int h = 0; h < 2; ++h) {
                            int R[64][8];
                            for (int l = 0; l < 64; ++l) {
                                const int off = b_frag_off<C>(ks, j, wn0, l, h);
                                if (off < 0 || off + 8 > C::B_BYTES) FAIL("B read out of region");
                                for (int e = 0; e < 8; ++e) R[l][e] = decode<D>(&lds[C::A_BYTES + off + e]);
                            }
                            for (int l = 0; l < 64; ++l)
                                for (int e = 0; e < 8; ++e) {
                                    const int i16 = l & 15, blk = l & ~15;
                                    bf[l][8 * h + e] = R[blk + 2 * e + i16 / 8][i16 % 8];
                                }
                        }
                    } else {
                        for (int jm = 0; jm < 4; ++jm)
                            for (int l = 0; l < 64; ++l) {
                                const int off = b_frag_off<C>(ks, j, wn0, l, jm);
                                if (off < 0 || off + 4 > C::B_BYTES) FAIL("B read out of region");
                                bf[l][jm] = decode<D>(&lds[C::A_BYTES + off]);
                            }
                    }
                    // MFMA(s) of this block and K step
                    long dblk[16][16] = {};
                    if constexpr (D == DT_F32) {
                        for (int jm = 0; jm < 4; ++jm)
                            for (int r = 0; r < 16; ++r)
                                for (int c = 0; c < 16; ++c)
                                    for (int g = 0; g < 4; ++g)
                                        dblk[r][c] += (long)af[r + 16 * g][jm] * bf[c + 16 * g][jm];
                    } else {
                        constexpr int KPL = (D == DT_I8) ? 16 : 8;  // K per lane group
                        for (int r = 0; r < 16; ++r)
                            for (int c = 0; c < 16; ++c)
                                for (int k = 0; k < 4 * KPL; ++k)
                                    dblk[r][c] += (long)af[r + 16 * (k / KPL)][k % KPL] * bf[c + 16 * (k / KPL)][k % KPL];
                    }
                    for (int r = 0; r < 16; ++r)
                        for (int c = 0; c < 16; ++c) out[(wm0 + 16 * i + r) * C::BN + wn0 + 16 * j + c] += dblk[r][c];
                }
    }
    for (int r = 0; r < C::BM; ++r)
        for (int c = 0; c < C::BN; ++c) {
            long ref = 0;
            for (int k = 0; k < C::BK; ++k) ref += (long)A[r * C::BK + k] * B[k * C::BN + c];
            if (out[r * C::BN + c] != ref) FAIL("C[%d][%d] = %ld, want %ld", r, c, out[r * C::BN + c], ref);
        }
}


// The generic producer reads a whole 16-byte chunk wherever chunk_fits says
// so.  Brute force over small matrices: the allocation ends at the largest
// r*ld + c over the matrix's elements; every admitted read must end there or
// before, and every chunk lying wholly inside one row must be admitted.
static int check_chunk_fits() {
    const char* name = "chunk_fits";
    int cases = 0;
    for (int epc : {4, 8, 16})
        for (int rows = 1; rows <= 5; ++rows)
            for (int cols = 1; cols <= 40; ++cols)
                for (int ld = cols; ld <= cols + 20; ++ld) {
                    long last = -1;
                    for (int r = 0; r < rows; ++r)
                        for (int c = 0; c < cols; ++c) last = std::max(last, (long)r * ld + c);
                    for (int r = 0; r < rows; ++r)
                        for (int c = 0; c < cols; ++c) {
                            const bool fits = chunk_fits(r, c, ld, rows, cols, epc);
                            const long end = (long)r * ld + c + epc - 1;
                            if (fits && end > last) FAIL("read of %d at (%d,%d) ld %d ends past the matrix", epc, r, c, ld);
                            if (!fits && c + epc <= cols) FAIL("in-row chunk at (%d,%d) rejected", r, c);
                            if (!fits && end <= last) FAIL("in-bounds chunk at (%d,%d) ld %d rejected", r, c, ld);
                            ++cases;
                        }
                }
    return cases;
}

// The generic producer's choice of whole 16-byte loads for a K tile
// (whole_loads), over the exact chunk sets of tile class C, for remaining
// extents k_left, n_left around every boundary and leading dimensions from the
// smallest up.  Whenever whole loads are chosen, every in-range chunk's read
// ends at or before the last element of its matrix, and no in-range A chunk
// reaches past K (elements past N in a B chunk feed only outputs that are
// never stored).  K tiles before the last one always take whole loads when
// ldb >= EPC.
template <class C>
static int check_whole_loads(const char* name) {
    constexpr int EPC = C::EPC, BK = C::BK, BN = C::BN;
    std::vector<std::pair<int, int>> ach, bch;
    for (int w = 0; w < C::NW; ++w)
        for (int l = 0; l < 64; ++l) {
            for (int q = 0; q < C::A_INSTR; ++q) {
                int row, kel;
                a_chunk<C>(w, l, q, row, kel);
                ach.push_back({row, kel});
            }
            for (int q = 0; q < C::B_INSTR; ++q) {
                int krow, nel;
                b_chunk<C>(w, l, q, krow, nel);
                bch.push_back({krow, nel});
            }
        }
    int cases = 0;
    std::vector<int> ks = {-BK, 3 * BK + 5};
    for (int k = -1; k <= 2 * BK + 1; ++k) ks.push_back(k);
    std::vector<int> ns;
    for (int n = 1; n <= 3 * EPC; ++n) ns.push_back(n);
    for (int n = BN - 3 * EPC; n <= BN + 2 * EPC; ++n) ns.push_back(n);
    for (int k_left : ks)
        for (int n_left : ns)
            for (int ldb = n_left; ldb <= n_left + EPC + 1; ++ldb) {
                const bool whole = whole_loads<C>(k_left, n_left, ldb);
                if (!whole && k_left > BK && ldb >= EPC) FAIL("K tile before the last not on whole loads");
                if (!whole || k_left <= 0) continue;
                ++cases;
                const long b_last = (long)(k_left - 1) * ldb + n_left - 1;
                if (!C::B_DMA)  // a B moved by LDS-DMA meets the 16-byte rules: N is whole chunks
                    for (auto [krow, nel] : bch)
                        if (krow < k_left && nel < n_left && (long)krow * ldb + nel + EPC - 1 > b_last)
                            FAIL("B chunk (%d,%d) k_left %d n_left %d ldb %d reads past B", krow, nel, k_left, n_left,
                                 ldb);
                if (C::A_DMA) continue;  // likewise an A moved by LDS-DMA: K is whole chunks
                for (auto [row, kel] : ach)
                    if (kel < k_left && kel + EPC > k_left) FAIL("A chunk (%d,%d) straddles K, k_left %d", row, kel, k_left);
                if (n_left != ns[0] || ldb != n_left) continue;  // A's reads do not depend on N
                for (int rows_left : {1, 2, C::BM})
                    for (int lda : {k_left, k_left + 1, k_left + EPC}) {
                        const long a_last = (long)(rows_left - 1) * lda + k_left - 1;
                        for (auto [row, kel] : ach)
                            if (row < rows_left && kel < k_left && (long)row * lda + kel + EPC - 1 > a_last)
                                FAIL("A chunk (%d,%d) reads past A", row, kel);
                    }
            }
    return cases;
}

// DIRECT on a K that is not whole 16-byte chunks, in the K tile that holds
// the end of K (k_left < BK, k_left % EPC != 0): LDS-DMA moves only whole A
// chunks (every element it reads lies before k_left in a row that exists),
// lanes with a straddling chunk receive zeros, and the tail patch writes the
// chunk's elements before k_left over them.  The A region must then hold the
// zero-padded tile exactly, as DIRECT would on a copy with K rounded up.
template <class C>
static int check_dma_tail(const char* name) {
    constexpr int EPC = C::EPC, BK = C::BK;
    int cases = 0;
    for (int k_left = 1; k_left < BK; ++k_left) {
        if (k_left % EPC == 0) continue;
        for (int rows_left : {1, C::BM / 2 + 3, C::BM}) {
            // element (row, k) of the global tile holds 1 + row * BK + k; -1 marks "never written"
            std::vector<long> lds(C::A_BYTES / C::ES, -1);
            for (int w = 0; w < C::NW; ++w)
                for (int l = 0; l < 64; ++l)
                    for (int q = 0; q < C::A_INSTR; ++q) {
                        int row, kel;
                        a_chunk<C>(w, l, q, row, kel);
                        const long base = ((long)(w * C::A_INSTR + q) * 1024 + l * 16) / C::ES;
                        const bool ok = row < rows_left && kel + EPC <= k_left;  // dma_piece
                        for (int e = 0; e < EPC; ++e) {
                            if (ok && kel + e >= k_left) FAIL("LDS-DMA reads past K: k %d k_left %d", kel + e, k_left);
                            lds[base + e] = ok ? 1 + (long)row * BK + kel + e : 0;
                        }
                        // dma_patch (after the pieces have landed)
                        if (row < rows_left && kel < k_left && kel + EPC > k_left)
                            for (int e = 0; e < EPC; ++e) lds[base + e] = kel + e < k_left ? 1 + (long)row * BK + kel + e : 0;
                    }
            // compare with the zero-padded tile, placed by the A swizzle
            for (int row = 0; row < C::BM; ++row)
                for (int kc = 0; kc < C::KC; ++kc)
                    for (int e = 0; e < EPC; ++e) {
                        const int k = kc * EPC + e;
                        const long want = row < rows_left && k < k_left ? 1 + (long)row * BK + k : 0;
                        const long got = lds[a_off<C::KC>(row, kc) / C::ES + e];
                        if (got != want)
                            FAIL("tail tile: row %d k %d k_left %d rows_left %d holds %ld, want %ld", row, k, k_left,
                                 rows_left, got, want);
                    }
            ++cases;
        }
    }
    return cases;
}

// Hazard demonstrator indexing (hazard_demo.hpp), for the shapes and leading
// dimensions the entry point admits: every global read (tiles 0, 1 and, per
// iteration, t+2 or t) lies inside the caller's rows x cols, every LDS index
// inside a stage, every row sum and timeline stamp inside its buffer; the
// producers fill each stage chunk exactly once and the consumers read each
// exactly once, wave w the rows 4w..4w+3; and every wave's rows are written
// by other waves, so a missing reuse barrier can corrupt them.
static int check_hazard_indexing() {
    using namespace hazard;
    const char* name = "hazard";
    int cases = 0;
    for (int rows : {16, 48})
        for (int cols : {256, 512, 1280})
            for (int ldx : {cols, cols + 4, cols + 260}) {
                const int nT = cols / TC, grid = rows / RB;
                for (int b = 0; b < grid; ++b)
                    for (int t = -1; t < nT; ++t) {
                        // t = -1: the prologue's tiles 0 and 1; else the loop's load
                        std::vector<int> tiles;
                        if (t < 0) {
                            tiles.push_back(0);
                            if (nT > 1) tiles.push_back(1);
                        } else {
                            tiles.push_back(t + 2 < nT ? t + 2 : t);
                        }
                        for (int tt : tiles)
                            for (int tid = 0; tid < NTH; ++tid)
                                for (int j = 0; j < CPT; ++j) {
                                    const int c = prod_chunk(tid, j);
                                    if (c < 0 || c >= CHUNKS) FAIL("stage index %d", c);
                                    const int64_t off = (int64_t)b * RB * ldx + x_offset(ldx, chunk_row(c), tt, chunk_col(c));
                                    const int64_t r = off / ldx, col = off % ldx;
                                    if (off < 0 || r >= rows || col + 3 >= cols)
                                        FAIL("read (%lld,%lld) outside %dx%d ld %d", (long long)r, (long long)col, rows, cols, ldx);
                                    if (r != b * RB + chunk_row(c) || col != tt * TC + chunk_col(c)) FAIL("chunk placement");
                                    ++cases;
                                }
                    }
                for (int w = 0; w < NWAVE; ++w)
                    for (int t = 0; t < nT; ++t)
                        for (int e = 0; e < EV; ++e)
                            if (trace_index(w, nT, t, e) < 0 || trace_index(w, nT, t, e) >= (int64_t)NWAVE * EV * nT)
                                FAIL("trace index");
                for (int b = 0; b < grid; ++b)
                    for (int w = 0; w < NWAVE; ++w)
                        for (int rr = 0; rr < ROWS_PER_WAVE; ++rr)
                            if (b * RB + ROWS_PER_WAVE * w + rr >= rows) FAIL("row sum index");
            }
    std::vector<int> prod(CHUNKS, 0), cons(CHUNKS, 0);
    for (int tid = 0; tid < NTH; ++tid)
        for (int j = 0; j < CPT; ++j) prod[prod_chunk(tid, j)]++;
    for (int w = 0; w < NWAVE; ++w)
        for (int l = 0; l < 64; ++l)
            for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
                const int c = cons_chunk(w, l, rr);
                if (c < 0 || c >= CHUNKS) FAIL("consumer index %d", c);
                if (chunk_row(c) != ROWS_PER_WAVE * w + rr || chunk_col(c) != 4 * l) FAIL("consumer placement");
                cons[c]++;
            }
    for (int c = 0; c < CHUNKS; ++c)
        if (prod[c] != 1 || cons[c] != 1) FAIL("chunk %d produced %d, consumed %d times", c, prod[c], cons[c]);
    for (int w = 0; w < NWAVE; ++w) {
        bool foreign = false;
        for (int tid = 0; tid < NTH; ++tid)
            for (int j = 0; j < CPT; ++j) {
                const int row = chunk_row(prod_chunk(tid, j));
                if (tid / 64 != w && row / ROWS_PER_WAVE == w) foreign = true;
            }
        if (!foreign) FAIL("rows of wave %d written only by itself", w);
    }
    return cases;
}

// Work split: for every tile count and grid (a multiple of 8, at most one
// workgroup per tile rounded up to 8, as the host launches), each logical tile
// goes to exactly one workgroup, each XCD (b % 8) gets a contiguous range,
// and the grouped raster maps the logical tiles onto the tile grid one to one.
static int check_work_split() {
    const char* name = "work_split";
    int cases = 0;
    for (int G = 1; G <= 300; G += (G < 40 ? 1 : 7)) {
        const int full = (G + 7) / 8 * 8;
        for (int nb = 8; nb <= full; nb += 8) {
            std::vector<int> owner(G, -1);
            for (int b = 0; b < nb; ++b) {
                const WgTiles w = wg_tiles_of(G, b, nb);
                if (nb == full && w.count > 1) FAIL("G %d: default grid gives wg %d %d tiles", G, b, w.count);
                for (int i = 0; i < w.count; ++i) {
                    const int L = w.start + w.lb + i * w.nl;
                    if (L < 0 || L >= G) FAIL("G %d grid %d: wg %d tile %d out of range", G, nb, b, L);
                    if (owner[L] >= 0) FAIL("G %d grid %d: tile %d owned twice", G, nb, L);
                    if ((owner[L] = b) % 8 != (b & 7)) FAIL("bad XCD");
                }
            }
            for (int L = 0; L < G; ++L)
                if (owner[L] < 0) FAIL("G %d grid %d: tile %d unowned", G, nb, L);
            for (int L = 1; L < G; ++L)
                if ((owner[L] & 7) < (owner[L - 1] & 7)) FAIL("G %d grid %d: XCD ranges not contiguous", G, nb);
            ++cases;
        }
    }
    for (int tm = 1; tm <= 20; ++tm)
        for (int tn = 1; tn <= 20; ++tn)
            for (int gm = 1; gm <= 20; ++gm) {
                std::vector<int> hit(tm * tn, 0);
                for (int L = 0; L < tm * tn; ++L) {
                    int a, b;
                    raster(L, tm, tn, gm, a, b);
                    if (a < 0 || a >= tm || b < 0 || b >= tn) FAIL("raster %d of %dx%d out of range", L, tm, tn);
                    hit[a * tn + b]++;
                }
                for (int x : hit)
                    if (x != 1) FAIL("raster %dx%d group %d not a bijection", tm, tn, gm);
                ++cases;
            }
    return cases;
}

#define CHECK(D, BM, BN, BK, WGM, WGN)                                              \
    do {                                                                           \
        emulate<Cfg<D, BM, BN, BK, 2, WGM, WGN, PROD_DIRECT>>(#D " " #BM "x" #BN "x" #BK); \
        wl += check_whole_loads<Cfg<D, BM, BN, BK, 2, WGM, WGN, PROD_GENERIC>>("whole_loads " #D); \
        wl += check_whole_loads<Cfg<D, BM, BN, BK, 2, WGM, WGN, PROD_STAGED_A>>("whole_loads staged A " #D); \
        wl += check_whole_loads<Cfg<D, BM, BN, BK, 2, WGM, WGN, PROD_STAGED_B>>("whole_loads staged B " #D); \
        dt += check_dma_tail<Cfg<D, BM, BN, BK, 2, WGM, WGN, PROD_DIRECT>>("dma tail " #D);   \
        ++n;                                                                       \
        printf("class %d %d %d %d %d %d\n", D, BM, BN, BK, WGM, WGN);              \
    } while (0)

int main() {
    int n = 0, wl = 0, dt = 0;
    CHECK(DT_BF16, 256, 256, 32, 2, 4);
    CHECK(DT_BF16, 256, 256, 64, 2, 4);
    CHECK(DT_BF16, 128, 128, 64, 2, 2);
    CHECK(DT_F16, 256, 256, 32, 2, 4);
    CHECK(DT_F16, 256, 256, 64, 2, 4);
    CHECK(DT_F16, 128, 128, 64, 2, 2);
    CHECK(DT_I8, 256, 256, 64, 2, 4);
    CHECK(DT_I8, 256, 256, 128, 2, 4);
    CHECK(DT_I8, 128, 128, 128, 2, 2);
    CHECK(DT_F32, 128, 64, 16, 2, 2);
    CHECK(DT_F32, 256, 256, 32, 2, 4);
    CHECK(DT_F32, 128, 128, 32, 2, 2);
    printf("whole_loads %d cases\n", wl);
    printf("dma_tail %d cases\n", dt);
    printf("chunk_fits %d cases\n", check_chunk_fits());
    printf("work_split %d cases\n", check_work_split());
    printf("hazard %d cases\n", check_hazard_indexing());
    printf("OK %d\n", n);
    return 0;
}
