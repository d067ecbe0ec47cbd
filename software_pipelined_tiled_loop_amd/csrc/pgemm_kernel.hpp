// pgemm_kernel.hpp -- the software-pipelined tiled GEMM kernel for gfx950.
//
// A workgroup computes BM x BN tiles of C = alpha*A*B + beta*C.  Its K loop
// runs over a ring of S LDS stages, following the prologue / steady state /
// epilogue structure of page "Software pipelines and asynchronous copies"
// (section "Prologue, steady state, and epilogue") and the one-barrier
// double-buffered loop of page "Double Buffering: Software Pipelining the
// K-Loop" (section "Two Stages, One Barrier"), generalised to S stages:
//
//   prologue      issue K tiles 0 .. S-2 into stages 0 .. S-2
//   iteration t   s_waitcnt: tile t+1 has landed (the loads of the S-2 later
//                 tiles may still be in flight: vmcnt = loads-per-stage times
//                 their count); s_barrier: ready edge of tile t+1's stage for
//                 every wave, and reuse edge of tile t's stage (every wave
//                 finished reading it); issue tile t+S into that stage; MFMA
//                 work on tile t (its last K step after the barrier)
//   drain         the loop body is the same for every t: a slot past the last
//                 K tile issues the same number of loads with every lane out
//                 of range (zeros into a stage nobody reads), so the wait
//                 count is a constant and the loop has no drain branches; the
//                 workgroup waits for everything before it retires.
//
// S == 1 is the single-buffer loop (load, wait, barrier, compute, barrier) of
// the first page's section on kernel 10; with the REGISTER producer it is the
// single-LDS-buffer register-prefetch variant of page "GPU-Kernel pipelinen",
// step 1 (two barriers per tile, the loads of tile t+1 in flight during the
// arithmetic on tile t).
//
// Producers (page "Double Buffering...", section "Two Stages, One Barrier";
// page "GPU-Kernel pipelinen", step 2):
//   DIRECT    buffer_load_dwordx4 ... lds: global memory straight into the LDS
//             stage without registers; completion observed with vmcnt.  Slots
//             that load a whole K tile of a whole output tile pass each lane's
//             offset unselected (no range check can fail there).
//   REGISTER  buffer_load_dwordx4 into VGPRs at the top of the iteration,
//             ds_write_b128 into the stage after the MFMA work.
//   GENERIC   as REGISTER for any element-aligned layout: 16-byte loads at
//             unaligned addresses; in the last K tile, elements past K zeroed
//             in registers and element loads for a chunk at the very end of a
//             matrix.
//   STAGED_A  one producer per operand: A as GENERIC (any alignment), B by
//   STAGED_B  LDS-DMA; or A by LDS-DMA, B as GENERIC.  The operand that is a
//             straight aligned copy goes direct while the other goes through
//             registers (the split of the first page's kernel 11, which copies
//             B asynchronously and stages A in registers).  Two-stage ring.
// All of them write the same LDS bytes for every element inside the matrix and
// zeros past K and M (the generic producer may leave other values in columns
// past N, which feed only outputs that are never stored), so the stored result
// does not depend on the producer or on S.
//
// Launches: one workgroup per output tile (the per-tile pipeline, epilogue
// after it), or persistent workgroups that stream the K tiles of all their
// output tiles through one ring, the fused alpha/beta epilogue of each tile
// between them.
//
// LDS layout (per stage): A tile as BM rows of BK elements (K contiguous),
// B tile as BK rows of BN elements (N contiguous) -- both straight copies of
// global memory, so both can use the direct producer.  16-byte chunks are
// XOR-swizzled within each row against bank conflicts; the direct producer
// realises the swizzle by choosing which global chunk each lane fetches (an
// LDS-DMA instruction writes 1 KiB contiguously, lane l at byte 16*l).
// MFMA operands: A fragments with ds_read_b128; B fragments with the gfx950
// transposing reads ds_read_b64_tr_b16 (fp16/bf16) and ds_read_b64_tr_b8
// (int8), which deliver K-contiguous fragments from the N-contiguous rows;
// fp32 B fragments with ds_read_b32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgemm {

enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3 };
enum Producer : int { PROD_DIRECT = 1, PROD_REGISTER = 2, PROD_GENERIC = 3, PROD_STAGED_A = 4, PROD_STAGED_B = 5 };
// Parts of the steady state that a parts-ladder build (PartsCfg) can leave
// out: the LDS-DMA pieces, the ready-edge barrier, the A and the B fragment
// reads.
enum Part : int { PART_DMA = 1, PART_BARRIER = 2, PART_AREADS = 4, PART_BREADS = 8, PART_ALL = 15 };

struct KernelArgs {
    const void* A;
    const void* B;
    void* C;
    int64_t lda, ldb, ldc;  // elements
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;            // tile-rows per raster group
    float alpha, beta;      // float dtypes
    int ialpha, ibeta;      // int8
    int beta_nonzero;
    int dbg_sleep;          // test hook: wave (t % NW) sleeps dbg_sleep x 8128 cycles per K tile (0 = off)
    long long* probe;       // wait-profile builds only (ProbeCfg): per-wave clock totals, else unused
};

// Test hook for stress runs: skew one wave per K tile (rotating) so that the
// stage protocol is exercised with waves far apart.  Off (one scalar compare)
// unless the caller asks for it.
__device__ __forceinline__ void debug_skew(const KernelArgs& g, int t, int wave, int nw) {
    if (g.dbg_sleep != 0 && wave == t % nw) {
        for (int i = 0; i < g.dbg_sleep; ++i) __builtin_amdgcn_s_sleep(127);
    }
}

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

#define PGEMM_LDS __attribute__((address_space(3)))

template <int D> struct Traits;
template <> struct Traits<DT_F32> {
    static constexpr int ES = 4;       // element bytes
    static constexpr int EPC = 4;      // elements per 16-byte chunk
    static constexpr int KSTEP = 16;   // K covered when each lane reads one A chunk
    typedef f32x4 Acc;
    typedef float Out;                 // element type of C
};
template <> struct Traits<DT_F16> {
    static constexpr int ES = 2, EPC = 8, KSTEP = 32;
    typedef f32x4 Acc;
    typedef float Out;
};
template <> struct Traits<DT_BF16> {
    static constexpr int ES = 2, EPC = 8, KSTEP = 32;
    typedef f32x4 Acc;
    typedef float Out;
};
template <> struct Traits<DT_I8> {
    static constexpr int ES = 1, EPC = 16, KSTEP = 64;
    typedef i32x4 Acc;
    typedef int Out;
};

// Buffer resource covering [base, base + 2^31): the kernel decides validity
// itself and sends invalid lanes to offset 2^31, which the hardware range
// check turns into zeros (no memory access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x80000000, 0x00020000);
}
// The same descriptor as four scalar dwords, for the inline-asm LDS-DMA load.
__device__ __forceinline__ i32x4 make_rsrc_sgpr(const void* base) {
    const uint64_t p = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu));  // stride 0
    r[2] = (int)0x80000000u;                                                          // num_records
    r[3] = 0x00020000;                                                                // 32-bit data format
    return r;
}
static constexpr uint32_t OOB = 0x80000000u;

// LDS-DMA: 16 bytes from buffer offset `voff` of lane l land at LDS byte
// `lds_base + 16*l` (lds_base is wave-uniform and goes through M0).  The
// load is issued from inline asm so that the compiler does not treat it as a
// pending LDS write: it would otherwise wait for every outstanding LDS-DMA
// (vmcnt(0)) before each later LDS read and serialise the pipeline.  The
// kernel owns vmcnt for these loads and waits for them explicitly.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t voff, uint32_t lds_base) {
    // s_nop: one wait state between an SALU write of M0 and an LDS-DMA load.
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most VM vector-memory loads of this wave are outstanding and
// all its LDS operations are done, then the workgroup barrier.  One asm
// statement, so neither the compiler's scheduler nor its memory model moves
// anything across it or adds a vmcnt(0).
// The leading builtin lgkmcnt(0) is there for the compiler's own bookkeeping:
// it then knows every earlier LDS read has completed and does not hold back
// the next MFMAs on reads issued after the barrier.
__device__ __forceinline__ void lgkm_drain() {
    __builtin_amdgcn_s_waitcnt((15 & 15) | (7 << 4) | (0 << 8) | (3 << 14));  // vmcnt(63) expcnt(7) lgkmcnt(0)
}
template <int VM>
__device__ __forceinline__ void wait_barrier() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt is 6 bits");
    lgkm_drain();
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(VM) : "memory");
}
__device__ __forceinline__ void lgkm_barrier() {
    lgkm_drain();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// ---- LDS swizzles --------------------------------------------------------
// A: rows of KC 16-byte chunks, read by ds_read_b128 fragments that touch 16
// consecutive rows at 4 consecutive chunks.  Measured on gfx950 (per-variant
// SQ_LDS_BANK_CONFLICT), the LDS serves a ds_read_b128 16 lanes per cycle
// across 64 banks (256 bytes), grouping lanes that share lane-id bits 0 and
// 5: eight rows of one parity at two adjacent chunks.
//  * 64-byte rows (KC = 4): chunk L = row*KC + kc sits in 128-byte line L/8
//    at slot (L%8) ^ (line%8) ^ (line/8 %2) -- conflict-free.
//  * 128-byte rows (KC = 8): rows of one parity would all fall in the same
//    half of the 256-byte bank window (a 2-way conflict for any XOR inside a
//    line), so the swizzle works on 256-byte super-lines of two rows: slot
//    ((row%2)*8 + kc) ^ 2*(superline%8).  This removed the 2-way conflict
//    (8 -> 4 LDS cycles per fragment read).
#define PGEMM_HD __host__ __device__ __forceinline__

template <int KC>
PGEMM_HD constexpr int a_off(int row, int kc) {
    if constexpr (KC == 8) {
        const int sl = row >> 1;
        const int u = ((row & 1) << 3) + kc;
        return (sl << 8) + ((u ^ ((sl & 7) << 1)) << 4);
    } else {
        const int L = row * KC + kc;
        const int line = L >> 3;
        return (line << 7) + ((((L & 7) ^ (line & 7) ^ ((line >> 3) & 1))) << 4);
    }
}
// Inverse of a_off: the (row, chunk) stored at LDS byte `off` of the A region.
template <int KC>
PGEMM_HD void a_inv(int off, int& row, int& kc) {
    if constexpr (KC == 8) {
        const int sl = off >> 8;
        const int u = ((off >> 4) & 15) ^ ((sl & 7) << 1);
        row = (sl << 1) + (u >> 3);
        kc = u & 7;
    } else {
        const int line = off >> 7;
        const int L = (line << 3) + (((off >> 4) & 7) ^ (line & 7) ^ ((line >> 3) & 1));
        row = L / KC;
        kc = L % KC;
    }
}
// B: rows k of NCH chunks; chunk c of row k sits at c ^ pb(k).  pb spreads the
// rows that one transposing read touches over distinct banks.
template <int D, int NCH>
PGEMM_HD constexpr int b_swz(int k) {
    if constexpr (D == DT_I8) {
        return ((k & 7) + (((k >> 4) & 1) << 3)) & (NCH - 1);
    } else if constexpr (D == DT_F32) {
        return (((k >> 2) & 3) << 2) & (NCH - 1);
    } else {
        return (((k & 3) << 1) + (((k >> 3) & 1) << 3)) & (NCH - 1);
    }
}

template <int D, int BM_, int BN_, int BK_, int S_, int WGM_, int WGN_, int P_>
struct Cfg {
    static constexpr int Dt = D, BM = BM_, BN = BN_, BK = BK_, S = S_, WGM = WGM_, WGN = WGN_, P = P_;
    typedef Traits<D> T;
    static constexpr int ES = T::ES, EPC = T::EPC, KSTEP = T::KSTEP;
    static constexpr int NW = WGM * WGN;
    static constexpr int NT = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int FM = WM / 16, FN = WN / 16;
    static constexpr int KC = BK * ES / 16;           // chunks per A row
    static constexpr int NCH = BN * ES / 16;          // chunks per B row
    static constexpr int A_BYTES = BM * BK * ES;
    static constexpr int B_BYTES = BK * BN * ES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = S * STAGE_BYTES;
    static constexpr int A_INSTR = A_BYTES / 1024 / NW;   // 1-KiB chunk blocks per wave per stage
    static constexpr int B_INSTR = B_BYTES / 1024 / NW;
    static constexpr int LPS = A_INSTR + B_INSTR;         // vector loads per thread per stage
    static constexpr int B_ROWS_PER_KB = 1024 / (BN * ES);  // B rows per 1-KiB block
    static constexpr int A_ROWS_PER_KB = 1024 / (BK * ES);
    static constexpr int NKS = BK / KSTEP;               // MFMA K steps per tile
    // MFMA groups of a K step that the DMA blocks of the next tile are spread
    // over (see mfma_step).  Measured on MI355X at 4096^3 (whole-tile loads,
    // alternating rounds): fp32 (one long MFMA per block) is fastest with the
    // blocks in the first four groups (0.3 % ahead of two, 0.4 % of eight),
    // bf16 and int8 2-3 % faster with them spread over all eight than over
    // four.
    static constexpr int DMA_GROUPS = D == DT_F32 ? 4 : 8;
    // Which operands the LDS-DMA producer moves; the others are staged
    // through registers.  LDS-DMA pieces q of a K tile are [DMA_P0, DMA_P1):
    // A's blocks are 0 .. A_INSTR-1, B's A_INSTR .. LPS-1.
    static constexpr bool A_DMA = P == PROD_DIRECT || P == PROD_STAGED_B;
    static constexpr bool B_DMA = P == PROD_DIRECT || P == PROD_STAGED_A;
    static constexpr bool ANY_DMA = A_DMA || B_DMA;
    static constexpr bool ANY_STAGED = !(A_DMA && B_DMA);
    static constexpr bool MIXED = ANY_DMA && ANY_STAGED;
    static constexpr int DMA_P0 = A_DMA ? 0 : A_INSTR;
    static constexpr int DMA_P1 = B_DMA ? LPS : A_INSTR;
    static constexpr int STAGED_LOADS = LPS - (DMA_P1 - DMA_P0);  // register loads per thread per K tile
    // K tiles ahead of the one being multiplied that are loaded: S for the
    // LDS-DMA pieces, one more for register-staged operands, which hold a
    // K tile in registers before it is written to its stage.
    static constexpr int LA_DMA = S;
    static constexpr int LA_REG = S + 1;
    // MFMA groups of a K step (mfma_step), and the first group after the
    // last one that issues LDS-DMA blocks: the register-staged loads of a
    // one-producer-per-operand ring go there, behind every piece.
    static constexpr int NGROUPS = FM * FN < 8 ? FM * FN : 8;
    static constexpr int DMA_NG = DMA_GROUPS < NGROUPS ? DMA_GROUPS : NGROUPS;
    static constexpr int DMA_PPG = (DMA_P1 - DMA_P0 + DMA_NG - 1) / (DMA_NG > 0 ? DMA_NG : 1);
    static constexpr int REG_GROUP = MIXED ? (DMA_P1 - DMA_P0 + DMA_PPG - 1) / DMA_PPG : 1;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be whole 16x16 blocks");
    static_assert(BK % KSTEP == 0, "BK must be a multiple of the MFMA K step");
    static_assert(KC == 4 || KC == 8, "A rows must be 64 or 128 bytes");
    static_assert((NCH & (NCH - 1)) == 0 && NCH >= 4, "B rows must be a power-of-two number of chunks");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "stage must split into 1 KiB per wave");
    static_assert(BN * ES <= 1024 && 1024 % (BN * ES) == 0, "B row must divide 1 KiB");
    static_assert(LDS_BYTES <= 163840, "LDS ring exceeds 160 KiB");
    static_assert(S >= 1 && S <= 4, "1..4 stages");
    static_assert(LPS * (S > 2 ? S - 2 : 0) <= 63, "vmcnt is a 6-bit counter");
    static_assert(P >= PROD_DIRECT && P <= PROD_STAGED_B, "unknown producer");
    // Wait-profile builds (ProbeCfg) stamp the shader clock around the waits
    // of every ready edge; the GEMM's own variants never do.
    static constexpr bool PROBE = false;
    // Parts-ladder builds (PartsCfg) leave parts of the K loop out and stamp
    // the clocks at the start and end of each workgroup; the GEMM's own
    // variants run every part and stamp nothing.
    static constexpr int PARTS = PART_ALL;
    static constexpr bool CLOCK = false;
    static_assert(!MIXED || S == 2, "one producer per operand runs a two-stage ring");
};

// ---- producers -------------------------------------------------------------

// Chunk q (0..A_INSTR-1) that this lane moves for the A tile: the LDS byte of
// the chunk is (wave*A_INSTR + q)*1024 + 16*lane within the stage's A region;
// returns the (row, first element k) of global memory that belongs there.
template <class C>
PGEMM_HD void a_chunk(int wave, int lane, int q, int& row, int& kel) {
    int kc;
    a_inv<C::KC>((wave * C::A_INSTR + q) * 1024 + lane * 16, row, kc);
    kel = kc * C::EPC;
}
// Same for the B tile: (row k, first element n).
template <class C>
PGEMM_HD void b_chunk(int wave, int lane, int q, int& krow, int& nel) {
    const int lds_off = (wave * C::B_INSTR + q) * 1024 + lane * 16;
    krow = lds_off / (C::BN * C::ES);
    const int pc = (lds_off % (C::BN * C::ES)) >> 4;
    nel = (pc ^ b_swz<C::Dt, C::NCH>(krow)) * C::EPC;
}

// A parts-ladder build of tile configuration C: the same kernel with parts
// of its steady state left out (PARTS, a set of Part bits), for measuring
// what each part costs.  Left-out LDS-DMA pieces leave the two stages holding
// the prologue's K tiles (real operand data, so the matrix cores see the
// same kind of values); left-out fragment reads leave the registers holding
// the previous step's fragments (both fragment buffers start from operand
// data); a left-out barrier keeps its s_waitcnt.
// The prologue's ready edge always keeps its barrier.  Results are correct
// only with every part in.  Wave 0 of each workgroup stamps the shader and
// 100 MHz clocks at its start and after its last store (kClockWords).
template <class Base, int PARTS_>
struct PartsCfg : Base {
    static constexpr int PARTS = PARTS_;
    static constexpr bool CLOCK = true;
};

// Entries per workgroup of a parts-ladder build's clock output: shader clock
// and 100 MHz clock at the start, then both after the last store.
constexpr int kClockWords = 4;

// A wait-profile build of tile configuration C: the same kernel, with shader
// clock stamps around the vmcnt wait and the barrier of each ready edge
// (sync_ring), summed per wave.
template <class Base>
struct ProbeCfg : Base {
    static constexpr bool PROBE = true;
};

// Per-wave clock totals of a wait-profile build: cycles spent in the vmcnt
// wait of the ready edges, cycles from there through the barrier, the
// number of ready edges, and the time (100 MHz clock) the first ready edge
// (the end of the prologue) was passed.
template <bool P>
struct ProbeSlots {};
template <>
struct ProbeSlots<true> {
    long long vm = 0, bar = 0, n = 0, rt_ready0 = 0;
};

// Entries per wave of the wait-profile output.
constexpr int kProbeWords = 8;

template <class C>
struct Staging : ProbeSlots<C::PROBE> {
    i32x4 a[C::A_INSTR];
    i32x4 b[C::B_INSTR];
};

// True when EPC elements read from element (r, c) of a row-major matrix with
// `rows` rows, `cols` columns and leading dimension `ld` end at or before the
// matrix's last element, so that a 16-byte read of a chunk that is partly
// outside the columns never leaves the caller's allocation.
PGEMM_HD bool chunk_fits(int r, int c, int64_t ld, int rows, int cols, int epc) {
    return c + epc <= cols || (int64_t)r * ld + c + epc <= (int64_t)(rows - 1) * ld + cols;
}

// Element-wise load of one 16-byte chunk: elements at or beyond `valid` are
// zero.  `off` is the byte offset of the first element.
template <int ES>
__device__ __forceinline__ i32x4 load_chunk_elementwise(__amdgpu_buffer_rsrc_t r, uint32_t off, int valid) {
    i32x4 v = {0, 0, 0, 0};
    if constexpr (ES == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t o = (e < valid) ? off + 4u * e : OOB;
            v[e] = (int)__builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
        }
    } else if constexpr (ES == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t o = (e < valid) ? off + 2u * e : OOB;
            const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, 0);
            v[e >> 1] |= (int)(h << (16 * (e & 1)));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t o = (e < valid) ? off + (uint32_t)e : OOB;
            const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(r, o, 0, 0);
            v[e >> 2] |= (int)(b << (8 * (e & 3)));
        }
    }
    return v;
}

// Zero the elements of a chunk at or beyond `valid` (0 <= valid <= 16/ES).
template <int ES>
__device__ __forceinline__ i32x4 zero_tail(i32x4 v, int valid) {
    const int vbytes = valid * ES;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int keep = vbytes - 4 * d;  // bytes of dword d that stay
        const uint32_t m = keep >= 4 ? 0xffffffffu : keep <= 0 ? 0u : (0xffffffffu >> (8 * (4 - keep)));
        v[d] = (int)((uint32_t)v[d] & m);
    }
    return v;
}

// GENERIC producer: any element-aligned address.  One 16-byte load when the
// 16 bytes lie inside the caller's matrix (`vec_ok`; the target runs in
// unaligned-access mode, which the compiler itself relies on for unaligned
// vector accesses), with the tail beyond `valid` zeroed; element-wise loads
// for a partial chunk at the very end of the matrix, where a 16-byte load
// could run past the allocation.
template <int ES>
__device__ __forceinline__ i32x4 load_chunk_any(__amdgpu_buffer_rsrc_t r, uint32_t off, int valid, bool vec_ok) {
    if (valid <= 0) return i32x4{0, 0, 0, 0};
    if (vec_ok) {
        const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        return valid >= 16 / ES ? v : zero_tail<ES>(v, valid);
    }
    return load_chunk_elementwise<ES>(r, off, valid);
}

// GENERIC producer (and the staged operand of STAGED_A / STAGED_B): true
// when every register-staged chunk of the K tile whose remaining extents from
// the tile origin are k_left and n_left may be read as one whole 16-byte load,
// so the tile's loads form one straight run with no waits between them.  Chunks start at multiples of EPC, so no A chunk straddles the
// end of K when the K tile is whole or k_left is a multiple of EPC; likewise
// for B and N.  A B chunk that does straddle N carries the first elements of
// B's next row into columns >= N, which feed only outputs that are never
// stored; before the last K tile (k_left > BK) at least one more row of B lies
// beyond it, which holds the overrun when ldb >= EPC.  Otherwise (only ever in
// the last K tile) each chunk is loaded by load_chunk_any.  Past the last K
// tile (k_left <= 0) every chunk is out of range and loads nothing.
template <class C>
PGEMM_HD bool whole_loads(int k_left, int n_left, int64_t ldb) {
    const bool a_whole = C::A_DMA || k_left >= C::BK || k_left % C::EPC == 0;
    const bool b_whole = C::B_DMA || n_left >= C::BN || n_left % C::EPC == 0 || (k_left > C::BK && ldb >= C::EPC);
    return k_left <= 0 || (a_whole && b_whole);
}

// DIRECT producer state for one K tile: buffer descriptors of the tile's A
// and B panels, the LDS bases of the stage and the remaining extents.
struct DmaTile {
    i32x4 ra, rb;
    uint32_t sa, sb;
    int rows_left, k_left, n_left;
};

template <class C>
__device__ __forceinline__ DmaTile dma_setup(const KernelArgs& g, int m0, int n0, int kt, char PGEMM_LDS* stage,
                                             int wave) {
    constexpr int ES = C::ES;
    const int k0 = kt * C::BK;
    DmaTile d;
    // Tile-local bases keep every byte offset below 2^31.
    d.ra = make_rsrc_sgpr((const char*)g.A + ((int64_t)m0 * g.lda + k0) * ES);
    d.rb = make_rsrc_sgpr((const char*)g.B + ((int64_t)k0 * g.ldb + n0) * ES);
    d.sa = (uint32_t)(size_t)stage + (uint32_t)(wave * C::A_INSTR) * 1024u;
    d.sb = (uint32_t)(size_t)stage + (uint32_t)C::A_BYTES + (uint32_t)(wave * C::B_INSTR) * 1024u;
    d.rows_left = g.M - m0;
    d.k_left = g.K - k0;
    d.n_left = g.N - n0;
    return d;
}

// Load piece q (0..LPS-1) of the tile: one 1-KiB LDS-DMA block of A (q <
// A_INSTR) or of B.  FULL: the caller guarantees a whole K tile of a whole
// output tile (k_left >= BK, rows_left >= BM, n_left >= BN), so every lane is
// in range and its offset goes to the load as it is, with no per-lane select
// (the select's destination would be a temporary register written right
// under the MFMAs, which stalls the matrix pipe when the register was one of
// their operands).
//
//
// Only whole A chunks are moved: a chunk that straddles the end of K (K not
// whole chunks, in the K tile that holds its end) would run past the row's K
// elements, into the caller's padding or past the allocation.  Its lane
// receives zeros like a lane outside the matrix, and dma_patch then writes
// the chunk's elements before K over them.
template <class C, bool FULL = false>
__device__ __forceinline__ void dma_piece(const KernelArgs& g, const DmaTile& d, int q, int wave, int lane) {
    constexpr int ES = C::ES;
    if (q < C::A_INSTR) {
        int row, kel;
        a_chunk<C>(wave, lane, q, row, kel);
        const bool ok = FULL || (row < d.rows_left && kel + C::EPC <= d.k_left);
        dma16(d.ra, ok ? (uint32_t)(row * (int)g.lda + kel) * ES : OOB, d.sa + (uint32_t)q * 1024u);
    } else {
        const int qb = q - C::A_INSTR;
        int krow, nel;
        b_chunk<C>(wave, lane, qb, krow, nel);
        const bool ok = FULL || (krow < d.k_left && nel < d.n_left);
        dma16(d.rb, ok ? (uint32_t)(krow * (int)g.ldb + nel) * ES : OOB, d.sb + (uint32_t)qb * 1024u);
    }
}

// LDS-DMA pieces of K tile `kt` for the operands the DMA producer moves,
// straight into LDS stage `stage`.  Lanes whose chunk lies outside the matrix
// get offset 2^31 and receive zeros.  FULL as for dma_piece.
template <class C, bool FULL = false>
__device__ __forceinline__ void issue_dma(const KernelArgs& g, int m0, int n0, int kt, char PGEMM_LDS* stage,
                                          int wave, int lane) {
    const DmaTile d = dma_setup<C>(g, m0, n0, kt, stage, wave);
#pragma unroll
    for (int q = C::DMA_P0; q < C::DMA_P1; ++q) dma_piece<C, FULL>(g, d, q, wave, lane);
    if constexpr (!FULL && C::P == PROD_DIRECT) {
        if (tail_tile<C>(g, kt)) dma_patch<C>(g, m0, kt, stage, wave, lane);
    }
}

// Whether K tile kt holds the end of a K that is not whole 16-byte chunks
// (uniform): the one K tile whose A chunks can straddle the end of K.  Only
// the DIRECT producer meets it: STAGED_B, the other one that moves A by
// LDS-DMA, is admitted only when A's rows are whole chunks.
template <class C>
__device__ __forceinline__ bool tail_tile(const KernelArgs& g, int kt) {
    const int k_left = g.K - kt * C::BK;
    return C::P == PROD_DIRECT && k_left > 0 && k_left < C::BK && k_left % C::EPC != 0;
}

// The K tail of an A moved by LDS-DMA when K is not whole 16-byte chunks: in
// the tail K tile each row's chunk that straddles K (zeros from dma_piece) is
// loaded element by element, zero past K, and written over its place in the
// stage.  Called after the tile's LDS-DMA pieces and before the barrier that
// makes the stage ready.  Waiting for its own loads before the LDS writes, it
// waits for every earlier load of the wave (vmcnt counts in order), so the
// pieces' zeros have landed before they are overwritten.  Once per output
// tile.
template <class C>
__device__ __forceinline__ void dma_patch(const KernelArgs& g, int m0, int kt, char PGEMM_LDS* stage, int wave,
                                          int lane) {
    if constexpr (C::A_DMA) {
        const int k0 = kt * C::BK, k_left = g.K - k0;
        const int rows_left = g.M - m0;
        const __amdgpu_buffer_rsrc_t r = make_rsrc((const char*)g.A + ((int64_t)m0 * g.lda + k0) * C::ES);
#pragma unroll
        for (int q = 0; q < C::A_INSTR; ++q) {
            int row, kel;
            a_chunk<C>(wave, lane, q, row, kel);
            if (row < rows_left && kel < k_left && kel + C::EPC > k_left) {
                const i32x4 v =
                    load_chunk_elementwise<C::ES>(r, (uint32_t)(row * (int)g.lda + kel) * C::ES, k_left - kel);
                *(i32x4 PGEMM_LDS*)(stage + (wave * C::A_INSTR + q) * 1024 + lane * 16) = v;
            }
        }
    }
}

// Global loads of K tile `kt` for the register-staged operands, into the
// staging registers.  Lanes whose chunk lies outside the matrix load zeros.
template <class C>
__device__ __forceinline__ void issue_regs(const KernelArgs& g, int m0, int n0, int kt, Staging<C>& st, int wave,
                                           int lane) {
    constexpr int ES = C::ES;
    const int k0 = kt * C::BK;
    // Tile-local bases keep every byte offset below 2^31.
    const char* a_base = (const char*)g.A + ((int64_t)m0 * g.lda + k0) * ES;
    const char* b_base = (const char*)g.B + ((int64_t)k0 * g.ldb + n0) * ES;
    const int rows_left = g.M - m0, k_left = g.K - k0, n_left = g.N - n0;
    // With a ring (S >= 2) the chunk offsets are recomputed from an opaque
    // copy of the lane id at every issue: hoisted out of the K loop they
    // would hold a dozen registers for the whole loop next to the doubled
    // fragment set and, at the register limit, spill.
    if constexpr (C::S > 1) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" : "+v"(lane));
    }
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base);
    if (C::P == PROD_REGISTER || whole_loads<C>(k_left, n_left, g.ldb)) {
        if constexpr (!C::A_DMA) {
#pragma unroll
            for (int q = 0; q < C::A_INSTR; ++q) {
                int row, kel;
                a_chunk<C>(wave, lane, q, row, kel);
                const bool ok = row < rows_left && kel < k_left;
                st.a[q] = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? (uint32_t)(row * (int)g.lda + kel) * ES : OOB,
                                                                0, 0);
            }
        }
        if constexpr (!C::B_DMA) {
#pragma unroll
            for (int q = 0; q < C::B_INSTR; ++q) {
                int krow, nel;
                b_chunk<C>(wave, lane, q, krow, nel);
                const bool ok = krow < k_left && nel < n_left;
                st.b[q] = __builtin_amdgcn_raw_buffer_load_b128(rb, ok ? (uint32_t)(krow * (int)g.ldb + nel) * ES : OOB,
                                                                0, 0);
            }
        }
    } else {
        if constexpr (!C::A_DMA) {
#pragma unroll
            for (int q = 0; q < C::A_INSTR; ++q) {
                int row, kel;
                a_chunk<C>(wave, lane, q, row, kel);
                const bool ok = row < rows_left && kel < k_left;
                const uint32_t off = (uint32_t)(row * (int)g.lda + kel) * ES;
                const bool vec_ok = chunk_fits(row, kel, g.lda, rows_left, k_left, C::EPC);
                st.a[q] = load_chunk_any<ES>(ra, off, ok ? min(C::EPC, k_left - kel) : 0, vec_ok);
            }
        }
        if constexpr (!C::B_DMA) {
#pragma unroll
            for (int q = 0; q < C::B_INSTR; ++q) {
                int krow, nel;
                b_chunk<C>(wave, lane, q, krow, nel);
                const bool ok = krow < k_left && nel < n_left;
                const uint32_t off = (uint32_t)(krow * (int)g.ldb + nel) * ES;
                const bool vec_ok = chunk_fits(krow, nel, g.ldb, k_left, n_left, C::EPC);
                st.b[q] = load_chunk_any<ES>(rb, off, ok ? min(C::EPC, n_left - nel) : 0, vec_ok);
            }
        }
    }
}

// Register-staged operands: write the staged chunks to the same LDS bytes
// the direct producer fills.
template <class C>
__device__ __forceinline__ void store_tile(char PGEMM_LDS* stage, const Staging<C>& st, int wave, int lane) {
    if constexpr (!C::A_DMA) {
#pragma unroll
        for (int q = 0; q < C::A_INSTR; ++q)
            *(i32x4 PGEMM_LDS*)(stage + (wave * C::A_INSTR + q) * 1024 + lane * 16) = st.a[q];
    }
    if constexpr (!C::B_DMA) {
#pragma unroll
        for (int q = 0; q < C::B_INSTR; ++q)
            *(i32x4 PGEMM_LDS*)(stage + C::A_BYTES + (wave * C::B_INSTR + q) * 1024 + lane * 16) = st.b[q];
    }
}

// All loads of K tile `kt` that go to stage `stage` now: every operand for
// DIRECT, the register loads for REGISTER / GENERIC (written to the stage
// later by store_tile).  Used by the single-buffer loop.
template <class C>
__device__ __forceinline__ void issue_tile(const KernelArgs& g, int m0, int n0, int kt, char PGEMM_LDS* stage,
                                           Staging<C>& st, int wave, int lane) {
    static_assert(!C::MIXED, "the one-producer-per-operand ring issues its two parts separately");
    if constexpr (C::ANY_DMA)
        issue_dma<C>(g, m0, n0, kt, stage, wave, lane);
    else
        issue_regs<C>(g, m0, n0, kt, st, wave, lane);
}

// ---- consumer: MFMA fragments from one LDS stage ------------------------------

template <class C>
struct Frags {
    i32x4 a[C::FM];
    i32x4 b[C::FN];  // fp32: the B values of the four MFMAs of a K step
};

// LDS byte offset (within the stage's A region) of lane `lane`'s 16-byte A
// fragment for K step ks and 16-row block i of the wave.
template <class C>
PGEMM_HD int a_frag_off(int ks, int i, int wm0, int lane) {
    return a_off<C::KC>(wm0 + 16 * i + (lane & 15), ks * 4 + (lane >> 4));
}

// LDS byte offset (within the stage's B region) that lane `lane` addresses
// for B block j: h selects the half (0/1) of a 16-bit / 8-bit fragment
// (two transposing reads), or the MFMA jm (0..3) of an fp32 K step.
//  * ds_read_b64_tr_b16: lane i of a 16-lane block receives element i%4 of
//    the 4-element row piece addressed by lane 4e + i/4 (e = 0..3), so lane
//    j addresses row kb + j/4, columns nb + 4*(j%4), and lane i ends up with
//    B[kb + e][nb + i], e = 0..3.
//  * ds_read_b64_tr_b8: lane i receives byte i%8 of the 8-byte row piece
//    addressed by lane 2e + i/8 (e = 0..7): lane j addresses row kb + j/2,
//    columns nb + 8*(j%2).
//  * fp32: MFMA jm of the K step takes k = 4*lg + jm in lane group lg
//    (element jm of the lane's A chunk), so lane l reads B[k][nb + l%16].
template <class C>
PGEMM_HD int b_frag_off(int ks, int j, int wn0, int lane, int h) {
    constexpr int D = C::Dt;
    constexpr int ROWB = C::BN * C::ES;
    const int li = lane & 15, lg = lane >> 4;
    const int nb = wn0 + 16 * j;
    int k, n;
    if constexpr (D == DT_F16 || D == DT_BF16) {
        k = ks * C::KSTEP + 8 * lg + 4 * h + (li >> 2);
        n = nb + 4 * (li & 3);
    } else if constexpr (D == DT_I8) {
        k = ks * C::KSTEP + 16 * lg + 8 * h + (li >> 1);
        n = nb + 8 * (li & 1);
    } else {
        k = ks * C::KSTEP + 4 * lg + h;
        n = nb + li;
    }
    return k * ROWB + (((n / C::EPC) ^ b_swz<D, C::NCH>(k)) << 4) + (n % C::EPC) * C::ES;
}

template <class C>
__device__ __forceinline__ void read_a(const char PGEMM_LDS* stage, int ks, int i, int wm0, int lane, i32x4& out) {
    out = *(const i32x4 PGEMM_LDS*)(stage + a_frag_off<C>(ks, i, wm0, lane));
}

template <class C>
__device__ __forceinline__ void read_b(const char PGEMM_LDS* stage, int ks, int j, int wn0, int lane, i32x4& out) {
    constexpr int D = C::Dt;
    const char PGEMM_LDS* bs = stage + C::A_BYTES;
    if constexpr (D == DT_F16 || D == DT_BF16) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 PGEMM_LDS*)(bs + b_frag_off<C>(ks, j, wn0, lane, h)));
            const i32x2 w = __builtin_bit_cast(i32x2, v);
            out[2 * h] = w[0];
            out[2 * h + 1] = w[1];
        }
    } else if constexpr (D == DT_I8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 PGEMM_LDS*)(bs + b_frag_off<C>(ks, j, wn0, lane, h)));
            out[2 * h] = w[0];
            out[2 * h + 1] = w[1];
        }
    } else {
#pragma unroll
        for (int jm = 0; jm < 4; ++jm) out[jm] = *(const int PGEMM_LDS*)(bs + b_frag_off<C>(ks, j, wn0, lane, jm));
    }
}

template <class C>
__device__ __forceinline__ void read_frags(const char PGEMM_LDS* stage, int ks, int wm0, int wn0, int lane,
                                           Frags<C>& f) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) read_a<C>(stage, ks, i, wm0, lane, f.a[i]);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) read_b<C>(stage, ks, j, wn0, lane, f.b[j]);
}

// The r-th fragment read of a K step, in the order the MFMAs consume them
// (MFMA blocks run row-major: block (i, j) needs a[i] and b[j]):
// b0, a0, b1 .. b(FN-1), a1 .. a(FM-1).
template <class C>
__device__ __forceinline__ void read_item(const char PGEMM_LDS* stage, int ks, int r, int wm0, int wn0, int lane,
                                          Frags<C>& f) {
    if (r == 0) {
        read_b<C>(stage, ks, 0, wn0, lane, f.b[0]);
    } else if (r == 1) {
        read_a<C>(stage, ks, 0, wm0, lane, f.a[0]);
    } else if (r <= C::FN) {
        read_b<C>(stage, ks, r - 1, wn0, lane, f.b[r - 1]);
    } else {
        read_a<C>(stage, ks, r - C::FN, wm0, lane, f.a[r - C::FN]);
    }
}

// Whether fragment read item r (read_item's order: items 0 and 2 .. FN are B
// fragments, the others A) belongs to a part the build runs.
template <class C>
PGEMM_HD constexpr bool item_in_parts(int r) {
    const bool is_b = r == 0 || (r >= 2 && r <= C::FN);
    return (C::PARTS & (is_b ? PART_BREADS : PART_AREADS)) != 0;
}

template <class C>
__device__ __forceinline__ void mfma_block(typename C::T::Acc& acc, const i32x4& a, const i32x4& b) {
    constexpr int D = C::Dt;
    if constexpr (D == DT_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                      acc, 0, 0, 0);
    } else if constexpr (D == DT_F16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc,
                                                     0, 0, 0);
    } else if constexpr (D == DT_I8) {
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
    } else {
        // Bit-cast whole vectors, then index: hipcc (clang 22) lowers
        // __builtin_bit_cast(float, v[i]) of an int vector element to element 0
        // for every i, which silently fed the first k of the chunk to all four
        // MFMAs.
        const f32x4 af = __builtin_bit_cast(f32x4, a);
        const f32x4 bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
        for (int jm = 0; jm < 4; ++jm) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[jm], bf[jm], acc, 0, 0, 0);
    }
}

template <class C>
__device__ __forceinline__ void mfma_all(typename C::T::Acc (&acc)[C::FM][C::FN], const Frags<C>& f) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mfma_block<C>(acc[i][j], f.a[i], f.b[j]);
}

// ---- stage protocol -------------------------------------------------------------

// The MFMA work of one K step, cut into (up to) eight groups.  After each of
// the first C::DMA_GROUPS groups: a share of the producer's work (LDS-DMA
// blocks of the tile being issued); after every group: a share of the next
// step's fragment reads, so none of that issue time leaves the matrix pipe
// idle.  sched_barrier keeps the groups in this order.
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};

// `hook(gi)` runs after the MFMAs of group gi, before its DMA blocks: the
// register-staged producers put their stage writes and next loads there.
template <class C, bool READS, bool DMA, bool FULL = false, class Hook = NoHook>
__device__ __forceinline__ void mfma_step(typename C::T::Acc (&acc)[C::FM][C::FN], const Frags<C>& use,
                                          Frags<C>& nxt, const char PGEMM_LDS* rstage, int rks,
                                          const KernelArgs& g, const DmaTile& d, int wave, int lane, int wm0,
                                          int wn0, Hook hook = Hook{}) {
    constexpr int NMF = C::FM * C::FN;
    constexpr int NG = NMF < 8 ? NMF : 8;
    constexpr int GS = NMF / NG;
    constexpr int NR = C::FM + C::FN;
    constexpr int RPG = (NR + NG - 1) / NG;
    constexpr int NP = C::DMA_P1 - C::DMA_P0;
    constexpr int DG = C::DMA_GROUPS < NG ? C::DMA_GROUPS : NG;
    constexpr int PPG = (NP + DG - 1) / DG;  // DMA blocks per group, in the first DG groups
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
        for (int m = gi * GS; m < (gi + 1) * GS; ++m) mfma_block<C>(acc[m / C::FN][m % C::FN], use.a[m / C::FN], use.b[m % C::FN]);
        hook(gi);
        if constexpr (DMA && (C::PARTS & PART_DMA) != 0) {
#pragma unroll
            for (int p = gi * PPG; p < (gi + 1) * PPG; ++p)
                if (p < NP) dma_piece<C, FULL>(g, d, C::DMA_P0 + p, wave, lane);
        }
        if constexpr (READS) {
#pragma unroll
            for (int r = gi * RPG; r < (gi + 1) * RPG; ++r)
                if (r < NR && item_in_parts<C>(r)) read_item<C>(rstage, rks, r, wm0, wn0, lane, nxt);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Barrier of the uniform pipelined loop: every K-tile slot issues exactly
// LPS loads (real, or all-out-of-range for slots past nK), so when tile t+1
// must have landed the loads of the S-2 later slots may still be in flight.
// Register producers wait for their loads where the registers are written to
// LDS (the compiler's own vmcnt, after the barrier: each wave waits for its
// own loads only, not for the slowest wave's), so their barrier needs only
// lgkmcnt.  With one producer per operand (two stages) each slot issues its
// LDS-DMA pieces and then the register loads of the slot after it, so when
// slot t+1's pieces must have landed only those register loads may still be
// in flight: vmcnt(STAGED_LOADS), and they are waited for after the barrier.
// A workgroup barrier after s_waitcnt vmcnt(VM) lgkmcnt(0) (VM < 0: lgkmcnt
// only); in a wait-profile build, with the clock stamps described at
// ProbeCfg.  READY: the barrier is a ready edge (counted in st.n).
template <class C, int VM, bool READY = true>
__device__ __forceinline__ void probed_barrier(Staging<C>& st) {
    if constexpr (C::PROBE) {
        // the same waits, split by clock stamps: vmcnt (with lgkmcnt), then
        // the barrier; each stamp's own latency lands in the second part
        lgkm_drain();
        const long long t0 = (long long)__builtin_amdgcn_s_memtime();
        if constexpr (VM >= 0)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" : : "n"(VM) : "memory");
        else
            asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        const long long t1 = (long long)__builtin_amdgcn_s_memtime();
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
        const long long t2 = (long long)__builtin_amdgcn_s_memtime();
        st.vm += t1 - t0;
        st.bar += t2 - t1;
        if (READY && st.n == 0) st.rt_ready0 = (long long)__builtin_amdgcn_s_memrealtime();
        st.n += READY ? 1 : 0;
    } else if constexpr ((C::PARTS & PART_BARRIER) == 0) {
        // parts-ladder build without the barrier: the waits alone
        lgkm_drain();
        if constexpr (VM >= 0)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" : : "n"(VM) : "memory");
        else
            asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    } else if constexpr (VM >= 0) {
        wait_barrier<(VM >= 0 ? VM : 0)>();
    } else {
        lgkm_barrier();
    }
}

template <class C>
__device__ __forceinline__ void sync_ring(Staging<C>& st) {
    probed_barrier<C, C::P == PROD_DIRECT ? C::LPS * (C::S - 2) : C::MIXED ? C::STAGED_LOADS : -1>(st);
}

// Start of a K loop, and its end: a wait-profile build writes the wave's
// totals to g.probe[(workgroup * waves + wave) * kProbeWords + i]: i = 0
// vmcnt cycles, 1 barrier cycles, 2 ready edges, 3 shader cycles of the
// whole loop, 7 the 100 MHz time of the first ready edge (the kernel writes
// 4..6, see probe_times).
template <class C>
__device__ __forceinline__ long long probe_start() {
    if constexpr (C::PROBE) return (long long)__builtin_amdgcn_s_memtime();
    return 0;
}
template <class C>
__device__ __forceinline__ void probe_end(const KernelArgs& g, const Staging<C>& st, long long t_begin, int wave,
                                          int lane) {
    if constexpr (C::PROBE) {
        const long long t_end = (long long)__builtin_amdgcn_s_memtime();
        if (lane == 0) {
            long long* o = g.probe + ((int64_t)blockIdx.x * C::NW + wave) * kProbeWords;
            o[0] = st.vm;
            o[1] = st.bar;
            o[2] = st.n;
            o[3] = t_end - t_begin;
            o[7] = st.rt_ready0;
        }
    }
}

// Work of one workgroup and the K-tile slots it streams through the ring.
//
// Workgroups are dealt round-robin over the 8 XCDs (workgroup b runs on XCD
// b % 8, each XCD with its own L2).  The grid is a multiple of 8.  XCD x owns
// a contiguous range of logical tiles; its nl workgroups take tiles start+lb,
// start+lb+nl, ... of that range, and a grouped raster turns the range into a
// compact block of tile-rows x tile-columns, so the XCD's L2 serves the
// shared A and B panels.  With one workgroup per tile every workgroup gets one
// tile; with fewer (persistent workgroups) each one loops over its tiles.
struct WgTiles {
    int start, lb, nl, count;
};

// Tiles of workgroup b of a grid of `nb` workgroups (nb a multiple of 8) over
// G logical tiles.
PGEMM_HD WgTiles wg_tiles_of(int G, int b, int nb) {
    const int x = b & 7, lb = b >> 3, nl = nb >> 3;
    const int per = G >> 3, rem = G & 7;
    const int start = x * per + (x < rem ? x : rem);
    const int size = per + (x < rem ? 1 : 0);
    return WgTiles{start, lb, nl, lb < size ? (size - lb + nl - 1) / nl : 0};
}

// Logical tile L -> (tile row, tile column): grouped raster, group_m tile-rows
// per group, column-major inside a group.
PGEMM_HD void raster(int L, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    const int width = group_m * tiles_n;
    const int grp = L / width;
    const int first = grp * group_m;
    const int gm = (tiles_m - first < group_m) ? tiles_m - first : group_m;
    const int r = L - grp * width;
    tm = first + r % gm;
    tn = r / gm;
}

__device__ __forceinline__ WgTiles wg_tiles(const KernelArgs& g) {
    return wg_tiles_of(g.tiles_m * g.tiles_n, (int)blockIdx.x, (int)gridDim.x);
}

// Origin of this workgroup's i-th tile; past its last tile the origin is
// (M, N), so every chunk of such a slot lies outside the matrices and loads
// nothing.
template <class C>
__device__ __forceinline__ void wg_tile_origin(const KernelArgs& g, const WgTiles& w, int i, int& m0, int& n0) {
    if (i >= w.count) {
        m0 = g.M;
        n0 = g.N;
        return;
    }
    int tm, tn;
    raster(w.start + w.lb + i * w.nl, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    m0 = tm * C::BM;
    n0 = tn * C::BN;
}

// A K-tile slot to load: K tile kt of the workgroup's i-th output tile, at
// tile origin (m0, n0).  Slots run through all K tiles of one output tile,
// then the next.
struct Cursor {
    int kt, m0, n0;
};

// Cursor of absolute slot `slot` (uniform; one division, so it stays out of
// the hot loop).
template <class C>
__device__ __forceinline__ Cursor cursor_at(const KernelArgs& g, const WgTiles& w, int nK, int slot) {
    Cursor c;
    const int i = slot / nK;
    c.kt = slot - i * nK;
    wg_tile_origin<C>(g, w, i, c.m0, c.n0);
    return c;
}

// One K tile of the S >= 2 pipeline.  Fragments for K step ks+1 are read
// while the MFMAs of step ks run; for the tile's last step the next reads
// belong to the next slot, so barrier B_{s+1} and the producer's issue sit
// right before them -- after the last LDS reads of slot s and before its last
// MFMAs.  The body is the same for every slot: slots past the workgroup's
// last K tile load nothing (every lane out of range, zeros land in a stage
// nobody reads), so the loop has no drain branches and the wait count is a
// constant.  `dc` is the slot whose LDS-DMA pieces are issued now (s+S), `rc`
// the slot loaded into registers now (s+S+1: the registers hold one more K
// tile, slot s+S, which is written to the freed stage right after the
// barrier).  PAR is the fragment buffer holding step 0 of this slot.
template <class C, int PAR, bool FULL = false>
__device__ __forceinline__ void tile_body(const KernelArgs& g, const Cursor& dc, const Cursor& rc, int s,
                                          char PGEMM_LDS* smem, int& cur, Staging<C>& st, Frags<C> (&f)[2],
                                          typename C::T::Acc (&acc)[C::FM][C::FN], int wave, int lane, int wm0,
                                          int wn0) {
    constexpr int NKS = C::BK / C::KSTEP;
    const char PGEMM_LDS* cstage = smem + cur * C::STAGE_BYTES;
    const int nstage = (cur + 1 == C::S) ? 0 : cur + 1;
    const DmaTile none{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        Frags<C>& use = f[(PAR + ks) & 1];
        Frags<C>& nxt = f[(PAR + ks + 1) & 1];
        if (ks + 1 < NKS) {
            mfma_step<C, true, false>(acc, use, nxt, cstage, ks + 1, g, none, wave, lane, wm0, wn0);
        } else {
            sync_ring<C>(st);  // B_{s+1}: slot s+1 ready, stage of slot s free
            debug_skew(g, s, wave, C::NW);
            const char PGEMM_LDS* rstage = smem + nstage * C::STAGE_BYTES;
            char PGEMM_LDS* freed = smem + cur * C::STAGE_BYTES;
            // The LDS-DMA descriptors of slot s+S are formed after the
            // barrier: formed before it (measured), they delay the last wave
            // to arrive, whose arrival sets the K tile's period, and the
            // loop ran 1 % slower.
            const DmaTile d = C::ANY_DMA ? dma_setup<C>(g, dc.m0, dc.n0, dc.kt, freed, wave) : none;
            if constexpr (C::ANY_STAGED) {
                // Spread over the MFMA groups: after group 0 the staged
                // operand of slot s+S (in registers since B_s) is written to
                // the freed stage, then the LDS-DMA pieces of slot s+S (if
                // any) follow in the first groups, and after group REG_GROUP
                // the register loads of slot s+S+1 -- behind every piece, so
                // the next barrier waits for the pieces only.
                auto staged = [&](int gi) {
                    if (gi == 0) store_tile<C>(freed, st, wave, lane);
                    if (gi == C::REG_GROUP) issue_regs<C>(g, rc.m0, rc.n0, rc.kt, st, wave, lane);
                };
                mfma_step<C, true, C::ANY_DMA, FULL>(acc, use, nxt, rstage, 0, g, d, wave, lane, wm0, wn0, staged);
            } else {
                mfma_step<C, true, true, FULL>(acc, use, nxt, rstage, 0, g, d, wave, lane, wm0, wn0);  // slot s+S
            }
            // slot s+S holds the end of a K that is not whole chunks: its
            // straddling A chunks are completed after the pieces
            if constexpr (!FULL && C::P == PROD_DIRECT) {
                if (tail_tile<C>(g, dc.kt)) dma_patch<C>(g, dc.m0, dc.kt, freed, wave, lane);
            }
        }
    }
    cur = nstage;
}

template <class C>
__device__ __forceinline__ void zero_acc(typename C::T::Acc (&acc)[C::FM][C::FN]) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = typename C::T::Acc{0, 0, 0, 0};
}

template <class C>
__device__ __forceinline__ void store_c(const KernelArgs& g, int m0, int n0, int wm0, int wn0, int lane,
                                        typename C::T::Acc (&acc)[C::FM][C::FN]);

// The S >= 2 pipeline of one output tile: prologue, steady state, drain.
// The slots to load are LA_DMA = S K tiles ahead for LDS-DMA pieces and
// LA_REG = S+1 for register-staged operands; past the last K tile those lie
// beyond K, so every lane is out of range and the slot loads nothing.
template <class C>
__device__ __forceinline__ void pertile_loop(const KernelArgs& g, int m0, int n0, int nK, char PGEMM_LDS* smem,
                                             typename C::T::Acc (&acc)[C::FM][C::FN], int wave, int lane, int wm0,
                                             int wn0) {
    constexpr int NKS = C::BK / C::KSTEP;
    constexpr int LD = C::LA_DMA, LR = C::LA_REG;
    Staging<C> st;
    Frags<C> f[2];
    const long long t_begin = probe_start<C>();
    // Prologue: K tiles 0 .. S-2 into stages 0 .. S-2.
#pragma unroll
    for (int p = 0; p < C::S - 1; ++p) {
        if constexpr (C::ANY_STAGED) issue_regs<C>(g, m0, n0, p, st, wave, lane);
        if constexpr (C::ANY_DMA) issue_dma<C>(g, m0, n0, p, smem + p * C::STAGE_BYTES, wave, lane);
        if constexpr (C::ANY_STAGED) store_tile<C>(smem + p * C::STAGE_BYTES, st, wave, lane);
    }
    if constexpr (C::ANY_STAGED) issue_regs<C>(g, m0, n0, C::S - 1, st, wave, lane);
    sync_ring<C>(st);  // B_0
    if constexpr ((C::PARTS & PART_BARRIER) == 0) lgkm_barrier();  // parts build: the prologue keeps its barrier
    // Stage S-1 has never been used: K tile S-1 goes there now (the staged
    // operand from registers, then the LDS-DMA pieces), then K tile S into
    // registers -- the order of every slot of the loop.
    if constexpr (C::ANY_STAGED) store_tile<C>(smem + (C::S - 1) * C::STAGE_BYTES, st, wave, lane);
    if constexpr (C::ANY_DMA) issue_dma<C>(g, m0, n0, C::S - 1, smem + (C::S - 1) * C::STAGE_BYTES, wave, lane);
    if constexpr (C::ANY_STAGED) issue_regs<C>(g, m0, n0, C::S, st, wave, lane);
    read_frags<C>(smem, 0, wm0, wn0, lane, f[0]);
    // Parts build without some fragment reads: both fragment buffers start
    // from operand data (K steps 0 and 1 of the first K tile), so the steps
    // that keep stale fragments still multiply operand values, never
    // uninitialised registers.
    if constexpr (C::PARTS != PART_ALL) read_frags<C>(smem, 1 % NKS, wm0, wn0, lane, f[1]);
    int cur = 0;
    // Slots t < nfull load a whole K tile of a whole output tile by LDS-DMA
    // (issued without per-lane range selects); the rest, up to LD + 1 of
    // them, take the general path.
    const bool whole = C::ANY_DMA && (!C::A_DMA || m0 + C::BM <= g.M) && (!C::B_DMA || n0 + C::BN <= g.N);
    const int nfull = whole && g.K / C::BK > LD ? g.K / C::BK - LD : 0;
    if constexpr (NKS % 2 == 0) {
        int t = 0;
        for (; t < nfull; ++t)
            tile_body<C, 0, true>(g, Cursor{t + LD, m0, n0}, Cursor{t + LR, m0, n0}, t, smem, cur, st, f, acc, wave,
                                  lane, wm0, wn0);
        for (; t < nK; ++t)
            tile_body<C, 0>(g, Cursor{t + LD, m0, n0}, Cursor{t + LR, m0, n0}, t, smem, cur, st, f, acc, wave, lane,
                            wm0, wn0);
    } else {
        int t = 0;
        for (; t + 1 < nfull; t += 2) {
            tile_body<C, 0, true>(g, Cursor{t + LD, m0, n0}, Cursor{t + LR, m0, n0}, t, smem, cur, st, f, acc, wave,
                                  lane, wm0, wn0);
            tile_body<C, 1, true>(g, Cursor{t + 1 + LD, m0, n0}, Cursor{t + 1 + LR, m0, n0}, t + 1, smem, cur, st, f,
                                  acc, wave, lane, wm0, wn0);
        }
        for (; t + 1 < nK; t += 2) {
            tile_body<C, 0>(g, Cursor{t + LD, m0, n0}, Cursor{t + LR, m0, n0}, t, smem, cur, st, f, acc, wave, lane,
                            wm0, wn0);
            tile_body<C, 1>(g, Cursor{t + 1 + LD, m0, n0}, Cursor{t + 1 + LR, m0, n0}, t + 1, smem, cur, st, f, acc,
                            wave, lane, wm0, wn0);
        }
        if (t < nK)
            tile_body<C, 0>(g, Cursor{t + LD, m0, n0}, Cursor{t + LR, m0, n0}, t, smem, cur, st, f, acc, wave, lane,
                            wm0, wn0);
    }
    // No load may still be writing LDS when the workgroup retires.
    __builtin_amdgcn_s_waitcnt(0);
    probe_end<C>(g, st, t_begin, wave, lane);
}

// The S >= 2 pipeline over all K-tile slots of the workgroup's tiles: one
// ring, one prologue, one drain.  A workgroup with one tile runs exactly the
// per-tile pipeline; with several, tile j+1's first K tiles load while tile
// j's last ones are multiplied and stored.
//
// Each output tile's K loop has two phases.  In phase A every slot to load
// (LA_DMA and LA_REG slots ahead) lies in the same output tile, so its
// cursor is plain arithmetic: this is the hot loop.  Phase B covers the last
// LA slots, whose loads belong to later tiles.
template <class C>
__device__ __forceinline__ void stream_loop(const KernelArgs& g, const WgTiles& w, int nK, char PGEMM_LDS* smem,
                                            typename C::T::Acc (&acc)[C::FM][C::FN], int wave, int lane, int wm0,
                                            int wn0) {
    constexpr int NKS = C::BK / C::KSTEP;
    constexpr int LD = C::LA_DMA, LR = C::LA_REG;
    constexpr int LA = C::ANY_STAGED ? LR : LD;
    Staging<C> st;
    Frags<C> f[2];
    const long long t_begin = probe_start<C>();
    // Prologue: slots 0 .. S-2 into stages 0 .. S-2.
#pragma unroll
    for (int p = 0; p < C::S - 1; ++p) {
        const Cursor c = cursor_at<C>(g, w, nK, p);
        if constexpr (C::ANY_STAGED) issue_regs<C>(g, c.m0, c.n0, c.kt, st, wave, lane);
        if constexpr (C::ANY_DMA) issue_dma<C>(g, c.m0, c.n0, c.kt, smem + p * C::STAGE_BYTES, wave, lane);
        if constexpr (C::ANY_STAGED) store_tile<C>(smem + p * C::STAGE_BYTES, st, wave, lane);
    }
    if constexpr (C::ANY_STAGED) {
        const Cursor c = cursor_at<C>(g, w, nK, C::S - 1);
        issue_regs<C>(g, c.m0, c.n0, c.kt, st, wave, lane);  // slot S-1 into registers
    }
    sync_ring<C>(st);  // B_0
    // Stage S-1 has never been used: slot S-1 goes there now (the staged
    // operand from registers, then the LDS-DMA pieces), then slot S into
    // registers -- the order of every slot of the loop.
    if constexpr (C::ANY_STAGED) store_tile<C>(smem + (C::S - 1) * C::STAGE_BYTES, st, wave, lane);
    if constexpr (C::ANY_DMA) {
        const Cursor c = cursor_at<C>(g, w, nK, C::S - 1);
        issue_dma<C>(g, c.m0, c.n0, c.kt, smem + (C::S - 1) * C::STAGE_BYTES, wave, lane);
    }
    if constexpr (C::ANY_STAGED) {
        const Cursor c = cursor_at<C>(g, w, nK, C::S);
        issue_regs<C>(g, c.m0, c.n0, c.kt, st, wave, lane);  // slot S into registers
    }
    read_frags<C>(smem, 0, wm0, wn0, lane, f[0]);
    int cur = 0;
    // Outer loop: the workgroup's output tiles (epilogue between them); the
    // ring and the look-ahead fragments carry over from tile to tile.
    for (int i = 0; i < w.count; ++i) {
        const int s0 = i * nK;
        int m0, n0;
        wg_tile_origin<C>(g, w, i, m0, n0);
        const int nA = nK > LA ? nK - LA : 0;
        // phase B cursors: the slot LD (LR) ahead of slot s0 + kt, in whatever
        // output tile it falls
        auto dc_at = [&](int kt) { return C::ANY_DMA ? cursor_at<C>(g, w, nK, s0 + kt + LD) : Cursor{0, 0, 0}; };
        auto rc_at = [&](int kt) { return C::ANY_STAGED ? cursor_at<C>(g, w, nK, s0 + kt + LR) : Cursor{0, 0, 0}; };
        int kt = 0;
        if constexpr (NKS % 2 == 0) {
            for (; kt < nA; ++kt)
                tile_body<C, 0>(g, Cursor{kt + LD, m0, n0}, Cursor{kt + LR, m0, n0}, s0 + kt, smem, cur, st, f, acc,
                                wave, lane, wm0, wn0);
            for (; kt < nK; ++kt)
                tile_body<C, 0>(g, dc_at(kt), rc_at(kt), s0 + kt, smem, cur, st, f, acc, wave, lane, wm0, wn0);
        } else {
            // Pairs of slots keep the fragment buffers' roles fixed at the
            // back edge of the hot loop (one buffer live between slots).
            for (; kt + 1 < nA; kt += 2) {
                tile_body<C, 0>(g, Cursor{kt + LD, m0, n0}, Cursor{kt + LR, m0, n0}, s0 + kt, smem, cur, st, f, acc,
                                wave, lane, wm0, wn0);
                tile_body<C, 1>(g, Cursor{kt + 1 + LD, m0, n0}, Cursor{kt + 1 + LR, m0, n0}, s0 + kt + 1, smem, cur,
                                st, f, acc, wave, lane, wm0, wn0);
            }
            // The rest (at most LA + 1 slots): one slot at a time, the look-ahead
            // fragments moved back to buffer 0 after each, so a single buffer
            // is live at every join.
            for (; kt < nK; ++kt) {
                const Cursor dc = kt < nA ? Cursor{kt + LD, m0, n0} : dc_at(kt);
                const Cursor rc = kt < nA ? Cursor{kt + LR, m0, n0} : rc_at(kt);
                tile_body<C, 0>(g, dc, rc, s0 + kt, smem, cur, st, f, acc, wave, lane, wm0, wn0);
                f[0] = f[1];
            }
        }
        // Fused alpha/beta epilogue; the loads of the next tile's first slots
        // are already in flight.
        store_c<C>(g, m0, n0, wm0, wn0, lane, acc);
        zero_acc<C>(acc);
    }
    // No load may still be writing LDS when the workgroup retires.
    __builtin_amdgcn_s_waitcnt(0);
    probe_end<C>(g, st, t_begin, wave, lane);
}

// MFMA work on one stage with the fragments of step ks+1 read under step ks.
template <class C>
__device__ __forceinline__ void compute_stage(const char PGEMM_LDS* stage, int wm0, int wn0, int lane,
                                              typename C::T::Acc (&acc)[C::FM][C::FN]) {
    constexpr int NKS = C::BK / C::KSTEP;
    Frags<C> f[2];
    read_frags<C>(stage, 0, wm0, wn0, lane, f[0]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (ks > 0) lgkm_drain();
        if (ks + 1 < NKS) read_frags<C>(stage, ks + 1, wm0, wn0, lane, f[(ks + 1) & 1]);
        mfma_all<C>(acc, f[ks & 1]);
    }
}

// Single LDS buffer.  DIRECT: load, wait, barrier, compute, barrier (nothing
// of the load overlaps the arithmetic).  REGISTER/GENERIC: tile t+1 is
// prefetched into registers before the arithmetic on tile t and written after
// the second barrier.
template <class C>
__device__ __forceinline__ void single_buffer_loop(const KernelArgs& g, int m0, int n0, int nK, char PGEMM_LDS* smem,
                                                   typename C::T::Acc (&acc)[C::FM][C::FN], int wave, int lane,
                                                   int wm0, int wn0) {
    Staging<C> st;
    const long long t_begin = probe_start<C>();
    if constexpr (C::P == PROD_DIRECT) {
        for (int t = 0; t < nK; ++t) {
            issue_tile<C>(g, m0, n0, t, smem, st, wave, lane);
            probed_barrier<C, 0>(st);          // ready
            debug_skew(g, t, wave, C::NW);
            compute_stage<C>(smem, wm0, wn0, lane, acc);
            probed_barrier<C, -1, false>(st);  // reuse
        }
    } else {
        issue_tile<C>(g, m0, n0, 0, smem, st, wave, lane);
        store_tile<C>(smem, st, wave, lane);
        for (int t = 0; t < nK; ++t) {
            probed_barrier<C, -1>(st);  // ready
            debug_skew(g, t, wave, C::NW);
            const bool more = t + 1 < nK;
            if (more) issue_tile<C>(g, m0, n0, t + 1, smem, st, wave, lane);
            compute_stage<C>(smem, wm0, wn0, lane, acc);
            probed_barrier<C, -1, false>(st);  // reuse
            if (more) store_tile<C>(smem, st, wave, lane);
        }
    }
    probe_end<C>(g, st, t_begin, wave, lane);
}

// ---- epilogue: C = alpha*acc + beta*C (fused, as in the pages' kernel) -------------

// The wave's block of C starts at a uniform address; a lane's element sits at
// a 32-bit offset from it (row 4*lg + 16*i + r, column li + 16*j), split into
// a uniform row part, one per-lane part and an immediate column part, so the
// epilogue holds one address register per lane rather than one per row.
// Byte offsets stay below 2^31 because ldc * 4 * 256 < 2^31 (checked on the
// host).
//
// With beta != 0 the old C is read one 16-row block (i) at a time: all reads
// of a block in flight together, then the block is combined and written.  A
// bounded number of registers (the next tile's fragments may be live here)
// and no serialised read-wait-write per element.  MASK: the tile is cut by the edge
// of C; the bounds are compared in a lane-invariant form (4*lg against a
// uniform limit) so no per-row lane values have to stay live.
template <class C, bool MASK, bool BETA>
__device__ __forceinline__ void store_c_impl(const KernelArgs& g, int m0, int n0, int wm0, int wn0, int lane,
                                             typename C::T::Acc (&acc)[C::FM][C::FN]) {
    using E = typename C::T::Out;
    const int li = lane & 15, lg4 = 4 * (lane >> 4);
    const int rows_left = g.M - m0 - wm0, n_left = g.N - n0 - wn0;
    const int ldc4 = (int)g.ldc * 4;
    char* cw = (char*)g.C + ((int64_t)(m0 + wm0) * g.ldc + n0 + wn0) * 4;
    const uint32_t voff = (uint32_t)(lg4 * ldc4 + 4 * li);
    auto at = [&](int i, int r, int j) -> E* { return (E*)(cw + (uint32_t)((16 * i + r) * ldc4) + voff) + 16 * j; };
    auto inside = [&](int i, int r, int j) -> bool {
        return !MASK || (lg4 < rows_left - 16 * i - r && li < n_left - 16 * j);
    };
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        E old[4][C::FN];
        if constexpr (BETA) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < C::FN; ++j) old[r][j] = inside(i, r, j) ? *at(i, r, j) : E(0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                if (!inside(i, r, j)) continue;
                if constexpr (C::Dt == DT_I8) {
                    uint32_t v = (uint32_t)g.ialpha * (uint32_t)acc[i][j][r];
                    if constexpr (BETA) v += (uint32_t)g.ibeta * (uint32_t)old[r][j];
                    *at(i, r, j) = (int)v;
                } else {
                    float v = g.alpha * acc[i][j][r];
                    if constexpr (BETA) v = fmaf(g.beta, old[r][j], v);
                    *at(i, r, j) = v;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <class C>
__device__ __forceinline__ void store_c(const KernelArgs& g, int m0, int n0, int wm0, int wn0, int lane,
                                        typename C::T::Acc (&acc)[C::FM][C::FN]) {
    const bool full = m0 + C::BM <= g.M && n0 + C::BN <= g.N;
    if (g.beta_nonzero) {
        if (full)
            store_c_impl<C, false, true>(g, m0, n0, wm0, wn0, lane, acc);
        else
            store_c_impl<C, true, true>(g, m0, n0, wm0, wn0, lane, acc);
    } else {
        if (full)
            store_c_impl<C, false, false>(g, m0, n0, wm0, wn0, lane, acc);
        else
            store_c_impl<C, true, false>(g, m0, n0, wm0, wn0, lane, acc);
    }
}

// ---- the kernel -------------------------------------------------------------------------

// STREAM = false: one output tile per workgroup (the launch gives every
// workgroup at most one tile), the per-tile pipeline with the epilogue after
// it.  STREAM = true: persistent workgroups, one ring across all their tiles.
template <class C, bool STREAM>
__global__ void __launch_bounds__(C::NT) gemm_kernel(KernelArgs g) {
    __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
    char PGEMM_LDS* smem = (char PGEMM_LDS*)smem_raw;

    const long long rt_start = C::PROBE || C::CLOCK ? (long long)__builtin_amdgcn_s_memrealtime() : 0;
    const long long cy_start = C::CLOCK ? (long long)__builtin_amdgcn_s_memtime() : 0;
    const WgTiles w = wg_tiles(g);
    if (w.count == 0) return;  // more workgroups than tiles in this XCD's range
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm0 = (wave / C::WGN) * C::WM;
    const int wn0 = (wave % C::WGN) * C::WN;
    const int nK = (g.K + C::BK - 1) / C::BK;

    typename C::T::Acc acc[C::FM][C::FN];
    zero_acc<C>(acc);

    if constexpr (STREAM && C::S > 1) {
        if (nK > 0) {
            stream_loop<C>(g, w, nK, smem, acc, wave, lane, wm0, wn0);
            return;
        }
    }
    if constexpr (!STREAM) {
        int m0, n0;
        wg_tile_origin<C>(g, w, 0, m0, n0);
        if (nK > 0) {
            if constexpr (C::S == 1)
                single_buffer_loop<C>(g, m0, n0, nK, smem, acc, wave, lane, wm0, wn0);
            else
                pertile_loop<C>(g, m0, n0, nK, smem, acc, wave, lane, wm0, wn0);
        }
        const long long rt_loop = C::PROBE ? (long long)__builtin_amdgcn_s_memrealtime() : 0;
        store_c<C>(g, m0, n0, wm0, wn0, lane, acc);
        if constexpr (C::CLOCK) {
            // parts-ladder build: wave 0's clocks at its start and after its stores
            __builtin_amdgcn_s_waitcnt(0);
            const long long cy_end = (long long)__builtin_amdgcn_s_memtime();
            const long long rt_end = (long long)__builtin_amdgcn_s_memrealtime();
            if (wave == 0 && lane == 0) {
                long long* o = g.probe + (int64_t)blockIdx.x * kClockWords;
                o[0] = cy_start;
                o[1] = rt_start;
                o[2] = cy_end;
                o[3] = rt_end;
            }
        }
        if constexpr (C::PROBE) {
            // the wave's timeline on the 100 MHz clock: start, end of the K
            // loop, and its C stores complete
            __builtin_amdgcn_s_waitcnt(0);
            const long long rt_end = (long long)__builtin_amdgcn_s_memrealtime();
            if (lane == 0) {
                long long* o = g.probe + ((int64_t)blockIdx.x * C::NW + wave) * kProbeWords;
                o[4] = rt_start;
                o[5] = rt_loop;
                o[6] = rt_end;
            }
        }
    } else {
        // Persistent with one ring slot (S = 1), or K = 0: tile by tile.
        for (int i = 0; i < w.count; ++i) {
            int m0, n0;
            wg_tile_origin<C>(g, w, i, m0, n0);
            if constexpr (C::S == 1) {
                if (nK > 0) single_buffer_loop<C>(g, m0, n0, nK, smem, acc, wave, lane, wm0, wn0);
            }
            store_c<C>(g, m0, n0, wm0, wn0, lane, acc);
            zero_acc<C>(acc);
        }
    }
}

}  // namespace pgemm
