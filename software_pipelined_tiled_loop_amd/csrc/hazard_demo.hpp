// Index functions of the consume-before-reuse hazard demonstrator (page
// "Software pipelines and asynchronous copies", section "Practice"): a
// two-stage tiled copy-and-reduce of an int32 array into row sums.  Shared by
// the kernel (hazard_demo.hip) and the host emulator, which checks by brute
// force that every address stays inside its buffer.
//
// A workgroup of 4 waves owns RB = 16 rows.  Column tile t (TC = 256 int32)
// of those rows is 1024 16-byte chunks: chunk c holds row c / 64, columns
// 4*(c % 64) .. +3, and lives at index c of an LDS stage.  Thread tid
// produces chunks tid + 256*j (j = 0..3), so each wave writes rows of every
// other wave; wave w consumes rows 4w .. 4w+3, lane l the chunk at column 4l.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#define HAZARD_HD __host__ __device__ __forceinline__

namespace hazard {

constexpr int RB = 16;                       // rows per workgroup
constexpr int TC = 256;                      // columns per tile
constexpr int NTH = 256;                     // threads per workgroup
constexpr int NWAVE = NTH / 64;              // 4 waves
constexpr int CH_PER_ROW = TC / 4;           // 16-byte chunks per tile row
constexpr int CHUNKS = RB * CH_PER_ROW;      // chunks per tile (one LDS stage)
constexpr int CPT = CHUNKS / NTH;            // chunks each thread produces
constexpr int ROWS_PER_WAVE = RB / NWAVE;    // rows each wave reduces
constexpr int EV = 6;                        // timeline stamps per wave and tile

HAZARD_HD int prod_chunk(int tid, int j) { return tid + NTH * j; }
HAZARD_HD int chunk_row(int c) { return c / CH_PER_ROW; }
HAZARD_HD int chunk_col(int c) { return (c % CH_PER_ROW) * 4; }
HAZARD_HD int cons_chunk(int wave, int lane, int rr) { return (ROWS_PER_WAVE * wave + rr) * CH_PER_ROW + lane; }
// Element offset of a chunk of tile t from the workgroup's first row.
HAZARD_HD int64_t x_offset(int64_t ldx, int row, int t, int col) {
    return (int64_t)row * ldx + (int64_t)t * TC + col;
}
HAZARD_HD int64_t trace_index(int wave, int nT, int t, int e) { return ((int64_t)wave * nT + t) * EV + e; }

}  // namespace hazard
