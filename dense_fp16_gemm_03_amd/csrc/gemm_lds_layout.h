// LDS layout of an operand tile row, shared by the kernels and by the host
// test hook gemm_f16_lds_chunk (the same code on both sides, so the CPU tests
// check what the kernels use).
#pragma once

#include "gemm_schedule.h"  // G16_HD

namespace g16 {

// Position of logical 16-byte chunk `chunk` of tile row `row` inside the row.
// A fragment read puts lane l on row l % DIM, chunk l / DIM of its k-step
// (DIM = 32 or 16, the MFMA block height). On gfx950 the LDS serves a
// ds_read_b128 in four passes of 16 lanes, and the passes are not runs of
// consecutive lanes: measured, one pass holds lanes 0-3, 12-15, 20-23 and
// 24-27, another 4-11, 16-19 and 28-31 (and the same two sets shifted by
// 32). With 64 banks of 4 bytes a pass is conflict-free when its 16 lanes
// land in 16 different 16-byte bank groups; each f below is one-to-one where
// that requires it (checked on the host, through gemm_f16_lds_chunk, for
// every pass, k-step and block row of every kernel's tile).
//   DIM 32, 128-byte rows: f = (row ^ (row >> 3)) & 7
//   DIM 32,  64-byte rows: f = (row >> 2) & 3
//   DIM 16, 128-byte rows: f = (row >> 1) & 7
//   DIM 16,  64-byte rows: f = ((row >> 2) ^ ((row >> 1) & 2)) & 3
template <int CHUNKS, int DIM>
G16_HD int swz(int row, int chunk) {
  if constexpr (DIM == 32) {
    if constexpr (CHUNKS == 8) return chunk ^ ((row ^ (row >> 3)) & 7);
    else return chunk ^ ((row >> 2) & 3);
  } else {
    if constexpr (CHUNKS == 8) return chunk ^ ((row >> 1) & 7);
    else return chunk ^ (((row >> 2) ^ ((row >> 1) & 2)) & 3);
  }
}

}  // namespace g16
