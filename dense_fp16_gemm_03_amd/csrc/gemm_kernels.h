// Kernel configurations and launch entry points of the gfx950 GEMM kernels.
// Host code (gemm_api.cpp) picks a configuration and a schedule; the kernels
// in gemm_kernels.hip run it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_schedule.h"

namespace g16 {

// Tiled MFMA kernel variants: macro tile BM x BN, k-tile BK, ring depth
// STAGES, and a WGM x WGN grid of waves (each wave owns BM/WGM x BN/WGN).
enum KernelId : int32_t {
  KID_256x256x64_S2_W4 = 0,
  KID_256x256x32_S4_W4 = 1,
  KID_256x256x64_S2_W8 = 2,
  KID_256x128x64_S3_W4 = 3,
  KID_128x128x64_S4_W4 = 4,
  KID_128x64x64_S4_W4 = 5,
  KID_64x64x64_S4_W4 = 6,
  KID_256x256x32_S5_W4 = 7,
  KID_256x256x32_S4_W8 = 8,
  KID_256x256x32_S5_W8 = 9,
  KID_COUNT = 10,
  KID_GENERAL = 100  // any shape and alignment, 64 x 64 tiles, no LDS
};

struct KernelInfo {
  int32_t bm, bn, bk, stages, waves;
  int32_t lds_bytes;
  const char* name;
};

// Static description of a tiled kernel id (nullptr for unknown ids).
const KernelInfo* kernel_info(int32_t kid);

typedef float f32x4_storage __attribute__((ext_vector_type(4)));

struct GemmParams {
  const uint16_t* A;
  const uint16_t* B;
  float* C;
  f32x4_storage* partials;  // [tiles][s.slots] partial tiles (split-K / stream-K only)
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t c_vec4;  // C base and ldc allow 16-byte stores
  Sched s;
};

// Launches the tiled kernel `kid` with p.s.grid workgroups on `stream`, and
// for split-K / stream-K schedules the reduce pass after it.
hipError_t launch_tiled(int32_t kid, const GemmParams& p, hipStream_t stream);

// Launches the general kernel over ceil(M/64) x ceil(N/64) workgroups.
hipError_t launch_general(const GemmParams& p, hipStream_t stream);

// Workgroups of kernel `kid` that fit on one CU at once (0 on error).
int32_t tiled_occupancy(int32_t kid);

}  // namespace g16
