// Kernel configurations and launch entry points of the gfx950 GEMM kernels.
// Host code (gemm_api.cpp) picks a configuration and a schedule; the kernels
// in gemm_kernels.hip run it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_f16.h"
#include "gemm_schedule.h"

namespace g16 {

// Tiled MFMA kernel variants: macro tile BM x BN, k-tile BK, ring depth
// STAGES, a WGM x WGN grid of waves (each wave owns BM/WGM x BN/WGN) and the
// MFMA shape (32: v_mfma_f32_32x32x16_f16, 16: v_mfma_f32_16x16x32_f16).
// X(id, enum name, BM, BN, BK, STAGES, WGM, WGN, MFMA, RS, PP); RS 1 issues
// each next-k-step fragment read right after the last use of the one it
// replaces; PP 1 selects the ping-pong main loop (two wave groups, one
// computing while the other reads LDS and issues loads), PP 2 its form with
// two stages 64 wide in k (whole 128-byte rows per load), PP 3 its form with
// the A and B halves of 64-wide stages in STAGES separate slots (five 32 KiB
// slots: two and a half stages).
// Built: the kernels the shape rule picks (16, 18, 27, 37, 38) and three the
// plan override can select for comparisons on the same schedule: 35, the
// two-stage form of 37's loop, and 28 and 36, the v_mfma_f32_32x32x16_f16
// forms of the two ping-pong loops. Ids are stable: a removed variant's id is
// never reused.
#define G16_TILED_KERNELS(X)                                           \
  X(16, KID_128x128x64_S4_W4_M16, 128, 128, 64, 4, 2, 2, 16, 0, 0)     \
  X(18, KID_64x64x64_S4_W4_M16, 64, 64, 64, 4, 2, 2, 16, 0, 0)         \
  X(27, KID_256x256x32_S3_W8_M16_PP, 256, 256, 32, 3, 2, 4, 16, 0, 1)  \
  X(28, KID_256x256x32_S5_W8_PP, 256, 256, 32, 5, 2, 4, 32, 0, 1)      \
  X(35, KID_256x256x64_S2_W8_M16_PP, 256, 256, 64, 2, 2, 4, 16, 0, 2)  \
  X(36, KID_256x256x64_S2_W8_PP, 256, 256, 64, 2, 2, 4, 32, 0, 2)      \
  X(37, KID_256x256x64_H5_W8_M16_PP, 256, 256, 64, 5, 2, 4, 16, 0, 3)  \
  X(38, KID_32x32x64_S5_W4_M16, 32, 32, 64, 5, 2, 2, 16, 0, 0)

// Kernel ids also built for bfloat16 operands (the shape rule's picks).
#define G16_BF16_KERNELS(X) X(16) X(18) X(27) X(37) X(38)

// Operand element types.
enum DType : int32_t { DT_F16 = 0, DT_BF16 = 1 };

#define G16_KID_ENUM(id, name, ...) name = id,
enum KernelId : int32_t {
  G16_TILED_KERNELS(G16_KID_ENUM)
  KID_COUNT = 39,  // one past the largest id (ids in between may be unused)
  KID_GENERAL = 100,  // any shape and alignment, 64 x 64 tiles, no LDS
  KID_DIRECT = 101    // 16 x 16 tiles, one wave each, no LDS (operands loadable directly)
};
#undef G16_KID_ENUM

struct KernelInfo {
  int32_t bm, bn, bk, stages, waves;
  int32_t lds_bytes;
  int32_t mfma;  // 32 or 16 (MFMA block size)
  const char* name;
};

// Static description of a tiled kernel id (nullptr for unknown ids).
const KernelInfo* kernel_info(int32_t kid);

typedef float f32x4_storage __attribute__((ext_vector_type(4)));

struct GemmParams {
  const uint16_t* A;  // binary16 or bfloat16 bit patterns
  const uint16_t* B;
  float* C;
  f32x4_storage* partials;  // [tiles][s.slots] partial tiles (split-K / stream-K only)
  int64_t lda, ldb, ldc;
  int32_t M, N, K;
  int32_t c_vec4;  // C base and ldc allow 16-byte stores
  Sched s;
  // Clock probe (nullptr: off). Workgroup 0 of the main kernel adds the
  // shader-clock cycles and the 100 MHz real-time ticks between its start and
  // its end to clock_probe[0] and clock_probe[1].
  unsigned long long* clock_probe;
};

// Launches the tiled kernel `kid` for operand type `dt` with p.s.grid
// workgroups on `stream`, and for split-K / stream-K schedules the reduce
// pass after it.
hipError_t launch_tiled(int32_t kid, int32_t dt, const GemmParams& p, hipStream_t stream);

// True when tiled kernel `kid` is built for operand type `dt`.
bool tiled_has(int32_t kid, int32_t dt);

// Launches the direct kernel (one 64-lane workgroup per 16x16 tile of C; A
// and B must be loadable directly: 16-byte aligned rows of a multiple of 8
// elements, K a multiple of 8).
hipError_t launch_direct(int32_t dt, const GemmParams& p, hipStream_t stream);

// Launches the general kernel over ceil(M/64) x ceil(N/64) workgroups.
hipError_t launch_general(int32_t dt, const GemmParams& p, hipStream_t stream);

// Copies `rows` rows of K 16-bit elements (row i at src + i * ld, any 2-byte
// alignment) to dst as rows of kp elements (kp = K rounded up to 8, dst
// 16-byte aligned), zero-filling elements K .. kp - 1.
hipError_t launch_pack(const uint16_t* src, int64_t ld, int32_t K, int64_t rows, int32_t kp,
                       void* dst, hipStream_t stream);

// The binary16 entry point's path with its workspace in `scratch` (a device
// buffer of scratch_bytes the library does not allocate; NULL where no device
// is current). A plan whose partial tiles need more returns GEMM_ERR_SCRATCH;
// operands that would be packed into more run the general kernel.
gemm_status_t run_in_scratch(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             const void* B, int64_t ldb, float* C, int64_t ldc, void* scratch,
                             size_t scratch_bytes, void* stream);

// Workgroups of kernel `kid` that fit on one CU at once (0 on error).
int32_t tiled_occupancy(int32_t kid);

}  // namespace g16
