/*
 * gemm_f16.h — C ABI of libgemm_f16.so: C = A * B^T on an AMD Instinct MI355X
 * (gfx950), binary16 inputs, binary32 accumulation and output.
 *
 * The operation is the one "SASS-Level Kernel Generation for Blackwell"
 * measures (section "The numbers", Setup): fp16 inputs, fp32 accumulation and
 * output, C = A B^T. Nothing here depends on PyTorch; pointers are plain
 * device (or host, where stated) addresses and sizes are element counts.
 *
 * Layouts (all row-major, elements):
 *   A : M x K binary16, element (i, k) at A[i*lda + k]      (K contiguous)
 *   B : N x K binary16, element (j, k) at B[j*ldb + k]      (K contiguous)
 *   C : M x N binary32, element (i, j) at C[i*ldc + j]
 *   C[i][j] = sum over k < K of A[i][k] * B[j][k], accumulated in binary32.
 * C is overwritten (no alpha/beta; its prior contents never matter). K = 0
 * writes zeros; M = 0 or N = 0 is a no-op.
 *
 * Execution: work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) of the current HIP device and the call returns without waiting.
 * The caller owns A, B, C and any workspace and keeps them alive until the
 * stream work finishes. The library never frees or retains caller pointers.
 * Argument errors (including a caller workspace that is too small) are
 * reported before anything is enqueued; the call may query the current
 * device first. Device faults surface at the caller's next synchronisation.
 * The library never aborts or prints.
 *
 * Plans (kernel, tile, schedule) depend only on the shape, the row strides,
 * whether each of A, B and C is 16-byte aligned, the operand type and the
 * device's compute-unit count; they are made once per such signature and
 * cached, so repeated calls pay only the argument checks and the launches.
 */
#ifndef GEMM_F16_H
#define GEMM_F16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_VALUE = 1, /* negative size, ld too small, NULL with work, C overlaps A/B */
  GEMM_ERR_NOT_SUPPORTED = 2, /* shape/alignment outside what any kernel here handles */
  GEMM_ERR_HIP = 3,           /* a HIP runtime call failed (launch, allocation of events...) */
  GEMM_ERR_ALLOC = 4,         /* library-owned workspace could not be allocated */
  GEMM_ERR_WORKSPACE = 5,     /* caller workspace too small or misaligned */
  GEMM_ERR_SCRATCH = 6        /* gemm_f16_f32_abt_noalloc: plan needs more than its scratch */
} gemm_status_t;

/* C = A * B^T (see the layout block above). A, B, C are device pointers.
 * Requirements: M, N, K >= 0; lda >= K; ldb >= K; ldc >= N; A, B, C non-NULL
 * when M*N > 0 (A, B may be NULL when K = 0); C must not overlap A or B.
 * M, N and K above 2147482623 (2^31 - 1025; the kernels index in 32 bits)
 * return GEMM_ERR_NOT_SUPPORTED, as do strides that would make an operand
 * span 2^60 bytes or more; strides and byte sizes may otherwise exceed 2^31.
 * Any alignment of pointers and strides is accepted: 16-byte aligned A, B
 * with lda, ldb, K multiples of 8 take the tiled MFMA kernels directly. When
 * an operand breaks these rules and M*N*K >= 2^22, a pack kernel first copies
 * it into the workspace as rows of K rounded up to 8 elements (zero past K)
 * and the tiled kernels run on the copy; smaller products take a slower
 * general kernel. Split-K and stream-K plans (the latter also for the tiles
 * left after whole data-parallel rounds) write fp32 partial tiles
 * to a workspace and a second kernel on the same stream sums them, in a fixed
 * (k) order, into C, so results do not depend on timing. The workspace is
 * library-owned, allocated once per (device, stream) on first use and grown
 * when a larger one is needed; calls sharing a stream are ordered by it,
 * calls on different streams do not share one. Calls from several host
 * threads at once are safe, on one stream or on several.
 * Graph capture: a call on a stream that is being captured returns
 * GEMM_ERR_WORKSPACE if its plan needs a workspace (a later call could free
 * or replace the library-owned one while the graph still holds its address);
 * use gemm_f16_f32_abt_ws with a caller workspace inside captured regions.
 * Plans without a workspace (data-parallel, aligned operands) capture as
 * they are. */
gemm_status_t gemm_f16_f32_abt(int64_t M, int64_t N, int64_t K,
                               const void* A, int64_t lda,
                               const void* B, int64_t ldb,
                               float* C, int64_t ldc, void* stream);

/* Bytes of workspace gemm_f16_f32_abt_ws needs for this shape (0 if none) on
 * the current device (its CU count sets the plan; 256 when no device is
 * visible), for 16-byte aligned operands with row strides a multiple of 8;
 * when K is not a multiple of 8 it includes the packed copies of both
 * operands. */
size_t gemm_f16_f32_abt_workspace_size(int64_t M, int64_t N, int64_t K);

/* As gemm_f16_f32_abt, with a caller-owned device workspace of at least
 * gemm_f16_f32_abt_workspace_size(M, N, K) bytes, 256-byte aligned. Its
 * contents on entry do not matter. Two calls in flight at once must not share
 * it. workspace may be NULL when the size is 0. Operands that would be packed
 * are packed only if the workspace also holds their copies; otherwise the
 * call runs the general kernel (never an error for that reason). */
gemm_status_t gemm_f16_f32_abt_ws(int64_t M, int64_t N, int64_t K,
                                  const void* A, int64_t lda,
                                  const void* B, int64_t ldb,
                                  float* C, int64_t ldc,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* bfloat16 inputs: as gemm_f16_f32_abt, with A and B holding bfloat16 bit
 * patterns (the upper 16 bits of an IEEE binary32: 1 sign bit, 8 exponent
 * bits with bias 127, 7 fraction bits) instead of binary16. Same layouts,
 * semantics, alignment rules, workspace and error behaviour; accumulation
 * and output stay binary32. bfloat16 is the 16-bit type the cuBLASDx "BLAS
 * Performance Guide" handles beside half (section "Build Card", on the half
 * and bfloat16 conversions its headers need); the path is otherwise the
 * fp16 one, on the bf16 forms of the same MFMA instructions. */
gemm_status_t gemm_bf16_f32_abt(int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t lda,
                                const void* B, int64_t ldb,
                                float* C, int64_t ldc, void* stream);

/* Bytes of workspace gemm_bf16_f32_abt_ws needs for this shape (0 if none);
 * the same as gemm_f16_f32_abt_workspace_size. */
size_t gemm_bf16_f32_abt_workspace_size(int64_t M, int64_t N, int64_t K);

/* gemm_bf16_f32_abt with a caller-owned workspace, as gemm_f16_f32_abt_ws. */
gemm_status_t gemm_bf16_f32_abt_ws(int64_t M, int64_t N, int64_t K,
                                   const void* A, int64_t lda,
                                   const void* B, int64_t ldb,
                                   float* C, int64_t ldc,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. As
 * gemm_f16_f32_abt, but every workspace the call needs (split-K and stream-K
 * partial tiles, packed operands) lives in a static device array of 64 MiB
 * (67108864 bytes) inside the library, so the call never allocates or frees
 * memory (no hipMalloc, no hipFree). Each device the entry point runs on
 * holds its own copy of the array from the first call on it until the
 * process ends; its address is looked up once per device with
 * hipGetSymbolAddress. The array covers every split-K plan and the five
 * reference workloads; a plan whose partial tiles need more returns
 * GEMM_ERR_SCRATCH before anything is enqueued (operands that would be packed
 * into more run the general kernel instead). Nothing in the array needs to
 * start at zero and it keeps the last call's contents. All calls on one
 * device share the one array: calls that can overlap in time on one device
 * (on different streams, or from threads without ordering) race and corrupt
 * each other's results; order them on one stream. Calls are safe to capture
 * in a HIP graph. Same arguments, layouts and other errors as
 * gemm_f16_f32_abt (binary16 operands). */
gemm_status_t gemm_f16_f32_abt_noalloc(int64_t M, int64_t N, int64_t K,
                                       const void* A, int64_t lda,
                                       const void* B, int64_t ldb,
                                       float* C, int64_t ldc, void* stream);

/* Static text for a status code (never NULL). */
const char* gemm_status_string(gemm_status_t s);

/* Writes a one-line description of the plan chosen for (M, N, K) on a
 * 256-CU device (a whole MI355X, unless the plan override names another CU
 * count) into the host buffer buf (NUL-terminated, truncated to len).
 * Touches no device.
 * Same size limits as gemm_f16_f32_abt (GEMM_ERR_NOT_SUPPORTED beyond them). */
gemm_status_t gemm_f16_f32_abt_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t len);

/* Frees the library-owned workspaces of the current device after waiting for
 * their streams. Call only when no gemm on those streams is in flight. */
void gemm_f16_release_workspaces(void);

/* Host-side schedule model (no device is touched): fills out[] with one row
 * of 7 int64 per (workgroup, segment) of the persistent schedule for
 * (M, N, K) on a 256-CU device with `grid` workgroups (grid <= 0: the plan's own grid; only
 * data-parallel, stream-K and rounds-then-stream-K plans accept another grid):
 *   { workgroup, tile, k_iter_begin, k_iter_end, role, shares, index }
 * role 0 = the tile's only unit (stores C directly); role 1 = one of `shares`
 * units of a tile, `index` its position in k order (writes its partial tile
 * to workspace slot `index`; the reduce kernel sums the slots into C).
 * Returns the number of rows (writes at most `cap`), or -1 on bad arguments or
 * when the plan has no persistent schedule (the general and direct kernels).
 * *k_iters and *tiles (if non-NULL) receive the plan's k-iterations per tile
 * and its output-tile count. Used by tests to check that every (tile, k-iter)
 * is covered exactly once and that the shares of a tile are numbered 0..s-1
 * in k order. */
int64_t gemm_f16_schedule_dump(int64_t M, int64_t N, int64_t K, int64_t grid,
                               int64_t* out, int64_t cap, int64_t* k_iters, int64_t* tiles);

/* Host-side view of the kernels' LDS layout (no device is touched): the
 * position, within an LDS tile row of `chunks_per_row` 16-byte chunks (4 for
 * 32-element k-stages, 8 for 64), at which the kernels store logical chunk
 * `chunk` of tile row `row`, for MFMA block height `block_dim` (16 or 32).
 * Returns -1 for other arguments. The same function runs in the kernels;
 * tests use this to check that every row's chunks form a permutation and
 * that the fragment reads (ds_read_b128) meet no LDS bank conflicts. */
int32_t gemm_f16_lds_chunk(int32_t chunks_per_row, int32_t block_dim, int32_t row,
                           int32_t chunk);

/* Plan override for tests and experiments (host only; no device is touched).
 * `text` is a comma-separated list of key=integer pairs, any subset of
 *   kid=<tiled kernel id>  mode=<0 data-parallel, 1 split-K, 2 stream-K,
 *   3 whole data-parallel rounds then stream-K>  splits=<k-shares per tile>
 *   grid=<workgroups>  group=<tile rows per band>  xcd=<0|1 renumbering>
 *   cus=<compute units to plan for>  general=1 (the general kernel)
 *   direct=<1: the direct 16x16 kernel where the operands allow it, 0: never>;
 * keys the shape does not allow are ignored, so every plan stays correct.
 * NULL or "" restores the default rule. The override applies to every later
 * call in the process (all threads) and empties the plan cache. At first use
 * the library takes its initial value from the environment variable
 * GEMM_F16_PLAN; later changes to that variable are not read. */
void gemm_f16_set_plan_override(const char* text);

/* Clock probe for measurement (host only; nothing is launched). With
 * `counters` a device pointer to two unsigned 64-bit integers, every later
 * launch of a tiled main kernel (any host thread, any stream) has its first
 * wave of workgroup 0 add, with device-scope atomics, the shader-clock cycles
 * (s_memtime) to counters[0] and the 100 MHz real-time ticks (s_memrealtime)
 * to counters[1] between the workgroup's start and its end. Over a set of
 * launches, 100 MHz * counters[0] / counters[1] is then the average shader
 * clock while they ran, which is what the MFMA peak scales with (of the XCD
 * workgroup 0 runs on: at the board's power limit the XCDs' clocks can differ
 * by several percent). The caller
 * zeroes the counters, keeps them alive while such launches are in flight,
 * and passes NULL to turn the probe off (the default). The general, direct
 * and reduce kernels are not probed. */
void gemm_f16_set_clock_probe(unsigned long long* counters);


#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_H */
