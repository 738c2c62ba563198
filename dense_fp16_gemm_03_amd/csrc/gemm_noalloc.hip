// gemm_f16_f32_abt_noalloc: the binary16 entry point for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Its workspace (partial tiles of split-K
// and stream-K plans, packed operands) is a static device array of this
// file, so no call allocates or frees anything. Contract in
// include/gemm_f16.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gemm_f16.h"
#include "gemm_kernels.h"

namespace {

// 64 MiB: every split-K plan (256 units of at most one 256x256 fp32 partial
// tile each) and all five reference workloads fit.
constexpr size_t kScratchBytes = (size_t)64 << 20;

// The array itself. Host code never uses this name as an address: in host
// code it is a stand-in for the symbol, and each device holds its own copy at
// its own address, which scratch_address() looks up.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `dev`'s copy of the array (dev is the current device),
// looked up once per device.
gemm_status_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();  // clear it, so a later launch check does not report it
      return GEMM_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GEMM_OK;
}

}  // namespace

extern "C" gemm_status_t gemm_f16_f32_abt_noalloc(int64_t M, int64_t N, int64_t K,
                                                  const void* A, int64_t lda, const void* B,
                                                  int64_t ldb, float* C, int64_t ldc,
                                                  void* stream) {
  // With no current device the address stays NULL: argument and size errors
  // are still reported, and the call stops before any launch.
  void* ws = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess) {
    const gemm_status_t st = scratch_address(dev, &ws);
    if (st != GEMM_OK) return st;
  } else {
    (void)hipGetLastError();
  }
  return g16::run_in_scratch(M, N, K, A, lda, B, ldb, C, ldc, ws, kScratchBytes, stream);
}
