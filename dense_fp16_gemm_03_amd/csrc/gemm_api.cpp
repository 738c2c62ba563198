// C ABI of libgemm_f16.so: argument checks, the shape -> plan rule, the
// split-K / stream-K workspace, and kernel launch. Declarations and the
// contract of every entry point are in include/gemm_f16.h.
#include "gemm_f16.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <unordered_map>
#include <utility>

#include "gemm_kernels.h"
#include "gemm_lds_layout.h"

namespace {

using namespace g16;

constexpr int32_t kDefaultCUs = 256;  // MI355X: 8 XCDs x 32 CUs
// Largest M, N or K accepted. The kernels index rows, columns and k in 32-bit
// integers, and a tile's first index plus its extent (at most 256, plus the
// ring's masked tail stages in k) must not pass 2^31 - 1.
constexpr int64_t kMaxDim = 0x7FFFFFFF - 1024;
// Kernel for large tiles with K below 2048: 256x256 tiles, 16x16x32 MFMA,
// two waves per SIMD in the ping-pong main loop over a 32-wide ring.
constexpr int32_t KID_LARGE = KID_256x256x32_S3_W8_M16_PP;
// The same tiles over 64-wide stages (whole 128-byte rows per load) held as
// A and B halves in five LDS slots: for at least a round of tiles with
// K >= 2048, and for long K split over the CUs.
constexpr int32_t KID_LARGE64 = KID_256x256x64_H5_W8_M16_PP;

// Whether the tiles left after whole data-parallel rounds of 256x256 tiles
// are shared by stream-K (see make_plan).
bool share_last_round(int64_t tiles, int64_t k32, int32_t cus) {
  const int64_t left = tiles % cus;
  return tiles > cus && left > 0 && (cus - left) * k32 >= 44 * (int64_t)cus;
}

// Smallest product (M*N*K multiply-adds) for which operands the tiled
// kernels cannot load directly are packed first; below it the general kernel
// is as fast as the extra pack launches.
constexpr double kPackMinWork = (double)(1 << 22);

struct Plan {
  int32_t kid = -1;       // tiled kernel id, KID_GENERAL, or -1 (nothing to do)
  Sched s{};
  bool c_vec4 = false;
  size_t workspace = 0;   // bytes: partial tiles, then packed operands (0 if none)
  size_t partial_bytes = 0;  // the partial tiles at the start of the workspace
  bool pack_a = false, pack_b = false;  // operand copied to aligned rows first
  int64_t kp = 0;         // K of the packed operands (K rounded up to 8)
};

size_t round256(int64_t bytes) { return (size_t)((bytes + 255) / 256 * 256); }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Predicted GPU time (us) of a plan for shapes with fewer 256x256 tiles than
// CUs: `splits` k-shares of every tile of kernel `kid` (one of the 64-wide
// kernels KID_LARGE64, 128x128 or 64x64), units laid out in rounds of `cus`
// workgroups. Each round costs a fixed start plus a time per 64-wide
// k-iteration of one unit; a split plan adds the reduce pass, a fixed cost
// plus the partial tiles and C it streams. The constants are a least-squares
// fit (relative error) to calls-alone medians of 627 plans over 60 shapes
// (M, N in 512..3072, K in 2048..16384) on one MI355X: median error 4%,
// 90th percentile 11%.
double predicted_us(int64_t M, int64_t N, int64_t K, int32_t kid, int64_t splits, int32_t cus) {
  const KernelInfo* ki = kernel_info(kid);
  double start, per_iter;
  if (kid == KID_LARGE64) {
    start = 10.49, per_iter = 0.9955;
  } else if (kid == KID_128x128x64_S4_W4_M16) {
    start = 8.69, per_iter = 0.3727;
  } else {
    start = 5.14, per_iter = 0.1999;
  }
  const int64_t tiles = cdiv(M, ki->bm) * cdiv(N, ki->bn);
  const int64_t iters = cdiv(cdiv(K, 64), splits);
  const int64_t rounds = cdiv(tiles * splits, cus);
  double us = (double)rounds * (start + per_iter * (double)iters);
  if (splits > 1) {
    const double bytes = (double)tiles * splits * ki->bm * ki->bn * 4 + 4.0 * M * N;
    us += 2.56 + 0.318e-6 * bytes;
  }
  return us;
}

// For shapes with fewer 256x256 tiles than CUs, the rule's plan (kernel
// `*kid`, `*splits` k-shares) is replaced by the plan of least predicted time
// among the 64-wide kernels with 256x256, 128x128 and 64x64 tiles and every
// split that keeps one round and two or more k-iterations a share, when its
// prediction beats the rule's by more than 10% (near ties keep the rule).
// Measured on the same 60 shapes: calls alone 1.28x the best plan's time on
// average (geometric mean) with the rule alone, 1.007x with this choice; the
// largest gains where the rule's split leaves most CUs idle (1024x1024x4096
// 46.9 -> 21.6 us, 512x512x8192 44.8 -> 17.9 us).
void choose_by_prediction(int64_t M, int64_t N, int64_t K, int32_t cus, int32_t* kid,
                          int32_t* splits) {
  if (K < 64) return;
  const int32_t kids[3] = {KID_LARGE64, KID_128x128x64_S4_W4_M16, KID_64x64x64_S4_W4_M16};
  double best = -1.0;
  int32_t best_kid = *kid, best_splits = *splits;
  for (int32_t c : kids) {
    const KernelInfo* ki = kernel_info(c);
    const int64_t tiles = cdiv(M, ki->bm) * cdiv(N, ki->bn);
    const int64_t max_splits =
        tiles >= cus ? 1 : std::max<int64_t>(1, std::min<int64_t>(cus / tiles, cdiv(K, 64) / 2));
    for (int64_t sp = 1; sp <= max_splits; ++sp) {
      const double us = predicted_us(M, N, K, c, sp, cus);
      if (best < 0 || us < best) {
        best = us;
        best_kid = c;
        best_splits = (int32_t)sp;
      }
    }
  }
  if (predicted_us(M, N, K, *kid, std::max(*splits, 1), cus) > 1.1 * best) {
    *kid = best_kid;
    *splits = best_splits;
  }
}

bool ranges_overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (abytes == 0 || bbytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

size_t span_bytes(int64_t rows, int64_t ld, int64_t cols, size_t elem) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)((rows - 1) * ld + cols) * elem;
}

// A row stride whose operand would span 2^60 bytes or more (far beyond any
// device's address space) is refused, so spans and offsets never overflow.
bool stride_fits(int64_t rows, int64_t ld, int64_t elem) {
  return rows <= 1 || ld <= ((int64_t)1 << 60) / (rows * elem);
}

gemm_status_t validate(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       const void* B, int64_t ldb, const float* C, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_VALUE;
  if (lda < K || ldb < K || ldc < N) return GEMM_ERR_INVALID_VALUE;
  if (M == 0 || N == 0) return GEMM_OK;
  if (C == nullptr) return GEMM_ERR_INVALID_VALUE;
  if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_ERR_INVALID_VALUE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_ERR_NOT_SUPPORTED;
  if (!stride_fits(M, lda, 2) || !stride_fits(N, ldb, 2) || !stride_fits(M, ldc, 4))
    return GEMM_ERR_NOT_SUPPORTED;
  const size_t cbytes = span_bytes(M, ldc, N, 4);
  if (K > 0 && (ranges_overlap(C, cbytes, A, span_bytes(M, lda, K, 2)) ||
                ranges_overlap(C, cbytes, B, span_bytes(N, ldb, K, 2))))
    return GEMM_ERR_INVALID_VALUE;
  if (((uintptr_t)A & 1) || ((uintptr_t)B & 1) || ((uintptr_t)C & 3))
    return GEMM_ERR_NOT_SUPPORTED;
  return GEMM_OK;
}

// Plan override for experiments and tests, from text such as
// "kid=35,mode=1,splits=16,grid=256,group=4,xcd=0,cus=32" (any subset of
// keys), or "general=1" for the general kernel; unknown keys are ignored.
// `cus` plans for that many compute units instead of the device's (the grid
// never exceeds it). Set at first use from the environment variable
// GEMM_F16_PLAN, and afterwards only by gemm_f16_set_plan_override.
struct Override {
  int32_t kid = -1, mode = -1, splits = -1, grid = -1, group = -1, xcd = -1;
  int32_t general = 0;  // 1: the general kernel, whatever the operands
  int32_t direct = -1;  // 1: the direct kernel when the operands allow it; 0: never
  int32_t cus = -1;
};

Override parse_override(const char* text) {
  Override o;
  if (!text) return o;
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s", text);
  char* save = nullptr;
  for (char* tok = strtok_r(buf, ",", &save); tok; tok = strtok_r(nullptr, ",", &save)) {
    char key[32];
    int val = 0;
    if (std::sscanf(tok, "%31[^=]=%d", key, &val) != 2) continue;
    if (!std::strcmp(key, "kid")) o.kid = val;
    else if (!std::strcmp(key, "mode")) o.mode = val;
    else if (!std::strcmp(key, "splits")) o.splits = val;
    else if (!std::strcmp(key, "grid")) o.grid = val;
    else if (!std::strcmp(key, "group")) o.group = val;
    else if (!std::strcmp(key, "xcd")) o.xcd = val;
    else if (!std::strcmp(key, "general")) o.general = val;
    else if (!std::strcmp(key, "direct")) o.direct = val;
    else if (!std::strcmp(key, "cus")) o.cus = val;
  }
  return o;
}

// True when the tiled kernels can load an operand directly: 16-byte aligned
// rows of a multiple of 8 elements, and buffer offsets within a tile of
// `tile_rows` rows (row * ld + k, in bytes) below 2^31.
bool operand_loadable(const void* X, int64_t ld, int64_t K, int32_t tile_rows, int32_t bk) {
  if (((uintptr_t)X & 15) || ld % 8 || K % 8) return false;
  const int64_t limit = (int64_t)1 << 31;
  return (int64_t)(tile_rows - 1) * ld * 2 + (K + bk) * 2 < limit;
}

bool tiled_eligible(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                    int64_t ldb, int32_t kid) {
  const KernelInfo* ki = kernel_info(kid);
  if (!ki || K <= 0) return false;
  (void)M;
  (void)N;
  return operand_loadable(A, lda, K, ki->bm, ki->bk) && operand_loadable(B, ldb, K, ki->bn, ki->bk);
}

// Shape -> kernel and schedule. The pages' rule (section "Inside the kernels"
// of "SASS-Level Kernel Generation for Blackwell") picks per shape a tile, a
// ring depth and how K is divided; this is the same kind of rule for 256 CUs,
// set from measurements on the MI355X:
//   * at least one 256x256 tile per CU: 256x256 tiles, data-parallel,
//     persistent grid walking the tiles by stride; with K >= 4096 the main
//     loop over 64-wide stages in five half-stage slots;
//   * fewer tiles but long K (>= 128 k-steps of 32): the same tiles and main
//     loop with K split so tiles x splits fills the CUs (each share keeps
//     >= 64 k-steps of 32);
//   * smaller problems: 128x128 tiles, or 64x64 tiles when 128x128 ones
//     would fill fewer than half the CUs, or 32x32 tiles when even those
//     number no more than the CUs (their per-workgroup chain of loads, MFMAs
//     and stores is the shortest), data-parallel (at these sizes the reduce
//     pass of a split costs more than it gains); and when 16x16 tiles number
//     no more than the CUs and K <= 256, the direct kernel (no LDS);
//   * more 256x256 tiles than CUs, when the last round's idle CUs times the
//     k-iterations is large enough: whole rounds data-parallel, the tiles
//     left by stream-K (DP_SK).
Plan make_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
               int64_t ldb, const float* C, int64_t ldc, int32_t cus, int32_t dt,
               const Override& o, bool allow_pack = true);

// DP_SK: tiles below shared_base form whole data-parallel rounds of s.grid
// tiles; the rest are shared by stream-K. Without a whole round it is plain
// stream-K, and without a remainder plain data-parallel.
void set_shared_base(Sched& s) {
  if (s.mode != MODE_DP_SK) {
    s.shared_base = 0;
    return;
  }
  const int64_t whole = (int64_t)(s.tiles / s.grid) * s.grid;
  if (whole == 0) {
    s.mode = MODE_STREAM_K;
    s.shared_base = 0;
  } else if (whole == s.tiles) {
    s.mode = MODE_DATA_PARALLEL;
    s.shared_base = 0;
  } else {
    s.shared_base = (int32_t)whole;
  }
}

// Operands the tiled kernels cannot load directly (a pointer off 16 bytes, a
// row stride or K not a multiple of 8, a stride past the offset limit): for a
// large enough product each such operand is first copied into rows of K
// rounded up to 8 elements, zero-filled past K, at the end of the workspace,
// and the tiled plan runs on the copies. Otherwise the general kernel.
Plan packed_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                 int64_t ldb, const float* C, int64_t ldc, int32_t cus, int32_t dt, int32_t kid,
                 const Override& o) {
  Plan general;
  general.kid = KID_GENERAL;
  if (K <= 0 || (double)M * (double)N * (double)K < kPackMinWork) return general;
  const KernelInfo* ki = kernel_info(kid);
  const int64_t kp = cdiv(K, 8) * 8;
  const bool pa = !operand_loadable(A, lda, K, ki->bm, ki->bk);
  const bool pb = !operand_loadable(B, ldb, K, ki->bn, ki->bk);
  const void* aligned = (const void*)(uintptr_t)256;
  Plan p = make_plan(M, N, kp, pa ? aligned : A, pa ? kp : lda, pb ? aligned : B,
                     pb ? kp : ldb, C, ldc, cus, dt, o, false);
  if (p.kid < 0 || p.kid == KID_GENERAL) return general;
  p.pack_a = pa;
  p.pack_b = pb;
  p.kp = kp;
  p.partial_bytes = p.workspace;
  if (pa) p.workspace += round256(M * kp * 2);
  if (pb) p.workspace += round256(N * kp * 2);
  return p;
}

Plan make_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
               int64_t ldb, const float* C, int64_t ldc, int32_t cus, int32_t dt,
               const Override& o, bool allow_pack) {
  Plan plan;
  if (M == 0 || N == 0) return plan;
  plan.c_vec4 = ((uintptr_t)C % 16 == 0) && (ldc % 4 == 0);
  if (o.general == 1) {
    plan.kid = KID_GENERAL;
    return plan;
  }

  int32_t kid = KID_LARGE;
  int32_t mode = MODE_DATA_PARALLEL;
  int32_t splits = 1;
  {
    const int64_t t256 = cdiv(M, 256) * cdiv(N, 256);
    const int64_t k32 = cdiv(K, 32);
    if (t256 >= cus) {
      // 64-wide stages from K = 2048 on: calls alone, one box, against the
      // 32-wide ring: 4096^2 x 2048 64.2 -> 62.7 us, x 3072 89.4 -> 85.3,
      // 8192^2 x 2048 234.7 -> 225.6. At K = 1024 they tie (4096^2: 39.8 /
      // 40.0 us) or the ring wins (16384 x 4096: 139.0 / 141.3).
      kid = k32 >= 64 ? KID_LARGE64 : KID_LARGE;
    } else if (k32 >= 128) {
      kid = KID_LARGE64;
      int64_t sp = cus / t256;
      if (sp > k32 / 64) sp = k32 / 64;  // each share keeps >= 64 k-steps of 32
      splits = (int32_t)std::max<int64_t>(sp, 1);
      mode = splits > 1 ? MODE_SPLIT : MODE_DATA_PARALLEL;
    } else {
      kid = 2 * cdiv(M, 128) * cdiv(N, 128) >= cus ? KID_128x128x64_S4_W4_M16
            : cdiv(M, 32) * cdiv(N, 32) <= cus       ? KID_32x32x64_S5_W4_M16
                                                    : KID_64x64x64_S4_W4_M16;
    }
  }
  if (o.kid < 0 && o.mode < 0 && o.splits < 1 && cdiv(M, 256) * cdiv(N, 256) < cus &&
      (kid == KID_LARGE64 || kid == KID_128x128x64_S4_W4_M16 || kid == KID_64x64x64_S4_W4_M16)) {
    choose_by_prediction(M, N, K, cus, &kid, &splits);
    mode = splits > 1 ? MODE_SPLIT : MODE_DATA_PARALLEL;
  }
  if (o.kid >= 0 && kernel_info(o.kid) && tiled_has(o.kid, dt)) kid = o.kid;
  if (o.mode >= 0 && o.mode <= MODE_DP_SK) mode = o.mode;
  if (o.splits >= 1) splits = o.splits;

  if (!tiled_eligible(M, N, K, A, lda, B, ldb, kid)) {
    if (allow_pack) return packed_plan(M, N, K, A, lda, B, ldb, C, ldc, cus, dt, kid, o);
    plan.kid = KID_GENERAL;
    return plan;
  }
  // The smallest products (16x16 tiles no more than the CUs, K of one chunk
  // of loads) take the direct kernel: no LDS, one wave a tile. Measured
  // (kernel traces, same box): 256^3 3.64 -> 3.20 us against 32x32 tiles;
  // ties at 256x512x256 and 128x128x1024, losses from 384^3 and at K = 1024.
  const bool tiny = cdiv(M, 16) * cdiv(N, 16) <= cus && K <= 256;
  if (o.direct == 1 || (tiny && o.kid < 0 && o.mode < 0 && o.direct != 0)) {
    plan.kid = KID_DIRECT;
    return plan;
  }
  const KernelInfo* ki = kernel_info(kid);
  Sched& s = plan.s;
  s.tiles_m = (int32_t)cdiv(M, ki->bm);
  s.tiles_n = (int32_t)cdiv(N, ki->bn);
  const int64_t tiles = (int64_t)s.tiles_m * s.tiles_n;
  s.k_iters = (int32_t)cdiv(K, ki->bk);
  if (tiles > 0x3FFFFFFF || (int64_t)tiles * s.k_iters > ((int64_t)1 << 40)) {
    plan.kid = KID_GENERAL;
    return plan;
  }
  s.tiles = (int32_t)tiles;
  // After whole data-parallel rounds of 256x256 tiles, the tiles left are
  // shared by all workgroups (stream-K) when the CUs a last data-parallel
  // round would leave idle cost more than sharing does. Measured: the partial
  // tiles and the reduce pass cost about 40 us, an idle CU about 0.85 us per
  // k-iteration of 32, so sharing pays from (idle CUs / CUs) * k-iterations
  // of about 44.
  if (o.mode < 0 && mode == MODE_DATA_PARALLEL && (kid == KID_LARGE || kid == KID_LARGE64) &&
      share_last_round(tiles, cdiv(K, 32), cus))
    mode = MODE_DP_SK;
  s.group_m = o.group > 0 ? o.group : 4;
  if (s.group_m > s.tiles_m) s.group_m = s.tiles_m;
  s.xcd_remap = o.xcd >= 0 ? (o.xcd != 0) : 1;
  s.mode = mode;
  if (mode == MODE_SPLIT) {
    if (splits > s.k_iters) splits = s.k_iters;
    if (splits <= 1) s.mode = MODE_DATA_PARALLEL;
  }
  s.splits = s.mode == MODE_SPLIT ? splits : 1;

  // Persistent grid: at most one workgroup per CU at a time (the tiled
  // kernels' LDS use allows one per CU).
  const int64_t resident = cus;
  int64_t grid;
  if (s.mode == MODE_STREAM_K) {
    grid = std::min<int64_t>((int64_t)tiles * s.k_iters, resident);
    if (o.grid > 0) grid = std::min<int64_t>(grid, o.grid);
  } else if (s.mode == MODE_SPLIT) {
    grid = std::min<int64_t>((int64_t)tiles * s.splits, resident);
    if (o.grid > 0) grid = std::min<int64_t>(grid, o.grid);
  } else if (s.mode == MODE_DP_SK) {
    grid = std::min<int64_t>((int64_t)tiles * s.k_iters, resident);
    if (o.grid > 0) grid = std::min<int64_t>(grid, o.grid);
  } else {
    grid = std::min<int64_t>(tiles, resident);
    if (o.grid > 0) grid = std::min<int64_t>(o.grid, tiles);
  }
  s.grid = (int32_t)std::max<int64_t>(grid, 1);
  set_shared_base(s);
  s.slots = max_shares(s);
  plan.kid = kid;
  if (s.mode != MODE_DATA_PARALLEL)
    plan.workspace =
        (size_t)((int64_t)(tiles - s.shared_base) * s.slots * ki->bm * ki->bn * 4);
  return plan;
}

const char* mode_name(int32_t m) {
  switch (m) {
    case MODE_DATA_PARALLEL: return "data_parallel";
    case MODE_SPLIT: return "split";
    case MODE_STREAM_K: return "stream_k";
    case MODE_DP_SK: return "dp_stream_k";
    default: return "?";
  }
}

// Device CU counts, cached per device (0: not asked yet).
constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_cus[kMaxDevices];

int32_t device_cus(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
  int32_t n = g_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  int q = 0;
  if (hipDeviceGetAttribute(&q, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || q <= 0)
    q = kDefaultCUs;
  g_cus[dev].store(q, std::memory_order_relaxed);
  return q;
}

// Plans are cached per call signature: the shape, the row strides, whether
// each of A, B and C is 16-byte aligned (all make_plan looks at in the
// pointers), the operand type and the CU count. The override is part of the
// state the cache holds; changing it empties the cache.
struct PlanKey {
  int64_t M, N, K, lda, ldb, ldc;
  int32_t aligned;  // bit 0: A, bit 1: B, bit 2: C 16-byte aligned
  int32_t dt, cus;
  bool operator==(const PlanKey& o) const {
    return M == o.M && N == o.N && K == o.K && lda == o.lda && ldb == o.ldb && ldc == o.ldc &&
           aligned == o.aligned && dt == o.dt && cus == o.cus;
  }
};

struct PlanKeyHash {
  size_t operator()(const PlanKey& k) const {
    uint64_t h = 0x9E3779B97F4A7C15ull;
    const int64_t v[9] = {k.M, k.N, k.K, k.lda, k.ldb, k.ldc, k.aligned, k.dt, k.cus};
    for (int64_t x : v) {
      h ^= (uint64_t)x + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    }
    return (size_t)h;
  }
};

constexpr size_t kPlanCacheMax = 4096;  // emptied when it grows past this
std::mutex g_plan_mu;
bool g_override_set = false;
Override g_override;
std::unordered_map<PlanKey, Plan, PlanKeyHash> g_plans;

// The caller holds g_plan_mu.
const Override& current_override() {
  if (!g_override_set) {
    g_override = parse_override(std::getenv("GEMM_F16_PLAN"));
    g_override_set = true;
  }
  return g_override;
}

// CU count plans are made for: the override's, else the device's (dev >= 0),
// else a whole MI355X. The caller holds g_plan_mu.
int32_t planning_cus(int dev) {
  const Override& o = current_override();
  if (o.cus > 0) return o.cus;
  return dev >= 0 ? device_cus(dev) : kDefaultCUs;
}

// The plan for a call (cached). dev: the current device, or -1 for none.
Plan lookup_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                 int64_t ldb, const float* C, int64_t ldc, int32_t dt, int dev) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  const int32_t cus = planning_cus(dev);
  const PlanKey key{M, N, K, lda, ldb, ldc,
                    (((uintptr_t)A & 15) == 0 ? 1 : 0) | (((uintptr_t)B & 15) == 0 ? 2 : 0) |
                        (((uintptr_t)C & 15) == 0 ? 4 : 0),
                    dt, cus};
  auto it = g_plans.find(key);
  if (it != g_plans.end()) return it->second;
  const Plan plan = make_plan(M, N, K, A, lda, B, ldb, C, ldc, cus, dt, current_override());
  if (g_plans.size() >= kPlanCacheMax) g_plans.clear();
  g_plans.emplace(key, plan);
  return plan;
}

// The plan the entry points take for aligned operands with row strides of K
// (rounded up to 8) and ldc = N: what describe, workspace_size and the
// schedule model report. dev as in lookup_plan.
Plan reference_plan(int64_t M, int64_t N, int64_t K, int dev) {
  const void* aligned = (const void*)(uintptr_t)256;
  const int64_t ld = K % 8 ? K + (8 - K % 8) : K;
  return lookup_plan(M, N, K, aligned, ld, aligned, ld, (const float*)aligned, N, DT_F16, dev);
}

// Clock probe counters for every later launch (nullptr: off).
std::atomic<unsigned long long*> g_clock_probe{nullptr};

// The current device, or -1 when none is usable.
int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

// Library-owned workspaces (partial tiles of split-K / stream-K plans), one
// per (device, stream). g_ws_mu is held from taking a workspace until the
// kernels that use it are enqueued, so a call from another host thread that
// grows the same workspace cannot free it in between.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// The caller holds g_ws_mu.
gemm_status_t library_workspace(int dev, hipStream_t stream, size_t need, void** out) {
  Workspace& w = g_ws[{dev, stream}];
  if (w.bytes >= need) {
    *out = w.ptr;
    return GEMM_OK;
  }
  if (w.ptr) {
    // Earlier calls on this stream may still use the old buffer.
    if (hipStreamSynchronize(stream) != hipSuccess) return GEMM_ERR_HIP;
    (void)hipFree(w.ptr);
    w.ptr = nullptr;
    w.bytes = 0;
  }
  size_t bytes = need < 65536 ? 65536 : need;
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();  // clear it, so a later launch check does not report it
    return GEMM_ERR_ALLOC;
  }
  w.ptr = p;
  w.bytes = bytes;
  *out = p;
  return GEMM_OK;
}

bool workspace_fits(const Plan& plan, const void* ws, size_t ws_bytes) {
  return plan.workspace == 0 || (ws != nullptr && ws_bytes >= plan.workspace &&
                                 ((uintptr_t)ws & 255) == 0);
}

// The plan for a call with a caller workspace: a plan that packs operands but
// does not fit the workspace runs the general kernel instead (packing is an
// optimisation; partial tiles are not).
Plan caller_plan(Plan plan, const void* ws, size_t ws_bytes) {
  if ((plan.pack_a || plan.pack_b) && !workspace_fits(plan, ws, ws_bytes)) {
    Plan general;
    general.kid = KID_GENERAL;
    general.c_vec4 = plan.c_vec4;
    return general;
  }
  return plan;
}

// Where a call's workspace comes from: the library's per-stream allocation,
// the caller's buffer, or the static scratch array of the no-allocation
// entry point.
enum WsSource { WS_LIBRARY, WS_CALLER, WS_STATIC };

gemm_status_t run(int32_t dt, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                  const void* B, int64_t ldb, float* C, int64_t ldc, WsSource src, void* ws,
                  size_t ws_bytes, void* stream_v) {
  gemm_status_t st = validate(M, N, K, A, lda, B, ldb, C, ldc);
  if (st != GEMM_OK) return st;
  if (M == 0 || N == 0) return GEMM_OK;
  hipStream_t stream = (hipStream_t)stream_v;
  const bool caller_ws = src != WS_LIBRARY;
  // One plan per call, for the CU count gemm_f16_f32_abt_workspace_size also
  // uses; the caller's workspace is checked against it before anything is
  // enqueued.
  const int dev = current_device();
  Plan plan = lookup_plan(M, N, K, A, lda, B, ldb, C, ldc, dt, dev);
  if (src == WS_CALLER) {
    plan = caller_plan(plan, ws, ws_bytes);
    if (!workspace_fits(plan, ws, ws_bytes)) return GEMM_ERR_WORKSPACE;
  } else if (src == WS_STATIC && plan.workspace > ws_bytes) {
    // Packing is an optimisation (the general kernel needs no workspace);
    // partial tiles beyond the scratch array are an error.
    if (!(plan.pack_a || plan.pack_b)) return GEMM_ERR_SCRATCH;
    Plan general;
    general.kid = KID_GENERAL;
    general.c_vec4 = plan.c_vec4;
    plan = general;
  }
  if (dev < 0) return GEMM_ERR_HIP;
  if (src == WS_STATIC && plan.workspace > 0 && ws == nullptr) return GEMM_ERR_HIP;
  if (plan.kid != KID_GENERAL && plan.kid != KID_DIRECT && !tiled_has(plan.kid, dt))
    return GEMM_ERR_NOT_SUPPORTED;
  if (plan.workspace > 0 && !caller_ws) {
    // A library-owned workspace can be freed and replaced by a later call on
    // this stream; a captured graph would keep its old address. Calls being
    // captured therefore need a caller workspace.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return GEMM_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return GEMM_ERR_WORKSPACE;
  }
  GemmParams p{};
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
  p.C = C;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.M = (int32_t)M;
  p.N = (int32_t)N;
  p.K = (int32_t)K;
  p.c_vec4 = plan.c_vec4 ? 1 : 0;
  p.s = plan.s;
  p.clock_probe = g_clock_probe.load(std::memory_order_relaxed);
  if (plan.kid == KID_GENERAL) {
    return launch_general(dt, p, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
  }
  std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);
  if (plan.workspace > 0) {
    void* w = nullptr;
    if (caller_ws) {
      w = ws;
    } else {
      ws_lock.lock();  // released once the kernels are enqueued
      st = library_workspace(dev, stream, plan.workspace, &w);
      if (st == GEMM_ERR_ALLOC && (plan.pack_a || plan.pack_b)) {
        // No room for the packed copies: the general kernel needs none.
        ws_lock.unlock();
        return launch_general(dt, p, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
      }
      if (st != GEMM_OK) return st;
    }
    p.partials = (f32x4_storage*)w;  // partial tiles, when the schedule has any
    // Packed operands follow the partial tiles: rows of kp elements, 16-byte
    // aligned, zero past K. The tiled plan then runs over kp.
    char* next = (char*)w + plan.partial_bytes;
    if (plan.pack_a) {
      if (launch_pack(p.A, lda, (int32_t)K, M, (int32_t)plan.kp, next, stream) != hipSuccess)
        return GEMM_ERR_HIP;
      p.A = (const uint16_t*)next;
      p.lda = plan.kp;
      next += round256(M * plan.kp * 2);
    }
    if (plan.pack_b) {
      if (launch_pack(p.B, ldb, (int32_t)K, N, (int32_t)plan.kp, next, stream) != hipSuccess)
        return GEMM_ERR_HIP;
      p.B = (const uint16_t*)next;
      p.ldb = plan.kp;
    }
    if (plan.pack_a || plan.pack_b) p.K = (int32_t)plan.kp;
  }
  if (plan.kid == KID_DIRECT)
    return launch_direct(dt, p, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
  return launch_tiled(plan.kid, dt, p, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

}  // namespace

namespace g16 {

gemm_status_t run_in_scratch(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             const void* B, int64_t ldb, float* C, int64_t ldc, void* scratch,
                             size_t scratch_bytes, void* stream) {
  return run(DT_F16, M, N, K, A, lda, B, ldb, C, ldc, WS_STATIC, scratch, scratch_bytes, stream);
}

}  // namespace g16

extern "C" {

gemm_status_t gemm_f16_f32_abt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                               const void* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(DT_F16, M, N, K, A, lda, B, ldb, C, ldc, WS_LIBRARY, nullptr, 0, stream);
}

gemm_status_t gemm_bf16_f32_abt(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                const void* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(DT_BF16, M, N, K, A, lda, B, ldb, C, ldc, WS_LIBRARY, nullptr, 0, stream);
}

size_t gemm_f16_f32_abt_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K < 0) return 0;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  // Aligned operands with K as the row stride: the plan the fast path takes,
  // for the CU count the calls plan with (a partitioned device has fewer CUs
  // and may plan differently). With K not a multiple of 8 the rows of both
  // operands are packed (no row stride makes them 16-byte aligned), and this
  // includes the copies. Other misaligned operands pack only into a caller
  // workspace large enough for them; otherwise that call runs the general
  // kernel.
  return reference_plan(M, N, K, current_device()).workspace;
}

gemm_status_t gemm_f16_f32_abt_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                  const void* B, int64_t ldb, float* C, int64_t ldc,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return run(DT_F16, M, N, K, A, lda, B, ldb, C, ldc, WS_CALLER, workspace, workspace_bytes,
             stream);
}

size_t gemm_bf16_f32_abt_workspace_size(int64_t M, int64_t N, int64_t K) {
  // The plan rule does not depend on the element type.
  return gemm_f16_f32_abt_workspace_size(M, N, K);
}

gemm_status_t gemm_bf16_f32_abt_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                   const void* B, int64_t ldb, float* C, int64_t ldc,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return run(DT_BF16, M, N, K, A, lda, B, ldb, C, ldc, WS_CALLER, workspace, workspace_bytes,
             stream);
}

const char* gemm_status_string(gemm_status_t s) {
  switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_VALUE: return "GEMM_ERR_INVALID_VALUE: invalid argument";
    case GEMM_ERR_NOT_SUPPORTED: return "GEMM_ERR_NOT_SUPPORTED: shape or alignment not supported";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP: a HIP runtime call failed";
    case GEMM_ERR_ALLOC: return "GEMM_ERR_ALLOC: workspace allocation failed";
    case GEMM_ERR_WORKSPACE: return "GEMM_ERR_WORKSPACE: workspace too small or misaligned";
    case GEMM_ERR_SCRATCH:
      return "GEMM_ERR_SCRATCH: the plan needs more workspace than the static scratch array "
             "of gemm_f16_f32_abt_noalloc holds";
    default: return "unknown gemm_status_t";
  }
}

gemm_status_t gemm_f16_f32_abt_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t len) {
  if (buf == nullptr || len == 0) return GEMM_ERR_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_VALUE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_ERR_NOT_SUPPORTED;
  const Plan plan = reference_plan(M, N, K, -1);
  if (plan.kid < 0) {
    std::snprintf(buf, len, "M=%lld N=%lld K=%lld: nothing to do", (long long)M, (long long)N,
                  (long long)K);
  } else if (plan.kid == KID_GENERAL) {
    std::snprintf(buf, len, "M=%lld N=%lld K=%lld kernel=general_64x64", (long long)M,
                  (long long)N, (long long)K);
  } else if (plan.kid == KID_DIRECT) {
    char pack[64] = "";
    if (plan.pack_a || plan.pack_b)
      std::snprintf(pack, sizeof(pack), " pack=%s%s kp=%lld", plan.pack_a ? "A" : "",
                    plan.pack_b ? "B" : "", (long long)plan.kp);
    std::snprintf(buf, len, "M=%lld N=%lld K=%lld kernel=direct_16x16 kid=%d tiles=%lld%s",
                  (long long)M, (long long)N, (long long)K, KID_DIRECT,
                  (long long)(cdiv(M, 16) * cdiv(N, 16)), pack);
  } else {
    const KernelInfo* ki = kernel_info(plan.kid);
    const Sched& s = plan.s;
    char pack[64] = "";
    if (plan.pack_a || plan.pack_b)
      std::snprintf(pack, sizeof(pack), " pack=%s%s kp=%lld", plan.pack_a ? "A" : "",
                    plan.pack_b ? "B" : "", (long long)plan.kp);
    std::snprintf(buf, len,
                  "M=%lld N=%lld K=%lld kernel=%s kid=%d mode=%s splits=%d tiles=%d (%dx%d) "
                  "k_iters=%d grid=%d group_m=%d xcd_remap=%d slots=%d lds=%d workspace=%zu%s",
                  (long long)M, (long long)N, (long long)K, ki->name, plan.kid,
                  mode_name(s.mode), s.splits, s.tiles, s.tiles_m, s.tiles_n, s.k_iters, s.grid,
                  s.group_m, s.xcd_remap, s.slots, ki->lds_bytes, plan.workspace, pack);
  }
  return GEMM_OK;
}

void gemm_f16_release_workspaces(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  for (auto it = g_ws.begin(); it != g_ws.end();) {
    if (it->first.first == dev) {
      (void)hipStreamSynchronize(it->first.second);
      (void)hipFree(it->second.ptr);
      it = g_ws.erase(it);
    } else {
      ++it;
    }
  }
}

int32_t gemm_f16_lds_chunk(int32_t chunks_per_row, int32_t block_dim, int32_t row,
                           int32_t chunk) {
  if (row < 0 || chunk < 0 || chunk >= chunks_per_row) return -1;
  if (chunks_per_row == 8 && block_dim == 32) return swz<8, 32>(row, chunk);
  if (chunks_per_row == 4 && block_dim == 32) return swz<4, 32>(row, chunk);
  if (chunks_per_row == 8 && block_dim == 16) return swz<8, 16>(row, chunk);
  if (chunks_per_row == 4 && block_dim == 16) return swz<4, 16>(row, chunk);
  return -1;
}

int64_t gemm_f16_schedule_dump(int64_t M, int64_t N, int64_t K, int64_t grid, int64_t* out,
                               int64_t cap, int64_t* k_iters, int64_t* tiles) {
  if (M <= 0 || N <= 0 || K <= 0 || cap < 0 || (cap > 0 && out == nullptr)) return -1;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return -1;
  Plan plan = reference_plan(M, N, K, -1);
  if (plan.kid < 0 || plan.kid == KID_GENERAL || plan.kid == KID_DIRECT) return -1;
  Sched s = plan.s;
  if (grid > 0) {
    if ((s.mode == MODE_STREAM_K || s.mode == MODE_DP_SK) &&
        grid > (int64_t)s.tiles * s.k_iters)
      return -1;
    s.grid = (int32_t)grid;
    set_shared_base(s);  // DP_SK: its whole rounds depend on the grid
  }
  if (k_iters) *k_iters = s.k_iters;
  if (tiles) *tiles = s.tiles;
  int64_t rows = 0;
  for (int32_t w = 0; w < s.grid; ++w) {
    const int32_t v = virtual_wg(w, s.grid, s.xcd_remap);
    Segment seg;
    for (int32_t n = 0; seg_at(s, v, n, &seg); ++n) {
      if (rows < cap) {
        int64_t* r = out + rows * 7;
        r[0] = w;
        r[1] = seg.tile;
        r[2] = seg.k_begin;
        r[3] = seg.k_end;
        r[4] = seg.role;
        r[5] = seg.contributors;
        r[6] = seg.index;
      }
      ++rows;
    }
  }
  return rows;
}


void gemm_f16_set_clock_probe(unsigned long long* counters) {
  g_clock_probe.store(counters, std::memory_order_relaxed);
}

void gemm_f16_set_plan_override(const char* text) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  g_override = parse_override(text);
  g_override_set = true;
  g_plans.clear();
}

}  // extern "C"
