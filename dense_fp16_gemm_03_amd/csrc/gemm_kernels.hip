// gfx950 kernels for C = A * B^T (binary16 in, binary32 accumulate and out).
//
// Tiled kernel, per workgroup and per unit of the persistent schedule:
//   * global -> LDS: buffer_load_dwordx4 ... lds (16 bytes a lane, written by
//     the load unit straight into LDS, no registers), the gfx950 counterpart
//     of the asynchronous copies of the handbook page "Asynchronous copies and
//     the Hopper/Blackwell features" (section "cp.async and multi-stage
//     pipelines"). Each tile row of BK halves is stored with its 16-byte
//     chunks XOR-permuted by a function of the row, so the MFMA fragment
//     reads below hit distinct LDS banks (the role of the 128-byte swizzle in
//     that page's TMA section).
//   * a ring of STAGES such buffers: loads for k-iteration i+STAGES-1 are in
//     flight while iteration i computes; a wait on the load counter plus a
//     workgroup barrier hands a stage over, and the tail waits on fewer loads
//     when no more are issued (the "commit empty groups" rule of that page).
//   * LDS -> registers with ds_read_b128 (8 halves a lane) and
//     v_mfma_f32_32x32x16_f16 into per-wave register-blocked accumulators.
//     The next stage is handed over before the last k-step's MFMAs are issued,
//     so its first fragments load while those MFMAs run ("asking a stage
//     ahead" in "SASS-Level Kernel Generation for Blackwell", section "Inside
//     the kernels").
//   * the B tile is fed as the MFMA's first operand and the A tile as its
//     second (SwapAB in the same section), so each lane ends up holding runs
//     of 4 consecutive columns of C and stores them as one 16-byte write,
//     straight from the registers ("stored from the registers").
//   * split-K / stream-K: the share holding a tile's first k-iteration stores
//     the tile and raises the tile's flag; every other share waits for the
//     flag and adds its partial sums with fp32 atomics at device scope
//     (section "Inside the kernels", "Stream-K and split-K, added in the L2").
//     The last adder puts the flag and arrival count back to zero, so the
//     workspace is zero whenever no call is running.
#include "gemm_kernels.h"

#include <hip/hip_runtime.h>

namespace g16 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Flag waits that gave up (see kSpinLimit); read by read_wait_timeouts().
__device__ unsigned long long g_wait_timeouts = 0;

namespace {

// A lane whose buffer offset is >= the descriptor's record count reads zeros:
// rows past M and k past K are masked this way.
constexpr uint32_t kMaskedOffset = 0x80000000u;
constexpr int32_t kNumRecords = 0x7FFFFFF0;
constexpr int32_t kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format
// Polls of a tile flag before a waiting workgroup gives up (~seconds).
constexpr uint32_t kSpinLimit = 1u << 22;

template <int BM_, int BN_, int BK_, int STAGES_, int WGM_, int WGN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int WGM = WGM_, WGN = WGN_;
  static constexpr int WAVES = WGM * WGN;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  static constexpr int FM = WM / 32, FN = WN / 32;    // 32x32 MFMA blocks per wave
  static constexpr int KSTEPS = BK / 16;              // MFMA k-steps per stage
  static constexpr int ROW_BYTES = BK * 2;
  static constexpr int CHUNKS = BK / 8;               // 16-byte chunks per tile row
  static constexpr int RPL = 64 / CHUNKS;             // tile rows per 1 KiB wave load
  static constexpr int A_BYTES = BM * ROW_BYTES;
  static constexpr int B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGE_BYTES * STAGES;
  static constexpr int A_LOADS = BM / RPL / WAVES;    // per wave per stage
  static constexpr int B_LOADS = BN / RPL / WAVES;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int WAVES_PER_EU = WAVES / 4;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "every wave loads A and B");
  static_assert(A_LOADS * RPL * WAVES == BM && B_LOADS * RPL * WAVES == BN, "load split");
  static_assert(STAGES >= 2 && LOADS * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 163840, "gfx950 LDS limit");
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
};

// Position of logical 16-byte chunk `chunk` of tile row `row` inside the row.
// CHUNKS == 8: f(row) = (row ^ (row >> 3)) & 7. Any 8 consecutive rows get
// distinct f, and so do the 8 even (and the 8 odd) rows of any 16 aligned
// rows, so the 8- and 16-lane phases of a ds_read_b128 fragment read (lanes
// on consecutive rows, one chunk) never meet in a bank.
// CHUNKS == 4: the same property for 64-byte rows with f in 0..3.
template <int CHUNKS>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (CHUNKS == 8) {
    return chunk ^ ((row ^ (row >> 3)) & 7);
  } else {
    return chunk ^ (((row >> 1) ^ (row >> 3)) & 3);
  }
}

// s_waitcnt immediates (gfx9 layout): vmcnt bits [3:0] and [15:14],
// expcnt [6:4], lgkmcnt [11:8]; a field at its maximum does not wait.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kLgkmZero = 15 | (7 << 4) | (0 << 8) | (3 << 14);

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// Wait until at most `pending` whole stages of this wave's loads are in flight.
template <class C>
__device__ __forceinline__ void wait_vm_stages(int pending) {
  if constexpr (C::STAGES == 2) {
    wait_vm<0>();
  } else if constexpr (C::STAGES == 3) {
    if (pending >= 1) wait_vm<C::LOADS>(); else wait_vm<0>();
  } else if constexpr (C::STAGES == 4) {
    if (pending >= 2) wait_vm<2 * C::LOADS>();
    else if (pending == 1) wait_vm<C::LOADS>();
    else wait_vm<0>();
  } else {
    static_assert(C::STAGES <= 4, "add a case");
  }
}

__device__ __forceinline__ void wait_lgkm_zero() { __builtin_amdgcn_s_waitcnt(kLgkmZero); }

template <class C>
struct Frags {
  half8 a[C::FM];
  half8 b[C::FN];
};

// Per-lane LDS byte offsets of the fragments of k-step ks (relative to a stage).
// A fragment fm: rows wm*WM + fm*32 + lane%32, k = 16*ks + 8*(lane/32) .. +7.
template <class C>
__device__ __forceinline__ int frag_off(int tile_row, int ks, int lane) {
  const int c = 2 * ks + (lane >> 5);
  return tile_row * C::ROW_BYTES + swz<C::CHUNKS>(tile_row, c) * 16;
}

template <class C>
__device__ __forceinline__ void read_frags(const char* stage, int ks, int wm, int wn, int lane,
                                           Frags<C>& f) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int row = wm * C::WM + i * 32 + (lane & 31);
    f.a[i] = *reinterpret_cast<const half8*>(stage + frag_off<C>(row, ks, lane));
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const int row = wn * C::WN + j * 32 + (lane & 31);
    f.b[j] = *reinterpret_cast<const half8*>(stage + C::A_BYTES + frag_off<C>(row, ks, lane));
  }
}

template <class C>
__device__ __forceinline__ void mfma_step(const Frags<C>& f, f32x16 (&acc)[C::FM][C::FN]) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// Buffer offsets (bytes, relative to the tile's first row at k = 0) of this
// lane's 16-byte pieces of one stage, and the logical chunk each one holds.
template <class C, int LOADS_OF>
struct LoadMap {
  uint32_t off[LOADS_OF];
  int32_t chunk8[LOADS_OF];  // first k (relative to the stage) of the piece
};

template <class C, int LOADS_OF>
__device__ __forceinline__ void make_load_map(LoadMap<C, LOADS_OF>& m, int wave, int lane,
                                              int rows_valid, int64_t ld) {
#pragma unroll
  for (int j = 0; j < LOADS_OF; ++j) {
    const int group = wave * LOADS_OF + j;
    const int row = group * C::RPL + lane / C::CHUNKS;
    const int chunk = swz<C::CHUNKS>(row, lane % C::CHUNKS);  // XOR: its own inverse
    m.chunk8[j] = chunk * 8;
    m.off[j] = row < rows_valid ? (uint32_t)(row * ld * 2 + chunk * 16) : kMaskedOffset;
  }
}

// Issue this wave's share of one stage: A pieces then B pieces.
// k0 = first k of the stage; `tail` masks pieces at k >= K.
template <class C>
__device__ __forceinline__ void issue_stage(char* stage, __amdgpu_buffer_rsrc_t ra,
                                            __amdgpu_buffer_rsrc_t rb,
                                            const LoadMap<C, C::A_LOADS>& ma,
                                            const LoadMap<C, C::B_LOADS>& mb, int wave, int k0,
                                            bool tail, int K) {
  const int soff = k0 * 2;
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    uint32_t off = ma.off[j];
    if (tail && k0 + ma.chunk8[j] >= K) off = kMaskedOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        ra, (lds_void_ptr)(stage + (wave * C::A_LOADS + j) * 1024), 16, off, soff, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    uint32_t off = mb.off[j];
    if (tail && k0 + mb.chunk8[j] >= K) off = kMaskedOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (lds_void_ptr)(stage + C::A_BYTES + (wave * C::B_LOADS + j) * 1024), 16, off, soff,
        0, 0);
  }
}

// Bounded wait for a tile's flag; counts a give-up in g_wait_timeouts.
__device__ void wait_flag(uint32_t* flag) {
  uint32_t polls = 0;
  while (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != 1u) {
    __builtin_amdgcn_s_sleep(2);
    if (++polls == kSpinLimit) {
      atomicAdd(&g_wait_timeouts, 1ull);
      break;
    }
  }
}

// Write (role ONLY / STORER) or add (role ADDER) the wave's accumulators to C.
// Lane l holds, for block (i, j) and register v = 4g + q:
//   row    m = m_base + 32 i + l % 32
//   column n = n_base + 32 j + 8 g + 4 (l / 32) + q
template <class C>
__device__ __forceinline__ void epilogue(const GemmParams& p, const f32x16 (&acc)[C::FM][C::FN],
                                         int m_base, int n_base, int lane, bool add) {
  const bool full = m_base + C::WM <= p.M && n_base + C::WN <= p.N;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int m = m_base + i * 32 + (lane & 31);
    float* crow = p.C + (int64_t)m * p.ldc;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n_base + j * 32 + 8 * g + 4 * (lane >> 5);
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3]};
        if (!add) {
          if (full && p.c_vec4) {
            *reinterpret_cast<f32x4*>(crow + n) = v;
          } else if (m < p.M) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n + q < p.N) crow[n + q] = v[q];
          }
        } else if (m < p.M) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < p.N) unsafeAtomicAdd(crow + n + q, v[q]);
        }
      }
    }
  }
}

template <class C>
__global__ __launch_bounds__(C::THREADS)
__attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU, C::WAVES_PER_EU)))
void gemm_tiled_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WGN;
  const int wn = wave % C::WGN;
  const int v = virtual_wg(blockIdx.x, p.s.grid);
  uint32_t* flags = p.flags;
  uint32_t* counts = p.flags + p.s.tiles;
  const bool k_tail = (p.K % C::BK) != 0;

  Segment seg;
  for (int n = 0; seg_at(p.s, v, n, &seg); ++n) {
    const int m0 = seg.tm * C::BM;
    const int n0 = seg.tn * C::BN;
    const int nk = seg.k_end - seg.k_begin;

    // Operand windows for this tile: rows m0.. of A and n0.. of B.
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.A + (int64_t)m0 * p.lda), (short)0, kNumRecords, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.B + (int64_t)n0 * p.ldb), (short)0, kNumRecords, kBufferWord3);
    LoadMap<C, C::A_LOADS> ma;
    LoadMap<C, C::B_LOADS> mb;
    make_load_map<C, C::A_LOADS>(ma, wave, lane, p.M - m0, p.lda);
    make_load_map<C, C::B_LOADS>(mb, wave, lane, p.N - n0, p.ldb);

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

    // Every wave has finished reading LDS from the previous unit.
    __syncthreads();

    const int last_kt = p.s.k_iters - 1;
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s) {
      if (s < nk) {
        const int kt = seg.k_begin + s;
        issue_stage<C>(smem + s * C::STAGE_BYTES, ra, rb, ma, mb, wave, kt * C::BK,
                       k_tail && kt == last_kt, p.K);
      }
    }

    Frags<C> cur, nxt;
    if (nk > 0) {
      wait_vm_stages<C>(min_of(C::STAGES - 2, nk - 1));
      __syncthreads();
      read_frags<C>(smem, 0, wm, wn, lane, cur);
    }

    for (int it = 0; it < nk; ++it) {
      const int st = it % C::STAGES;
      const char* stage = smem + st * C::STAGE_BYTES;
      // The buffer of iteration it-1 was released at the last barrier.
      if (it + C::STAGES - 1 < nk) {
        const int kt = seg.k_begin + it + C::STAGES - 1;
        issue_stage<C>(smem + ((it + C::STAGES - 1) % C::STAGES) * C::STAGE_BYTES, ra, rb, ma,
                       mb, wave, kt * C::BK, k_tail && kt == last_kt, p.K);
      }
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS - 1; ++ks) {
        read_frags<C>(stage, ks + 1, wm, wn, lane, nxt);
        mfma_step<C>(cur, acc);
        cur = nxt;
      }
      if (it + 1 < nk) {
        // Hand over the next stage, then start its first reads while the
        // last k-step of this stage runs on the matrix cores.
        wait_vm_stages<C>(min_of(C::STAGES - 2, nk - 2 - it));
        wait_lgkm_zero();
        __syncthreads();
        read_frags<C>(smem + ((it + 1) % C::STAGES) * C::STAGE_BYTES, 0, wm, wn, lane, nxt);
      }
      mfma_step<C>(cur, acc);
      cur = nxt;
    }

    const int m_base = m0 + wm * C::WM;
    const int n_base = n0 + wn * C::WN;
    if (seg.role != ROLE_ADDER) {
      epilogue<C>(p, acc, m_base, n_base, lane, false);
      if (seg.role == ROLE_STORER) {
        __syncthreads();
        if (tid == 0) __hip_atomic_store(&flags[seg.tile], 1u, __ATOMIC_RELEASE,
                                         __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      if (tid == 0) wait_flag(&flags[seg.tile]);
      __syncthreads();
      epilogue<C>(p, acc, m_base, n_base, lane, true);
      __syncthreads();
      if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(&counts[seg.tile], 1u, __ATOMIC_ACQ_REL,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        if (before == (uint32_t)(seg.contributors - 2)) {
          // Last adder: every adder has seen the flag; leave both words zero.
          __hip_atomic_store(&counts[seg.tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&flags[seg.tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// General kernel: any shape, stride and (element-natural) alignment. One
// workgroup of 4 waves per 64 x 64 tile of C, each wave a 32 x 32 block;
// operands go straight from global memory into MFMA registers, element by
// element with bounds checks. Slow; taken only when the tiled kernels'
// alignment rules do not hold.
__global__ __launch_bounds__(256) void gemm_general_kernel(GemmParams p, int32_t tiles_n) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tm = blockIdx.x / tiles_n;
  const int tn = blockIdx.x % tiles_n;
  const int m0 = tm * 64 + (wave >> 1) * 32;
  const int n0 = tn * 64 + (wave & 1) * 32;
  const int ar = m0 + (lane & 31);
  const int br = n0 + (lane & 31);
  const int kk = 8 * (lane >> 5);
  const bool a_ok = ar < p.M;
  const bool b_ok = br < p.N;
  const uint16_t* arow = p.A + (int64_t)(a_ok ? ar : 0) * p.lda;
  const uint16_t* brow = p.B + (int64_t)(b_ok ? br : 0) * p.ldb;
  f32x16 acc = {};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    half8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = k0 + kk + e;
      const bool kin = k < p.K;
      a[e] = (a_ok && kin) ? __builtin_bit_cast(_Float16, arow[k]) : (_Float16)0;
      b[e] = (b_ok && kin) ? __builtin_bit_cast(_Float16, brow[k]) : (_Float16)0;
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, acc, 0, 0, 0);
  }
  const int m = m0 + (lane & 31);
  if (m < p.M) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = n0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (n < p.N) p.C[(int64_t)m * p.ldc + n] = acc[r];
    }
  }
}

using C0 = Cfg<256, 256, 64, 2, 2, 2>;
using C1 = Cfg<256, 256, 32, 4, 2, 2>;
using C2 = Cfg<256, 256, 64, 2, 2, 4>;
using C3 = Cfg<256, 128, 64, 3, 2, 2>;
using C4 = Cfg<128, 128, 64, 4, 2, 2>;
using C5 = Cfg<128, 64, 64, 4, 2, 2>;
using C6 = Cfg<64, 64, 64, 4, 2, 2>;

template <class C>
constexpr KernelInfo info_of(const char* name) {
  return KernelInfo{C::BM, C::BN, C::BK, C::STAGES, C::WAVES, C::LDS_BYTES, name};
}

constexpr KernelInfo kInfos[KID_COUNT] = {
    info_of<C0>("256x256x64_s2_w4"), info_of<C1>("256x256x32_s4_w4"),
    info_of<C2>("256x256x64_s2_w8"), info_of<C3>("256x128x64_s3_w4"),
    info_of<C4>("128x128x64_s4_w4"), info_of<C5>("128x64x64_s4_w4"),
    info_of<C6>("64x64x64_s4_w4"),
};

template <class C>
hipError_t launch_cfg(const GemmParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_tiled_kernel<C>, dim3(p.s.grid), dim3(C::THREADS), 0, stream, p);
  return hipGetLastError();
}

template <class C>
int32_t occupancy_cfg() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_tiled_kernel<C>, C::THREADS, 0) !=
      hipSuccess)
    return 0;
  return n;
}

}  // namespace

const KernelInfo* kernel_info(int32_t kid) {
  if (kid < 0 || kid >= KID_COUNT) return nullptr;
  return &kInfos[kid];
}

hipError_t launch_tiled(int32_t kid, const GemmParams& p, hipStream_t stream) {
  switch (kid) {
    case KID_256x256x64_S2_W4: return launch_cfg<C0>(p, stream);
    case KID_256x256x32_S4_W4: return launch_cfg<C1>(p, stream);
    case KID_256x256x64_S2_W8: return launch_cfg<C2>(p, stream);
    case KID_256x128x64_S3_W4: return launch_cfg<C3>(p, stream);
    case KID_128x128x64_S4_W4: return launch_cfg<C4>(p, stream);
    case KID_128x64x64_S4_W4: return launch_cfg<C5>(p, stream);
    case KID_64x64x64_S4_W4: return launch_cfg<C6>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

int32_t tiled_occupancy(int32_t kid) {
  switch (kid) {
    case KID_256x256x64_S2_W4: return occupancy_cfg<C0>();
    case KID_256x256x32_S4_W4: return occupancy_cfg<C1>();
    case KID_256x256x64_S2_W8: return occupancy_cfg<C2>();
    case KID_256x128x64_S3_W4: return occupancy_cfg<C3>();
    case KID_128x128x64_S4_W4: return occupancy_cfg<C4>();
    case KID_128x64x64_S4_W4: return occupancy_cfg<C5>();
    case KID_64x64x64_S4_W4: return occupancy_cfg<C6>();
    default: return 0;
  }
}

hipError_t launch_general(const GemmParams& p, hipStream_t stream) {
  const int64_t tiles_m = (p.M + 63) / 64;
  const int64_t tiles_n = (p.N + 63) / 64;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_general_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, p,
                     (int32_t)tiles_n);
  return hipGetLastError();
}

hipError_t read_wait_timeouts(unsigned long long* out, bool reset) {
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_wait_timeouts), sizeof(*out), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess || !reset) return e;
  const unsigned long long zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_wait_timeouts), &zero, sizeof(zero), 0,
                           hipMemcpyHostToDevice);
}

}  // namespace g16
