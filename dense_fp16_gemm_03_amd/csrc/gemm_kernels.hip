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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

namespace {

// A lane whose buffer offset is >= the descriptor's record count reads zeros:
// rows past M and k past K are masked this way.
constexpr uint32_t kMaskedOffset = 0x80000000u;
constexpr int32_t kNumRecords = 0x7FFFFFF0;
constexpr int32_t kBufferWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kReduceThreads = 256;

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

__device__ __forceinline__ void wait_lgkm_zero() { __builtin_amdgcn_s_waitcnt(kLgkmZero); }

// Workgroup barrier for the LDS ring: s_barrier alone. __syncthreads() would
// also wait for every outstanding global load (its fence drains vmcnt), which
// empties the prefetch ring at each stage; the waits the ring needs are the
// explicit vmcnt / lgkmcnt ones placed before each call. The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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

// Buffer offsets (bytes, relative to the tile's first row at k = 0) of this
// lane's 16-byte pieces of one stage, and for each piece the bound its stage's
// first k must stay below for the piece to be loaded (else it is masked and the
// LDS slot is zero-filled without a memory access).
template <class C, int LOADS_OF>
struct LoadMap {
  uint32_t off[LOADS_OF];
  int32_t lim[LOADS_OF];
};

// k_limit: loads cover k < k_limit only (the unit's k range, and K).
template <class C, int LOADS_OF>
__device__ __forceinline__ void make_load_map(LoadMap<C, LOADS_OF>& m, int wave, int lane,
                                              int rows_valid, int64_t ld, int k_limit) {
#pragma unroll
  for (int j = 0; j < LOADS_OF; ++j) {
    const int group = wave * LOADS_OF + j;
    const int row = group * C::RPL + lane / C::CHUNKS;
    const int chunk = swz<C::CHUNKS>(row, lane % C::CHUNKS);  // XOR: its own inverse
    m.off[j] = row < rows_valid ? (uint32_t)(row * ld * 2 + chunk * 16) : kMaskedOffset;
    m.lim[j] = k_limit - chunk * 8;
  }
}

struct Operands {
  __amdgpu_buffer_rsrc_t ra, rb;
};

// Load j (A pieces first, then B pieces) of the stage whose first k is k0,
// into the stage buffer `dst`.
template <class C>
__device__ __forceinline__ void issue_one(int j, char* dst, const Operands& op,
                                          const LoadMap<C, C::A_LOADS>& ma,
                                          const LoadMap<C, C::B_LOADS>& mb, int wave, int k0) {
  if (j < C::A_LOADS) {
    const uint32_t off = k0 < ma.lim[j] ? ma.off[j] : kMaskedOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        op.ra, (lds_void_ptr)(dst + (wave * C::A_LOADS + j) * 1024), 16, off, k0 * 2, 0, 0);
  } else {
    const int jb = j - C::A_LOADS;
    const uint32_t off = k0 < mb.lim[jb] ? mb.off[jb] : kMaskedOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        op.rb, (lds_void_ptr)(dst + C::A_BYTES + (wave * C::B_LOADS + jb) * 1024), 16, off,
        k0 * 2, 0, 0);
  }
}

// How many of n items spread evenly over nm MFMAs fall after MFMA m.
constexpr int items_at(int n, int nm, int m) {
  int c = 0;
  for (int r = 0; r < n; ++r) c += (r * nm / n == m);
  return c;
}

// Scheduling groups for one k-step: MFMA m, then its reads, then its loads.
template <int NM, int NR, int NL, int M>
__device__ __forceinline__ void sched_pattern() {
  if constexpr (M < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int nr = items_at(NR, NM, M);
    constexpr int nl = items_at(NL, NM, M);
    if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);  // LDS reads
    if constexpr (nl > 0) __builtin_amdgcn_sched_group_barrier(0x010, nl, 0);  // loads
    sched_pattern<NM, NR, NL, M + 1>();
  }
}

// One MFMA k-step on `cur`, interleaved with (a) the fragment reads of the
// next k-step (k-step rks of stage buffer rstage) into `nxt` and (b) loads
// [LFIRST, LFIRST + NL) of the stage being prefetched into lstage. The
// scheduling groups pin the interleave: after each MFMA come the reads and
// loads assigned to it, so neither the LDS reads nor the load issue (which
// can stall while the address FIFO is full) holds back a run of MFMAs.
template <class C, int LFIRST, int NL>
__device__ __forceinline__ void kstep(f32x16 (&acc)[C::FM][C::FN], const Frags<C>& cur,
                                      Frags<C>& nxt, const char* rstage, int rks, int wm, int wn,
                                      int lane, char* lstage, const Operands& op,
                                      const LoadMap<C, C::A_LOADS>& ma,
                                      const LoadMap<C, C::B_LOADS>& mb, int wave, int k0) {
  constexpr int NM = C::FM * C::FN;
  constexpr int NR = C::FM + C::FN;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int i = m / C::FN, j = m % C::FN;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (r * NM / NR == m) {
        if (r < C::FM) {
          const int row = wm * C::WM + r * 32 + (lane & 31);
          nxt.a[r] = *reinterpret_cast<const half8*>(rstage + frag_off<C>(row, rks, lane));
        } else {
          const int row = wn * C::WN + (r - C::FM) * 32 + (lane & 31);
          nxt.b[r - C::FM] =
              *reinterpret_cast<const half8*>(rstage + C::A_BYTES + frag_off<C>(row, rks, lane));
        }
      }
    }
#pragma unroll
    for (int l = 0; l < NL; ++l)
      if (NL > 0 && l * NM / NL == m) issue_one<C>(LFIRST + l, lstage, op, ma, mb, wave, k0);
  }
  sched_pattern<NM, NR, NL, 0>();
}

// The k-steps of one stage. K-steps 0..LK-1 also issue the loads of the stage
// entering the ring (all in k-step 0 with a 2-deep ring, whose next stage must
// land within this one). Before the last k-step the next stage is handed over
// (its loads landed in every wave, all reads of the freed buffer done), and
// that k-step reads the next stage's first fragments.
template <class C, int KS>
__device__ __forceinline__ void run_ksteps(f32x16 (&acc)[C::FM][C::FN], Frags<C> (&fr)[2],
                                           const char* stage, const char* nstage, int wm, int wn,
                                           int lane, char* lstage, const Operands& op,
                                           const LoadMap<C, C::A_LOADS>& ma,
                                           const LoadMap<C, C::B_LOADS>& mb, int wave, int k0) {
  static_assert(C::KSTEPS % 2 == 0, "fragment double buffer alternates per k-step");
  constexpr int LK = C::STAGES == 2 ? 1 : C::KSTEPS - 1;
  constexpr int LF = KS < LK ? KS * C::LOADS / LK : 0;
  constexpr int NL = KS < LK ? (KS + 1) * C::LOADS / LK - LF : 0;
  if constexpr (KS < C::KSTEPS - 1) {
    kstep<C, LF, NL>(acc, fr[KS & 1], fr[(KS + 1) & 1], stage, KS + 1, wm, wn, lane, lstage, op,
                     ma, mb, wave, k0);
    run_ksteps<C, KS + 1>(acc, fr, stage, nstage, wm, wn, lane, lstage, op, ma, mb, wave, k0);
  } else {
    wait_vm<C::LOADS * (C::STAGES - 2)>();
    wait_lgkm_zero();
    lds_barrier();
    kstep<C, LF, NL>(acc, fr[KS & 1], fr[(KS + 1) & 1], nstage, 0, wm, wn, lane, lstage, op, ma,
                     mb, wave, k0);
  }
}

// Partial tiles in the workspace are kept in the accumulators' own layout:
// float4 number (((i * FN + j) * 4 + g) * WAVES + wave) * 64 + lane holds
// registers 4g..4g+3 of block (i, j) of that wave and lane, so each store and
// each load of a wave covers 1 KiB of consecutive bytes.
template <class C>
__device__ __forceinline__ void write_partial(f32x4* part, const f32x16 (&acc)[C::FM][C::FN],
                                              int wave, int lane) {
  // Buffer stores: the tile's base in the descriptor, one per-lane offset, and
  // each store's fixed offset in a scalar register (no per-store addresses).
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)part, (short)0, kNumRecords, kBufferWord3);
  const int voff = (wave * 64 + lane) * 16;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, v), r, voff, ((i * C::FN + j) * 4 + g) * C::WAVES * 64 * 16,
            0);
      }
}

// Sums float4s [begin, end) of a tile's `shares` partials, over the shares in
// k order, and writes them to C (the tile's rows m0.., columns n0..).
template <class C>
__device__ __forceinline__ void reduce_range(const GemmParams& p, const f32x4* parts, int shares,
                                             int begin, int end, int m0, int n0) {
  constexpr int L = C::BM * C::BN / 4;  // float4s per partial tile
  constexpr int EB = 4;                 // elements per thread in flight
  constexpr int CB = 4;                 // partials per element in flight
  constexpr int T = kReduceThreads;
  for (int e0 = begin + (int)threadIdx.x; e0 < end; e0 += T * EB) {
    f32x4 sum[EB];
#pragma unroll
    for (int b = 0; b < EB; ++b) sum[b] = f32x4{};
    for (int c0 = 0; c0 < shares; c0 += CB) {
      f32x4 v[CB][EB];
#pragma unroll
      for (int cc = 0; cc < CB; ++cc)
#pragma unroll
        for (int b = 0; b < EB; ++b) {
          const int e = e0 + b * T;
          v[cc][b] = (c0 + cc < shares && e < end) ? parts[(int64_t)(c0 + cc) * L + e] : f32x4{};
        }
#pragma unroll
      for (int cc = 0; cc < CB; ++cc)
#pragma unroll
        for (int b = 0; b < EB; ++b) sum[b] += v[cc][b];
    }
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      const int e = e0 + b * T;
      if (e >= end) continue;
      const int lane = e % 64;
      const int wave = (e / 64) % C::WAVES;
      const int rest = e / (64 * C::WAVES);
      const int g = rest % 4;
      const int i = (rest / 4) / C::FN;
      const int j = (rest / 4) % C::FN;
      const int m = m0 + (wave / C::WGN) * C::WM + i * 32 + (lane & 31);
      const int n = n0 + (wave % C::WGN) * C::WN + j * 32 + 8 * g + 4 * (lane >> 5);
      if (m >= p.M) continue;
      float* crow = p.C + (int64_t)m * p.ldc;
      if (n + 3 < p.N && p.c_vec4) {
        *reinterpret_cast<f32x4*>(crow + n) = sum[b];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n + q < p.N) crow[n + q] = sum[b][q];
      }
    }
  }
}

// Write the wave's accumulators to C (a tile computed by one unit alone).
// Lane l holds, for block (i, j) and register v = 4g + q:
//   row    m = m_base + 32 i + l % 32
//   column n = n_base + 32 j + 8 g + 4 (l / 32) + q
template <class C>
__device__ __forceinline__ void epilogue(const GemmParams& p, const f32x16 (&acc)[C::FM][C::FN],
                                         int m_base, int n_base, int lane) {
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
        if (full && p.c_vec4) {
          *reinterpret_cast<f32x4*>(crow + n) = v;
        } else if (m < p.M) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < p.N) crow[n + q] = v[q];
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
  const int v = virtual_wg(blockIdx.x, p.s.grid, p.s.xcd_remap);

  Segment seg;
  for (int n = 0; seg_at(p.s, v, n, &seg); ++n) {
    const int m0 = seg.tm * C::BM;
    const int n0 = seg.tn * C::BN;
    const int nk = seg.k_end - seg.k_begin;
    // Loads cover this unit's k range only; the stages past its end that the
    // ring still issues are fully masked (zero-filled, no memory access).
    const int k_limit = min_of(p.K, seg.k_end * C::BK);

    // Operand windows for this tile: rows m0.. of A and n0.. of B.
    Operands op;
    op.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + (int64_t)m0 * p.lda), (short)0,
                                              kNumRecords, kBufferWord3);
    op.rb = __builtin_amdgcn_make_buffer_rsrc((void*)(p.B + (int64_t)n0 * p.ldb), (short)0,
                                              kNumRecords, kBufferWord3);
    LoadMap<C, C::A_LOADS> ma;
    LoadMap<C, C::B_LOADS> mb;
    make_load_map<C, C::A_LOADS>(ma, wave, lane, p.M - m0, p.lda, k_limit);
    make_load_map<C, C::B_LOADS>(mb, wave, lane, p.N - n0, p.ldb, k_limit);

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

    // The previous unit's loads have landed and every wave has finished
    // reading LDS, so the ring buffers can be refilled.
    wait_vm<0>();
    wait_lgkm_zero();
    lds_barrier();

#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s) {
#pragma unroll
      for (int j = 0; j < C::LOADS; ++j)
        issue_one<C>(j, smem + s * C::STAGE_BYTES, op, ma, mb, wave, (seg.k_begin + s) * C::BK);
    }

    Frags<C> fr[2];
    wait_vm<C::LOADS * (C::STAGES - 2)>();
    lds_barrier();
    read_frags<C>(smem, 0, wm, wn, lane, fr[0]);

    int st = 0;  // ring buffer holding stage `it`
    for (int it = 0; it < nk; ++it) {
      const int st_next = st + 1 == C::STAGES ? 0 : st + 1;
      const int st_load = st == 0 ? C::STAGES - 1 : st - 1;  // freed at the last barrier
      const char* stage = smem + st * C::STAGE_BYTES;
      char* lstage = smem + st_load * C::STAGE_BYTES;
      const int k0_load = (seg.k_begin + it + C::STAGES - 1) * C::BK;
      run_ksteps<C, 0>(acc, fr, stage, smem + st_next * C::STAGE_BYTES, wm, wn, lane, lstage, op,
                       ma, mb, wave, k0_load);
      st = st_next;
    }

    if (seg.role == ROLE_ONLY) {
      epilogue<C>(p, acc, m0 + wm * C::WM, n0 + wn * C::WN, lane);
    } else {
      // One share of a tile: its partial goes to the workspace; the reduce
      // kernel that follows on the stream sums the shares into C.
      write_partial<C>(p.partials + ((int64_t)seg.tile * p.s.slots + seg.index) * (C::BM * C::BN / 4),
                       acc, wave, lane);
    }
  }
}

// Shares of output tile t under schedule s (1: the tile was stored directly).
__device__ __forceinline__ int tile_shares(const Sched& s, int t) {
  if (s.mode == MODE_SPLIT) return s.splits;
  if (s.mode != MODE_STREAM_K) return 1;
  const int64_t lo = (int64_t)t * s.k_iters;
  return (int)(sk_owner(s, lo + s.k_iters - 1) - sk_owner(s, lo) + 1);
}

// Reduce pass for split-K / stream-K: workgroup b handles slice b % slices
// of tile b / slices. Partials are summed in k order, so the result does not
// depend on timing.
template <class C>
__global__ __launch_bounds__(kReduceThreads) void gemm_reduce_kernel(GemmParams p, int32_t slices) {
  constexpr int L = C::BM * C::BN / 4;
  const int t = blockIdx.x / slices;
  const int slice = blockIdx.x % slices;
  const int shares = tile_shares(p.s, t);
  if (shares <= 1) return;
  int tm, tn;
  tile_coords(p.s, t, &tm, &tn);
  const int begin = (int)((int64_t)slice * L / slices);
  const int end = (int)((int64_t)(slice + 1) * L / slices);
  reduce_range<C>(p, p.partials + (int64_t)t * p.s.slots * L, shares, begin, end, tm * C::BM,
                  tn * C::BN);
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
using C7 = Cfg<256, 256, 32, 5, 2, 2>;
using C8 = Cfg<256, 256, 32, 4, 2, 4>;
using C9 = Cfg<256, 256, 32, 5, 2, 4>;

template <class C>
constexpr KernelInfo info_of(const char* name) {
  return KernelInfo{C::BM, C::BN, C::BK, C::STAGES, C::WAVES, C::LDS_BYTES, name};
}

constexpr KernelInfo kInfos[KID_COUNT] = {
    info_of<C0>("256x256x64_s2_w4"), info_of<C1>("256x256x32_s4_w4"),
    info_of<C2>("256x256x64_s2_w8"), info_of<C3>("256x128x64_s3_w4"),
    info_of<C4>("128x128x64_s4_w4"), info_of<C5>("128x64x64_s4_w4"),
    info_of<C6>("64x64x64_s4_w4"), info_of<C7>("256x256x32_s5_w4"),
    info_of<C8>("256x256x32_s4_w8"), info_of<C9>("256x256x32_s5_w8"),
};

template <class C>
hipError_t launch_cfg(const GemmParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_tiled_kernel<C>, dim3(p.s.grid), dim3(C::THREADS), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.s.mode == MODE_DATA_PARALLEL) return e;
  // Slices per tile: enough workgroups to cover the CUs, at least 4 KiB each.
  const int max_slices = C::BM * C::BN / 4 / 256;
  int slices = (256 + p.s.tiles - 1) / p.s.tiles;
  if (slices > max_slices) slices = max_slices;
  if (slices < 1) slices = 1;
  hipLaunchKernelGGL(gemm_reduce_kernel<C>, dim3(p.s.tiles * slices), dim3(kReduceThreads), 0,
                     stream, p, slices);
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
    case KID_256x256x32_S5_W4: return launch_cfg<C7>(p, stream);
    case KID_256x256x32_S4_W8: return launch_cfg<C8>(p, stream);
    case KID_256x256x32_S5_W8: return launch_cfg<C9>(p, stream);
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
    case KID_256x256x32_S5_W4: return occupancy_cfg<C7>();
    case KID_256x256x32_S4_W8: return occupancy_cfg<C8>();
    case KID_256x256x32_S5_W8: return occupancy_cfg<C9>();
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

}  // namespace g16
