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
//     workgroup barrier hands a stage over. Past the end of K the ring still
//     issues (fully masked) loads, so every wait counts the same number of
//     loads; that page makes its pipeline's group count uniform the same way.
//   * LDS -> registers with ds_read_b128 (8 halves a lane) and an fp16 MFMA
//     (v_mfma_f32_32x32x16_f16 or v_mfma_f32_16x16x32_f16) into per-wave
//     register-blocked accumulators. The next stage is handed over before the
//     last k-step's MFMAs are issued, so its first fragments load while those
//     MFMAs run (requesting data one stage early, as "SASS-Level Kernel
//     Generation for Blackwell" does, section "Inside the kernels").
//   * the B tile is fed as the MFMA's first operand and the A tile as its
//     second (SwapAB in the same section), so each lane ends up holding runs
//     of 4 consecutive columns of C and stores them as one 16-byte write,
//     straight from the registers with no staging through LDS.
//   * split-K / stream-K (section "Inside the kernels", where the shares of a
//     tile are added in the L2): a tile whose k-iterations are shared among
//     workgroups is not added in place. Every share writes its fp32 partial
//     tile to a workspace slot, and a reduce kernel that follows on the same
//     stream sums the slots of each tile in k order and writes C, so the
//     result does not depend on timing and needs no flags or atomics.
#include "gemm_kernels.h"
#include "gemm_lds_layout.h"

#include <hip/hip_runtime.h>

namespace g16 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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
// Buffer-store cache policy for C in the ping-pong kernels: streaming and
// write-through to the system coherence point (nt sc1). Their rounds of
// 256x256 tiles write tens of MiB of C at once; measured faster than
// streaming stores alone.
constexpr int kStoreNtSc1 = 2 | 16;

// The two MFMA shapes with fp32 accumulation on gfx950, for binary16 (DT_F16)
// or bfloat16 (DT_BF16) operands. Both take 8 elements of each operand per
// lane; the B tile is the first operand and the A tile the second (SwapAB),
// so a block's accumulators run along N.
//   32x32x16: operand lane l holds row l % 32, k = 8 (l / 32) .. +7 of the
//     k-step; accumulator register 4g + q of lane l is row (m) l % 32,
//     column (n) 8g + 4 (l / 32) + q of the block.
//   16x16x32: operand lane l holds row l % 16, k = 8 (l / 16) .. +7;
//     accumulator register q of lane l is row l % 16, column 4 (l / 16) + q.
// The operand layouts do not depend on the element type. On random data the
// 16x16x32 form reaches a higher sustained clock under the board's power
// limit, for the same work.
template <int MI>
struct MmaShape;

template <>
struct MmaShape<32> {
  static constexpr int DIM = 32;    // rows (and columns) of an accumulator block
  static constexpr int KW = 16;     // k per instruction
  static constexpr int GROUPS = 4;  // runs of 4 consecutive columns per lane
  typedef f32x16 acc_t;
  static __device__ __forceinline__ int frag_row(int lane) { return lane & 31; }
  static __device__ __forceinline__ int frag_chunk(int ks, int lane) { return 2 * ks + (lane >> 5); }
  static __device__ __forceinline__ int acc_m(int lane) { return lane & 31; }
  static __device__ __forceinline__ int acc_n(int g, int lane) { return 8 * g + 4 * (lane >> 5); }
};

template <>
struct MmaShape<16> {
  static constexpr int DIM = 16;
  static constexpr int KW = 32;
  static constexpr int GROUPS = 1;
  typedef f32x4 acc_t;
  static __device__ __forceinline__ int frag_row(int lane) { return lane & 15; }
  static __device__ __forceinline__ int frag_chunk(int ks, int lane) { return 4 * ks + (lane >> 4); }
  static __device__ __forceinline__ int acc_m(int lane) { return lane & 15; }
  static __device__ __forceinline__ int acc_n(int, int lane) { return 4 * (lane >> 4); }
};

template <int MI, int DT>
struct Mma;

template <>
struct Mma<32, DT_F16> : MmaShape<32> {
  typedef half8 frag_t;
  typedef _Float16 elem_t;
  static __device__ __forceinline__ acc_t mma(frag_t b, frag_t a, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c, 0, 0, 0);
  }
};

template <>
struct Mma<16, DT_F16> : MmaShape<16> {
  typedef half8 frag_t;
  typedef _Float16 elem_t;
  static __device__ __forceinline__ acc_t mma(frag_t b, frag_t a, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
  }
};

template <>
struct Mma<32, DT_BF16> : MmaShape<32> {
  typedef bf16x8 frag_t;
  typedef __bf16 elem_t;
  static __device__ __forceinline__ acc_t mma(frag_t b, frag_t a, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
  }
};

template <>
struct Mma<16, DT_BF16> : MmaShape<16> {
  typedef bf16x8 frag_t;
  typedef __bf16 elem_t;
  static __device__ __forceinline__ acc_t mma(frag_t b, frag_t a, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, c, 0, 0, 0);
  }
};

// RS_: when the fragment reads of the next k-step are issued. 0: spread
// evenly over the k-step's MFMAs; 1: each right after the last MFMA that uses
// the fragment it replaces, so the current and next fragments barely overlap
// in registers (for register-bound variants).
// PP_: 1 selects the ping-pong main loop (gemm_pingpong_kernel, 8 waves), 2 the
// same loop over two 64-wide stages (gemm_pingpong64_kernel).
// DT_: operand element type (DT_F16 or DT_BF16).
template <int BM_, int BN_, int BK_, int STAGES_, int WGM_, int WGN_, int MI_ = 32, int RS_ = 0,
          int PP_ = 0, int DT_ = DT_F16>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int WGM = WGM_, WGN = WGN_;
  static constexpr int MI = MI_;
  static constexpr int RS = RS_;
  static constexpr int PP = PP_;
  static constexpr int DT = DT_;
  using M = Mma<MI, DT>;
  using acc_t = typename M::acc_t;
  static constexpr int WAVES = WGM * WGN;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  static constexpr int FM = WM / M::DIM, FN = WN / M::DIM;  // MFMA blocks per wave
  static constexpr int KSTEPS = BK / M::KW;                 // MFMA k-steps per stage
  static constexpr int ROW_BYTES = BK * 2;
  static constexpr int CHUNKS = BK / 8;               // 16-byte chunks per tile row
  static constexpr int RPL = 64 / CHUNKS;             // tile rows per 1 KiB wave load
  static constexpr int A_BYTES = BM * ROW_BYTES;
  static constexpr int B_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  // PP 3 keeps the A and B halves of its 64-wide stages in STAGES separate
  // slots of one half each (gemm_pingpong_ring_kernel).
  static constexpr int LDS_BYTES = PP == 3 ? A_BYTES * STAGES : STAGE_BYTES * STAGES;
  static constexpr int A_LOADS = BM / RPL / WAVES;    // per wave per stage
  static constexpr int B_LOADS = BN / RPL / WAVES;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int WAVES_PER_EU = WAVES / 4;
  static_assert(WM % M::DIM == 0 && WN % M::DIM == 0, "wave tile must be whole MFMA blocks");
  static_assert(KSTEPS >= 1, "a stage holds at least one k-step");
  static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "every wave loads A and B");
  static_assert(A_LOADS * RPL * WAVES == BM && B_LOADS * RPL * WAVES == BN, "load split");
  static_assert(STAGES >= 2 && LOADS * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 163840, "gfx950 LDS limit");
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
};

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

// seg_at computes the same segment in every lane (its inputs are the
// schedule and the workgroup index); this says so to the compiler, which
// otherwise may keep the segment in vector registers and wrap each buffer
// store that depends on it in a per-lane loop.
__device__ __forceinline__ bool seg_at_uniform(const Sched& s, int32_t v, int32_t n, Segment* out) {
  Segment t;
  if (!seg_at(s, v, n, &t)) return false;
  out->tile = __builtin_amdgcn_readfirstlane(t.tile);
  out->tm = __builtin_amdgcn_readfirstlane(t.tm);
  out->tn = __builtin_amdgcn_readfirstlane(t.tn);
  out->k_begin = __builtin_amdgcn_readfirstlane(t.k_begin);
  out->k_end = __builtin_amdgcn_readfirstlane(t.k_end);
  out->role = __builtin_amdgcn_readfirstlane(t.role);
  out->contributors = __builtin_amdgcn_readfirstlane(t.contributors);
  out->index = __builtin_amdgcn_readfirstlane(t.index);
  return true;
}

// A workgroup barrier that nothing is scheduled across, not even
// instructions without memory operands (the ping-pong phases depend on
// which MFMAs sit between which barriers).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Clock probe: wave 0 of workgroup 0 reads the shader-clock counter
// (s_memtime) and the constant 100 MHz real-time counter (s_memrealtime) when
// it starts and when it ends, and lane 0 adds both differences to the
// caller's counters, so their ratio over any number of launches is the
// average shader clock while those launches ran. Off (one uniform branch)
// when the pointer is null.
struct ClockProbe {
  unsigned long long cycles = 0, ticks = 0;
  bool on = false;
};

__device__ __forceinline__ ClockProbe probe_start(const GemmParams& p, int wave) {
  ClockProbe c;
  c.on = p.clock_probe != nullptr && blockIdx.x == 0 && wave == 0;
  if (c.on) {
    c.cycles = __builtin_amdgcn_s_memtime();
    c.ticks = __builtin_amdgcn_s_memrealtime();
  }
  return c;
}

__device__ __forceinline__ void probe_end(const GemmParams& p, const ClockProbe& c, int lane) {
  if (c.on) {
    const unsigned long long cycles = __builtin_amdgcn_s_memtime() - c.cycles;
    const unsigned long long ticks = __builtin_amdgcn_s_memrealtime() - c.ticks;
    if (lane == 0) {
      atomicAdd(p.clock_probe, cycles);
      atomicAdd(p.clock_probe + 1, ticks);
    }
  }
}

template <class C>
struct Frags {
  typename C::M::frag_t a[C::FM];
  typename C::M::frag_t b[C::FN];
};

// Per-lane LDS byte offset (relative to a stage) of the fragment of k-step
// ks whose block starts at tile row `block_row`.
template <class C>
__device__ __forceinline__ int frag_off(int block_row, int ks, int lane) {
  const int row = block_row + C::M::frag_row(lane);
  return row * C::ROW_BYTES + swz<C::CHUNKS, C::M::DIM>(row, C::M::frag_chunk(ks, lane)) * 16;
}

template <class C>
__device__ __forceinline__ void read_frags(const char* stage, int ks, int wm, int wn, int lane,
                                           Frags<C>& f) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    f.a[i] = *reinterpret_cast<const typename C::M::frag_t*>(
        stage + frag_off<C>(wm * C::WM + i * C::M::DIM, ks, lane));
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    f.b[j] = *reinterpret_cast<const typename C::M::frag_t*>(
        stage + C::A_BYTES + frag_off<C>(wn * C::WN + j * C::M::DIM, ks, lane));
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
    const int chunk = swz<C::CHUNKS, C::M::DIM>(row, lane % C::CHUNKS);  // XOR: own inverse
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

// Items spread evenly over nm MFMAs: item r goes after MFMA r * nm / n.
// items_at: how many go after MFMA m; items_before: how many before it.
constexpr int items_at(int n, int nm, int m) {
  int c = 0;
  for (int r = 0; r < n; ++r) c += (r * nm / n == m);
  return c;
}
constexpr int items_before(int n, int nm, int m) {
  int c = 0;
  for (int r = 0; r < n; ++r) c += (r * nm / n < m);
  return c;
}

// Fragment reads of the next k-step, in issue order r = 0 .. FM + FN - 1.
// MFMAs run row by row (block (i, j) is MFMA i * FN + j), so A fragment i is
// last used by MFMA i * FN + FN - 1 and B fragment j by (FM - 1) * FN + j.
//   RS 0: read r is A fragment r (r < FM), else B fragment r - FM, issued
//         after MFMA r * NM / NR.
//   RS 1: A fragments 0 .. FM - 2, then the B fragments, then A fragment
//         FM - 1, each issued after the last use of the one it replaces.
// read_frag(r): fragment id (A i -> i, B j -> FM + j); read_slot(r): MFMA.
constexpr int read_frag(int rs, int fm, int fn, int r) {
  if (rs == 0) return r;
  if (r < fm - 1) return r;
  if (r < fm - 1 + fn) return fm + (r - (fm - 1));
  return fm - 1;
}
constexpr int read_slot(int rs, int fm, int fn, int r) {
  const int nm = fm * fn, nr = fm + fn;
  if (rs == 0) return r * nm / nr;
  const int f = read_frag(rs, fm, fn, r);
  return f < fm ? f * fn + fn - 1 : (fm - 1) * fn + (f - fm);
}
constexpr int reads_at(int rs, int fm, int fn, int m) {
  int c = 0;
  for (int r = 0; r < fm + fn; ++r) c += (read_slot(rs, fm, fn, r) == m);
  return c;
}
constexpr int reads_before(int rs, int fm, int fn, int m) {
  int c = 0;
  for (int r = 0; r < fm + fn; ++r) c += (read_slot(rs, fm, fn, r) < m);
  return c;
}
constexpr bool read_slots_sorted(int rs, int fm, int fn) {
  for (int r = 1; r < fm + fn; ++r)
    if (read_slot(rs, fm, fn, r) < read_slot(rs, fm, fn, r - 1)) return false;
  return true;
}

// Scheduling groups for one k-step: MFMA m, then its reads, then its loads.
template <class C, int NL, int M>
__device__ __forceinline__ void sched_pattern() {
  constexpr int NM = C::FM * C::FN;
  if constexpr (M < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int nr = reads_at(C::RS, C::FM, C::FN, M);
    constexpr int nl = items_at(NL, NM, M);
    if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);  // LDS reads
    if constexpr (nl > 0) __builtin_amdgcn_sched_group_barrier(0x010, nl, 0);  // loads
    sched_pattern<C, NL, M + 1>();
  }
}

// Fragment read R of the next k-step (A fragments first, then B).
template <class C, int R>
__device__ __forceinline__ void read_one(Frags<C>& nxt, const char* rstage, int rks, int wm,
                                         int wn, int lane) {
  if constexpr (R < C::FM) {
    nxt.a[R] = *reinterpret_cast<const typename C::M::frag_t*>(
        rstage + frag_off<C>(wm * C::WM + R * C::M::DIM, rks, lane));
  } else {
    nxt.b[R - C::FM] = *reinterpret_cast<const typename C::M::frag_t*>(
        rstage + C::A_BYTES + frag_off<C>(wn * C::WN + (R - C::FM) * C::M::DIM, rks, lane));
  }
}

template <class C, int R, int END>
__device__ __forceinline__ void read_range(Frags<C>& nxt, const char* rstage, int rks, int wm,
                                           int wn, int lane) {
  if constexpr (R < END) {
    read_one<C, read_frag(C::RS, C::FM, C::FN, R)>(nxt, rstage, rks, wm, wn, lane);
    read_range<C, R + 1, END>(nxt, rstage, rks, wm, wn, lane);
  }
}

// MFMA M of one k-step on `cur`, followed by the fragment reads and the loads
// assigned to it; recursion keeps every accumulator and fragment index a
// compile-time constant, whatever the number of blocks.
template <class C, int LFIRST, int NL, int M>
__device__ __forceinline__ void kstep_from(typename C::acc_t (&acc)[C::FM][C::FN],
                                           const Frags<C>& cur, Frags<C>& nxt, const char* rstage,
                                           int rks, int wm, int wn, int lane, char* lstage,
                                           const Operands& op, const LoadMap<C, C::A_LOADS>& ma,
                                           const LoadMap<C, C::B_LOADS>& mb, int wave, int k0) {
  constexpr int NM = C::FM * C::FN;
  static_assert(read_slots_sorted(C::RS, C::FM, C::FN), "reads must be in slot order");
  if constexpr (M < NM) {
    constexpr int i = M / C::FN, j = M % C::FN;
    acc[i][j] = C::M::mma(cur.b[j], cur.a[i], acc[i][j]);
    constexpr int r0 = reads_before(C::RS, C::FM, C::FN, M);
    read_range<C, r0, r0 + reads_at(C::RS, C::FM, C::FN, M)>(nxt, rstage, rks, wm, wn, lane);
    if constexpr (NL > 0) {
      constexpr int l0 = items_before(NL, NM, M);
      constexpr int nl = items_at(NL, NM, M);
#pragma unroll
      for (int l = 0; l < nl; ++l) issue_one<C>(LFIRST + l0 + l, lstage, op, ma, mb, wave, k0);
    }
    kstep_from<C, LFIRST, NL, M + 1>(acc, cur, nxt, rstage, rks, wm, wn, lane, lstage, op, ma, mb,
                                     wave, k0);
  }
}

// One MFMA k-step on `cur`, interleaved with (a) the fragment reads of the
// next k-step (k-step rks of stage buffer rstage) into `nxt` and (b) loads
// [LFIRST, LFIRST + NL) of the stage being prefetched into lstage. The
// scheduling groups pin the interleave: after each MFMA come the reads and
// loads assigned to it, so neither the LDS reads nor the load issue (which
// can stall while the address FIFO is full) holds back a run of MFMAs.
template <class C, int LFIRST, int NL>
__device__ __forceinline__ void kstep(typename C::acc_t (&acc)[C::FM][C::FN], const Frags<C>& cur,
                                      Frags<C>& nxt, const char* rstage, int rks, int wm, int wn,
                                      int lane, char* lstage, const Operands& op,
                                      const LoadMap<C, C::A_LOADS>& ma,
                                      const LoadMap<C, C::B_LOADS>& mb, int wave, int k0) {
  kstep_from<C, LFIRST, NL, 0>(acc, cur, nxt, rstage, rks, wm, wn, lane, lstage, op, ma, mb, wave,
                               k0);
  sched_pattern<C, NL, 0>();
}

// The k-steps of one stage. K-steps 0..LK-1 also issue the loads of the stage
// entering the ring (all in k-step 0 with a 2-deep ring, whose next stage must
// land within this one). Before the last k-step the next stage is handed over
// (its loads landed in every wave, all reads of the freed buffer done), and
// that k-step reads the next stage's first fragments. Fragment buffers
// alternate per k-step: k-step KS computes from fr[(KS + PH) & 1], PH being
// the parity of the k-steps before this stage (always 0 when KSTEPS is even).
template <class C, int KS, int PH>
__device__ __forceinline__ void run_ksteps(typename C::acc_t (&acc)[C::FM][C::FN], Frags<C> (&fr)[2],
                                           const char* stage, const char* nstage, int wm, int wn,
                                           int lane, char* lstage, const Operands& op,
                                           const LoadMap<C, C::A_LOADS>& ma,
                                           const LoadMap<C, C::B_LOADS>& mb, int wave, int k0) {
  constexpr int LK = C::STAGES == 2 || C::KSTEPS == 1 ? 1 : C::KSTEPS - 1;
  constexpr int LF = KS < LK ? KS * C::LOADS / LK : 0;
  constexpr int NL = KS < LK ? (KS + 1) * C::LOADS / LK - LF : 0;
  // At the hand-over barrier the stages after the next one may still be in
  // flight: S - 2 of them when this stage's loads were issued before the
  // barrier, one fewer when they go out with the last k-step (KSTEPS == 1).
  constexpr bool kLoadsBefore = LK <= C::KSTEPS - 1;
  constexpr int kPending = C::LOADS * (C::STAGES - 2 - (kLoadsBefore ? 0 : 1));
  static_assert(kLoadsBefore || C::STAGES >= 3, "one k-step per stage needs 3 or more stages");
  if constexpr (KS < C::KSTEPS - 1) {
    kstep<C, LF, NL>(acc, fr[(KS + PH) & 1], fr[(KS + PH + 1) & 1], stage, KS + 1, wm, wn, lane,
                     lstage, op, ma, mb, wave, k0);
    run_ksteps<C, KS + 1, PH>(acc, fr, stage, nstage, wm, wn, lane, lstage, op, ma, mb, wave, k0);
  } else {
    wait_vm<kPending>();
    // With several k-steps a stage, this barrier also frees the current
    // buffer (refilled from the next stage's first k-step), so every read of
    // it must have returned. With one, the buffer refilled after it was last
    // read before the previous barrier, and the fragments in flight are only
    // waited for where the MFMAs use them.
    if constexpr (C::KSTEPS > 1) wait_lgkm_zero();
    lds_barrier();
    kstep<C, LF, NL>(acc, fr[(KS + PH) & 1], fr[(KS + PH + 1) & 1], nstage, 0, wm, wn, lane, lstage,
                     op, ma, mb, wave, k0);
  }
}

// One stage of the main loop: k-iteration `kit` (absolute, in BK units),
// held in ring buffer st; loads k-iteration kit + STAGES - 1 into the buffer
// freed at the last barrier and advances st.
template <class C, int PH>
__device__ __forceinline__ void run_stage(typename C::acc_t (&acc)[C::FM][C::FN],
                                          Frags<C> (&fr)[2], char* smem, int& st, int kit, int wm,
                                          int wn, int lane, const Operands& op,
                                          const LoadMap<C, C::A_LOADS>& ma,
                                          const LoadMap<C, C::B_LOADS>& mb, int wave) {
  const int st_next = st + 1 == C::STAGES ? 0 : st + 1;
  const int st_load = st == 0 ? C::STAGES - 1 : st - 1;
  run_ksteps<C, 0, PH>(acc, fr, smem + st * C::STAGE_BYTES, smem + st_next * C::STAGE_BYTES, wm,
                       wn, lane, smem + st_load * C::STAGE_BYTES, op, ma, mb, wave,
                       (kit + C::STAGES - 1) * C::BK);
  st = st_next;
}

// Partial tiles in the workspace are kept in the accumulators' own layout:
// float4 number (((i * FN + j) * GROUPS + g) * WAVES + wave) * 64 + lane
// holds registers 4g..4g+3 of block (i, j) of that wave and lane, so each
// store and each load of a wave covers 1 KiB of consecutive bytes.
template <class C>
__device__ __forceinline__ void write_partial(f32x4* part,
                                              const typename C::acc_t (&acc)[C::FM][C::FN],
                                              int wave, int lane) {
  constexpr int G = C::M::GROUPS;
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
      for (int g = 0; g < G; ++g) {
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, v), r, voff, ((i * C::FN + j) * G + g) * C::WAVES * 64 * 16,
            0);  // cached: the reduce pass reads the partials right back
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
      const int g = rest % C::M::GROUPS;
      const int i = (rest / C::M::GROUPS) / C::FN;
      const int j = (rest / C::M::GROUPS) % C::FN;
      const int m = m0 + (wave / C::WGN) * C::WM + i * C::M::DIM + C::M::acc_m(lane);
      const int n = n0 + (wave % C::WGN) * C::WN + j * C::M::DIM + C::M::acc_n(g, lane);
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
// Lane l holds, for block (i, j) and register v = 4g + q, row
// m_base + DIM i + acc_m(l) and column n_base + DIM j + acc_n(g, l) + q.
// Non-temporal: C is written once and not read back, and the workgroups of
// an XCD together write more C per round of tiles than its L2 holds, which
// would otherwise push out the A and B panels the next round reads.
template <class C>
__device__ __forceinline__ void epilogue(const GemmParams& p,
                                         const typename C::acc_t (&acc)[C::FM][C::FN],
                                         int m_base, int n_base, int lane) {
  const bool full = m_base + C::WM <= p.M && n_base + C::WN <= p.N;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int m = m_base + i * C::M::DIM + C::M::acc_m(lane);
    float* crow = p.C + (int64_t)m * p.ldc;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
#pragma unroll
      for (int g = 0; g < C::M::GROUPS; ++g) {
        const int n = n_base + j * C::M::DIM + C::M::acc_n(g, lane);
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3]};
        if (full && p.c_vec4) {
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(crow + n));
        } else if (m < p.M) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < p.N) __builtin_nontemporal_store(v[q], crow + n + q);
        }
      }
    }
  }
}

// Store instructions one wave's epilogue_stream issues on its vector path
// (16-byte stores of 4 consecutive columns from every accumulator group).
template <class C>
constexpr int epilogue_stores() {
  return C::FM * C::FN * C::M::GROUPS;
}

// True when the wave's block of C takes the vector path of epilogue_stream:
// all of it inside C, 16-byte aligned rows, and byte offsets within the
// block below 2^31. Uniform across the wave.
template <class C>
__device__ __forceinline__ bool epilogue_vector(const GemmParams& p, int m_base, int n_base) {
  return m_base + C::WM <= p.M && n_base + C::WN <= p.N && p.c_vec4 &&
         (int64_t)C::WM * p.ldc * 4 < ((int64_t)1 << 31);
}

// epilogue() for the ping-pong kernels: on the vector path every group of 4
// goes out as one 16-byte buffer store (exactly epilogue_stores<C>()
// instructions, which the next unit's first stage waits count on) with the
// nt sc1 policy; ragged blocks fall back to epilogue().
template <class C>
__device__ __forceinline__ void epilogue_stream(const GemmParams& p,
                                                const typename C::acc_t (&acc)[C::FM][C::FN],
                                                int m_base, int n_base, int lane) {
  if (!epilogue_vector<C>(p, m_base, n_base)) {
    epilogue<C>(p, acc, m_base, n_base, lane);
    return;
  }
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.C + (int64_t)m_base * p.ldc + n_base), (short)0, kNumRecords, kBufferWord3);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int row = i * C::M::DIM + C::M::acc_m(lane);
#pragma unroll
    for (int g = 0; g < C::M::GROUPS; ++g) {
      const int voff = (row * (int)p.ldc + C::M::acc_n(g, lane)) * 4;
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rc, voff,
                                               j * C::M::DIM * 4, kStoreNtSc1);
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
  const ClockProbe probe = probe_start(p, wave);

  Segment seg;
  for (int n = 0; seg_at_uniform(p.s, v, n, &seg); ++n) {
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

    typename C::acc_t acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = typename C::acc_t{};

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
    if constexpr (C::KSTEPS % 2 == 0) {
      for (int it = 0; it < nk; ++it)
        run_stage<C, 0>(acc, fr, smem, st, seg.k_begin + it, wm, wn, lane, op, ma, mb, wave);
    } else {
      // One k-step per stage: the fragment buffers swap roles every stage,
      // so stages go in pairs and each copy of the body has fixed roles.
      int it = 0;
      for (; it + 1 < nk; it += 2) {
        run_stage<C, 0>(acc, fr, smem, st, seg.k_begin + it, wm, wn, lane, op, ma, mb, wave);
        run_stage<C, 1>(acc, fr, smem, st, seg.k_begin + it + 1, wm, wn, lane, op, ma, mb, wave);
      }
      if (it < nk)
        run_stage<C, 0>(acc, fr, smem, st, seg.k_begin + it, wm, wn, lane, op, ma, mb, wave);
    }

    if (seg.role == ROLE_ONLY) {
      epilogue<C>(p, acc, m0 + wm * C::WM, n0 + wn * C::WN, lane);
    } else {
      // One share of a tile: its partial goes to the workspace; the reduce
      // kernel that follows on the stream sums the shares into C.
      write_partial<C>(p.partials + ((int64_t)(seg.tile - p.s.shared_base) * p.s.slots + seg.index) *
                                        (C::BM * C::BN / 4),
                       acc, wave, lane);
    }
  }
  probe_end(p, probe, lane);
}

// Per-unit state of the load stream: operand windows, per-lane load map and
// k range of one unit (output tile, or share of one).
template <class C>
struct UnitLoads {
  Operands op;
  LoadMap<C, C::A_LOADS> ma;
  LoadMap<C, C::B_LOADS> mb;
  int m0, n0, k_begin, nk;
};

template <class C>
__device__ __forceinline__ void unit_loads(const GemmParams& p, const Segment& seg, int wave,
                                           int lane, UnitLoads<C>& u) {
  u.m0 = seg.tm * C::BM;
  u.n0 = seg.tn * C::BN;
  u.k_begin = seg.k_begin;
  u.nk = seg.k_end - seg.k_begin;
  // Loads cover this unit's k range only; the stages past its end that the
  // ring still issues are fully masked (zero-filled, no memory access).
  const int k_limit = min_of(p.K, seg.k_end * C::BK);
  u.op.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + (int64_t)u.m0 * p.lda), (short)0,
                                              kNumRecords, kBufferWord3);
  u.op.rb = __builtin_amdgcn_make_buffer_rsrc((void*)(p.B + (int64_t)u.n0 * p.ldb), (short)0,
                                              kNumRecords, kBufferWord3);
  make_load_map<C, C::A_LOADS>(u.ma, wave, lane, p.M - u.m0, p.lda, k_limit);
  make_load_map<C, C::B_LOADS>(u.mb, wave, lane, p.N - u.n0, p.ldb, k_limit);
}

// Ping-pong main loop (8 waves, two per SIMD). The waves form two groups,
// one wave of each on every SIMD (group 0: waves 0-3, group 1: waves 4-7),
// and group 1 runs one phase behind group 0. A stage takes two phases per
// wave, separated by workgroup barriers:
//   memory phase:  read all of the stage's fragments from LDS, issue this
//                  wave's loads of stage it + STAGES - 1, wait until stage
//                  it + 1 has landed and the fragments have arrived;
//   compute phase: the stage's MFMAs, from registers only.
// So while one group computes, the other does its memory work and is
// already waiting at the barrier when the computing group arrives: the MFMA
// pipe of every SIMD is fed by one wave or the other through each barrier
// (the ping-pong schedule the CUTLASS Hopper post describes for two consumer
// warp groups, here across the waves sharing a SIMD).
// Buffer reuse: stage j's buffer is refilled in memory phases j + 1 (group 0
// after its compute phase j, which follows group 1's read of stage j across
// a barrier) and later; stage j + 1 is complete in LDS before either group
// reads it, since every wave waits for its share of it before the barrier
// that opens group 0's memory phase j + 1.
//
// Between units, each wave issues the first STAGES - 1 stages of its next
// unit as soon as its last compute phase is done (no wave reads the ring
// any more by then: group 1's last reads end before the barrier that closes
// group 0's last compute phase), and only then the stores of the finished
// unit. The next unit's first STAGES - 2 stage waits leave those stores
// in flight (their count is exact on the epilogue's vector path and for
// partial tiles), so the write of C overlaps the start of the next unit
// instead of stalling it: vector-memory operations retire in issue order,
// and the stores are younger than every stage waited for until stage
// STAGES - 1, which is issued after them.
template <class C>
__global__ __launch_bounds__(C::THREADS)
__attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU, C::WAVES_PER_EU)))
void gemm_pingpong_kernel(GemmParams p) {
  static_assert(C::WAVES == 8, "ping-pong pairs two waves per SIMD");
  static_assert(C::STAGES >= 3, "a stage is awaited while the next two are in flight");
  constexpr int kStage = C::LOADS * (C::STAGES - 2);  // loads younger than an awaited stage
  constexpr int kStores = epilogue_stores<C>();
  static_assert(kStage + kStores <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool late = wave >= 4;  // group 1
  const int wm = wave / C::WGN;
  const int wn = wave % C::WGN;
  const int v = virtual_wg(blockIdx.x, p.s.grid, p.s.xcd_remap);
  const ClockProbe probe = probe_start(p, wave);

  Segment seg;
  if (!seg_at_uniform(p.s, v, 0, &seg)) return;
  UnitLoads<C> u;
  unit_loads<C>(p, seg, wave, lane, u);
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s) {
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j)
      issue_one<C>(j, smem + s * C::STAGE_BYTES, u.op, u.ma, u.mb, wave, (u.k_begin + s) * C::BK);
  }
  // True when the previous unit's kStores stores were issued after this
  // unit's first stages (so they may stay in flight through its first
  // STAGES - 2 stage waits).
  bool stores_behind = false;

  for (int n = 0;; ++n) {
    typename C::acc_t acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = typename C::acc_t{};

    if (stores_behind)
      wait_vm<kStage + kStores>();
    else
      wait_vm<kStage>();
    phase_barrier();
    if (late) phase_barrier();  // group 1 starts one phase behind

    Frags<C> fr[C::KSTEPS];
    int st = 0;
    for (int it = 0; it < u.nk; ++it) {
      const int st_load = st == 0 ? C::STAGES - 1 : st - 1;
      const char* stage = smem + st * C::STAGE_BYTES;
      // Memory phase.
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) read_frags<C>(stage, ks, wm, wn, lane, fr[ks]);
      const int k0 = (u.k_begin + it + C::STAGES - 1) * C::BK;
#pragma unroll
      for (int j = 0; j < C::LOADS; ++j)
        issue_one<C>(j, smem + st_load * C::STAGE_BYTES, u.op, u.ma, u.mb, wave, k0);
      if (stores_behind && it < C::STAGES - 2)
        wait_vm<kStage + kStores>();
      else
        wait_vm<kStage>();
      wait_lgkm_zero();
      phase_barrier();
      // Compute phase. Serpentine order: block rows alternate the column
      // direction, so every MFMA shares an operand register with the one
      // before it (measured ~1% faster at 8192^3 than plain row order).
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int jj = 0; jj < C::FN; ++jj) {
            const int j = (i & 1) ? C::FN - 1 - jj : jj;
            acc[i][j] = C::M::mma(fr[ks].b[j], fr[ks].a[i], acc[i][j]);
          }
      phase_barrier();
      st = st + 1 == C::STAGES ? 0 : st + 1;
    }

    // Group 0 is here while group 1 runs its last compute phase; group 1
    // follows one phase later. The loads still in flight are the masked
    // tail stages (no memory access): let them land before the ring is
    // refilled, then start the next unit's stream.
    const Segment done = seg;
    const int m_base = u.m0 + wm * C::WM;
    const int n_base = u.n0 + wn * C::WN;
    const bool more = seg_at_uniform(p.s, v, n + 1, &seg);
    if (more) {
      wait_vm<0>();
      unit_loads<C>(p, seg, wave, lane, u);
#pragma unroll
      for (int s = 0; s < C::STAGES - 1; ++s) {
#pragma unroll
        for (int j = 0; j < C::LOADS; ++j)
          issue_one<C>(j, smem + s * C::STAGE_BYTES, u.op, u.ma, u.mb, wave,
                       (u.k_begin + s) * C::BK);
      }
    }
    if (done.role == ROLE_ONLY) {
      stores_behind = more && epilogue_vector<C>(p, m_base, n_base);
      epilogue_stream<C>(p, acc, m_base, n_base, lane);
    } else {
      // write_partial issues epilogue_stores<C>() buffer stores as well.
      stores_behind = more;
      write_partial<C>(p.partials + ((int64_t)(done.tile - p.s.shared_base) * p.s.slots + done.index) *
                                        (C::BM * C::BN / 4),
                       acc, wave, lane);
    }
    // Matches group 1's extra barrier at the start of the unit.
    if (!late) phase_barrier();
    if (!more) break;
  }
  probe_end(p, probe, lane);
}

// Ping-pong main loop over stages 64 wide in k, two of them in LDS (128 KiB),
// with the same two wave groups and phases as gemm_pingpong_kernel, one
// memory and one compute phase per 32-wide k-step. A stage's rows are 128
// bytes, a whole cache line each: every load of a wave covers 8 rows x 128
// bytes instead of 16 rows x 64 bytes, which the memory system delivers at
// nearly twice the rate (same addresses otherwise).
//   k-step 0 of stage it: read its fragments, issue this wave's loads of
//     stage it + 1 into the other buffer (last read in the memory phase just
//     before the previous barrier, so free);
//   k-step 1 of stage it: read its fragments, wait until stage it + 1 has
//     landed.
// A load is thus awaited one k-step after it was issued, as in the 32-wide
// three-stage ring. Between units the next unit's first stage goes out
// before the finished unit's stores, which stay in flight through the next
// unit's first wait; the wait for its stage 1 drains them.
template <class C>
__global__ __launch_bounds__(C::THREADS)
__attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU, C::WAVES_PER_EU)))
void gemm_pingpong64_kernel(GemmParams p) {
  static_assert(C::WAVES == 8, "ping-pong pairs two waves per SIMD");
  static_assert(C::STAGES == 2 && C::BK == 64, "two stages 64 wide in k");
  // MFMA k-steps per phase: a phase covers 32 of k (one 16x16x32 k-step, or
  // two 32x32x16 ones).
  constexpr int KPP = C::KSTEPS / 2;
  constexpr int kStores = epilogue_stores<C>();
  static_assert(C::LOADS + kStores <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool late = wave >= 4;  // group 1
  const int wm = wave / C::WGN;
  const int wn = wave % C::WGN;
  const int v = virtual_wg(blockIdx.x, p.s.grid, p.s.xcd_remap);
  const ClockProbe probe = probe_start(p, wave);

  Segment seg;
  if (!seg_at_uniform(p.s, v, 0, &seg)) return;
  UnitLoads<C> u;
  unit_loads<C>(p, seg, wave, lane, u);
#pragma unroll
  for (int j = 0; j < C::LOADS; ++j)
    issue_one<C>(j, smem, u.op, u.ma, u.mb, wave, u.k_begin * C::BK);
  bool stores_behind = false;

  for (int n = 0;; ++n) {
    typename C::acc_t acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = typename C::acc_t{};

    if (stores_behind)
      wait_vm<kStores>();
    else
      wait_vm<0>();
    phase_barrier();
    if (late) phase_barrier();  // group 1 starts one phase behind

    Frags<C> fr[KPP];
    for (int it = 0; it < u.nk; ++it) {
      const char* stage = smem + (it & 1) * C::STAGE_BYTES;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // Memory phase.
#pragma unroll
        for (int kk = 0; kk < KPP; ++kk) read_frags<C>(stage, ks * KPP + kk, wm, wn, lane, fr[kk]);
        if (ks == 0) {
          if (it + 1 < u.nk) {
            const int k0 = (u.k_begin + it + 1) * C::BK;
#pragma unroll
            for (int j = 0; j < C::LOADS; ++j)
              issue_one<C>(j, smem + ((it & 1) ^ 1) * C::STAGE_BYTES, u.op, u.ma, u.mb, wave, k0);
          }
        } else {
          wait_vm<0>();
        }
        wait_lgkm_zero();
        phase_barrier();
        // Compute phase (serpentine order, as in gemm_pingpong_kernel).
#pragma unroll
        for (int kk = 0; kk < KPP; ++kk)
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < C::FN; ++jj) {
              const int j = (i & 1) ? C::FN - 1 - jj : jj;
              acc[i][j] = C::M::mma(fr[kk].b[j], fr[kk].a[i], acc[i][j]);
            }
        phase_barrier();
      }
    }

    // Group 0 is here while group 1 runs its last compute phase: no wave
    // reads LDS any more, so the next unit's first stage can go out.
    const Segment done = seg;
    const int m_base = u.m0 + wm * C::WM;
    const int n_base = u.n0 + wn * C::WN;
    const bool more = seg_at_uniform(p.s, v, n + 1, &seg);
    if (more) {
      wait_vm<0>();
      unit_loads<C>(p, seg, wave, lane, u);
#pragma unroll
      for (int j = 0; j < C::LOADS; ++j)
        issue_one<C>(j, smem, u.op, u.ma, u.mb, wave, u.k_begin * C::BK);
    }
    if (done.role == ROLE_ONLY) {
      stores_behind = more && epilogue_vector<C>(p, m_base, n_base);
      epilogue_stream<C>(p, acc, m_base, n_base, lane);
    } else {
      stores_behind = more;
      write_partial<C>(p.partials + ((int64_t)(done.tile - p.s.shared_base) * p.s.slots + done.index) *
                                        (C::BM * C::BN / 4),
                       acc, wave, lane);
    }
    // Matches group 1's extra barrier at the start of the unit.
    if (!late) phase_barrier();
    if (!more) break;
  }
  probe_end(p, probe, lane);
}

// Fragments of the A tile (all FM blocks of the wave) or of the B tile (all
// FN blocks) for MFMA k-step ks, from an LDS slot holding that tile alone.
template <class C>
__device__ __forceinline__ void read_a_frags(const char* slot, int ks, int wm, int lane,
                                             typename C::M::frag_t (&a)[C::FM]) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
    a[i] = *reinterpret_cast<const typename C::M::frag_t*>(
        slot + frag_off<C>(wm * C::WM + i * C::M::DIM, ks, lane));
}

template <class C>
__device__ __forceinline__ void read_b_frags(const char* slot, int ks, int wn, int lane,
                                             typename C::M::frag_t (&b)[C::FN]) {
#pragma unroll
  for (int j = 0; j < C::FN; ++j)
    b[j] = *reinterpret_cast<const typename C::M::frag_t*>(
        slot + frag_off<C>(wn * C::WN + j * C::M::DIM, ks, lane));
}

// This wave's loads of the A (or B) half of the stage whose first k is k0,
// into an LDS slot holding that half alone.
template <class C>
__device__ __forceinline__ void issue_a_half(char* slot, const UnitLoads<C>& u, int wave, int k0) {
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const uint32_t off = k0 < u.ma.lim[j] ? u.ma.off[j] : kMaskedOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        u.op.ra, (lds_void_ptr)(slot + (wave * C::A_LOADS + j) * 1024), 16, off, k0 * 2, 0, 0);
  }
}

template <class C>
__device__ __forceinline__ void issue_b_half(char* slot, const UnitLoads<C>& u, int wave, int k0) {
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const uint32_t off = k0 < u.mb.lim[j] ? u.mb.off[j] : kMaskedOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        u.op.rb, (lds_void_ptr)(slot + (wave * C::B_LOADS + j) * 1024), 16, off, k0 * 2, 0, 0);
  }
}

// Ping-pong main loop over 64-wide stages held as separate A and B halves in
// five LDS slots of 32 KiB (the whole 160 KiB), with the same two wave groups
// and phases as gemm_pingpong64_kernel (one memory and one compute phase per
// 32-wide k-step). The memory phase of a stage's first k-step reads the B
// fragments of both its k-steps (and the A fragments of the first), so the
// stage's B half is free after both groups' first memory phase and its A half
// after their second. Stage s takes A slot 2 (s mod 3) and B slot
// 1 + 2 (s mod 2), so each half of stage s + 2 goes into the slot its
// counterpart of stage s - 1 (A) or s (B) has just freed:
//   k-step 0 of stage it: read A(it) k-step 0 and B(it) both k-steps; issue
//     this wave's loads of A(it + 2) into A(it - 1)'s slot;
//   k-step 1 of stage it: read A(it) k-step 1; issue B(it + 2) into
//     B(it)'s slot; wait until stage it + 1 has landed (group 1 here, group 0
//     after its compute phase, both before the barrier that opens stage
//     it + 1).
// A half is thus awaited four to seven phases after it was issued, where the
// two-stage loop of gemm_pingpong64_kernel awaits a stage two phases after
// issuing it. In steady state the loads younger than an awaited stage are
// exactly the next stage's A and B halves (LOADS). Units run one after
// another: the ring drains (masked tail stages) and every wave's stores are
// issued before the next unit's first loads.
template <class C>
__global__ __launch_bounds__(C::THREADS)
__attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU, C::WAVES_PER_EU)))
void gemm_pingpong_ring_kernel(GemmParams p) {
  static_assert(C::WAVES == 8, "ping-pong pairs two waves per SIMD");
  static_assert(C::BK == 64 && C::KSTEPS == 2 && C::STAGES == 5 && C::A_BYTES == C::B_BYTES,
                "five half-stage slots of 64-wide stages, one k-step per phase");
  constexpr int SLOT = C::A_BYTES;
  constexpr int kRing = C::LOADS;  // loads younger than an awaited stage
  typedef typename C::M::frag_t frag_t;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool late = wave >= 4;  // group 1
  const int wm = wave / C::WGN;
  const int wn = wave % C::WGN;
  const int v = virtual_wg(blockIdx.x, p.s.grid, p.s.xcd_remap);
  const ClockProbe probe = probe_start(p, wave);

  Segment seg;
  for (int n = 0; seg_at_uniform(p.s, v, n, &seg); ++n) {
    UnitLoads<C> u;
    unit_loads<C>(p, seg, wave, lane, u);
    typename C::acc_t acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = typename C::acc_t{};

    // The previous unit's loads (its masked tail) and stores are done and no
    // wave reads the slots any more.
    wait_vm<0>();
    wait_lgkm_zero();
    phase_barrier();
    // Stages 0 and 1 into slots 0-3; stage 0 awaited.
    issue_a_half<C>(smem, u, wave, u.k_begin * C::BK);
    issue_b_half<C>(smem + SLOT, u, wave, u.k_begin * C::BK);
    issue_a_half<C>(smem + 2 * SLOT, u, wave, (u.k_begin + 1) * C::BK);
    issue_b_half<C>(smem + 3 * SLOT, u, wave, (u.k_begin + 1) * C::BK);
    wait_vm<kRing>();
    phase_barrier();
    if (late) phase_barrier();  // group 1 starts one phase behind

    frag_t fa[C::FM], fb0[C::FN], fb1[C::FN];
    int ia = 0, ib = 0;  // it mod 3, it mod 2
    for (int it = 0; it < u.nk; ++it) {
      const char* sa = smem + 2 * ia * SLOT;
      char* sb = smem + (1 + 2 * ib) * SLOT;
      char* sa_next = smem + 2 * (ia == 0 ? 2 : ia - 1) * SLOT;  // slot of A(it - 1) = A(it + 2)
      const int k_next = (u.k_begin + it + 2) * C::BK;
      // Memory phase, k-step 0.
      read_a_frags<C>(sa, 0, wm, lane, fa);
      read_b_frags<C>(sb, 0, wn, lane, fb0);
      read_b_frags<C>(sb, 1, wn, lane, fb1);
      issue_a_half<C>(sa_next, u, wave, k_next);
      wait_lgkm_zero();
      phase_barrier();
      // Compute phase, k-step 0 (serpentine order, as in gemm_pingpong_kernel).
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < C::FN; ++jj) {
          const int j = (i & 1) ? C::FN - 1 - jj : jj;
          acc[i][j] = C::M::mma(fb0[j], fa[i], acc[i][j]);
        }
      phase_barrier();
      // Memory phase, k-step 1: both groups have read B(it), so its slot
      // takes B(it + 2).
      read_a_frags<C>(sa, 1, wm, lane, fa);
      issue_b_half<C>(sb, u, wave, k_next);
      if (late) wait_vm<kRing>();
      wait_lgkm_zero();
      phase_barrier();
      // Compute phase, k-step 1.
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < C::FN; ++jj) {
          const int j = (i & 1) ? C::FN - 1 - jj : jj;
          acc[i][j] = C::M::mma(fb1[j], fa[i], acc[i][j]);
        }
      __builtin_amdgcn_sched_barrier(0);
      if (!late) wait_vm<kRing>();
      phase_barrier();
      ia = ia == 2 ? 0 : ia + 1;
      ib ^= 1;
    }

    // Group 0 is here while group 1 runs its last compute phase.
    const int m_base = u.m0 + wm * C::WM;
    const int n_base = u.n0 + wn * C::WN;
    if (seg.role == ROLE_ONLY) {
      epilogue_stream<C>(p, acc, m_base, n_base, lane);
    } else {
      write_partial<C>(p.partials + ((int64_t)(seg.tile - p.s.shared_base) * p.s.slots + seg.index) *
                                        (C::BM * C::BN / 4),
                       acc, wave, lane);
    }
    // Matches group 1's extra barrier at the start of the unit.
    if (!late) phase_barrier();
  }
  probe_end(p, probe, lane);
}

// Shares of output tile t under schedule s (1: the tile was stored directly).
__device__ __forceinline__ int tile_shares(const Sched& s, int t) {
  if (s.mode == MODE_SPLIT) return s.splits;
  if ((s.mode != MODE_STREAM_K && s.mode != MODE_DP_SK) || t < s.shared_base) return 1;
  const int64_t lo = (int64_t)(t - s.shared_base) * s.k_iters;
  return (int)(sk_owner(s, lo + s.k_iters - 1) - sk_owner(s, lo) + 1);
}

// Reduce pass for split-K / stream-K: workgroup b handles slice b % slices
// of tile shared_base + b / slices. Partials are summed in k order, so the result does not
// depend on timing.
template <class C>
__global__ __launch_bounds__(kReduceThreads) void gemm_reduce_kernel(GemmParams p, int32_t slices) {
  constexpr int L = C::BM * C::BN / 4;
  const int t = p.s.shared_base + (int)(blockIdx.x / slices);
  const int slice = blockIdx.x % slices;
  const int shares = tile_shares(p.s, t);
  if (shares <= 1) return;
  int tm, tn;
  tile_coords(p.s, t, &tm, &tn);
  const int begin = (int)((int64_t)slice * L / slices);
  const int end = (int)((int64_t)(slice + 1) * L / slices);
  reduce_range<C>(p, p.partials + (int64_t)(t - p.s.shared_base) * p.s.slots * L, shares, begin,
                  end, tm * C::BM, tn * C::BN);
}

// General kernel: any shape, stride and (element-natural) alignment. 4 waves
// per 64 x 64 tile of C, each wave a 32 x 32 block; operands go straight from
// global memory into MFMA registers, element by element with bounds checks.
// Workgroups walk the tiles by stride, so the grid stays within the launch
// limits however many tiles there are. Slow; taken only when the tiled
// kernels' alignment rules do not hold.
template <int DT>
__global__ __launch_bounds__(256) void gemm_general_kernel(GemmParams p, int32_t tiles_n,
                                                           int64_t tiles) {
  using M = Mma<32, DT>;
  typedef typename M::elem_t elem_t;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int tm = (int)(t / tiles_n);
    const int tn = (int)(t % tiles_n);
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
      typename M::frag_t a, b;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + kk + e;
        const bool kin = k < p.K;
        a[e] = __builtin_bit_cast(elem_t, (a_ok && kin) ? arow[k] : (uint16_t)0);
        b[e] = __builtin_bit_cast(elem_t, (b_ok && kin) ? brow[k] : (uint16_t)0);
      }
      acc = M::mma(b, a, acc);
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
}

// Direct kernel for the smallest problems: one wave per 16x16 tile of C and
// no LDS. Each lane loads its own MFMA operand fragments (row l % 16 and
// elements 8 (l / 16) .. +7 of every 32-wide k-step, for A and B) straight
// from global memory with 16-byte buffer loads, all the k-steps of a chunk at
// once, and accumulates them with v_mfma_f32_16x16x32 into two accumulators
// (even and odd k-steps, added at the end), so that the dependent chain of
// MFMAs is half as long. Rows past M or N and k-steps past K are masked by
// out-of-range offsets (zeros, no memory access). Operands must follow the
// tiled kernels' loading rules (16-byte aligned rows of a multiple of 8
// elements). Each lane then holds 4 consecutive columns of one row of C and
// stores them as one 16-byte write. Workgroups walk the tiles by stride.
template <int DT>
__global__ __launch_bounds__(64) void gemm_direct_kernel(GemmParams p, int32_t tiles_n,
                                                         int64_t tiles) {
  using M = Mma<16, DT>;
  typedef typename M::frag_t frag_t;
  constexpr int CH = 8;  // k-steps of 32 loaded at once
  const int lane = threadIdx.x;
  const int r = lane & 15;
  const int kg = (lane >> 4) * 8;
  const int nks = (p.K + 31) / 32;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int m0 = (int)(t / tiles_n) * 16;
    const int n0 = (int)(t % tiles_n) * 16;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.A + (int64_t)m0 * p.lda), (short)0, kNumRecords, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.B + (int64_t)n0 * p.ldb), (short)0, kNumRecords, kBufferWord3);
    const uint32_t offa = m0 + r < p.M ? (uint32_t)(r * p.lda * 2 + kg * 2) : kMaskedOffset;
    const uint32_t offb = n0 + r < p.N ? (uint32_t)(r * p.ldb * 2 + kg * 2) : kMaskedOffset;
    f32x4 acc0 = {}, acc1 = {};
    for (int c = 0; c < nks; c += CH) {
      frag_t fa[CH], fb[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int k = (c + j) * 32;
        const bool kin = k + kg < p.K;  // K is a multiple of 8: all or none of the lane's 8
        fa[j] = __builtin_bit_cast(
            frag_t, __builtin_amdgcn_raw_buffer_load_b128(ra, kin ? offa : kMaskedOffset, k * 2, 0));
        fb[j] = __builtin_bit_cast(
            frag_t, __builtin_amdgcn_raw_buffer_load_b128(rb, kin ? offb : kMaskedOffset, k * 2, 0));
      }
#pragma unroll
      for (int j = 0; j < CH; j += 2) {
        if (c + j < nks) acc0 = M::mma(fb[j], fa[j], acc0);
        if (c + j + 1 < nks) acc1 = M::mma(fb[j + 1], fa[j + 1], acc1);
      }
    }
    const f32x4 acc = acc0 + acc1;
    const int m = m0 + M::acc_m(lane);
    const int n = n0 + M::acc_n(0, lane);
    if (m < p.M) {
      float* crow = p.C + (int64_t)m * p.ldc;
      if (n + 3 < p.N && p.c_vec4) {
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(crow + n));
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (n + q < p.N) __builtin_nontemporal_store(acc[q], crow + n + q);
      }
    }
  }
}

// Operand packing: one thread per 16-byte chunk (8 elements) of the packed
// copy. The chunk's source bytes start at any 2-byte boundary, so the thread
// loads the aligned 16-byte block holding its first element and, when a valid
// element lies past it, the next block; it shifts the 8 elements into place
// (v_alignbyte) and zeroes those at or past K. Neighbouring lanes load
// neighbouring blocks, so the loads coalesce. A block is loaded only if it
// holds a valid element of the row; an aligned 16-byte block never crosses a
// page, so the bytes read beside the valid ones are always mapped (their
// values are discarded). Workgroups walk the chunks by stride.
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint16_t* __restrict__ src,
                                                        int64_t ld, int32_t K,
                                                        int32_t chunks_per_row, int64_t chunks,
                                                        u32x4* __restrict__ dst) {
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < chunks; t += step) {
    const int64_t r = t / chunks_per_row;
    const int k0 = (int)(t - r * chunks_per_row) * 8;
    const int nvalid = min_of(8, K - k0);  // >= 1: chunks stop at K rounded up to 8
    const uint16_t* first = src + r * ld + k0;
    const int s = (int)((uintptr_t)first & 15);  // byte offset in its block (even)
    const u32x4* blk = (const u32x4*)((const char*)first - s);
    const u32x4 b0 = blk[0];
    const u32x4 b1 = s + 2 * nvalid > 16 ? blk[1] : u32x4{0u, 0u, 0u, 0u};
    const uint32_t w[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    const int q = s >> 2;  // first dword of the chunk in w
    uint32_t d[5];
#pragma unroll
    for (int k = 0; k < 5; ++k)
      d[k] = q == 0 ? w[k] : q == 1 ? w[k + 1] : q == 2 ? w[k + 2] : w[k + 3];
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = (s & 2) ? __builtin_amdgcn_alignbyte(d[i + 1], d[i], 2) : d[i];
      if (2 * i >= nvalid)
        o[i] = 0u;
      else if (2 * i + 1 >= nvalid)
        o[i] &= 0xffffu;
    }
    dst[t] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

#define G16_CFG(id, name, bm, bn, bk, st, wgm, wgn, mi, rs, pp) \
  using K##id = Cfg<bm, bn, bk, st, wgm, wgn, mi, rs, pp>;
G16_TILED_KERNELS(G16_CFG)
#undef G16_CFG

// The same configuration with bfloat16 operands.
template <class C>
using Bf16Of = Cfg<C::BM, C::BN, C::BK, C::STAGES, C::WGM, C::WGN, C::MI, C::RS, C::PP, DT_BF16>;

template <class C>
constexpr KernelInfo info_of(const char* name) {
  return KernelInfo{C::BM, C::BN, C::BK, C::STAGES, C::WAVES, C::LDS_BYTES, C::MI, name};
}

// Names: BMxBNxBK, ring depth, waves, "_m16" for the 16x16x32 MFMA and
// "_pp" for the ping-pong main loop.
constexpr KernelInfo kInfo16 = info_of<K16>("128x128x64_s4_w4_m16");
constexpr KernelInfo kInfo18 = info_of<K18>("64x64x64_s4_w4_m16");
constexpr KernelInfo kInfo27 = info_of<K27>("256x256x32_s3_w8_m16_pp");
constexpr KernelInfo kInfo28 = info_of<K28>("256x256x32_s5_w8_pp");
constexpr KernelInfo kInfo35 = info_of<K35>("256x256x64_s2_w8_m16_pp");
constexpr KernelInfo kInfo36 = info_of<K36>("256x256x64_s2_w8_pp");
constexpr KernelInfo kInfo37 = info_of<K37>("256x256x64_h5_w8_m16_pp");
constexpr KernelInfo kInfo38 = info_of<K38>("32x32x64_s5_w4_m16");

template <class C>
hipError_t launch_cfg(const GemmParams& p, hipStream_t stream) {
  if constexpr (C::PP == 3)
    hipLaunchKernelGGL(gemm_pingpong_ring_kernel<C>, dim3(p.s.grid), dim3(C::THREADS), 0, stream,
                       p);
  else if constexpr (C::PP == 2)
    hipLaunchKernelGGL(gemm_pingpong64_kernel<C>, dim3(p.s.grid), dim3(C::THREADS), 0, stream, p);
  else if constexpr (C::PP)
    hipLaunchKernelGGL(gemm_pingpong_kernel<C>, dim3(p.s.grid), dim3(C::THREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(gemm_tiled_kernel<C>, dim3(p.s.grid), dim3(C::THREADS), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.s.mode == MODE_DATA_PARALLEL) return e;
  // Slices per tile: enough workgroups to cover the CUs, at least 4 KiB each.
  const int max_slices = C::BM * C::BN / 4 / 256;
  const int shared_tiles = p.s.tiles - p.s.shared_base;  // tiles that may have partials
  if (shared_tiles <= 0) return e;
  int slices = (256 + shared_tiles - 1) / shared_tiles;
  if (slices > max_slices) slices = max_slices;
  if (slices < 1) slices = 1;
  hipLaunchKernelGGL(gemm_reduce_kernel<C>, dim3(shared_tiles * slices), dim3(kReduceThreads), 0,
                     stream, p, slices);
  return hipGetLastError();
}

template <class C>
int32_t occupancy_cfg() {
  int n = 0;
  hipError_t e;
  if constexpr (C::PP == 3)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_pingpong_ring_kernel<C>, C::THREADS,
                                                     0);
  else if constexpr (C::PP == 2)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_pingpong64_kernel<C>, C::THREADS, 0);
  else if constexpr (C::PP)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_pingpong_kernel<C>, C::THREADS, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_tiled_kernel<C>, C::THREADS, 0);
  if (e != hipSuccess) return 0;
  return n;
}

}  // namespace

const KernelInfo* kernel_info(int32_t kid) {
#define G16_INFO(id, name, ...) \
  case name: return &kInfo##id;
  switch (kid) {
    G16_TILED_KERNELS(G16_INFO)
    default: return nullptr;
  }
#undef G16_INFO
}

hipError_t launch_tiled(int32_t kid, int32_t dt, const GemmParams& p, hipStream_t stream) {
  if (dt == DT_BF16) {
#define G16_LAUNCH_BF16(id) \
  case id: return launch_cfg<Bf16Of<K##id>>(p, stream);
    switch (kid) {
      G16_BF16_KERNELS(G16_LAUNCH_BF16)
      default: return hipErrorInvalidValue;
    }
#undef G16_LAUNCH_BF16
  }
#define G16_LAUNCH(id, name, ...) \
  case name: return launch_cfg<K##id>(p, stream);
  switch (kid) {
    G16_TILED_KERNELS(G16_LAUNCH)
    default: return hipErrorInvalidValue;
  }
#undef G16_LAUNCH
}

bool tiled_has(int32_t kid, int32_t dt) {
  if (kernel_info(kid) == nullptr) return false;
  if (dt == DT_F16) return true;
  if (dt != DT_BF16) return false;
#define G16_HAS_BF16(id) if (kid == id) return true;
  G16_BF16_KERNELS(G16_HAS_BF16)
#undef G16_HAS_BF16
  return false;
}

int32_t tiled_occupancy(int32_t kid) {
#define G16_OCC(id, name, ...) \
  case name: return occupancy_cfg<K##id>();
  switch (kid) {
    G16_TILED_KERNELS(G16_OCC)
    default: return 0;
  }
#undef G16_OCC
}

hipError_t launch_general(int32_t dt, const GemmParams& p, hipStream_t stream) {
  const int64_t tiles_m = (p.M + 63) / 64;
  const int64_t tiles_n = (p.N + 63) / 64;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles <= 0) return hipSuccess;
  // A dispatch counts its work-items in 32 bits: cap the grid (2^20
  // workgroups of 256, far more than fit on the chip at once) and let
  // workgroups take further tiles by stride.
  const uint32_t grid = (uint32_t)min_of<int64_t>(tiles, (int64_t)1 << 20);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(gemm_general_kernel<DT_BF16>, dim3(grid), dim3(256), 0, stream, p,
                       (int32_t)tiles_n, tiles);
  else
    hipLaunchKernelGGL(gemm_general_kernel<DT_F16>, dim3(grid), dim3(256), 0, stream, p,
                       (int32_t)tiles_n, tiles);
  return hipGetLastError();
}

hipError_t launch_direct(int32_t dt, const GemmParams& p, hipStream_t stream) {
  const int64_t tiles_n = (p.N + 15) / 16;
  const int64_t tiles = (p.M + 15) / 16 * tiles_n;
  if (tiles <= 0) return hipSuccess;
  const uint32_t grid = (uint32_t)min_of<int64_t>(tiles, (int64_t)1 << 20);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(gemm_direct_kernel<DT_BF16>, dim3(grid), dim3(64), 0, stream, p,
                       (int32_t)tiles_n, tiles);
  else
    hipLaunchKernelGGL(gemm_direct_kernel<DT_F16>, dim3(grid), dim3(64), 0, stream, p,
                       (int32_t)tiles_n, tiles);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* src, int64_t ld, int32_t K, int64_t rows, int32_t kp,
                       void* dst, hipStream_t stream) {
  const int32_t per_row = kp / 8;
  const int64_t chunks = rows * per_row;
  if (chunks <= 0) return hipSuccess;
  const uint32_t grid = (uint32_t)min_of<int64_t>((chunks + 255) / 256, (int64_t)1 << 20);
  hipLaunchKernelGGL(pack_rows_kernel, dim3(grid), dim3(256), 0, stream, src, ld, K, per_row,
                     chunks, (u32x4*)dst);
  return hipGetLastError();
}

}  // namespace g16
