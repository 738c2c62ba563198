// Persistent tile schedule shared by the device kernels and the host-side
// schedule model (gemm_f16_schedule_dump). Every function here is plain
// integer arithmetic, callable from both sides, so the model the tests check
// is the very code the kernels run.
//
// Four modes, after the per-shape program rule of "SASS-Level Kernel
// Generation for Blackwell" (section "Inside the kernels"), which picks for
// each shape between a persistent grid over whole tiles, a split of K and
// stream-K:
//   DATA_PARALLEL  each output tile is one unit over all of K; a fixed grid
//                  of workgroups takes the units by stride.
//   SPLIT          the k-iterations of every tile are cut into `splits`
//                  contiguous, near-equal shares, each its own unit.
//   STREAM_K       the k-iterations of all tiles, laid end to end, are cut
//                  into one contiguous range per workgroup; a range may end
//                  part-way through a tile and start the next one.
//   DP_SK          whole rounds of tiles (grid tiles each) data-parallel,
//                  then STREAM_K over the tiles left, so a last round that
//                  would keep few workgroups busy is shared by all of them.
//                  Only those last tiles can have partial tiles.
// The shares of a tile are not added in place (the page adds them in L2):
// each share writes its fp32 partial tile to a workspace slot, and a reduce
// kernel launched after the main kernel on the same stream sums every tile's
// slots in k order and writes C. Nothing in the schedule requires the shares
// of a tile to run at the same time.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define G16_HD __host__ __device__ __forceinline__
#else
#define G16_HD inline
#endif

namespace g16 {

enum SchedMode : int32_t {
  MODE_DATA_PARALLEL = 0,
  MODE_SPLIT = 1,
  MODE_STREAM_K = 2,
  MODE_DP_SK = 3  // whole data-parallel rounds, then stream-K over the tiles left
};
enum SegRole : int32_t { ROLE_ONLY = 0, ROLE_SHARED = 1 };

struct Sched {
  int32_t tiles_m, tiles_n, tiles;  // output tiles (tiles = tiles_m * tiles_n)
  int32_t k_iters;                  // k-iterations (of BK) per tile
  int32_t mode;                     // SchedMode
  int32_t splits;                   // MODE_SPLIT: k-shares per tile (<= k_iters)
  int32_t grid;                     // workgroups launched
  int32_t group_m;                  // tile order: bands of group_m tile rows
  int32_t xcd_remap;                // 1: renumber workgroups XCD by XCD (virtual_wg)
  int32_t slots;                    // partial-tile slots per tile in the workspace
  int32_t shared_base;              // first tile that may be shared (DP_SK: the tiles of
                                    // the whole data-parallel rounds come before it);
                                    // partial tiles are indexed from it
};

struct Segment {
  int32_t tile;        // position in tile order (also the partial-tile slot group)
  int32_t tm, tn;      // tile coordinates
  int32_t k_begin;     // first k-iteration (inclusive)
  int32_t k_end;       // last k-iteration (exclusive)
  int32_t role;        // SegRole
  int32_t contributors;  // shares of this tile (1 for ROLE_ONLY)
  int32_t index;         // this share's position among them, in k order
};

template <class T>
G16_HD T min_of(T a, T b) { return a < b ? a : b; }
template <class T>
G16_HD T max_of(T a, T b) { return a > b ? a : b; }

// Workgroups are handed to the 8 XCDs round-robin (workgroup w runs on XCD
// w mod 8). Renumber them so each XCD gets a contiguous block of virtual
// indices: neighbouring units then share an XCD and its L2. XCD x holds
// grid / 8 workgroups, one more when x < grid mod 8, and its block starts
// after those of XCDs 0 .. x-1; for any grid this is a permutation of
// 0 .. grid-1. (Leaving a grid that is not a multiple of 8 unrenumbered
// spreads neighbouring units over all XCDs, which cost 13-31% on split
// plans of 27-50 tiles measured at K = 12288 and 24576.)
G16_HD int32_t virtual_wg(int32_t w, int32_t grid, int32_t remap = 1) {
  if (!remap) return w;
  const int32_t x = w % 8, per = grid / 8, extra = grid % 8;
  return x * per + min_of(x, extra) + w / 8;
}

// Tile order: bands of group_m tile rows, column-major inside a band, so a
// run of consecutive indices covers a compact block of C.
G16_HD void tile_coords(const Sched& s, int32_t idx, int32_t* tm, int32_t* tn) {
  const int32_t per_band = s.group_m * s.tiles_n;
  const int32_t band = idx / per_band;
  const int32_t first_m = band * s.group_m;
  const int32_t rows = min_of(s.tiles_m - first_m, s.group_m);
  const int32_t r = idx - band * per_band;
  *tm = first_m + r % rows;
  *tn = r / rows;
}

// STREAM_K and DP_SK: k-iterations of the stream-K region (tiles from
// shared_base on, laid end to end; iteration 0 is the first of tile
// shared_base).
G16_HD int64_t sk_total(const Sched& s) {
  return (int64_t)(s.tiles - s.shared_base) * s.k_iters;
}

// Workgroups that take part in the stream-K region: all of the grid, or as
// many as it has iterations (DP_SK's region can be smaller than the grid), so
// every range is non-empty and the owners of a tile are consecutive.
G16_HD int64_t sk_grid(const Sched& s) { return min_of<int64_t>(s.grid, sk_total(s)); }

// First stream-K iteration of virtual workgroup v (v <= sk_grid).
G16_HD int64_t sk_start(const Sched& s, int64_t v) { return v * sk_total(s) / sk_grid(s); }

// The workgroup whose range holds stream-K iteration i.
G16_HD int64_t sk_owner(const Sched& s, int64_t i) {
  return ((i + 1) * sk_grid(s) - 1) / sk_total(s);
}

// Number of units (DATA_PARALLEL, SPLIT) or segments a workgroup walks is
// found by iterating seg_at(...) until it returns false.
//
// DATA_PARALLEL / SPLIT: the n-th unit of virtual workgroup v is v + n*grid.
// STREAM_K: the n-th segment of v, counted from the end of v's range.
// DP_SK: first the whole tiles v + n*grid below shared_base (a multiple of
// grid), then v's stream-K segments over the remaining tiles.
G16_HD bool seg_at(const Sched& s, int32_t v, int32_t n, Segment* out) {
  if (s.mode == MODE_STREAM_K || s.mode == MODE_DP_SK) {
    const int32_t rounds = s.mode == MODE_DP_SK ? s.shared_base / s.grid : 0;
    if (n < rounds) {
      const int32_t t = v + n * s.grid;
      out->tile = t;
      tile_coords(s, t, &out->tm, &out->tn);
      out->k_begin = 0;
      out->k_end = s.k_iters;
      out->contributors = 1;
      out->index = 0;
      out->role = ROLE_ONLY;
      return true;
    }
    n -= rounds;
    if (v >= sk_grid(s)) return false;  // no stream-K range for this workgroup
    const int64_t a = sk_start(s, v);
    int64_t b = sk_start(s, (int64_t)v + 1);
    for (int32_t i = 0; b > a; ++i) {
      const int64_t t = (b - 1) / s.k_iters;  // tile within the stream-K region
      const int64_t tile_lo = t * s.k_iters;
      const int64_t lo = max_of(a, tile_lo);
      if (i == n) {
        out->tile = (int32_t)(s.shared_base + t);
        tile_coords(s, out->tile, &out->tm, &out->tn);
        out->k_begin = (int32_t)(lo - tile_lo);
        out->k_end = (int32_t)(b - tile_lo);
        const int64_t first = sk_owner(s, tile_lo);
        const int64_t last = sk_owner(s, tile_lo + s.k_iters - 1);
        out->contributors = (int32_t)(last - first + 1);
        out->index = (int32_t)(v - first);
        out->role = out->contributors == 1 ? ROLE_ONLY : ROLE_SHARED;
        return true;
      }
      b = lo;
    }
    return false;
  }
  const int32_t splits = s.mode == MODE_SPLIT ? s.splits : 1;
  const int64_t u = (int64_t)v + (int64_t)n * s.grid;
  if (u >= (int64_t)s.tiles * splits) return false;
  const int32_t share = (int32_t)(u / s.tiles);
  const int32_t t = (int32_t)(u - (int64_t)share * s.tiles);
  out->tile = t;
  tile_coords(s, t, &out->tm, &out->tn);
  out->k_begin = (int32_t)((int64_t)share * s.k_iters / splits);
  out->k_end = (int32_t)((int64_t)(share + 1) * s.k_iters / splits);
  out->contributors = splits;
  out->index = share;
  out->role = splits == 1 ? ROLE_ONLY : ROLE_SHARED;
  return true;
}

}  // namespace g16

namespace g16 {

// Most shares any tile has under schedule s (the workspace slots per tile).
inline int32_t max_shares(const Sched& s) {
  if (s.mode == MODE_SPLIT) return s.splits;
  if (s.mode != MODE_STREAM_K && s.mode != MODE_DP_SK) return 1;
  int64_t most = 1;
  for (int64_t t = 0; t < (int64_t)s.tiles - s.shared_base; ++t) {
    const int64_t lo = t * s.k_iters;
    const int64_t c = sk_owner(s, lo + s.k_iters - 1) - sk_owner(s, lo) + 1;
    if (c > most) most = c;
  }
  return (int32_t)most;
}

}  // namespace g16
