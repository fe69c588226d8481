// Internal declarations shared by the kernels and the C-ABI layer of libmsm.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ec.hpp"

namespace msmk {

constexpr int SCAN_ITEMS = 4;                        // counts per thread in a scan tile
constexpr uint32_t SCAN_TILE = 256 * SCAN_ITEMS;     // counts per scan block
constexpr uint32_t SCAN_PRE_ITEMS = 4;               // tile sums per thread of a down block
constexpr uint32_t SCAN_MAX_BLOCKS = 256 * SCAN_PRE_ITEMS;  // tiles of one scan
constexpr int MAX_LEVELS = 32;                       // pair-tree levels tracked
constexpr uint32_t XYZZ_QUAD_MAX_PAIRS = 65536;      // XYZZ levels this small use 4 lanes per add

constexpr int MAX_PLANES = 160;                      // reduction planes (at most 128 occur)
constexpr int MAX_PLANE_GROUPS = 10;                 // join groups (8 occur: 2, 2, 4, ..., 32 planes)

// Plan read back to the host after the sort (one small copy).
struct msm_stats {
  uint32_t range_flag;          // a GLV half-scalar came out >= 2^127 (never expected)
  uint32_t max_count;           // largest bucket
  uint32_t total;               // bucket entries E (non-zero digits)
  uint32_t bad_point;           // verify: some input point is off the curve or not reduced
  uint32_t pairs[MAX_LEVELS];   // pair adds at pair-tree level l
  uint32_t bad_out;             // verify: the result is off the curve (read after the MSM)
  uint32_t join[MAX_PLANE_GROUPS + 1];  // reduction: finished planes per group, groups
};

// The planes of the bucket reduction (k_reduce.hip): plane i has exponent e[i] & 0xff,
// window (e[i] >> 8) & 0xff and selector e[i] >> 16 (0: every segment's R + T; beta + 1:
// the segment totals T of segments with bit beta set). Passed to kernels by value.
struct plane_table {
  uint32_t n;        // planes, in order of decreasing exponent
  uint32_t nseg;     // segments per window (2^(hb + lb))
  uint32_t lambda;   // log2 of the slots per segment
  uint32_t hb, lb;   // segment index s = hi 2^lb + lo, hi < 2^hb, lo < 2^lb (lb >= hb)
  uint32_t pg;       // log2 of the segments per (R + T) group: 5, or 6 for 2048 or more
  uint32_t np;       // (R + T) group sums per window: ceil(nseg / 2^pg)
  uint32_t wstride;  // group sums per window: np, then 2^hb sums A_hi, then 2^lb sums B_lo
  uint32_t e[MAX_PLANES];
};

// XYZZ point as stored in device memory (X, Y, ZZ, ZZZ; 128 bytes).
struct xyzz_st {
  uint32_t w[32];
};

hipError_t launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
// verify != 0 also checks every input point (reduced coordinates, on the curve or
// (0, 0)) and sets st->bad_point when one fails.
hipError_t launch_glv_prep(const g1a* points, const uint32_t* scalars, uint32_t n, g1a* pts2,
                           uint32_t* halfs, msm_stats* st, int verify, int scalar_form, hipStream_t s);
// *flag |= 1 when the affine point p is neither (0, 0) nor a reduced point on the curve.
hipError_t launch_verify_point(const g1a* p, uint32_t* flag, hipStream_t s);
// Counting pass: per (chunk of half-scalars, window) LDS histograms into hist_blk
// (nwin nchunk 2^(c-1) words), turned into per-chunk prefixes, the bucket counts, and
// the plan statistics in st (largest bucket, total, pair adds per level).
hipError_t launch_hist(const uint32_t* halfs, uint32_t m, uint32_t c, uint32_t nwin,
                       uint32_t chunk, uint32_t nchunk, uint32_t* hist_blk, uint32_t* counts,
                       uint32_t* rank, msm_stats* st, hipStream_t s);
hipError_t launch_scatter(const uint32_t* halfs, uint32_t m, uint32_t c, uint32_t nwin,
                          uint32_t chunk, uint32_t nchunk, const uint32_t* offsets,
                          const uint32_t* hist_blk, const uint32_t* rank, uint32_t* sorted_idx,
                          hipStream_t s);
// Blocks of the tile scan over n values.
inline uint32_t scan_blocks(uint32_t n) {
  uint32_t nb = (n + SCAN_TILE - 1) / SCAN_TILE;
  return nb ? nb : 1;
}
// Exclusive scans of the per-bucket values of levels level0 .. level0 + nlev - 1 (level
// -1: the counts themselves; level l >= 0: the pair adds at pair-tree level l). Level
// level0 + y writes n + 1 values (the total last) at out + y out_stride; block_sums
// needs nlev (scan_blocks(n) + 1) words. With max_count (device, may be NULL), levels
// l >= 0 that a largest bucket of *max_count entries does not need are skipped.
hipError_t launch_scan(const uint32_t* counts, uint32_t n, int level0, int nlev,
                       uint32_t* block_sums, uint32_t* out, size_t out_stride,
                       const uint32_t* max_count, hipStream_t s);
hipError_t launch_bucket_init(const uint32_t* counts, const uint32_t* offsets, uint32_t K,
                              const uint32_t* sorted_idx, const g1a* points, xyzz_st* bsum,
                              hipStream_t s);
// Batched-affine pair-tree level; place selects the slot-state placement (0 private
// memory, bit 0 LDS, bit 1 cached denominators).
hipError_t launch_level(int S, int place, const g1a* in, const uint32_t* idx, g1a* out,
                        xyzz_st* bsum, const uint32_t* counts, const uint32_t* offsets,
                        const uint32_t* poff, uint32_t K, uint32_t npairs, int level,
                        hipStream_t s);
hipError_t launch_level_placed(int S, int place, const g1a* in, const uint32_t* idx, g1a* out,
                               xyzz_st* bsum, const uint32_t* counts, const uint32_t* offsets,
                               const uint32_t* poff, uint32_t K, uint32_t npairs, int level,
                               hipStream_t s);
hipError_t launch_level_xyzz(bool in_aff, const void* in, const uint32_t* idx, xyzz_st* out,
                             xyzz_st* bsum, const uint32_t* counts, const uint32_t* offsets,
                             const uint32_t* poff, uint32_t K, uint32_t npairs, int level,
                             hipStream_t s);
// Stream-walker accumulate (k_walk.hip): T lanes of S slots walk chunks of L entries of
// the E sorted entries. acc (16 Z words) and kst (Z words) are the device-side slot state
// (used when dev_state), head / tail (Z points) and head_k / tail_k (Z words) the partial
// sums of split buckets, Z = T S.
struct walk_args {
  const g1a* pts;
  const uint32_t* idx;
  const uint32_t* offsets;
  uint32_t K, E, T, L;
  uint32_t* acc;
  uint32_t* kst;
  xyzz_st* bsum;
  xyzz_st* head;
  xyzz_st* tail;
  uint32_t* head_k;
  uint32_t* tail_k;
};
constexpr uint32_t WALK_MAX_LANES = 65536;
constexpr uint32_t WALK_MIN_CHUNK = 16;  // aim for at least this many entries per slot
// Lanes of a walk over E entries with S slots per lane: enough for chunks of about
// WALK_MIN_CHUNK entries, a multiple of 64, at most WALK_MAX_LANES.
inline uint32_t walk_lanes(uint64_t E, int S) {
  uint64_t t = (E + (uint64_t)S * WALK_MIN_CHUNK - 1) / ((uint64_t)S * WALK_MIN_CHUNK);
  t = (t + 63) / 64 * 64;
  if (t < 64) t = 64;
  if (t > WALK_MAX_LANES) t = WALK_MAX_LANES;
  return (uint32_t)t;
}
// The walk kernel alone (slot state private, or on the device when dev_state).
hipError_t launch_walk(int S, bool dev_state, const walk_args& a, hipStream_t s);
// merge_passes pair passes over the partial sums, then the split buckets' sums.
hipError_t launch_walk_merge(int S, const walk_args& a, uint32_t merge_passes, hipStream_t s);

// Planes of the reduction for window width c and nwin windows (host side of the plan).
plane_table make_planes(uint32_t c, uint32_t nwin);

// Segment sums (tseg, pseg: nwin nseg points each) and the group sums the planes are
// made of (part: nwin wstride points).
hipError_t launch_reduce(const xyzz_st* bsum, uint32_t c, uint32_t nwin, const plane_table& pt,
                         xyzz_st* tseg, xyzz_st* pseg, xyzz_st* part, hipStream_t s);
// Doubling runs of every plane and their sum, in affine form, to out (res: n points,
// gres: MAX_PLANE_GROUPS points, join: the zeroed counters of msm_stats).
hipError_t launch_final(const xyzz_st* part, const plane_table& pt, xyzz_st* res, xyzz_st* gres,
                        uint32_t* join, g1a* out, hipStream_t s);
hipError_t launch_from_scalars(const uint32_t* ks, uint32_t n, g1a* out, hipStream_t s);
hipError_t launch_test_fp(int op, const uint32_t* a, const uint32_t* b, uint32_t* out, uint32_t n,
                          hipStream_t s);
hipError_t launch_test_rate(int op, uint32_t blocks, uint32_t iters, uint32_t seed, uint32_t* out,
                            hipStream_t s);
// Row-form field and doubling-run hooks (ops 0..6 of msm_test_row).
hipError_t launch_test_row(int op, const uint32_t* a, const uint32_t* b, uint32_t* out, uint32_t n,
                           uint32_t d, hipStream_t s);
hipError_t launch_test_glv(const uint32_t* scalars, uint32_t n, uint32_t* halfs, hipStream_t s);
hipError_t launch_test_pair_add(int S, const g1a* a, const g1a* b, g1a* out, uint32_t n,
                                hipStream_t s);

}  // namespace msmk
