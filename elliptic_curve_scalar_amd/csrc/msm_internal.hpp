// Internal declarations shared by the kernels and the C-ABI layer of libmsm.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ec.hpp"

namespace msmk {

constexpr int SCAN_ITEMS = 4;                        // counts per thread in a scan tile
constexpr uint32_t SCAN_TILE = 256 * SCAN_ITEMS;     // counts per scan block
constexpr int SCAN_TOP_ITEMS = 16;                   // block sums per thread in the top scan
constexpr uint32_t SCAN_MAX_BLOCKS = 256 * SCAN_TOP_ITEMS;
constexpr int MAX_LEVELS = 32;                       // pair-tree levels tracked
constexpr unsigned LEVEL_BLOCK = 128;                // lanes per block in k_level
constexpr uint32_t XYZZ_QUAD_MAX_PAIRS = 65536;      // XYZZ levels this small use 4 lanes per add

// Plan read back to the host after the sort (one 16 + 4 * MAX_LEVELS byte copy).
struct msm_stats {
  uint32_t range_flag;          // a GLV half-scalar came out >= 2^127 (never expected)
  uint32_t max_count;           // largest bucket
  uint32_t total;               // bucket entries E (non-zero digits)
  uint32_t bad_point;           // verify: some input point is off the curve or not reduced
  uint32_t pairs[MAX_LEVELS];   // pair adds at pair-tree level l
  uint32_t bad_out;             // verify: the result is off the curve (read after the MSM)
  uint32_t pad[3];
};

// XYZZ point as stored in device memory (X, Y, ZZ, ZZZ; 128 bytes).
struct xyzz_st {
  uint32_t w[32];
};

hipError_t launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
// verify != 0 also checks every input point (reduced coordinates, on the curve or
// (0, 0)) and sets st->bad_point when one fails.
hipError_t launch_glv_prep(const g1a* points, const uint32_t* scalars, uint32_t n, g1a* pts2,
                           uint32_t* halfs, msm_stats* st, int verify, hipStream_t s);
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
hipError_t launch_level(int S, const g1a* in, const uint32_t* idx, g1a* out, xyzz_st* bsum,
                        const uint32_t* counts, const uint32_t* offsets, const uint32_t* poff,
                        uint32_t K, uint32_t npairs, int level, hipStream_t s);
hipError_t launch_level_xyzz(bool in_aff, const void* in, const uint32_t* idx, xyzz_st* out,
                             xyzz_st* bsum, const uint32_t* counts, const uint32_t* offsets,
                             const uint32_t* poff, uint32_t K, uint32_t npairs, int level,
                             hipStream_t s);
// Blocks per window in the first pass of the segment-sum tree: 64 segments per block
// (one per quad), at most 64 blocks; every c has at most 4096 segments per window.
inline uint32_t reduce_blocks(uint32_t nseg) {
  uint32_t b = (nseg + 63) / 64;
  return b < 1 ? 1 : (b > 64 ? 64 : b);
}
hipError_t launch_reduce(const xyzz_st* bsum, uint32_t c, uint32_t nwin, uint32_t seg_len,
                         uint32_t nseg, xyzz_st* part, xyzz_st* win, hipStream_t s);
hipError_t launch_final(const xyzz_st* win, uint32_t nwin, uint32_t c, g1a* out, hipStream_t s);
hipError_t launch_from_scalars(const uint32_t* ks, uint32_t n, g1a* out, hipStream_t s);
hipError_t launch_test_fp(int op, const uint32_t* a, const uint32_t* b, uint32_t* out, uint32_t n,
                          hipStream_t s);
hipError_t launch_test_glv(const uint32_t* scalars, uint32_t n, uint32_t* halfs, hipStream_t s);
hipError_t launch_test_pair_add(int S, const g1a* a, const g1a* b, g1a* out, uint32_t n,
                                hipStream_t s);

}  // namespace msmk
