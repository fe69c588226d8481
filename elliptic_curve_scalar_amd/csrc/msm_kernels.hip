// Device kernels of the BN254 G1 bucket MSM for gfx950, and their launchers.
//
// Pipeline (one stream; W = ceil(128 / c) windows of signed digits over the 2n GLV
// half-scalars, 2^(c-1) buckets per window, digit 0 dropped since it adds nothing):
//   k_glv_prep    scalar -> two half-scalars below 2^127; points [P, phi(P)]
//   k_hist_tile   per (chunk of half-scalars, window): LDS histogram, rank per entry
//   k_chunk_scan  per bucket: prefix over the chunks, bucket count; plan statistics
//   k_scan_*      exclusive scan of the counts -> bucket offsets
//   -- the plan is copied to the host --
//   k_scatter     point indices into per-bucket lists (sorted_idx)
//   k_bucket_init buckets of size 0 / 1 are final at once
//   k_scan_*      pair offsets of every pair-tree level
//   -- the host reads the plan --
//   k_level<S>    pair-tree level 0: pair (2m, 2m+1) of every bucket -> element m,
//                 S pairs per lane with one inversion (batch_add.hpp)
//   k_level_xyzz  deeper levels in XYZZ coordinates (quad-cooperative when small)
//   k_rsum_tree   per window, segments of buckets: sum_b b * B_b by running sums,
//                 summed per block through an LDS tree
//   k_tree_sum    per window: the blocks' partial sums -> W_j
//   k_final       Q = sum_j 2^(c j) W_j by doubling, then affine
//
// The method is aztec-packages PR #23738 / #23736 / #23520 ("bb/msm"); its WebGPU
// kernels are prior art only: the level kernel takes S pairs per lane the way the
// pages' pair-tree accumulate takes S adds per invocation (PR #23520 "Summary").
#include <hip/hip_runtime.h>

#include "batch_add.hpp"
#include "glv.hpp"
#include "msm_internal.hpp"
#include "quad.hpp"

namespace msmk {

// ------------------------------------------------------------------ scalars
struct sc256 {
  uint32_t w[8];
};

__device__ __forceinline__ sc256 load_scalar(const uint32_t* s, uint32_t i) {
  const uint4* q = reinterpret_cast<const uint4*>(s + 8 * (size_t)i);
  uint4 a = q[0], b = q[1];
  sc256 r;
  r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
  r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
  return r;
}

// Bits [bit, bit + c) of s (c <= 16, bit < 256); bits past 255 read as 0.
__device__ __forceinline__ uint32_t window_digit(const sc256& s, uint32_t bit, uint32_t c) {
  uint32_t w = bit >> 5, sh = bit & 31u;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (uint32_t k = 0; k < 8; k++) {
    lo = (k == w) ? s.w[k] : lo;
    hi = (k == w + 1) ? s.w[k] : hi;
  }
  uint64_t v = ((uint64_t)hi << 32) | lo;
  return (uint32_t)(v >> sh) & ((1u << c) - 1u);
}

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Signed window digits: s = sum_j d_j 2^(c j) with d_j in [-2^(c-1), 2^(c-1)], found
// from the least significant window up with a carry (a window above 2^(c-1) becomes
// d - 2^c and carries 1); the top window is not recoded, which is why scalars must be
// below 2^(W c - 1). -P is free in affine coordinates, so a window needs only 2^(c-1)
// buckets, one per |d|. Calls f(j, slot, negative) for every non-zero digit, with
// slot = |d| - 1.
template <class F>
__device__ __forceinline__ void for_each_signed_digit(const sc256& s, uint32_t c, uint32_t nwin,
                                                      F&& f) {
  const uint32_t half = 1u << (c - 1);
  uint32_t carry = 0;
  for (uint32_t j = 0; j < nwin; j++) {
    const uint32_t raw = window_digit(s, j * c, c) + carry;
    const bool neg = (j + 1 < nwin) && raw > half;
    carry = neg ? 1u : 0u;
    const uint32_t mag = neg ? (1u << c) - raw : raw;
    if (mag) f(j, mag - 1, neg);
  }
}

// GLV split (glv.hpp): half-scalar i = |k1| of scalar i and half-scalar n + i = |k2|,
// each four words with the sign in bit 127; point i is P_i and point n + i is
// phi(P_i) = (beta x, y). Every later stage sees 2n points with 127-bit scalars.
__global__ void __launch_bounds__(128) k_glv_prep(const g1a* __restrict__ points,
                                                  const uint32_t* __restrict__ scalars, uint32_t n,
                                                  g1a* __restrict__ pts2, uint32_t* __restrict__ halfs,
                                                  msm_stats* st) {
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const sc256 sc = load_scalar(scalars, i);
  uint32_t s[8], k1[4], k2[4];
#pragma unroll
  for (int w = 0; w < 8; w++) s[w] = sc.w[w];
  bool bad = false;
  glv_split(s, k1, k2, bad);
  if (bad) atomicOr(&st->range_flag, 1u);
  reinterpret_cast<uint4*>(halfs)[i] = make_uint4(k1[0], k1[1], k1[2], k1[3]);
  reinterpret_cast<uint4*>(halfs)[n + i] = make_uint4(k2[0], k2[1], k2[2], k2[3]);
  aff a = aff_load(points + i);
  aff_store(pts2 + i, a);
  if (!aff_is_inf(a)) a.x = fp_mul(a.x, glv_beta());
  aff_store(pts2 + n + i, a);
}

// Half-scalar i: 127-bit magnitude in a 256-bit value, and its sign.
__device__ __forceinline__ sc256 load_half(const uint32_t* halfs, uint32_t i, bool& neg) {
  const uint4 h = reinterpret_cast<const uint4*>(halfs)[i];
  neg = (h.w >> 31) != 0;
  sc256 r;
  r.w[0] = h.x; r.w[1] = h.y; r.w[2] = h.z; r.w[3] = h.w & 0x7fffffffu;
  r.w[4] = r.w[5] = r.w[6] = r.w[7] = 0;
  return r;
}

// Slots per digit value in window j. The half-scalars have 127-bit magnitudes, so the
// top window's digits never exceed 2^(127 - c (W - 1)) while it has 2^(c-1) slots like
// every window: each of its digits is spread over 2^(c W - 128) slots, chosen by the
// half-scalar's index, which evens out the bucket sizes (at c = 13 the top window's
// buckets would otherwise be eight times fuller and the pair tree three levels deeper).
// The running sum weights slot b of window j by floor(b / spread) + 1.
__device__ __forceinline__ uint32_t window_spread(uint32_t c, uint32_t nwin, uint32_t j) {
  return (j + 1 == nwin) ? (1u << (c * nwin - 128)) : 1u;
}

// Slot of a digit of magnitude mag >= 1 in window j, for half-scalar i.
__device__ __forceinline__ uint32_t digit_slot(uint32_t c, uint32_t nwin, uint32_t j, uint32_t mag,
                                               uint32_t i) {
  const uint32_t f = window_spread(c, nwin, j);
  return (mag - 1) * f + (i & (f - 1));
}

// Signed digits of one half-scalar for a fixed maximum window count: slot[j] = |d_j| - 1
// and act[j] = (d_j != 0), the same recoding as for_each_signed_digit. Unrolled, so the
// per-window memory operations that follow can all be in flight together.
template <int MAXW>
__device__ __forceinline__ void signed_digits(const sc256& s, uint32_t c, uint32_t nwin,
                                              uint32_t (&slot)[MAXW], bool (&act)[MAXW],
                                              bool (&neg)[MAXW]) {
  const uint32_t half = 1u << (c - 1);
  uint32_t carry = 0;
#pragma unroll
  for (int j = 0; j < MAXW; j++) {
    const bool in = (uint32_t)j < nwin;
    const uint32_t raw = (in ? window_digit(s, j * c, c) : 0u) + carry;
    const bool ng = ((uint32_t)j + 1 < nwin) && raw > half;
    carry = ng ? 1u : 0u;
    const uint32_t mag = ng ? (1u << c) - raw : raw;
    act[j] = in && mag != 0;
    slot[j] = mag - 1;
    neg[j] = ng;
  }
}

// Signed digit of window jw of a half-scalar, the recoding of for_each_signed_digit:
// the carry is run up from window 0. mag = |d|, neg = d < 0.
__device__ __forceinline__ void signed_digit_at(const sc256& s, uint32_t c, uint32_t nwin,
                                                uint32_t jw, uint32_t& mag, bool& neg) {
  const uint32_t half = 1u << (c - 1);
  uint32_t carry = 0;
  for (uint32_t j = 0; j < jw; j++) carry = (window_digit(s, j * c, c) + carry > half) ? 1u : 0u;
  const uint32_t raw = window_digit(s, jw * c, c) + carry;
  neg = (jw + 1 < nwin) && raw > half;
  mag = neg ? (1u << c) - raw : raw;
}

// Counting pass of the counting sort, one block per (chunk of half-scalars, window):
// the block counts its entries into an LDS histogram of the window's 2^(c-1) buckets,
// the LDS atomic returning each entry's rank among the chunk's entries of its bucket
// (kept in rank[j m + i]), and writes the histogram to hist_blk[(j nchunk + chunk) H
// + slot]. No atomic leaves the block, so a bucket that collects a large share of the
// entries costs no more than any other.
__global__ void __launch_bounds__(1024) k_hist_tile(const uint32_t* __restrict__ halfs, uint32_t m,
                                                    uint32_t c, uint32_t nwin, uint32_t chunk,
                                                    uint32_t nchunk, uint32_t* __restrict__ hist_blk,
                                                    uint32_t* __restrict__ rank) {
  extern __shared__ uint32_t lds_hist[];
  const uint32_t H = 1u << (c - 1);
  const uint32_t ch = blockIdx.x, j = blockIdx.y;
  for (uint32_t k = threadIdx.x; k < H; k += blockDim.x) lds_hist[k] = 0;
  __syncthreads();
  const uint32_t i0 = ch * chunk, i1 = min(m, i0 + chunk);
  for (uint32_t i = i0 + threadIdx.x; i < i1; i += blockDim.x) {
    bool sneg;
    const sc256 s = load_half(halfs, i, sneg);
    uint32_t mag;
    bool neg;
    signed_digit_at(s, c, nwin, j, mag, neg);
    if (mag) rank[(size_t)j * m + i] = atomicAdd(&lds_hist[digit_slot(c, nwin, j, mag, i)], 1u);
  }
  __syncthreads();
  uint32_t* out = hist_blk + ((size_t)j * nchunk + ch) * H;
  for (uint32_t k = threadIdx.x; k < H; k += blockDim.x) out[k] = lds_hist[k];
}

// Entries of a bucket of cnt entries at pair-tree level `level`: ceil(cnt / 2^level).
__device__ __forceinline__ uint32_t level_count(uint32_t cnt, int level) {
  return (uint32_t)(((uint64_t)cnt + (1ull << level) - 1) >> level);
}

// ------------------------------------------------------------------ stats
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor(v, off, 64));
  return v;
}

// Largest bucket, total entries and the pair adds of every pair-tree level, from one
// bucket count per thread (0 for threads past the last bucket): reduced in registers,
// then over the block's four waves through LDS, then one atomic per value and block.
// Every thread of the 256-thread block must call it.
__device__ __forceinline__ void block_stats(uint32_t cnt, msm_stats* st) {
  __shared__ uint32_t red[4][MAX_LEVELS + 2];
  const uint32_t wave = threadIdx.x >> 6;
  const bool lead = (threadIdx.x & 63) == 0;
  const uint32_t mx = wave_max(cnt), tot = wave_sum(cnt);
  if (lead) {
    red[wave][MAX_LEVELS] = mx;
    red[wave][MAX_LEVELS + 1] = tot;
  }
#pragma unroll
  for (int l = 0; l < MAX_LEVELS; l++) {
    const uint32_t v = wave_sum(level_count(cnt, l) >> 1);
    if (lead) red[wave][l] = v;
  }
  __syncthreads();
  if (threadIdx.x < MAX_LEVELS + 2) {
    const uint32_t i = threadIdx.x;
    const uint32_t a = red[0][i], b = red[1][i], c = red[2][i], d = red[3][i];
    if (i == MAX_LEVELS) {
      atomicMax(&st->max_count, max(max(a, b), max(c, d)));
    } else {
      const uint32_t v = a + b + c + d;
      if (v) atomicAdd(i == MAX_LEVELS + 1 ? &st->total : &st->pairs[i], v);
    }
  }
}

// Per bucket (thread t = j 2^(c-1) + slot): the per-chunk counts become each chunk's
// exclusive prefix within the bucket, counts[t] the bucket's total, and the block's
// buckets go into the plan statistics (block_stats).
__global__ void __launch_bounds__(256) k_chunk_scan(uint32_t* __restrict__ hist_blk, uint32_t c,
                                                    uint32_t nwin, uint32_t nchunk,
                                                    uint32_t* __restrict__ counts, msm_stats* st) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t H = 1u << (c - 1);
  uint32_t run = 0;
  if (t < nwin * H) {
    const uint32_t j = t >> (c - 1), slot = t & (H - 1);
    uint32_t* const col = hist_blk + (size_t)j * nchunk * H + slot;  // chunk ch at col[ch H]
    uint32_t ch = 0;
    for (; ch + 8 <= nchunk; ch += 8) {  // eight loads in flight, then the running sum
      uint32_t v[8];
#pragma unroll
      for (int e = 0; e < 8; e++) v[e] = col[(size_t)(ch + e) * H];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        col[(size_t)(ch + e) * H] = run;
        run += v[e];
      }
    }
    for (; ch < nchunk; ch++) {
      const uint32_t v = col[(size_t)ch * H];
      col[(size_t)ch * H] = run;
      run += v;
    }
    counts[t] = run;
  }
  block_stats(run, st);
}

// Bucket lists hold point indices with the sign of (digit x half-scalar) in bit 31,
// written at the bucket's offset plus the chunk's prefix within the bucket plus the
// rank the counting pass handed out. MAXW > 0 unrolls over at most MAXW windows so
// that the loads of one half-scalar are all in flight together.
template <int MAXW>
__global__ void __launch_bounds__(256) k_scatter(const uint32_t* __restrict__ halfs, uint32_t m,
                                                 uint32_t c, uint32_t nwin, uint32_t chunk,
                                                 uint32_t nchunk,
                                                 const uint32_t* __restrict__ offsets,
                                                 const uint32_t* __restrict__ hist_blk,
                                                 const uint32_t* __restrict__ rank,
                                                 uint32_t* __restrict__ sorted_idx) {
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m) return;
  bool sneg;
  const sc256 s = load_half(halfs, i, sneg);
  const uint32_t sh = c - 1, ch = i / chunk;
  auto pos_of = [&](uint32_t j, uint32_t slot) -> uint32_t {
    return offsets[(j << sh) | slot] + hist_blk[(((size_t)j * nchunk + ch) << sh) + slot] +
           rank[(size_t)j * m + i];
  };
  if constexpr (MAXW > 0) {
    uint32_t slot[MAXW], pos[MAXW];
    bool act[MAXW], neg[MAXW];
    signed_digits<MAXW>(s, c, nwin, slot, act, neg);
#pragma unroll
    for (int j = 0; j < MAXW; j++)
      if (act[j]) pos[j] = pos_of((uint32_t)j, digit_slot(c, nwin, (uint32_t)j, slot[j] + 1, i));
#pragma unroll
    for (int j = 0; j < MAXW; j++)
      if (act[j]) sorted_idx[pos[j]] = i | ((neg[j] != sneg) ? 0x80000000u : 0u);
  } else {
    for_each_signed_digit(s, c, nwin, [&](uint32_t j, uint32_t sl, bool ng) {
      sorted_idx[pos_of(j, digit_slot(c, nwin, j, sl + 1, i))] = i | ((ng != sneg) ? 0x80000000u : 0u);
    });
  }
}

// ------------------------------------------------------------------ scan
// Value scanned for bucket k: its count (level < 0), or the number of pair adds
// it has at pair-tree level `level`: floor(ceil(count / 2^level) / 2).
__device__ __forceinline__ uint32_t scan_value(const uint32_t* counts, uint32_t k, uint32_t n,
                                               int level) {
  if (k >= n) return 0;
  uint32_t c = counts[k];
  return level < 0 ? c : (level_count(c, level) >> 1);
}

// Exclusive scan of 256 per-thread values in a block; returns this thread's prefix,
// *total gets the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds, uint32_t* total) {
  uint32_t t = threadIdx.x;
  lds[t] = v;
  __syncthreads();
  for (uint32_t off = 1; off < 256; off <<= 1) {
    uint32_t add = (t >= off) ? lds[t - off] : 0u;
    __syncthreads();
    lds[t] += add;
    __syncthreads();
  }
  uint32_t incl = lds[t];
  *total = lds[255];
  __syncthreads();
  return incl - v;
}

// Pair-tree levels needed for a largest bucket of max_count entries.
__device__ __forceinline__ bool level_needed(int level, const uint32_t* max_count) {
  return level < 0 || !max_count || ((uint64_t)1 << level) < *max_count;
}

// The scans run over several levels at once: blockIdx.y selects level level0 + y,
// whose block sums sit at block_sums + y (nb + 1) and whose output at out + y stride.
__global__ void __launch_bounds__(256) k_scan_reduce(const uint32_t* __restrict__ counts, uint32_t n,
                                                     int level0, uint32_t* __restrict__ block_sums,
                                                     uint32_t nb, const uint32_t* max_count) {
  __shared__ uint32_t lds[256];
  const int level = level0 + (int)blockIdx.y;
  if (!level_needed(level, max_count)) return;
  uint32_t base = blockIdx.x * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < SCAN_ITEMS; e++) sum += scan_value(counts, base + e, n, level);
  uint32_t total;
  block_exclusive_scan(sum, lds, &total);
  if (threadIdx.x == 0) block_sums[(size_t)blockIdx.y * (nb + 1) + blockIdx.x] = total;
}

// One block of 256 threads per level scans up to 256 * SCAN_TOP_ITEMS block sums in
// place (exclusive) and stores the grand total at block_sums[nb].
__global__ void __launch_bounds__(256) k_scan_top(uint32_t* block_sums_all, uint32_t nb, int level0,
                                                  const uint32_t* max_count) {
  __shared__ uint32_t lds[256];
  if (!level_needed(level0 + (int)blockIdx.x, max_count)) return;
  uint32_t* block_sums = block_sums_all + (size_t)blockIdx.x * (nb + 1);
  uint32_t base = threadIdx.x * SCAN_TOP_ITEMS;
  uint32_t v[SCAN_TOP_ITEMS];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < SCAN_TOP_ITEMS; e++) {
    v[e] = (base + e < nb) ? block_sums[base + e] : 0u;
    sum += v[e];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan(sum, lds, &total);
#pragma unroll
  for (int e = 0; e < SCAN_TOP_ITEMS; e++) {
    if (base + e < nb) block_sums[base + e] = run;
    run += v[e];
  }
  if (threadIdx.x == 0) block_sums[nb] = total;
}

__global__ void __launch_bounds__(256) k_scan_down(const uint32_t* __restrict__ counts, uint32_t n,
                                                   int level0, const uint32_t* __restrict__ block_sums_all,
                                                   uint32_t nb, uint32_t* __restrict__ out_all,
                                                   size_t out_stride, const uint32_t* max_count) {
  __shared__ uint32_t lds[256];
  const int level = level0 + (int)blockIdx.y;
  if (!level_needed(level, max_count)) return;
  const uint32_t* block_sums = block_sums_all + (size_t)blockIdx.y * (nb + 1);
  uint32_t* out = out_all + (size_t)blockIdx.y * out_stride;
  uint32_t base = blockIdx.x * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  uint32_t v[SCAN_ITEMS];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < SCAN_ITEMS; e++) {
    v[e] = scan_value(counts, base + e, n, level);
    sum += v[e];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan(sum, lds, &total) + block_sums[blockIdx.x];
#pragma unroll
  for (int e = 0; e < SCAN_ITEMS; e++) {
    if (base + e < n) out[base + e] = run;
    run += v[e];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) out[n] = block_sums[nb];
}

// ------------------------------------------------------------------ buckets
// Point named by a bucket-list entry: index in bits 0..30, negated when bit 31 is set
// (the negative of (x, y) is (x, -y); the infinity encoding (0, 0) stays put).
__device__ __forceinline__ aff load_entry(const g1a* points, uint32_t e) {
  aff a = aff_load(points + (e & 0x7fffffffu));
  if (e >> 31) a.y = fp_neg(a.y);
  return a;
}

__device__ __forceinline__ void xyzz_store(xyzz_st* p, const xyzz& a) {
#pragma unroll
  for (int i = 0; i < 8; i++) {
    p->w[i] = a.X.v[i];
    p->w[8 + i] = a.Y.v[i];
    p->w[16 + i] = a.ZZ.v[i];
    p->w[24 + i] = a.ZZZ.v[i];
  }
}

__device__ __forceinline__ xyzz xyzz_load(const xyzz_st* p) {
  xyzz a;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a.X.v[i] = p->w[i];
    a.Y.v[i] = p->w[8 + i];
    a.ZZ.v[i] = p->w[16 + i];
    a.ZZZ.v[i] = p->w[24 + i];
  }
  return a;
}

__global__ void __launch_bounds__(256) k_bucket_init(const uint32_t* __restrict__ counts,
                                                     const uint32_t* __restrict__ offsets, uint32_t K,
                                                     const uint32_t* __restrict__ sorted_idx,
                                                     const g1a* __restrict__ points,
                                                     xyzz_st* __restrict__ bsum) {
  uint32_t k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  uint32_t c = counts[k];
  if (c == 0) {
    xyzz_store(bsum + k, xyzz_inf());
  } else if (c == 1) {
    xyzz_store(bsum + k, xyzz_from_aff(load_entry(points, sorted_idx[offsets[k]])));
  }
}

// Start of bucket k's elements in the buffers of pair-tree levels >= 1: a level-l
// bucket holds at most ceil(count / 2) elements, and (offset + k) / 2 leaves exactly
// that much room before the next bucket.
__device__ __forceinline__ uint32_t half_base(uint32_t off, uint32_t k) { return (off + k) >> 1; }

// Bucket of a pair: the largest k in [0, n) with a[k] <= x, for the non-decreasing pair
// offsets a of a level (n + 1 entries, a[0] = 0 <= x < a[n]). Each read is a dependent
// load, so rather than bisecting all n buckets the search first tests, with two loads
// issued together, whether the answer lies within GUESS_SPAN buckets of a guess, and
// then bisects that bracket (about log2(2 GUESS_SPAN) reads) or, when it does not (skewed
// bucket sizes), the whole array. Every lane runs the same code path, so a wavefront
// waits for its slowest lane's reads and for nothing else.
constexpr uint32_t GUESS_SPAN = 128;

// Largest k in [lo, hi) with a[k] <= x, given a[lo] <= x < a[hi].
__device__ __forceinline__ uint32_t bisect_le(const uint32_t* a, uint32_t lo, uint32_t hi, uint32_t x) {
  while (hi - lo > 1) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (a[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The bucket of x, searched from the guess g.
__device__ __forceinline__ uint32_t bucket_of(const uint32_t* a, uint32_t n, uint32_t x, uint32_t g) {
  if (g >= n) g = n - 1;
  uint32_t lo = g > GUESS_SPAN ? g - GUESS_SPAN : 0u;
  uint32_t hi = min(g + GUESS_SPAN, n);
  const bool in = (a[lo] <= x) & (a[hi] > x);
  if (!in) {
    lo = 0;
    hi = n;
  }
  return bisect_le(a, lo, hi, x);
}

// Guess for the bucket of pair p: pairs spread evenly over the K buckets.
__device__ __forceinline__ uint32_t bucket_guess(uint32_t p, uint32_t K, uint32_t npairs) {
  return (uint32_t)(((uint64_t)p * K) / npairs);
}

// Operands of pair-tree level `level`: pair m of bucket k adds elements 2m and 2m+1
// of the bucket's list at this level. Level 0 reads the points through sorted_idx
// (bucket k's entries at offsets[k] + i); later levels read the previous level's
// buffer (entries at half_base(offsets[k], k) + i). Output m goes to
// half_base + m, or straight to the bucket sum when the bucket has exactly two
// elements left; the last pair of an odd list also moves the unpaired element along.
template <int S>
struct LevelSrc {
  const g1a* in;
  const uint32_t* idx;
  g1a* out;
  xyzz_st* bsum;
  const uint32_t* counts;
  const uint32_t* offsets;
  int level;
  uint32_t ea[S], eb[S], kb[S], mm[S];

  __device__ __forceinline__ uint32_t base(uint32_t k) const {
    return idx ? offsets[k] : half_base(offsets[k], k);
  }
  __device__ __forceinline__ uint32_t elem(uint32_t pos) const { return idx ? idx[pos] : pos; }
  __device__ __forceinline__ aff get(uint32_t e) const { return idx ? load_entry(in, e) : aff_load(in + e); }
  // the x-coordinate does not depend on the entry's sign bit
  __device__ __forceinline__ fp getx(uint32_t e) const { return fp_load_x(in + (idx ? (e & 0x7fffffffu) : e)); }
  __device__ __forceinline__ aff a(int s) const { return get(ea[s]); }
  __device__ __forceinline__ aff b(int s) const { return get(eb[s]); }
  __device__ __forceinline__ fp ax(int s) const { return getx(ea[s]); }
  __device__ __forceinline__ fp bx(int s) const { return getx(eb[s]); }
  __device__ __forceinline__ void put(int s, const aff& r) const {
    uint32_t k = kb[s], m = mm[s];
    uint32_t cl = level_count(counts[k], level);
    if (cl == 2) {
      xyzz_store(bsum + k, xyzz_from_aff(r));
      return;
    }
    uint32_t ob = half_base(offsets[k], k);
    aff_store(out + ob + m, r);
    uint32_t np = cl >> 1;
    if ((cl & 1u) && m == np - 1) aff_store(out + ob + np, get(elem(base(k) + cl - 1)));
  }
};

template <int S>
__global__ void __launch_bounds__(256) k_level(const g1a* __restrict__ in,
                                               const uint32_t* __restrict__ idx, g1a* out, xyzz_st* bsum,
                                               const uint32_t* __restrict__ counts,
                                               const uint32_t* __restrict__ offsets,
                                               const uint32_t* __restrict__ poff, uint32_t K,
                                               uint32_t npairs, int level) {
  uint64_t p0 = (uint64_t)(blockIdx.x * blockDim.x + threadIdx.x) * S;
  if (p0 >= npairs) return;
  int cnt = (int)min((uint64_t)S, (uint64_t)npairs - p0);
  LevelSrc<S> src{in, idx, out, bsum, counts, offsets, level, {}, {}, {}, {}};
  // bucket of the first pair; later pairs stay in it or move to a later bucket
  uint32_t k = bucket_of(poff, K, (uint32_t)p0, bucket_guess((uint32_t)p0, K, npairs));
#pragma unroll
  for (int s = 0; s < S; s++) {
    if (s < cnt) {
      uint32_t p = (uint32_t)p0 + s;
      if (p >= poff[k + 1]) {  // a later bucket: most often the next one
        k++;
        if (k + 1 < K && p >= poff[k + 1]) {
          const uint32_t hi = min(k + 9, K);
          k = bisect_le(poff, k + 1, poff[hi] > p ? hi : K, p);
        }
      }
      uint32_t m = p - poff[k];
      src.kb[s] = k;
      src.mm[s] = m;
      uint32_t pos = src.base(k) + 2 * m;
      src.ea[s] = src.elem(pos);
      src.eb[s] = src.elem(pos + 1);
    }
  }
  batch_affine_add<S>(src, cnt);
}


// Pair-tree level in XYZZ coordinates, one pair per lane and no inversion: the
// deep levels have few pairs, so their time is one addition's latency rather than an
// inversion's. Inputs are affine (IN_AFF, the output of a batched-affine level, or
// the points themselves through sorted_idx at level 0) or XYZZ; outputs are XYZZ.
template <bool IN_AFF>
__global__ void __launch_bounds__(128, 3) k_level_xyzz(const void* __restrict__ in_,
                                                    const uint32_t* __restrict__ idx,
                                                    xyzz_st* __restrict__ out, xyzz_st* bsum,
                                                    const uint32_t* __restrict__ counts,
                                                    const uint32_t* __restrict__ offsets,
                                                    const uint32_t* __restrict__ poff, uint32_t K,
                                                    uint32_t npairs, int level) {
  uint32_t p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= npairs) return;
  uint32_t k = bucket_of(poff, K, p, bucket_guess(p, K, npairs));
  uint32_t m = p - poff[k];
  uint32_t off = offsets[k];
  uint32_t base = idx ? off : half_base(off, k);
  uint32_t cl = level_count(counts[k], level);
  auto load_aff = [&](uint32_t pos) -> aff {
    const g1a* in = reinterpret_cast<const g1a*>(in_);
    return idx ? load_entry(in, idx[pos]) : aff_load(in + pos);
  };
  auto load = [&](uint32_t pos) -> xyzz {
    if (IN_AFF) return xyzz_from_aff(load_aff(pos));
    return xyzz_load(reinterpret_cast<const xyzz_st*>(in_) + pos);
  };
  xyzz r;
  if (IN_AFF) {
    uint32_t ia = base + 2 * m;
    r = xyzz_add_aa(load_aff(ia), load_aff(ia + 1));
  } else {
    r = xyzz_add(load(base + 2 * m), load(base + 2 * m + 1));
  }
  if (cl == 2) {
    xyzz_store(bsum + k, r);
    return;
  }
  uint32_t ob = half_base(off, k);
  xyzz_store(out + ob + m, r);
  uint32_t np = cl >> 1;
  if ((cl & 1u) && m == np - 1) xyzz_store(out + ob + np, load(base + cl - 1));
}

// The same level with one pair per quad (quad.hpp): for small levels, whose time is
// one addition's latency, four lanes share each addition.
template <bool IN_AFF>
__global__ void __launch_bounds__(128) k_level_xyzz_q(const void* __restrict__ in_,
                                                      const uint32_t* __restrict__ idx,
                                                      xyzz_st* __restrict__ out, xyzz_st* bsum,
                                                      const uint32_t* __restrict__ counts,
                                                      const uint32_t* __restrict__ offsets,
                                                      const uint32_t* __restrict__ poff,
                                                      uint32_t K, uint32_t npairs, int level) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t p = gid >> 2;
  const int q = (int)(gid & 3u);
  if (p >= npairs) return;
  uint32_t k = bucket_of(poff, K, p, bucket_guess(p, K, npairs));
  uint32_t m = p - poff[k];
  uint32_t off = offsets[k];
  uint32_t base = idx ? off : half_base(off, k);
  uint32_t cl = level_count(counts[k], level);
  auto load_aff = [&](uint32_t pos) -> aff {
    const g1a* in = reinterpret_cast<const g1a*>(in_);
    return idx ? load_entry(in, idx[pos]) : aff_load(in + pos);
  };
  auto load = [&](uint32_t pos) -> xyzz {
    if (IN_AFF) return xyzz_from_aff(load_aff(pos));
    return xyzz_load(reinterpret_cast<const xyzz_st*>(in_) + pos);
  };
  const xyzz r = IN_AFF ? quad_add_aa(load_aff(base + 2 * m), load_aff(base + 2 * m + 1), q)
                        : quad_add(load(base + 2 * m), load(base + 2 * m + 1), q);
  if (q != 0) return;
  if (cl == 2) {
    xyzz_store(bsum + k, r);
    return;
  }
  uint32_t ob = half_base(off, k);
  xyzz_store(out + ob + m, r);
  uint32_t np = cl >> 1;
  if ((cl & 1u) && m == np - 1) xyzz_store(out + ob + np, load(base + cl - 1));
}

// ------------------------------------------------------------------ reduction
// XYZZ point of lane (this lane xor `mask`), for a mask that is a multiple of 4 (a whole
// other quad); ds_bpermute, no LDS storage.
__device__ __forceinline__ xyzz xyzz_shfl_xor(const xyzz& a, int mask) {
  xyzz r;
  const int src = (((int)(threadIdx.x & 63)) ^ mask) << 2;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    r.X.v[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)a.X.v[i]);
    r.Y.v[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)a.Y.v[i]);
    r.ZZ.v[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)a.ZZ.v[i]);
    r.ZZZ.v[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)a.ZZZ.v[i]);
  }
  return r;
}

// Window j has 2^(c-1) bucket slots; slot b holds points whose digit has magnitude
// floor(b / f) + 1 (f = window_spread), so W_j = sum_b (floor(b / f) + 1) B_b. Segment s
// covers slots [lo, hi). Running from the top slot down, T sums the slots so far and R
// adds T at every slot that is a multiple of f; then R = sum_b (floor(b / f) -
// ceil(lo / f) + 1) B_b, and the segment's share of W_j is R + ceil(lo / f) T.
__device__ __forceinline__ xyzz rsum_segment(const xyzz_st* __restrict__ bsum, uint32_t c,
                                             uint32_t nwin, uint32_t seg_len, uint32_t j,
                                             uint32_t s, int q) {
  const uint32_t nb = 1u << (c - 1);
  const uint32_t lo = s * seg_len, hi = min(nb, (s + 1) * seg_len);
  const uint32_t f = window_spread(c, nwin, j);
  xyzz T = xyzz_inf(), R = xyzz_inf();
  for (uint32_t b = hi; b-- > lo;) {
    T = quad_add(T, xyzz_load(bsum + (size_t)j * nb + b), q);
    if ((b & (f - 1)) == 0) R = quad_add(R, T, q);
  }
  return quad_add(R, quad_mul_small(T, (lo + f - 1) / f, q), q);
}

// The 64 quads of a block add their points through an LDS tree; thread 0 stores the sum.
__device__ __forceinline__ void block_quad_sum(xyzz acc, xyzz_st* lds, xyzz_st* out) {
  const uint32_t quad = threadIdx.x >> 2;
  const int q = (int)(threadIdx.x & 3u);
  if (q == 0) xyzz_store(&lds[quad], acc);
  __syncthreads();
  for (uint32_t stride = 32; stride > 0; stride >>= 1) {
    if (quad < stride) {
      acc = quad_add(acc, xyzz_load(&lds[quad + stride]), q);
      if (q == 0) xyzz_store(&lds[quad], acc);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) xyzz_store(out, acc);
}

// Running sums and the first tree pass in one launch: block b of window j takes segments
// [64 b, 64 b + 64) of the window's nseg, one per quad, and writes their sum to
// out[j nblk + b] (nblk = ceil(nseg / 64); nseg <= 4096 for every c, so a window needs
// at most 64 blocks).
__global__ void __launch_bounds__(256) k_rsum_tree(const xyzz_st* __restrict__ bsum, uint32_t c,
                                                   uint32_t nwin, uint32_t seg_len, uint32_t nseg,
                                                   uint32_t nblk, xyzz_st* __restrict__ out) {
  __shared__ xyzz_st lds[64];
  const uint32_t j = blockIdx.x / nblk, b = blockIdx.x % nblk, quad = threadIdx.x >> 2;
  const int q = (int)(threadIdx.x & 3u);
  const uint32_t sg = b * 64 + quad;
  xyzz acc = xyzz_inf();
  if (sg < nseg) acc = rsum_segment(bsum, c, nwin, seg_len, j, sg, q);
  block_quad_sum(acc, lds, out + blockIdx.x);
}

// Sums of groups of n consecutive XYZZ points, one wavefront per group: quad g adds
// items g, g + 16, ..., then a butterfly over the 16 quads (ds_bpermute, four additions
// deep) leaves the sum in every quad. The second pass, from the partials of k_rsum_tree
// to the window sums.
__global__ void __launch_bounds__(64) k_tree_sum(const xyzz_st* __restrict__ in, uint32_t n,
                                                 xyzz_st* __restrict__ out) {
  const uint32_t g = blockIdx.x, quad = threadIdx.x >> 2;
  const int q = (int)(threadIdx.x & 3u);
  xyzz acc = xyzz_inf();
  for (uint32_t i = quad; i < n; i += 16) acc = quad_add(acc, xyzz_load(in + (size_t)g * n + i), q);
#pragma unroll
  for (int m = 4; m < 64; m <<= 1) acc = quad_add(acc, xyzz_shfl_xor(acc, m), q);
  if (threadIdx.x == 0) xyzz_store(out + g, acc);
}

// ---- window combine ----------------------------------------------------------------
// The combine is one long chain (c (W - 1) doublings), so its time is latency, not
// throughput. The four lanes of a quad split each round of products (quad.hpp): a run
// of doublings with one round of lookahead costs 2.5 product latencies per doubling,
// an addition 4. Every quad computes its own chain, so every branch is uniform within
// a quad.

// Q = sum_j 2^(c j) W_j, then to affine. Two wavefronts: wave 0 doubles the top window's
// sum c (W - 1) times. In wave 1, quad g doubles W_g c g times (at most c (W - 2)), and a
// tree over the quads adds the results (four additions deep), so no addition sits on the
// longest chain; with more than 17 windows (c <= 7) wave 1 runs Horner over the lower
// windows instead. One addition joins the two waves. W >= 8 for every c <= 16.
__global__ void __launch_bounds__(128) k_final(const xyzz_st* __restrict__ win, uint32_t nwin,
                                               uint32_t c, g1a* out) {
  __shared__ xyzz_st low;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane & 3;
  const uint32_t g = (uint32_t)lane >> 2;
  xyzz acc;
  if (wave == 0) {
    acc = quad_dbl_n(xyzz_load(win + nwin - 1), c * (nwin - 1), q);
  } else {
    if (nwin - 1 <= 16) {
      acc = (g < nwin - 1) ? quad_dbl_n(xyzz_load(win + g), c * g, q) : xyzz_inf();
#pragma unroll
      for (int m = 4; m < 64; m <<= 1) acc = quad_add(acc, xyzz_shfl_xor(acc, m), q);
    } else {
      acc = xyzz_load(win + nwin - 2);
      for (int j = (int)nwin - 3; j >= 0; j--) acc = quad_add(quad_dbl_n(acc, c, q), xyzz_load(win + j), q);
    }
    if (lane == 0) xyzz_store(&low, acc);
  }
  __syncthreads();
  if (wave == 0) {
    acc = quad_add(acc, xyzz_load(&low), q);
    const aff a = xyzz_to_aff(acc);
    if (lane == 0) aff_store(out, a);
  }
}

// ------------------------------------------------------------------ generator
__global__ void __launch_bounds__(128) k_from_scalars(const uint32_t* __restrict__ ks, uint32_t n,
                                                      g1a* __restrict__ out) {
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  sc256 k = load_scalar(ks, i);
  aff g;
  g.x = fp_from_u32(1);
  g.y = fp_from_u32(2);
  xyzz acc = xyzz_inf();
  for (int w = 7; w >= 0; w--) {
    uint32_t word = k.w[w];
    for (int b = 31; b >= 0; b--) {
      acc = xyzz_dbl(acc);
      if ((word >> b) & 1u) acc = xyzz_add_aff(acc, g);
    }
  }
  aff_store(out + i, xyzz_to_aff(acc));
}

// ------------------------------------------------------------------ test hooks
__device__ __forceinline__ fp fp_load_words(const uint32_t* p) {
  fp r;
#pragma unroll
  for (int i = 0; i < 8; i++) r.v[i] = p[i];
  return r;
}

__global__ void k_test_fp(int op, const uint32_t* a, const uint32_t* b, uint32_t* out, uint32_t n) {
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  fp x = fp_load_words(a + 8 * (size_t)i), y = fp_zero(), r;
  if (b) y = fp_load_words(b + 8 * (size_t)i);
  switch (op) {
    case 0: r = fp_mul(x, y); break;
    case 1: r = fp_add(x, y); break;
    case 2: r = fp_sub(x, y); break;
    case 3: r = fp_sqr(x); break;
    case 4: r = fp_is_zero(x) ? fp_zero() : fp_inv(x); break;
    case 5: r = fp_mul(x, fp_r2()); break;
    default: {
      fp one = fp_zero();
      one.v[0] = 1;
      r = fp_mul(x, one);
    }
  }
#pragma unroll
  for (int k = 0; k < 8; k++) out[8 * (size_t)i + k] = r.v[k];
}

template <int S>
struct PairSrc {
  const g1a* a_;
  const g1a* b_;
  g1a* out;
  uint32_t base;
  __device__ __forceinline__ aff a(int s) const { return aff_load(a_ + base + s); }
  __device__ __forceinline__ aff b(int s) const { return aff_load(b_ + base + s); }
  __device__ __forceinline__ fp ax(int s) const { return fp_load_x(a_ + base + s); }
  __device__ __forceinline__ fp bx(int s) const { return fp_load_x(b_ + base + s); }
  __device__ __forceinline__ void put(int s, const aff& r) const { aff_store(out + base + s, r); }
};

__global__ void __launch_bounds__(128) k_test_glv(const uint32_t* __restrict__ scalars, uint32_t n,
                                                  uint32_t* __restrict__ halfs) {
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const sc256 sc = load_scalar(scalars, i);
  uint32_t s[8], k1[4], k2[4];
#pragma unroll
  for (int w = 0; w < 8; w++) s[w] = sc.w[w];
  bool bad = false;
  glv_split(s, k1, k2, bad);
  reinterpret_cast<uint4*>(halfs)[i] = make_uint4(k1[0], k1[1], k1[2], k1[3]);
  reinterpret_cast<uint4*>(halfs)[n + i] = make_uint4(k2[0], k2[1], k2[2], k2[3]);
}

template <int S>
__global__ void __launch_bounds__(256) k_test_pair_add(const g1a* a, const g1a* b, g1a* out,
                                                       uint32_t n) {
  uint64_t p0 = (uint64_t)(blockIdx.x * blockDim.x + threadIdx.x) * S;
  if (p0 >= n) return;
  int cnt = (int)min((uint64_t)S, (uint64_t)n - p0);
  PairSrc<S> src{a, b, out, (uint32_t)p0};
  batch_affine_add<S>(src, cnt);
}

// ------------------------------------------------------------------ launchers
static inline unsigned grid_for(size_t n, unsigned block) { return (unsigned)((n + block - 1) / block); }

hipError_t launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_fill_u32<<<grid_for(n, 256), 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_glv_prep(const g1a* points, const uint32_t* scalars, uint32_t n, g1a* pts2,
                           uint32_t* halfs, msm_stats* st, hipStream_t s) {
  k_glv_prep<<<grid_for(n, 128), 128, 0, s>>>(points, scalars, n, pts2, halfs, st);
  return hipGetLastError();
}

hipError_t launch_hist(const uint32_t* halfs, uint32_t m, uint32_t c, uint32_t nwin,
                       uint32_t chunk, uint32_t nchunk, uint32_t* hist_blk, uint32_t* counts,
                       uint32_t* rank, msm_stats* st, hipStream_t s) {
  const size_t lds = ((size_t)1 << (c - 1)) * 4;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k_hist_tile,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  k_hist_tile<<<dim3(nchunk, nwin), 1024, lds, s>>>(halfs, m, c, nwin, chunk, nchunk, hist_blk, rank);
  const uint32_t K = nwin << (c - 1);
  k_chunk_scan<<<grid_for(K, 256), 256, 0, s>>>(hist_blk, c, nwin, nchunk, counts, st);
  return hipGetLastError();
}

hipError_t launch_scatter(const uint32_t* halfs, uint32_t m, uint32_t c, uint32_t nwin,
                          uint32_t chunk, uint32_t nchunk, const uint32_t* offsets,
                          const uint32_t* hist_blk, const uint32_t* rank, uint32_t* sorted_idx,
                          hipStream_t s) {
  if (nwin <= 16)
    k_scatter<16><<<grid_for(m, 256), 256, 0, s>>>(halfs, m, c, nwin, chunk, nchunk, offsets,
                                                    hist_blk, rank, sorted_idx);
  else
    k_scatter<0><<<grid_for(m, 256), 256, 0, s>>>(halfs, m, c, nwin, chunk, nchunk, offsets,
                                                   hist_blk, rank, sorted_idx);
  return hipGetLastError();
}

hipError_t launch_scan(const uint32_t* counts, uint32_t n, int level0, int nlev,
                       uint32_t* block_sums, uint32_t* out, size_t out_stride,
                       const uint32_t* max_count, hipStream_t s) {
  uint32_t nb = scan_blocks(n);
  if (nlev < 1) return hipSuccess;
  k_scan_reduce<<<dim3(nb, nlev), 256, 0, s>>>(counts, n, level0, block_sums, nb, max_count);
  k_scan_top<<<nlev, 256, 0, s>>>(block_sums, nb, level0, max_count);
  k_scan_down<<<dim3(nb, nlev), 256, 0, s>>>(counts, n, level0, block_sums, nb, out, out_stride,
                                              max_count);
  return hipGetLastError();
}


hipError_t launch_bucket_init(const uint32_t* counts, const uint32_t* offsets, uint32_t K,
                              const uint32_t* sorted_idx, const g1a* points, xyzz_st* bsum,
                              hipStream_t s) {
  k_bucket_init<<<grid_for(K, 256), 256, 0, s>>>(counts, offsets, K, sorted_idx, points, bsum);
  return hipGetLastError();
}

template <int S>
static hipError_t level_S(const g1a* in, const uint32_t* idx, g1a* out, xyzz_st* bsum,
                          const uint32_t* counts, const uint32_t* offsets, const uint32_t* poff,
                          uint32_t K, uint32_t npairs, int level, hipStream_t s) {
  size_t threads = (npairs + S - 1) / S;
  k_level<S><<<grid_for(threads, LEVEL_BLOCK), LEVEL_BLOCK, 0, s>>>(in, idx, out, bsum, counts,
                                                                    offsets, poff, K, npairs, level);
  return hipGetLastError();
}

hipError_t launch_level(int S, const g1a* in, const uint32_t* idx, g1a* out, xyzz_st* bsum,
                        const uint32_t* counts, const uint32_t* offsets, const uint32_t* poff,
                        uint32_t K, uint32_t npairs, int level, hipStream_t s) {
  switch (S) {
    case 4: return level_S<4>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    case 8: return level_S<8>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    case 16: return level_S<16>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    case 32: return level_S<32>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_level_xyzz(bool in_aff, const void* in, const uint32_t* idx, xyzz_st* out,
                             xyzz_st* bsum, const uint32_t* counts, const uint32_t* offsets,
                             const uint32_t* poff, uint32_t K, uint32_t npairs, int level,
                             hipStream_t s) {
  if (npairs <= XYZZ_QUAD_MAX_PAIRS) {  // small level: four lanes per addition
    unsigned g = grid_for((size_t)npairs * 4, 128);
    if (in_aff)
      k_level_xyzz_q<true><<<g, 128, 0, s>>>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level);
    else
      k_level_xyzz_q<false><<<g, 128, 0, s>>>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level);
    return hipGetLastError();
  }
  unsigned g = grid_for(npairs, 128);
  if (in_aff)
    k_level_xyzz<true><<<g, 128, 0, s>>>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level);
  else
    k_level_xyzz<false><<<g, 128, 0, s>>>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level);
  return hipGetLastError();
}

hipError_t launch_reduce(const xyzz_st* bsum, uint32_t c, uint32_t nwin, uint32_t seg_len,
                         uint32_t nseg, xyzz_st* part, xyzz_st* win, hipStream_t s) {
  const uint32_t nblk = reduce_blocks(nseg);
  if ((size_t)nblk * 64 < nseg) return hipErrorInvalidValue;  // one segment per quad
  k_rsum_tree<<<nwin * nblk, 256, 0, s>>>(bsum, c, nwin, seg_len, nseg, nblk, part);
  k_tree_sum<<<nwin, 64, 0, s>>>(part, nblk, win);
  return hipGetLastError();
}

hipError_t launch_final(const xyzz_st* win, uint32_t nwin, uint32_t c, g1a* out, hipStream_t s) {
  k_final<<<1, 128, 0, s>>>(win, nwin, c, out);
  return hipGetLastError();
}

hipError_t launch_from_scalars(const uint32_t* ks, uint32_t n, g1a* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  k_from_scalars<<<grid_for(n, 128), 128, 0, s>>>(ks, n, out);
  return hipGetLastError();
}

hipError_t launch_test_fp(int op, const uint32_t* a, const uint32_t* b, uint32_t* out, uint32_t n,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  k_test_fp<<<grid_for(n, 128), 128, 0, s>>>(op, a, b, out, n);
  return hipGetLastError();
}

hipError_t launch_test_glv(const uint32_t* scalars, uint32_t n, uint32_t* halfs, hipStream_t s) {
  k_test_glv<<<grid_for(n, 128), 128, 0, s>>>(scalars, n, halfs);
  return hipGetLastError();
}

hipError_t launch_test_pair_add(int S, const g1a* a, const g1a* b, g1a* out, uint32_t n,
                                hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t threads;
  switch (S) {
    case 4: threads = (n + 3) / 4; k_test_pair_add<4><<<grid_for(threads, 256), 256, 0, s>>>(a, b, out, n); break;
    case 8: threads = (n + 7) / 8; k_test_pair_add<8><<<grid_for(threads, 256), 256, 0, s>>>(a, b, out, n); break;
    case 16: threads = (n + 15) / 16; k_test_pair_add<16><<<grid_for(threads, 256), 256, 0, s>>>(a, b, out, n); break;
    case 32: threads = (n + 31) / 32; k_test_pair_add<32><<<grid_for(threads, 256), 256, 0, s>>>(a, b, out, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msmk
