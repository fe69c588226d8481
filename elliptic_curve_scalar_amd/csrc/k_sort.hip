// Decompose and counting-sort kernels of the BN254 G1 bucket MSM (gfx950), and their
// launchers:
//   k_glv_prep    scalar -> two half-scalars below 2^127; points [P, phi(P)]
//   k_hist_tile   per (chunk of half-scalars, window): LDS histogram, rank per entry
//   k_chunk_scan  per bucket: prefix over the chunks, bucket count; plan statistics
//   k_scan_*      exclusive scans of per-bucket values (counts, pairs per level)
//   k_scatter     point indices into per-bucket lists (sorted_idx)
//   k_bucket_init buckets of size 0 / 1 are final at once
// The sorted lists are the sorted_bucket_list / sorted_count_list of aztec-packages
// PR #23738 ("What would actually win"); how they are built is this library's.
#include <hip/hip_runtime.h>

#include "glv.hpp"
#include "kern_util.hpp"

namespace msmk {

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
                                                  msm_stats* st, int verify, int scalar_form) {
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const sc256 sc = load_scalar(scalars, i);
  uint32_t s[8], k1[4], k2[4];
#pragma unroll
  for (int w = 0; w < 8; w++) s[w] = sc.w[w];
  if (scalar_form) fr_from_mont(s);
  bool bad = false;
  glv_split(s, k1, k2, bad);
  if (bad) atomicOr(&st->range_flag, 1u);
  reinterpret_cast<uint4*>(halfs)[i] = make_uint4(k1[0], k1[1], k1[2], k1[3]);
  reinterpret_cast<uint4*>(halfs)[n + i] = make_uint4(k2[0], k2[1], k2[2], k2[3]);
  aff a = aff_load(points + i);
  if (verify && !aff_valid(a)) atomicOr(&st->bad_point, 1u);
  aff_store(pts2 + i, a);
  if (!aff_is_inf(a)) a.x = fp_mul(a.x, glv_beta());
  aff_store(pts2 + n + i, a);
}

// The curve check of msm_run's verify option on its result.
__global__ void __launch_bounds__(64) k_verify_point(const g1a* __restrict__ p, uint32_t* flag) {
  if (threadIdx.x == 0 && !aff_valid(aff_load(p))) atomicOr(flag, 1u);
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
  // level l has no pair in this wave once 2^l reaches the wave's largest count (every
  // bucket is down to one entry): only the levels below need a reduction
#pragma unroll
  for (int l = 0; l < MAX_LEVELS; l++) {
    uint32_t v = 0;
    if (((uint64_t)1 << l) < mx) v = wave_sum(level_count(cnt, l) >> 1);
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

// Writes the exclusive prefixes of every tile: each block adds up the sums of the tiles
// before it (nb <= SCAN_MAX_BLOCKS), and block 0 adds up all of them for the total.
__global__ void __launch_bounds__(256) k_scan_down(const uint32_t* __restrict__ counts, uint32_t n,
                                                   int level0, const uint32_t* __restrict__ block_sums_all,
                                                   uint32_t nb, uint32_t* __restrict__ out_all,
                                                   size_t out_stride, const uint32_t* max_count) {
  __shared__ uint32_t lds[256];
  __shared__ uint32_t wab[4][2];
  const int level = level0 + (int)blockIdx.y;
  if (!level_needed(level, max_count)) return;
  const uint32_t* block_sums = block_sums_all + (size_t)blockIdx.y * (nb + 1);
  uint32_t* out = out_all + (size_t)blockIdx.y * out_stride;
  // the sums of tiles 0 .. blockIdx.x - 1 and of all nb tiles, over the block's threads
  uint32_t a = 0, b = 0;
#pragma unroll
  for (uint32_t e = 0; e < SCAN_PRE_ITEMS; e++) {
    const uint32_t i = threadIdx.x + 256u * e;
    const uint32_t x = i < nb ? block_sums[i] : 0u;
    a += i < blockIdx.x ? x : 0u;
    b += x;
  }
  a = wave_sum(a);
  b = wave_sum(b);
  if ((threadIdx.x & 63u) == 0) {
    wab[threadIdx.x >> 6][0] = a;
    wab[threadIdx.x >> 6][1] = b;
  }
  __syncthreads();
  const uint32_t pre = wab[0][0] + wab[1][0] + wab[2][0] + wab[3][0];
  const uint32_t grand = wab[0][1] + wab[1][1] + wab[2][1] + wab[3][1];
  uint32_t base = blockIdx.x * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  uint32_t v[SCAN_ITEMS];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < SCAN_ITEMS; e++) {
    v[e] = scan_value(counts, base + e, n, level);
    sum += v[e];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan(sum, lds, &total) + pre;
#pragma unroll
  for (int e = 0; e < SCAN_ITEMS; e++) {
    if (base + e < n) out[base + e] = run;
    run += v[e];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) out[n] = grand;
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

// ------------------------------------------------------------------ launchers
hipError_t launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  k_fill_u32<<<grid_for(n, 256), 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_glv_prep(const g1a* points, const uint32_t* scalars, uint32_t n, g1a* pts2,
                           uint32_t* halfs, msm_stats* st, int verify, int scalar_form, hipStream_t s) {
  k_glv_prep<<<grid_for(n, 128), 128, 0, s>>>(points, scalars, n, pts2, halfs, st, verify,
                                                scalar_form);
  return hipGetLastError();
}

hipError_t launch_verify_point(const g1a* p, uint32_t* flag, hipStream_t s) {
  k_verify_point<<<1, 64, 0, s>>>(p, flag);
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
  if (nb > SCAN_MAX_BLOCKS) return hipErrorInvalidValue;  // K <= 2^18 buckets for c <= 16
  k_scan_reduce<<<dim3(nb, nlev), 256, 0, s>>>(counts, n, level0, block_sums, nb, max_count);
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

}  // namespace msmk
