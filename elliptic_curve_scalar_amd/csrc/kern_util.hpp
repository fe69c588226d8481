// Device helpers shared by the kernel files of libmsm: scalar words, the bucket-list
// entry format, XYZZ storage, wavefront reductions and the top-window spread.
#pragma once
#include <hip/hip_runtime.h>

#include "msm_internal.hpp"
#include "quad.hpp"

namespace msmk {

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

// Slots per digit value in window j. The half-scalars have 127-bit magnitudes, so the
// top window's digits never exceed 2^(127 - c (W - 1)) while it has 2^(c-1) slots like
// every window: each of its digits is spread over 2^(c W - 128) slots, chosen by the
// half-scalar's index, which evens out the bucket sizes (at c = 13 the top window's
// buckets would otherwise be eight times fuller and the pair tree three levels deeper).
// The running sum weights slot b of window j by floor(b / spread) + 1.
__device__ __forceinline__ uint32_t window_spread(uint32_t c, uint32_t nwin, uint32_t j) {
  return (j + 1 == nwin) ? (1u << (c * nwin - 128)) : 1u;
}

// Entries of a bucket of cnt entries at pair-tree level `level`: ceil(cnt / 2^level).
__device__ __forceinline__ uint32_t level_count(uint32_t cnt, int level) {
  return (uint32_t)(((uint64_t)cnt + (1ull << level) - 1) >> level);
}

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

inline unsigned grid_for(size_t n, unsigned block) { return (unsigned)((n + block - 1) / block); }

}  // namespace msmk
