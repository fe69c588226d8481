// Bucket reduction and window combine of the BN254 G1 bucket MSM (gfx950), and their
// launchers:
//   k_rsum_tree   per window, segments of buckets: sum_b b * B_b by running sums,
//                 summed per block through an LDS tree
//   k_tree_sum    per window: the blocks' partial sums -> W_j
//   k_final       Q = sum_j 2^(c j) W_j by doubling, then affine
#include <hip/hip_runtime.h>

#include "glv.hpp"
#include "kern_util.hpp"

namespace msmk {

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

// ------------------------------------------------------------------ launchers
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

}  // namespace msmk
