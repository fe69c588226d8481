// Bucket reduction and window combine of the BN254 G1 bucket MSM (gfx950), and their
// launchers.
//
// After the accumulate, window j (W windows of c bits over the GLV half-scalars) holds
// 2^(c-1) bucket sums B_{j,b}; slot b carries the weight w_b = floor(b / f_j) + 1 (f_j =
// window_spread), and the result is
//     Q = sum_j 2^(c j) W_j,   W_j = sum_b w_b B_{j,b}.
// A running sum over all slots of a window would be one chain of 2^c additions. Instead
// the slots are cut into segments of L = 2^lambda slots, s = 0 .. nseg - 1:
//     T_s = sum_{b in s} B_b,   R_s = sum_{b in s} (w_b - w_lo(s)) B_b,
// where w_lo(s) is the weight of the segment's first slot (R_s is a running sum over at
// most L slots), so that
//     W_j = sum_s (R_s + T_s) + sum_s (w_lo(s) - 1) T_s,
// and w_lo(s) - 1 = (s L) >> log2(f_j) is a bit field of s. Writing it out bit by bit,
//     Q = sum_j 2^(c j) sum_s (R_s + T_s) + sum_{j, kappa} 2^(c j + kappa) sum_{s : bit kappa
//         of w_lo(s) - 1 is set} T_s.
// Each term is a plane: a plain sum of segment values (no weights), which a tree adds in
// log depth, times a power of two e <= 126, which a run of e doublings gives. Every plane
// is summed and doubled in parallel, and the planes are then added in groups. The
// longest chain is one plane's doublings instead of a running sum per window followed
// by c (W - 1) doublings of the top window.
//
// The planes of segment totals share their sub-sums: with s = hi 2^lb + lo, the sums
// A_hi = sum_lo T_s and B_lo = sum_hi T_s are formed once per window, and the plane of
// bit beta is the sum of the B_lo whose lo has bit beta (beta < lb), or of the A_hi whose
// hi has bit beta - lb: about 2 nseg additions per window for all such planes, against
// nseg / 2 for each.
//
//   k_seg_sums     one quad per (window, segment): T_s and P_s = R_s + T_s
//   k_plane_sums   one wavefront per group: the A_hi and B_lo of every window, and the
//                  (R + T) planes in groups of 64 segments (butterfly over the quads)
//   k_plane_chain  one block of eight wavefronts per plane, in row form (rowpoint.hpp: each
//                  of a round's four products spread over the 16 lanes of a row): the
//                  plane's terms, then 2^e S by a run of doublings on one wavefront; the
//                  last block of each join group of planes adds the group, the last group
//                  adds the groups and converts the result to affine
#include <hip/hip_runtime.h>
#include <string.h>

#include "glv.hpp"
#include "kern_util.hpp"
#include "rowpoint.hpp"

namespace msmk {

// Sum over the first `used` quads of a wavefront (1 <= used <= 16; the others hold the
// point at infinity): a ds_bpermute butterfly over the smallest power-of-two group of quads
// that covers them, ceil(log2 used) additions deep. Quad 0 ends with the total.
__device__ __forceinline__ xyzz wave_quad_sum(xyzz acc, uint32_t used, int q) {
#pragma unroll 1
  for (uint32_t m = 4; m < 4 * used; m <<= 1) acc = quad_add(acc, xyzz_shfl_xor(acc, (int)m), q);
  return acc;
}

// Segment sums, one quad per (window j, segment s) at g = j nseg + s. Running from the
// segment's top slot down, T adds each slot and R adds T after the lowest slot of every
// weight group except the segment's lowest, so R = sum (w_b - w_lo) B_b.
__global__ void __launch_bounds__(256) k_seg_sums(const xyzz_st* __restrict__ bsum, uint32_t c,
                                                  uint32_t nwin, uint32_t lambda, uint32_t nseg,
                                                  xyzz_st* __restrict__ tseg,
                                                  xyzz_st* __restrict__ pseg) {
  const uint32_t g = (blockIdx.x * blockDim.x + threadIdx.x) >> 2;
  const int q = (int)(threadIdx.x & 3u);
  if (g >= nwin * nseg) return;  // whole quads leave together; no barrier follows
  const uint32_t j = g / nseg, s = g % nseg;
  const uint32_t slots = 1u << (c - 1);
  const uint32_t lo = s << lambda, hi = min(slots, (s + 1) << lambda);
  const uint32_t f = window_spread(c, nwin, j);
  const xyzz_st* B = bsum + (size_t)j * slots;
  xyzz T = xyzz_inf(), R = xyzz_inf();
  for (uint32_t b = hi; b-- > lo;) {
    T = quad_add(T, xyzz_load(B + b), q);
    if (b > lo && (b & (f - 1u)) == 0) R = quad_add(R, T, q);
  }
  const xyzz P = quad_add(R, T, q);
  if (q == 0) {
    xyzz_store(tseg + g, T);
    xyzz_store(pseg + g, P);
  }
}

// Join group of plane p: 0 for p < 2, else floor(log2 p) (group k >= 1 is [2^k, 2^(k+1))).
__device__ __forceinline__ uint32_t plane_group(uint32_t p) { return p < 2u ? 0u : 31u - __clz(p); }

// Spread t over the bits other than beta and set bit beta: the t-th index with bit beta set.
__device__ __forceinline__ uint32_t with_bit(uint32_t t, uint32_t beta) {
  return ((t >> beta) << (beta + 1)) | (1u << beta) | (t & ((1u << beta) - 1u));
}

// Group r of window j (r < pt.wstride), at part[j wstride + r]:
//   r < np:            P_s for the segments s in [r 2^pg, (r + 1) 2^pg) (fewer in the last)
//   r - np = hi < nA:  A_hi = sum of T_s, s = hi 2^lb + lo over lo  (2^lb terms)
//   else lo:           B_lo = sum of T_s, s = hi 2^lb + lo over hi  (2^hb terms)
// One wavefront per group (at most 64 terms), four groups per block: the 16 quads share
// the terms evenly (quad q adds its run of ceil(terms / 16)), then a butterfly over the
// quads (no barriers; whole wavefronts leave together).
__global__ void __launch_bounds__(256) k_plane_sums(const xyzz_st* __restrict__ tseg,
                                                    const xyzz_st* __restrict__ pseg,
                                                    plane_table pt, uint32_t nwin,
                                                    xyzz_st* __restrict__ part) {
  const uint32_t g = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (g >= nwin * pt.wstride) return;
  const uint32_t j = g / pt.wstride, r = g % pt.wstride;
  const uint32_t quad = (threadIdx.x & 63u) >> 2;
  const int q = (int)(threadIdx.x & 3u);
  const uint32_t nA = 1u << pt.hb;
  uint32_t cnt, base, stride;
  const xyzz_st* src = tseg + (size_t)j * pt.nseg;
  if (r < pt.np) {
    src = pseg + (size_t)j * pt.nseg;
    base = r << pt.pg;
    cnt = min(1u << pt.pg, pt.nseg - base);
    stride = 1;
  } else if (r - pt.np < nA) {
    base = (r - pt.np) << pt.lb;
    cnt = 1u << pt.lb;
    stride = 1;
  } else {
    base = r - pt.np - nA;
    cnt = nA;
    stride = 1u << pt.lb;
  }
  const uint32_t per = (cnt + 15u) / 16u;
  xyzz acc = xyzz_inf();
  for (uint32_t i = per * quad; i < per * quad + per && i < cnt; i++)
    acc = quad_add(acc, xyzz_load(src + base + i * stride), q);
  acc = wave_quad_sum(acc, min(16u, (cnt + per - 1u) / per), q);
  if ((threadIdx.x & 63u) == 0) xyzz_store(part + (size_t)j * pt.wstride + r, acc);
}

// Waves per block of k_plane_chain: at least the number of join groups (plane_group of the
// last plane, plus one).
constexpr uint32_t CHAIN_WAVES = 8;
static_assert(MAX_PLANES <= (1 << CHAIN_WAVES), "join groups must fit the block's waves");

// Sum of the points of the block's CHAIN_WAVES wavefronts (row form; LDS holds one point per
// wavefront), a butterfly three additions deep: wave 0 ends with the total. Every
// wavefront of the block calls it (barriers).
__device__ __forceinline__ rxyzz block_row_sum(rxyzz acc, uint32_t w, uint32_t (*sh)[32],
                                               row_consts& k) {
#pragma unroll 1
  for (uint32_t s = 1; s < CHAIN_WAVES; s <<= 1) {
    if ((w & (2u * s - 1u)) == s) rxyzz_to_lds(sh[w], acc);
    __syncthreads();
    if ((w & (2u * s - 1u)) == 0) acc = rxyzz_add(acc, rxyzz_from_lds(sh[w + s]), k);
  }
  return acc;
}

// One block of CHAIN_WAVES wavefronts per plane p, in row form throughout (rowpoint.hpp):
// S = the sum of the plane's terms among its window's group sums (the np (R + T) group
// sums, or the A_hi or B_lo of its bit; wavefront w adds terms w, w + CHAIN_WAVES, ...,
// then the block adds the wavefronts' sums), then 2^e S (e = the plane's exponent) by a
// run of doublings on wavefront 0 while the others wait at the barrier. Planes are in
// order of decreasing e, so the long runs start first. The last block to finish in each
// join group (counted by join[group]) adds the group's results, the block's wavefronts
// sharing them; the last group to finish (join[MAX_PLANE_GROUPS]) adds the group sums
// (one per wavefront) and writes the affine result (its one inversion on wavefront 0).
// The counters start at zero (cleared with the plan statistics before the MSM).
__global__ void __launch_bounds__(64 * CHAIN_WAVES)
k_plane_chain(const xyzz_st* __restrict__ part, plane_table pt, xyzz_st* res, xyzz_st* gres,
              uint32_t* join, g1a* out) {
  __shared__ uint32_t sh[CHAIN_WAVES][32];
  __shared__ uint32_t last_in_group, last_group;
  const uint32_t p = blockIdx.x, w = threadIdx.x >> 6;
  const uint32_t e = pt.e[p] & 0xffu, j = (pt.e[p] >> 8) & 0xffu, sel = pt.e[p] >> 16;
  // the plane's terms: term t is part[first + term_index(t)]
  const xyzz_st* grp_sums = part + (size_t)j * pt.wstride;
  uint32_t nterm, first, beta = 0;
  if (sel == 0) {
    nterm = pt.np;
    first = 0;
  } else if (sel - 1 < pt.lb) {  // B_lo with bit beta of lo
    beta = sel - 1;
    nterm = 1u << (pt.lb - 1);
    first = pt.np + (1u << pt.hb);
  } else {  // A_hi with bit beta - lb of hi
    beta = sel - 1 - pt.lb;
    nterm = 1u << (pt.hb - 1);
    first = pt.np;
  }
  row_consts k = row_consts_load();
  rxyzz acc = rxyzz_inf();
  for (uint32_t t = w; t < nterm; t += CHAIN_WAVES) {
    const uint32_t idx = sel ? with_bit(t, beta) : t;
    acc = rxyzz_add(acc, rxyzz_load(grp_sums + first + idx), k);
  }
  acc = block_row_sum(acc, w, sh, k);
  // join groups by finishing order: planes [0, 2), [2, 4), [4, 8), [8, 16), ... (group k >= 1
  // holds planes [2^k, 2^(k+1))). The long runs end last and sit in the small groups.
  const uint32_t grp = plane_group(p), ngroups = plane_group(pt.n - 1u) + 1u;
  const uint32_t g0 = grp ? (1u << grp) : 0u;
  const uint32_t gsize = min(grp ? (1u << grp) : 2u, pt.n - g0);
  if (w == 0) {
    acc = rxyzz_dbl_n(acc, e, k);
    rxyzz_store(res + p, acc, k);
    __threadfence();
    if (threadIdx.x == 0) last_in_group = (atomicAdd(&join[grp], 1u) + 1u == gsize) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_in_group) return;  // the whole block leaves
  __threadfence();
  acc = rxyzz_inf();
  for (uint32_t i = w; i < gsize; i += CHAIN_WAVES)
    acc = rxyzz_add(acc, rxyzz_load_coherent(res + g0 + i), k);
  acc = block_row_sum(acc, w, sh, k);
  if (w == 0) {
    rxyzz_store(gres + grp, acc, k);
    __threadfence();
    if (threadIdx.x == 0) last_group = (atomicAdd(&join[MAX_PLANE_GROUPS], 1u) + 1u == ngroups) ? 1u : 0u;
  }
  __syncthreads();
  if (!last_group) return;
  __threadfence();
  acc = (w < ngroups) ? rxyzz_load_coherent(gres + w) : rxyzz_inf();
  acc = block_row_sum(acc, w, sh, k);
  if (w == 0) {
    const aff a = xyzz_to_aff(rxyzz_to_fp(acc, k));
    if (threadIdx.x == 0) aff_store(out, a);
  }
}

// ------------------------------------------------------------------ host side
hipError_t launch_reduce(const xyzz_st* bsum, uint32_t c, uint32_t nwin, const plane_table& pt,
                         xyzz_st* tseg, xyzz_st* pseg, xyzz_st* part, hipStream_t s) {
  const size_t quads = (size_t)nwin * pt.nseg;
  k_seg_sums<<<grid_for(quads * 4, 256), 256, 0, s>>>(bsum, c, nwin, pt.lambda, pt.nseg, tseg, pseg);
  const uint32_t groups = nwin * pt.wstride;
  k_plane_sums<<<(groups + 3u) / 4u, 256, 0, s>>>(tseg, pseg, pt, nwin, part);
  return hipGetLastError();
}

hipError_t launch_final(const xyzz_st* part, const plane_table& pt, xyzz_st* res, xyzz_st* gres,
                        uint32_t* join, g1a* out, hipStream_t s) {
  k_plane_chain<<<pt.n, 64 * CHAIN_WAVES, 0, s>>>(part, pt, res, gres, join, out);
  return hipGetLastError();
}

}  // namespace msmk
