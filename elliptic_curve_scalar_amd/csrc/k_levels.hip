// Pair-tree level kernels of the BN254 G1 bucket MSM (gfx950), and their launchers:
//   k_level<S>    pair-tree level 0: pair (2m, 2m+1) of every bucket -> element m,
//                 S pairs per lane with one inversion (batch_add.hpp)
//   k_level_xyzz  deeper levels in XYZZ coordinates (quad-cooperative when small)
// The level kernel takes S pairs per lane the way the pair-tree accumulate of
// aztec-packages PR #23520 ("Summary") takes S adds per invocation.
#include <hip/hip_runtime.h>

#include "batch_add.hpp"
#include "kern_util.hpp"
#include "level_kernel.hpp"

namespace msmk {

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

// ------------------------------------------------------------------ launchers
template <int S>
static hipError_t level_S(const g1a* in, const uint32_t* idx, g1a* out, xyzz_st* bsum,
                          const uint32_t* counts, const uint32_t* offsets, const uint32_t* poff,
                          uint32_t K, uint32_t npairs, int level, hipStream_t s) {
  constexpr unsigned B = level_block<PLACE_PRIVATE>();
  size_t threads = (npairs + S - 1) / S;
  k_level<S, PLACE_PRIVATE><<<grid_for(threads, B), B, 0, s>>>(in, idx, out, bsum, counts, offsets,
                                                               poff, K, npairs, level);
  return hipGetLastError();
}

hipError_t launch_level(int S, int place, const g1a* in, const uint32_t* idx, g1a* out,
                        xyzz_st* bsum, const uint32_t* counts, const uint32_t* offsets,
                        const uint32_t* poff, uint32_t K, uint32_t npairs, int level,
                        hipStream_t s) {
  if (place != PLACE_PRIVATE)
    return launch_level_placed(S, place, in, idx, out, bsum, counts, offsets, poff, K, npairs,
                               level, s);
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

}  // namespace msmk
