// Pair-tree level kernels of the BN254 G1 bucket MSM (gfx950), and their launchers:
//   k_level<S>    pair-tree level 0: pair (2m, 2m+1) of every bucket -> element m,
//                 S pairs per lane with one inversion (batch_add.hpp)
//   k_level_xyzz  deeper levels in XYZZ coordinates (quad-cooperative when small)
// The level kernel takes S pairs per lane the way the pair-tree accumulate of
// aztec-packages PR #23520 ("Summary") takes S adds per invocation.
#include <hip/hip_runtime.h>

#include "batch_add.hpp"
#include "kern_util.hpp"

namespace msmk {

// Start of bucket k's elements in the buffers of pair-tree levels >= 1: a level-l
// bucket holds at most ceil(count / 2) elements, and (offset + k) / 2 leaves exactly
// that much room before the next bucket.
__device__ __forceinline__ uint32_t half_base(uint32_t off, uint32_t k) { return (off + k) >> 1; }

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

// ------------------------------------------------------------------ launchers
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

}  // namespace msmk
