// The batched-affine pair-tree level kernel (k_level): S pairs per lane, one inversion
// per lane, slot state placed by PLACE. Shared by the file with the default placement
// and the file with the other placements.
#pragma once
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

// Slot-state placements of the batched-affine level kernel (msm_ctx_set_prefix_store):
// bit 0 puts the prefix products in LDS instead of private memory, bit 1 adds the cached
// denominators (PR #23520 "Summary"); PLACE_CKPT keeps one prefix in CKPT_GROUP in
// private memory and rebuilds the others (batch_affine_add_ckpt).
enum : int { PLACE_PRIVATE = 0, PLACE_LDS = 1, PLACE_DX = 2, PLACE_CKPT = 4 };
constexpr int CKPT_GROUP = 4;  // slots per checkpoint of PLACE_CKPT

// Lanes per block of the level kernel: two wavefronts with private state; one with LDS
// state, whose size grows with S (S * 32 bytes per lane, twice that with the
// denominators).
template <int PLACE>
constexpr unsigned level_block() { return (PLACE & PLACE_LDS) ? 64u : 128u; }

template <int S, int PLACE>
__global__ void __launch_bounds__(128) k_level(const g1a* __restrict__ in,
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
  constexpr bool DX = (PLACE & PLACE_DX) != 0;
  if constexpr (PLACE == PLACE_CKPT) {
    PrefPrivate<S / CKPT_GROUP, false> st;
    batch_affine_add_ckpt<S, CKPT_GROUP>(src, cnt, st);
  } else if constexpr ((PLACE & PLACE_LDS) != 0) {
    extern __shared__ uint32_t lds_pref[];
    PrefLds<S, DX> st{lds_pref, blockDim.x, threadIdx.x};
    batch_affine_add<S, DX>(src, cnt, st);
  } else {
    PrefPrivate<S, DX> st;
    batch_affine_add<S, DX>(src, cnt, st);
  }
}

}  // namespace msmk
