// The batched-affine pair-tree level kernel with its slot state in LDS and/or with cached
// denominators (level_kernel.hpp), for the slot-state placement study of the
// accumulate; the default placement (private memory) is in k_levels.hip.
#include <hip/hip_runtime.h>

#include "level_kernel.hpp"

namespace msmk {

template <int S, int PLACE>
static hipError_t level_placed(const g1a* in, const uint32_t* idx, g1a* out, xyzz_st* bsum,
                               const uint32_t* counts, const uint32_t* offsets,
                               const uint32_t* poff, uint32_t K, uint32_t npairs, int level,
                               hipStream_t s) {
  constexpr unsigned B = level_block<PLACE>();
  constexpr bool LDS = (PLACE & PLACE_LDS) != 0;
  const size_t lds = LDS ? (size_t)pref_lds_bytes(S, (PLACE & PLACE_DX) != 0) * B : 0;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)k_level<S, PLACE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  size_t threads = (npairs + S - 1) / S;
  k_level<S, PLACE><<<grid_for(threads, B), B, lds, s>>>(in, idx, out, bsum, counts, offsets, poff,
                                                        K, npairs, level);
  return hipGetLastError();
}

template <int PLACE>
static hipError_t placed_S(int S, const g1a* in, const uint32_t* idx, g1a* out, xyzz_st* bsum,
                           const uint32_t* counts, const uint32_t* offsets, const uint32_t* poff,
                           uint32_t K, uint32_t npairs, int level, hipStream_t s) {
  switch (S) {
    case 4: return level_placed<4, PLACE>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    case 8: return level_placed<8, PLACE>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    case 16: return level_placed<16, PLACE>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    case 32: return level_placed<32, PLACE>(in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_level_placed(int S, int place, const g1a* in, const uint32_t* idx, g1a* out,
                               xyzz_st* bsum, const uint32_t* counts, const uint32_t* offsets,
                               const uint32_t* poff, uint32_t K, uint32_t npairs, int level,
                               hipStream_t s) {
  switch (place) {
    case PLACE_LDS:
      return placed_S<PLACE_LDS>(S, in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    case PLACE_DX:
      return placed_S<PLACE_DX>(S, in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    case PLACE_LDS | PLACE_DX:
      return placed_S<PLACE_LDS | PLACE_DX>(S, in, idx, out, bsum, counts, offsets, poff, K, npairs,
                                            level, s);
    case PLACE_CKPT:
      return placed_S<PLACE_CKPT>(S, in, idx, out, bsum, counts, offsets, poff, K, npairs, level, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msmk
