// Stream-walker accumulate of the BN254 G1 bucket MSM (gfx950), msm_run's
// MSM_SCHED_WALKER, and its launchers.
//
// The scheduling of aztec-packages PR #23736 ("Change") and PR #23738 ("TL;DR"): T lanes
// own S slots each; slot z = s T + t (slot s of lane t) walks chunk z of the sorted
// bucket lists, entries [z L, min(E, z L + L)) with L = ceil(E / (T S)). At every step
// each slot takes the next entry of its chunk, and the S slots of a lane add their
// entries to their accumulators as one batch of affine additions sharing one inversion
// (batch_add.hpp). An accumulator holds the sum of the current bucket's entries within
// the chunk. When the bucket or the chunk ends it is flushed: into the bucket sum when
// the bucket lies inside the chunk, else into the partial sums (partials_buf on the
// pages): the head partial of a chunk that starts inside a bucket, the tail partial of a
// chunk that ends inside one. A bucket split over chunks c0 < ... < c1 then sums
// tail(c0) + head(c0 + 1) + ... + head(c1), by pairs in log2(c1 - c0 + 1) passes
// (k_walk_merge), so that a bucket holding most of the entries is not a serial chain.
//
// Where the slot state lives is a template choice. DEV = false keeps the accumulators in
// per-lane arrays, which the compiler places in private memory, as the pages' walker does
// (PR #23738 "TL;DR"). DEV = true keeps them in a device buffer, word-major over slots so
// that the lanes of a wavefront touch consecutive words, as the pages propose (PR #23738
// "What would actually win"). The batch's prefix products are private in both.
#include <hip/hip_runtime.h>

#include "batch_add.hpp"
#include "kern_util.hpp"

namespace msmk {

constexpr uint32_t WALK_NONE = 0xffffffffu;

// Slot state and the batch interface of batch_affine_add: slot s adds entry ent[s] of
// its chunk to its accumulator, or starts it when the accumulator is empty (the adder's
// A = infinity case: d = 1, result B).
template <int S, bool DEV>
struct WalkSrc {
  const g1a* pts;
  uint32_t* acc;  // DEV: word w of slot z at acc[w Z + z]
  uint32_t Z, t, T;
  aff loc[DEV ? 1 : S];  // !DEV: the accumulators, private
  uint32_t ent[S];
  uint32_t valid;  // bit s: slot s's accumulator holds a partial sum

  __device__ __forceinline__ uint32_t zof(int s) const { return (uint32_t)s * T + t; }
  __device__ __forceinline__ bool has(int s) const { return (valid >> s) & 1u; }
  __device__ __forceinline__ aff acc_get(int s) const {
    if constexpr (DEV) {
      aff r;
      const uint32_t z = zof(s);
#pragma unroll
      for (int w = 0; w < 8; w++) {
        r.x.v[w] = acc[(size_t)w * Z + z];
        r.y.v[w] = acc[(size_t)(8 + w) * Z + z];
      }
      return r;
    } else {
      return loc[s];
    }
  }
  __device__ __forceinline__ fp acc_x(int s) const {
    if constexpr (DEV) {
      fp r;
      const uint32_t z = zof(s);
#pragma unroll
      for (int w = 0; w < 8; w++) r.v[w] = acc[(size_t)w * Z + z];
      return r;
    } else {
      return loc[s].x;
    }
  }
  __device__ __forceinline__ void acc_put(int s, const aff& a) {
    if constexpr (DEV) {
      const uint32_t z = zof(s);
#pragma unroll
      for (int w = 0; w < 8; w++) {
        acc[(size_t)w * Z + z] = a.x.v[w];
        acc[(size_t)(8 + w) * Z + z] = a.y.v[w];
      }
    } else {
      loc[s] = a;
    }
  }
  __device__ __forceinline__ fp ax(int s) const { return has(s) ? acc_x(s) : fp_zero(); }
  __device__ __forceinline__ fp bx(int s) const { return fp_load_x(pts + (ent[s] & 0x7fffffffu)); }
  __device__ __forceinline__ aff a(int s) const { return has(s) ? acc_get(s) : aff_inf(); }
  __device__ __forceinline__ aff b(int s) const { return load_entry(pts, ent[s]); }
  __device__ __forceinline__ void put(int s, const aff& r) { acc_put(s, r); }
};

// The walk. kst holds each slot's current bucket (private for !DEV, device for DEV).
// Partial sums go to head[z] / tail[z] (XYZZ) with their buckets in head_k[z] / tail_k[z]
// (WALK_NONE when the chunk has none); complete buckets go straight to bsum.
template <int S, bool DEV>
__global__ void __launch_bounds__(128) k_walk(const g1a* __restrict__ pts,
                                              const uint32_t* __restrict__ idx,
                                              const uint32_t* __restrict__ offsets, uint32_t K,
                                              uint32_t E, uint32_t T, uint32_t L, uint32_t* acc_dev,
                                              uint32_t* kst_dev, xyzz_st* bsum, xyzz_st* head,
                                              xyzz_st* tail, uint32_t* head_k, uint32_t* tail_k) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const uint32_t Z = T * (uint32_t)S;
  WalkSrc<S, DEV> src;
  src.pts = pts;
  src.acc = acc_dev;
  src.Z = Z;
  src.t = t;
  src.T = T;
  src.valid = 0;
  uint32_t kloc[DEV ? 1 : S];
  auto kget = [&](int s) -> uint32_t { return DEV ? kst_dev[src.zof(s)] : kloc[DEV ? 0 : s]; };
  auto kput = [&](int s, uint32_t k) {
    if (DEV) kst_dev[src.zof(s)] = k;
    else kloc[DEV ? 0 : s] = k;
  };
  // chunk index grows with s, so the slots that still have entries are a prefix
  // (chunk positions in 64 bits: Z L may exceed E by up to Z)
  int nact = 0;
  for (int s = 0; s < S; s++) {
    const uint32_t z = src.zof(s);
    head_k[z] = WALK_NONE;
    tail_k[z] = WALK_NONE;
    const uint64_t c0 = (uint64_t)z * L;
    if (c0 < E) {
      nact = s + 1;
      kput(s, bucket_of(offsets, K, (uint32_t)c0, bucket_guess((uint32_t)c0, K, E)));
    }
  }
  for (uint32_t step = 0; step < L; step++) {
    int cnt = 0;
    for (int s = 0; s < nact; s++)
      if ((uint64_t)src.zof(s) * L + step < E) cnt = s + 1;
    if (cnt == 0) break;
    for (int s = 0; s < cnt; s++) src.ent[s] = idx[src.zof(s) * L + step];
    batch_affine_add<S, true>(src, cnt);  // products as calls: see fp_mul_call
    for (int s = 0; s < cnt; s++) {
      const uint32_t z = src.zof(s);
      const uint32_t cstart = z * L;  // below E: slot s had an entry this step
      const uint32_t cend = (uint32_t)min((uint64_t)E, (uint64_t)cstart + L), next = cstart + step + 1;
      uint32_t k = kget(s);
      const uint32_t bstart = offsets[k], bend = offsets[k + 1];
      src.valid |= 1u << s;
      if (next == bend || next == cend) {
        const xyzz a = xyzz_from_aff(src.acc_get(s));
        if (bstart >= cstart && bend <= cend) {
          xyzz_store(bsum + k, a);  // the whole bucket lies in this chunk
        } else if (bstart < cstart) {
          xyzz_store(head + z, a);
          head_k[z] = k;
        } else {
          xyzz_store(tail + z, a);
          tail_k[z] = k;
        }
        src.valid &= ~(1u << s);
        if (next < cend) {  // the bucket of the next entry (empty buckets skipped)
          k = (offsets[k + 2] > next) ? k + 1 : bisect_le(offsets, k + 1, K, next);
          kput(s, k);
        }
      }
    }
  }
}

// Pass r of the partial merge, one quad per chunk c. A split bucket's partials are
// element 0 = tail(c0) and element i = head(c0 + i), i = 1 .. m; pass r adds element
// i + 2^r into element i for every i that is a multiple of 2^(r+1). Chunk c holds at most
// one element of each kind: its tail (always element 0 of its bucket) and its head.
__global__ void __launch_bounds__(256) k_walk_merge(const uint32_t* __restrict__ offsets,
                                                    uint32_t L, uint32_t Z, uint32_t r,
                                                    xyzz_st* head, xyzz_st* tail,
                                                    const uint32_t* __restrict__ head_k,
                                                    const uint32_t* __restrict__ tail_k) {
  const uint32_t c = (blockIdx.x * blockDim.x + threadIdx.x) >> 2;
  const int q = (int)(threadIdx.x & 3u);
  if (c >= Z) return;  // whole quads leave together; no barrier follows
  const uint32_t step = 1u << r;
  const uint32_t kt = tail_k[c];
  if (kt != WALK_NONE) {
    const uint32_t c1 = (offsets[kt + 1] - 1) / L;  // last chunk of the bucket
    if (c + step <= c1) {
      const xyzz s = quad_add(xyzz_load(tail + c), xyzz_load(head + c + step), q);
      if (q == 0) xyzz_store(tail + c, s);
    }
  }
  const uint32_t kh = head_k[c];
  if (kh != WALK_NONE) {
    const uint32_t c0 = offsets[kh] / L, c1 = (offsets[kh + 1] - 1) / L;
    const uint32_t i = c - c0;
    if ((i & (2 * step - 1)) == 0 && c + step <= c1) {
      const xyzz s = quad_add(xyzz_load(head + c), xyzz_load(head + c + step), q);
      if (q == 0) xyzz_store(head + c, s);
    }
  }
}

// Split buckets take their merged sum, tail(c0); one lane per chunk c whose tail starts a
// bucket.
__global__ void __launch_bounds__(256) k_walk_finish(uint32_t Z, const xyzz_st* __restrict__ tail,
                                                     const uint32_t* __restrict__ tail_k,
                                                     xyzz_st* bsum) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= Z) return;
  const uint32_t kt = tail_k[c];
  if (kt != WALK_NONE) xyzz_store(bsum + kt, xyzz_load(tail + c));
}

// ------------------------------------------------------------------ launchers
template <int S, bool DEV>
static hipError_t walk_S(const walk_args& a, hipStream_t s) {
  k_walk<S, DEV><<<grid_for(a.T, 128), 128, 0, s>>>(a.pts, a.idx, a.offsets, a.K, a.E, a.T, a.L,
                                                   a.acc, a.kst, a.bsum, a.head, a.tail, a.head_k,
                                                   a.tail_k);
  return hipGetLastError();
}

hipError_t launch_walk(int S, bool dev_state, const walk_args& a, hipStream_t s) {
  switch (S * 2 + (dev_state ? 1 : 0)) {
    case 8: return walk_S<4, false>(a, s);
    case 9: return walk_S<4, true>(a, s);
    case 16: return walk_S<8, false>(a, s);
    case 17: return walk_S<8, true>(a, s);
    case 32: return walk_S<16, false>(a, s);
    case 33: return walk_S<16, true>(a, s);
    case 64: return walk_S<32, false>(a, s);
    case 65: return walk_S<32, true>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_walk_merge(int S, const walk_args& a, uint32_t merge_passes, hipStream_t s) {
  const uint32_t Z = a.T * (uint32_t)S;
  for (uint32_t r = 0; r < merge_passes; r++)
    k_walk_merge<<<grid_for((size_t)Z * 4, 256), 256, 0, s>>>(a.offsets, a.L, Z, r, a.head, a.tail,
                                                              a.head_k, a.tail_k);
  k_walk_finish<<<grid_for(Z, 256), 256, 0, s>>>(Z, a.tail, a.tail_k, a.bsum);
  return hipGetLastError();
}

}  // namespace msmk
