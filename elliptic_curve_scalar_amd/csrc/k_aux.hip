// Input generator and unit-test hooks of libmsm (gfx950): the same device code as the
// MSM kernels, exposed for the tests and for building synthetic inputs.
#include <hip/hip_runtime.h>

#include "batch_add.hpp"
#include "glv.hpp"
#include "kern_util.hpp"
#include "rowpoint.hpp"

namespace msmk {

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
    case 7: r = fp_inv_fermat(x); break;
    case 8: r = fp_inv_bingcd(x); break;
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

// Row-form field operations (rowfp.hpp): wavefront w computes elements 4 w .. 4 w + 3, one
// per row; rows past n compute on zeros and store nothing. op 0 a b, 1 a + b, 2 a - b.
// One wavefront per 64-lane block.
__global__ void __launch_bounds__(64) k_test_row(int op, const uint32_t* __restrict__ a,
                                                 const uint32_t* __restrict__ b,
                                                 uint32_t* __restrict__ out, uint32_t n) {
  const uint32_t l = threadIdx.x & 15u, e = 4u * blockIdx.x + (threadIdx.x >> 4);
  const bool live = e < n && l < 8u;
  const uint32_t x = live ? a[8 * (size_t)e + l] : 0u, y = live ? b[8 * (size_t)e + l] : 0u;
  row_consts k = row_consts_load();
  uint32_t r;
  if (op == 0) r = row_mul(x, y, k);
  else if (op == 1) r = row_add(x, y, k);
  else r = row_sub(x, y, k);
  if (live) out[8 * (size_t)e + l] = r;
}

// XYZZ points (32 words each: X, Y, ZZ, ZZZ), one wavefront per point:
//   op 3  2^d P by a run of doublings in row form (rowpoint.hpp)
//   op 4  2^d P by the quad runs (quad.hpp)
//   op 7  P + Q in row form (every special case)
//   op 8  2P in row form
//   op 9  P in affine coordinates (16 words) by the uniform path of the window combine's
//         end (the inverse on scalar registers)
__global__ void __launch_bounds__(64) k_test_row_pts(int op, const uint32_t* __restrict__ pts,
                                                     const uint32_t* __restrict__ pts2, uint32_t d,
                                                     uint32_t* __restrict__ out) {
  const xyzz_st* src = reinterpret_cast<const xyzz_st*>(pts) + blockIdx.x;
  xyzz_st* dst = reinterpret_cast<xyzz_st*>(out) + blockIdx.x;
  if (op == 4) {
    const xyzz r = quad_dbl_n(xyzz_load(src), d, (int)(threadIdx.x & 3u));
    if (threadIdx.x == 0) xyzz_store(dst, r);
    return;
  }
  row_consts k = row_consts_load();
  const rxyzz a = rxyzz_load(src);
  if (op == 9) {
    const aff r = xyzz_to_aff(rxyzz_to_fp(a, k));
    if (threadIdx.x == 0) aff_store(reinterpret_cast<g1a*>(out) + blockIdx.x, r);
    return;
  }
  rxyzz r;
  if (op == 3) r = rxyzz_dbl_n(a, d, k);
  else if (op == 7) r = rxyzz_add(a, rxyzz_load(reinterpret_cast<const xyzz_st*>(pts2) + blockIdx.x), k);
  else r = rxyzz_dbl(a, k);
  rxyzz_store(dst, r, k);
}

// Latency probe, one wavefront: x <- x b, d times, for the four elements of a and b (8 words
// each): op 5 in row form (element r on row r), op 6 with the per-lane product (element
// i mod 4 on lane i). out gets the four results.
__global__ void __launch_bounds__(64) k_test_row_chain(int op, const uint32_t* __restrict__ a,
                                                       const uint32_t* __restrict__ b, uint32_t d,
                                                       uint32_t* __restrict__ out) {
  if (op == 5) {
    const uint32_t l = threadIdx.x & 15u, e = threadIdx.x >> 4;
    uint32_t x = l < 8u ? a[8 * e + l] : 0u;
    const uint32_t y = l < 8u ? b[8 * e + l] : 0u;
    row_consts k = row_consts_load();
    for (uint32_t i = 0; i < d; i++) x = row_mul(x, y, k);
    if (l < 8u) out[8 * e + l] = x;
  } else {
    const uint32_t e = threadIdx.x & 3u;
    fp x = fp_load_words(a + 8 * e);
    const fp y = fp_load_words(b + 8 * e);
    for (uint32_t i = 0; i < d; i++) x = fp_mul(x, y);
    if (threadIdx.x < 4u) {
#pragma unroll
      for (int w = 0; w < 8; w++) out[8 * e + w] = x.v[w];
    }
  }
}

// Instruction-rate probe: each lane runs `iters` rounds of 16 independent chains of one
// instruction class, then folds the chains into out[lane] so that nothing is dead.
//   op 0: 32 x 32 -> 64-bit multiply-add, the product's unit (v_mad_u64_u32)
//   op 1: 32-bit add (v_add_u32)
//   op 2: 32-bit add with carry in and out, the carry chains of field add/sub
//         (v_add_co_u32 / v_addc_co_u32)
// Timed over many waves per SIMD it gives the sustained issue rate of the class.
__global__ void __launch_bounds__(256) k_test_rate(int op, uint32_t iters, uint32_t seed,
                                                   uint32_t* __restrict__ out) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x[16];
#pragma unroll
  for (int k = 0; k < 16; k++) x[k] = gid * 2654435761u + (uint32_t)k * 40503u + seed;
  uint32_t fold = 0;
  if (op == 0) {
    uint64_t acc[16];
#pragma unroll
    for (int k = 0; k < 16; k++) acc[k] = x[k];
    for (uint32_t it = 0; it < iters; it++) {
#pragma unroll
      for (int k = 0; k < 16; k++) acc[k] = (uint64_t)(uint32_t)acc[k] * seed + acc[k];
    }
#pragma unroll
    for (int k = 0; k < 16; k++) fold ^= (uint32_t)acc[k] ^ (uint32_t)(acc[k] >> 32);
  } else if (op == 1) {
    for (uint32_t it = 0; it < iters; it++) {
#pragma unroll
      for (int k = 0; k < 16; k += 2) {  // eight Fibonacci pairs: no closed form to fold
        x[k] = x[k] + x[k + 1];
        x[k + 1] = x[k + 1] + x[k];
      }
    }
#pragma unroll
    for (int k = 0; k < 16; k++) fold ^= x[k];
  } else {
    uint32_t c = 0;
    for (uint32_t it = 0; it < iters; it++) {
#pragma unroll
      for (int k = 0; k < 16; k++) x[k] = __builtin_addc(x[k], seed, c, &c);
    }
#pragma unroll
    for (int k = 0; k < 16; k++) fold ^= x[k];
    fold ^= c;
  }
  out[gid] = fold;
}

// ------------------------------------------------------------------ launchers
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

hipError_t launch_test_row(int op, const uint32_t* a, const uint32_t* b, uint32_t* out, uint32_t n,
                           uint32_t d, hipStream_t s) {
  if (op <= 2) {
    if (n == 0) return hipSuccess;
    k_test_row<<<(n + 3) / 4, 64, 0, s>>>(op, a, b, out, n);
  } else if (op == 5 || op == 6) {
    k_test_row_chain<<<1, 64, 0, s>>>(op, a, b, d, out);
  } else {
    if (n == 0) return hipSuccess;
    k_test_row_pts<<<n, 64, 0, s>>>(op, a, b, d, out);
  }
  return hipGetLastError();
}

hipError_t launch_test_rate(int op, uint32_t blocks, uint32_t iters, uint32_t seed, uint32_t* out,
                            hipStream_t s) {
  k_test_rate<<<blocks, 256, 0, s>>>(op, iters, seed, out);
  return hipGetLastError();
}

}  // namespace msmk
