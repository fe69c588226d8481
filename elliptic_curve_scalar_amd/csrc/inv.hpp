// Field inversion by batched divsteps (Bernstein and Yang, "Fast constant-time gcd
// computation and modular inversion", 2019), the family of inverse the pages use
// ("safegcd", aztec-packages PR #23738 "Notes / caveats"; PR #23520 names the
// "safegcd inverse" as the accumulate's compute bound on Adreno).
//
// State: f odd, g, and delta; one divstep is
//   delta > 0 and g odd:  (delta, f, g) <- (1 - delta, g, (g - f) / 2)
//   g odd otherwise:      (delta, f, g) <- (1 + delta, f, (g + f) / 2)
//   g even:               (delta, f, g) <- (1 + delta, f, g / 2)
// Starting from f = p, g = x, delta = 1, g reaches 0 and f = +-1 within
// floor((49 * 254 + 80) / 17) = 736 steps for 254-bit inputs (the paper's bound);
// this code runs 25 batches of 30 = 750 steps, the same count for every lane, so a
// wavefront never diverges.
//
// A batch decides its 30 steps from the low 32 bits of f and g alone and records
// them as a 2x2 matrix [u v; q r] with 2^30 f' = u f + v g, 2^30 g' = q f + r g
// (every entry is at most 2^30 in magnitude). The matrix is then applied to the
// full f, g (exact division by 2^30) and to d, e with d x = f, e x = g (mod p),
// dividing by 2^30 mod p by first adding the multiple of p that clears the low
// 30 bits. At the end x^-1 = f d (f = +-1). |d| and |e| grow by less than p per
// batch, so they stay below 26 p and fit the nine signed 30-bit limbs.
#pragma once
#include "bingcd.hpp"
#include "fp.hpp"

namespace msmk {

#define MSM_M30 0x3fffffffu
#define MSM_NPINV30 0x24866389u  // -p^{-1} mod 2^30

__device__ __forceinline__ int32_t p30_limb(int k) {
  switch (k) {
    case 0: return 0x187cfd47;
    case 1: return 0x3082305b;
    case 2: return 0x071ca8d3;
    case 3: return 0x205aa45a;
    case 4: return 0x01585d97;
    case 5: return 0x0116da06;
    case 6: return 0x1a029b85;
    case 7: return 0x139cb84c;
    default: return 0x00003064;
  }
}

// g[k] = bits [30k, 30k + 30) of x (x < 2^256), as signed 30-bit limbs (all >= 0).
__device__ __forceinline__ void split30_signed(const fp& x, int32_t g[9]) {
#pragma unroll
  for (int k = 0; k < 9; k++) {
    const int o = 30 * k, w = o >> 5, sh = o & 31;
    const uint64_t pair = ((uint64_t)(w + 1 < 8 ? x.v[w + 1] : 0u) << 32) | x.v[w];
    g[k] = (int32_t)((uint32_t)(pair >> sh) & MSM_M30);
  }
}

// Eight 32-bit words of sum_k t[k] 2^(30k) for 0 <= value < 2^256, limbs in [0, 2^30).
__device__ __forceinline__ fp join30(const int32_t t[9]) {
  fp r;
#pragma unroll
  for (int w = 0; w < 8; w++) {
    const int b = 32 * w, k0 = b / 30, r0 = b % 30;
    uint32_t word = ((uint32_t)t[k0] >> r0) | ((uint32_t)t[k0 + 1] << (30 - r0));
    if (r0 > 28 && k0 + 2 < 9) word |= (uint32_t)t[k0 + 2] << (60 - r0);
    r.v[w] = word;
  }
  return r;
}

// Thirty divsteps on the low words of f and g; returns the transition matrix.
__device__ __forceinline__ void divsteps30(int32_t& delta, uint32_t f, uint32_t g, int32_t& u_o,
                                           int32_t& v_o, int32_t& q_o, int32_t& r_o) {
  int32_t u = 1, v = 0, q = 0, r = 1;
#pragma unroll 10
  for (int i = 0; i < 30; i++) {
    const int32_t odd = -(int32_t)(g & 1u);      // all ones when g is odd
    const int32_t pos = (-delta) >> 31;          // all ones when delta > 0
    const int32_t sw = odd & pos;                // swap rows this step
    // g' = (g + (sw ? -f : f) * [g odd]) / 2 ;  f' = sw ? g : f
    const uint32_t xf = (f ^ (uint32_t)sw) - (uint32_t)sw;
    const uint32_t nf = f ^ ((f ^ g) & (uint32_t)sw);
    g = (uint32_t)((int32_t)(g + (xf & (uint32_t)odd)) >> 1);
    f = nf;
    // rows: (q, r) += (sw ? -(u, v) : (u, v)) * [g odd];  (u, v) = 2 * (sw ? (q, r) : (u, v))
    const int32_t xu = (u ^ sw) - sw, xv = (v ^ sw) - sw;
    const int32_t nu = u ^ ((u ^ q) & sw), nv = v ^ ((v ^ r) & sw);
    q += xu & odd;
    r += xv & odd;
    u = (int32_t)((uint32_t)nu << 1);  // shift as unsigned: nu may be negative
    v = (int32_t)((uint32_t)nv << 1);
    delta = ((delta ^ sw) - sw) + 1;
  }
  u_o = u;
  v_o = v;
  q_o = q;
  r_o = r;
}

// (f, g) <- ([u v; q r] (f, g)) / 2^30, nine signed 30-bit limbs.
__device__ __forceinline__ void update_fg(int32_t f[9], int32_t g[9], int32_t u, int32_t v,
                                          int32_t q, int32_t r) {
  int64_t cf = (int64_t)u * f[0] + (int64_t)v * g[0];
  int64_t cg = (int64_t)q * f[0] + (int64_t)r * g[0];
  cf >>= 30;
  cg >>= 30;
#pragma unroll
  for (int k = 1; k < 9; k++) {
    cf += (int64_t)u * f[k] + (int64_t)v * g[k];
    cg += (int64_t)q * f[k] + (int64_t)r * g[k];
    f[k - 1] = (int32_t)((uint32_t)cf & MSM_M30);
    g[k - 1] = (int32_t)((uint32_t)cg & MSM_M30);
    cf >>= 30;
    cg >>= 30;
  }
  f[8] = (int32_t)cf;
  g[8] = (int32_t)cg;
}

// (d, e) <- ([u v; q r] (d, e) + (md, me) p) / 2^30, md and me clearing the low bits.
__device__ __forceinline__ void update_de(int32_t d[9], int32_t e[9], int32_t u, int32_t v,
                                          int32_t q, int32_t r) {
  int64_t cd = (int64_t)u * d[0] + (int64_t)v * e[0];
  int64_t ce = (int64_t)q * d[0] + (int64_t)r * e[0];
  const uint32_t md = ((uint32_t)cd * MSM_NPINV30) & MSM_M30;
  const uint32_t me = ((uint32_t)ce * MSM_NPINV30) & MSM_M30;
  cd += (int64_t)md * p30_limb(0);
  ce += (int64_t)me * p30_limb(0);
  cd >>= 30;
  ce >>= 30;
#pragma unroll
  for (int k = 1; k < 9; k++) {
    cd += (int64_t)u * d[k] + (int64_t)v * e[k] + (int64_t)md * p30_limb(k);
    ce += (int64_t)q * d[k] + (int64_t)r * e[k] + (int64_t)me * p30_limb(k);
    d[k - 1] = (int32_t)((uint32_t)cd & MSM_M30);
    e[k - 1] = (int32_t)((uint32_t)ce & MSM_M30);
    cd >>= 30;
    ce >>= 30;
  }
  d[8] = (int32_t)cd;
  e[8] = (int32_t)ce;
}

// MSMK_DIVSTEPS selects this inverse for fp_inv. It is off: it was switched on
// together with MSMK_MONT29 in the GPU run that stalled, and no cause has been found
// yet; a host build matches Python integers under ASan and UBSan.
#ifndef MSMK_DIVSTEPS
#define MSMK_DIVSTEPS 0
#endif

// x^-1 mod p for x != 0 given in Montgomery form: returns the Montgomery form of the
// inverse (0 maps to 0).
__device__ __forceinline__ fp fp_inv_divsteps(const fp& x) {
  int32_t f[9], g[9], d[9], e[9];
  split30_signed(x, g);
#pragma unroll
  for (int k = 0; k < 9; k++) {
    f[k] = p30_limb(k);
    d[k] = 0;
    e[k] = 0;
  }
  e[0] = 1;
  int32_t delta = 1;
  for (int b = 0; b < 25; b++) {
    int32_t u, v, q, r;
    divsteps30(delta, (uint32_t)f[0] | ((uint32_t)f[1] << 30),
               (uint32_t)g[0] | ((uint32_t)g[1] << 30), u, v, q, r);
    update_fg(f, g, u, v, q, r);
    update_de(d, e, u, v, q, r);
  }
  // f = +-1: x^-1 = f d. Bring f d + 26 p (in [0, 52 p)) into [0, p) by subtracting
  // 32p, 16p, ..., p where possible.
  const int32_t sgn = f[8] >> 31;  // f = -1 has all limbs of the two's-complement pattern
  int32_t t[9];
  {
    int64_t c = 0;
#pragma unroll
    for (int k = 0; k < 9; k++) {
      const int64_t dk = ((int64_t)d[k] ^ sgn) - sgn;  // -d limb-wise when f = -1
      c += dk + 26 * (int64_t)p30_limb(k);
      t[k] = (int32_t)((uint32_t)c & MSM_M30);
      c >>= 30;
    }
    t[8] += (int32_t)((uint64_t)c << 30);
  }
#pragma unroll
  for (int j = 5; j >= 0; j--) {
    int32_t s[9];
    int64_t c = 0;
#pragma unroll
    for (int k = 0; k < 9; k++) {
      // limb k of p * 2^j
      const int64_t pk = ((((int64_t)p30_limb(k) << j) & MSM_M30) |
                          (k ? ((int64_t)p30_limb(k - 1) >> (30 - j)) : 0)) +
                         (k == 8 ? (((int64_t)p30_limb(8) << j) & ~(int64_t)MSM_M30) : 0);
      c += (int64_t)t[k] - pk;
      s[k] = (int32_t)((uint32_t)c & MSM_M30);
      c >>= 30;
    }
    const bool keep = c < 0;  // t < 2^j p
#pragma unroll
    for (int k = 0; k < 9; k++) t[k] = keep ? t[k] : s[k];
  }
  fp inv = join30(t);
  // inv = X^-1 for the Montgomery-form input X = x R; x^-1 R = X^-1 R^2 = mont(inv, R^3)
  fp r3;
  r3.v[0] = 0xda1530dfu; r3.v[1] = 0xb1cd6dafu; r3.v[2] = 0xa7283db6u; r3.v[3] = 0x62f210e6u;
  r3.v[4] = 0x0ada0afbu; r3.v[5] = 0xef7f0b0cu; r3.v[6] = 0x2d592544u; r3.v[7] = 0x20fd6e90u;
  return fp_mul(inv, r3);
}

// fp_inv: the binary-GCD inverse (bingcd.hpp) unless MSMK_FERMAT_INV selects
// Fermat's x^(p-2) or MSMK_DIVSTEPS the divstep inverse above (off, see there).
#ifndef MSMK_FERMAT_INV
#define MSMK_FERMAT_INV 0
#endif
#if MSMK_DIVSTEPS
__device__ __forceinline__ fp fp_inv(const fp& x) { return fp_inv_divsteps(x); }
#elif MSMK_FERMAT_INV
__device__ __forceinline__ fp fp_inv(const fp& x) { return fp_inv_fermat(x); }
#else
__device__ __forceinline__ fp fp_inv(const fp& x) { return fp_inv_bingcd(x); }
#endif

}  // namespace msmk
