// Field inversion by the optimized binary GCD of T. Pornin ("Optimized Binary GCD for
// Modular Inversion", IACR ePrint 2020/972), the fast replacement for Fermat's x^(p-2).
//
// The exact binary GCD keeps a >= 0, b odd, and u, v with a = u y, b = v y (mod p),
// starting from (a, b, u, v) = (y, p, 1, 0). One step is
//   a odd and a < b:  swap (a, u) with (b, v)
//   a odd:            a <- a - b,  u <- u - v
//   always:           a <- a / 2,  u <- u / 2 (mod p)
// and 2 len(p) - 1 = 507 steps take a to 0 and b to gcd(y, p) = 1, so y^-1 = v.
//
// Batches of 30 steps decide everything from 64-bit stand-ins for a and b: their
// exact low 30 bits (enough for every parity test of the batch) under the 34 bits
// just below the top of max(a, b) (for the comparisons). The batch's steps are
// recorded as signed factors with
//   a' = (f0 a + g0 b) / 2^30,  b' = (f1 a + g1 b) / 2^30,  |f| + |g| <= 2^30,
// applied once to the full 254-bit a and b (a wrong comparison from the stand-ins
// shows up as a negative result, which is negated together with its factors) and to
// u, v, where the division by 2^30 is exact modular division: add the multiple of p
// that clears the low 30 bits, shift, then bring the result from (-p, 2p) into
// [0, p). Every lane of a wavefront runs the same batches, so the wavefront never
// diverges; it stops once every lane has reached a = 0, after which a batch would leave
// v unchanged. The exact algorithm needs at most 507 steps; random inputs need far fewer
// (of 40 million sampled, none needed more than 14 batches of 30), so at most 15 batches
// are run, and a lane whose b has not reached 1 (y = 0, or an input the batches do not
// cover) takes Fermat's inverse instead: the result is exact for every input.
#pragma once
#include "fp.hpp"

namespace msmk {

#define BG_STEPS 30        // steps per batch
#define BG_BATCHES 15      // batches: 450 steps
#define BG_NPINV30 0x24866389u  // -p^-1 mod 2^30

__device__ __forceinline__ uint32_t bg_p(int i) {
  switch (i) {
    case 0: return MSM_P0;
    case 1: return MSM_P1;
    case 2: return MSM_P2;
    case 3: return MSM_P3;
    case 4: return MSM_P4;
    case 5: return MSM_P5;
    case 6: return MSM_P6;
    default: return MSM_P7;
  }
}

// 64-bit stand-ins for a and b (see above); exact when both are below 2^64.
__device__ __forceinline__ void bg_approx(const uint32_t (&a)[8], const uint32_t (&b)[8],
                                          uint64_t& xa, uint64_t& xb) {
  uint32_t top = 0;
  int tw = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t o = a[i] | b[i];
    tw = o ? i : tw;
    top = o ? o : top;
  }
  const int n = 32 * tw + 32 - (top ? __builtin_clz(top) : 32);  // bit length of max(a, b)
  const uint64_t a01 = ((uint64_t)a[1] << 32) | a[0];
  const uint64_t b01 = ((uint64_t)b[1] << 32) | b[0];
  if (n <= 64) {
    xa = a01;
    xb = b01;
    return;
  }
  const int sh = n - 34;  // 30 .. 222: bits [sh, sh + 34) are the top 34 of max(a, b)
  const int q = sh >> 5, r = sh & 31;
  uint32_t a0 = 0, a1 = 0, a2 = 0, b0 = 0, b1 = 0, b2 = 0;  // words q, q + 1, q + 2
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a0 = (i == q) ? a[i] : a0;
    b0 = (i == q) ? b[i] : b0;
    a1 = (i == q + 1) ? a[i] : a1;
    b1 = (i == q + 1) ? b[i] : b1;
    a2 = (i == q + 2) ? a[i] : a2;
    b2 = (i == q + 2) ? b[i] : b2;
  }
  const uint64_t m34 = (1ull << 34) - 1;
  uint64_t ta = (((uint64_t)a1 << 32) | a0) >> r;
  uint64_t tb = (((uint64_t)b1 << 32) | b0) >> r;
  if (r) {
    ta |= (uint64_t)a2 << (64 - r);
    tb |= (uint64_t)b2 << (64 - r);
  }
  xa = ((ta & m34) << 30) | (a01 & 0x3fffffffull);
  xb = ((tb & m34) << 30) | (b01 & 0x3fffffffull);
}

// BG_STEPS binary-GCD steps on the stand-ins; returns the batch's factors.
__device__ __forceinline__ void bg_batch(uint64_t xa, uint64_t xb, int32_t& f0, int32_t& g0,
                                         int32_t& f1, int32_t& g1) {
  f0 = 1;
  g0 = 0;
  f1 = 0;
  g1 = 1;
#pragma unroll 10
  for (int j = 0; j < BG_STEPS; j++) {
    const bool odd = (xa & 1u) != 0;
    const bool sw = odd && xa < xb;
    const uint64_t na = sw ? xb : xa, nb = sw ? xa : xb;
    const int32_t nf0 = sw ? f1 : f0, ng0 = sw ? g1 : g0;
    const int32_t nf1 = sw ? f0 : f1, ng1 = sw ? g0 : g1;
    xa = (odd ? na - nb : na) >> 1;
    xb = nb;
    f0 = odd ? nf0 - nf1 : nf0;
    g0 = odd ? ng0 - ng1 : ng0;
    f1 = (int32_t)((uint32_t)nf1 << 1);
    g1 = (int32_t)((uint32_t)ng1 << 1);
  }
}

// t = x f + y g (+ k p when KP) as nine words of a two's-complement integer, for x, y
// below 2^254 and |f| + |g| <= 2^30. The factors are offset to f + 2^30 and g + 2^30
// (both in [0, 2^31]), so word i's products sum to s_i = x_i fo + y_i go (+ k p_i), below
// (2^32 - 1)(f + g + 2^31 + k) < 2^64 as f + g + 2^31 <= 3 2^30 and k < 2^30: the words'
// multiply-adds are independent of each other, and one add-with-carry chain joins them
// (t_i = lo(s_i) + hi(s_(i-1)) + carry). 2^30 (x + y) is subtracted once at the end.
template <bool KP>
__device__ __forceinline__ void bg_comb(const uint32_t (&x)[8], const uint32_t (&y)[8], int32_t f,
                                        int32_t g, uint32_t k, uint32_t (&t)[9]) {
  const uint32_t fo = (uint32_t)f + (1u << 30), go = (uint32_t)g + (1u << 30);
  uint64_t s[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    s[i] = (uint64_t)x[i] * fo;
    s[i] = (uint64_t)y[i] * go + s[i];
    if (KP) s[i] = (uint64_t)k * bg_p(i) + s[i];
  }
  uint32_t c = 0;
  t[0] = (uint32_t)s[0];
#pragma unroll
  for (int i = 1; i < 8; i++) t[i] = __builtin_addc((uint32_t)s[i], (uint32_t)(s[i - 1] >> 32), c, &c);
  t[8] = (uint32_t)(s[7] >> 32) + c;
  // subtract (x + y) << 30 (x + y < 2^255: nine words after the shift)
  uint32_t sum[8], cs = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) sum[i] = __builtin_addc(x[i], y[i], cs, &cs);
  uint32_t b = 0;
  t[0] = __builtin_subc(t[0], sum[0] << 30, b, &b);
#pragma unroll
  for (int i = 1; i < 8; i++) t[i] = __builtin_subc(t[i], (sum[i] << 30) | (sum[i - 1] >> 2), b, &b);
  t[8] = __builtin_subc(t[8], (cs << 30) | (sum[7] >> 2), b, &b);
}

// out = |a f + b g| / 2^30 (the sum is a multiple of 2^30); returns true when the sum
// was negative.
__device__ __forceinline__ bool bg_lin(const uint32_t (&a)[8], const uint32_t (&b)[8], int32_t f,
                                       int32_t g, uint32_t (&out)[8]) {
  uint32_t t[9];
  bg_comb<false>(a, b, f, g, 0u, t);
  const bool neg = (int32_t)t[8] < 0;
  const uint32_t m = neg ? 0xffffffffu : 0u;
  uint32_t c = neg ? 1u : 0u;
#pragma unroll
  for (int i = 0; i < 9; i++) t[i] = __builtin_addc(t[i] ^ m, 0u, c, &c);
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = (t[i] >> 30) | (t[i + 1] << 2);
  return neg;
}

// out = (u f + v g) / 2^30 mod p in [0, p), for u, v in [0, p) and |f| + |g| <= 2^30.
__device__ __forceinline__ void bg_lin_mod(const uint32_t (&u)[8], const uint32_t (&v)[8],
                                           int32_t f, int32_t g, uint32_t (&out)[8]) {
  // k p clears the low 30 bits: k = -(u f + v g) p^-1 mod 2^30
  const uint32_t lo = u[0] * (uint32_t)f + v[0] * (uint32_t)g;
  const uint32_t k = (lo * BG_NPINV30) & 0x3fffffffu;
  uint32_t t[9];
  bg_comb<true>(u, v, f, g, k, t);
  // r = t / 2^30 lies in (-p, 2p): nine words, the top one signed
  uint32_t r[9];
#pragma unroll
  for (int i = 0; i < 8; i++) r[i] = (t[i] >> 30) | (t[i + 1] << 2);
  r[8] = (uint32_t)((int32_t)t[8] >> 30);
  // r + p (used when r < 0) and r - p (used when r >= p)
  uint32_t rp[8], rm[8];
  uint32_t cp = 0, bm = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    rp[i] = __builtin_addc(r[i], bg_p(i), cp, &cp);
    rm[i] = __builtin_subc(r[i], bg_p(i), bm, &bm);
  }
  const bool neg = (int32_t)r[8] < 0;
  const bool ge = !neg && (r[8] != 0 || bm == 0);
#pragma unroll
  for (int i = 0; i < 8; i++) out[i] = neg ? rp[i] : ge ? rm[i] : r[i];
}

// x^-1 for x in Montgomery form (the Montgomery form of the inverse); 0 maps to 0.
//
// The steps keep a C = u y and b C = v y (mod p) for whatever constant C the run starts
// from with (a, b, u, v) = (y, p, C, 0), since every step is the same linear map on
// (a, b) and on (u, v). Here y = x R is the Montgomery representation, and starting
// from C = R^2 mod p the run ends (b = 1) with v = R^2 / (x R) = x^-1 R, the Montgomery
// form of the inverse itself: no Montgomery product converts the result afterwards.
// This is the "trim Montgomery form in the batched-inversion path" lever of the pages
// (PR #23738 "What would actually win", PR #23736 "Honest status") in the form it takes
// here: one product per inversion less.
__device__ __forceinline__ fp fp_inv_bingcd(const fp& x) {
  uint32_t a[8], b[8], u[8], v[8];
  const fp r2 = fp_r2();  // 2^512 mod p, as a plain integer below p
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[i] = x.v[i];
    b[i] = bg_p(i);
    u[i] = r2.v[i];
    v[i] = 0u;
  }
  for (int it = 0; it < BG_BATCHES; it++) {
    uint64_t xa, xb;
    bg_approx(a, b, xa, xb);
    int32_t f0, g0, f1, g1;
    bg_batch(xa, xb, f0, g0, f1, g1);
    uint32_t na[8], nb[8];
    if (bg_lin(a, b, f0, g0, na)) {
      f0 = -f0;
      g0 = -g0;
    }
    if (bg_lin(a, b, f1, g1, nb)) {
      f1 = -f1;
      g1 = -g1;
    }
    uint32_t nu[8], nv[8];
    bg_lin_mod(u, v, f0, g0, nu);
    bg_lin_mod(u, v, f1, g1, nv);
    uint32_t az = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      a[i] = na[i];
      b[i] = nb[i];
      u[i] = nu[i];
      v[i] = nv[i];
      az |= na[i];
    }
    // Once a = 0 a batch only halves a: its factors are (1, 0) and (0, 2^30), so b and v
    // stay as they are. The wavefront stops when every lane has got there.
    if (__all(az == 0)) break;
  }
  uint32_t one = b[0] ^ 1u;
#pragma unroll
  for (int i = 1; i < 8; i++) one |= b[i];
  fp r;
  if (one == 0) {
#pragma unroll
    for (int i = 0; i < 8; i++) r.v[i] = v[i];
  } else {
    r = fp_inv_fermat(x);  // x = 0, or b did not reach 1
  }
  return r;
}

// The field inverse every kernel uses.
__device__ __forceinline__ fp fp_inv(const fp& x) { return fp_inv_bingcd(x); }

}  // namespace msmk
