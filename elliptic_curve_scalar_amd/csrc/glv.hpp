// Scalar splitting by the BN254 G1 endomorphism (Gallant, Lambert and Vanstone,
// "Faster point multiplication on elliptic curves with efficient endomorphisms",
// CRYPTO 2001).
//
// p = 1 mod 3, so F_p has a primitive cube root of unity beta and phi(x, y) =
// (beta x, y) maps the curve to itself; on the prime-order group it acts as
// multiplication by lambda, a primitive cube root of unity mod r (beta and lambda
// are paired so that phi(G) = lambda G). Every scalar s splits as
// s = k1 + k2 lambda (mod r) with |k1|, |k2| < 2^127, found by rounding s against a
// short basis (a1, b1), (a2, b2) of the lattice {(a, b) : a + b lambda = 0 mod r}:
//   c1 = round(b2 s / r), c2 = round(-b1 s / r),
//   k1 = s - c1 a1 - c2 a2,  k2 = -c1 b1 - c2 b2.
// The divisions by r are products with g1 = floor(2^256 b2 / r) and
// g2 = floor(2^256 (-b1) / r); with s reduced below r the rounding error stays
// under 3/4 per coefficient, so |k| <= 3/4 (|a1| + |a2|) < 2^127.
//
// The bucket MSM then runs over 2n points (P_i and phi(P_i)) with 127-bit scalars:
// half the windows of the plain method and the same number of bucket entries. The
// constants were derived and are pinned in tests/test_glv_constants.py.
#pragma once
#include "fp.hpp"

namespace msmk {

// beta * 2^256 mod p (Montgomery form of the cube root of unity paired with lambda)
__device__ __forceinline__ fp glv_beta() {
  fp b;
  b.v[0] = 0x13e80b9cu; b.v[1] = 0x3350c88eu; b.v[2] = 0xdb5e56b9u; b.v[3] = 0x7dce557cu;
  b.v[4] = 0xb615564au; b.v[5] = 0x6001b4b8u; b.v[6] = 0x020217e0u; b.v[7] = 0x2682e617u;
  return b;
}

// out[0 .. na + nb) = a * b (little-endian 32-bit words), operand scanning.
template <int NA, int NB>
__device__ __forceinline__ void mul_words(const uint32_t (&a)[NA], const uint32_t (&b)[NB],
                                          uint32_t (&out)[NA + NB]) {
#pragma unroll
  for (int k = 0; k < NA + NB; k++) out[k] = 0;
#pragma unroll
  for (int i = 0; i < NA; i++) {
    uint64_t carry = 0;
#pragma unroll
    for (int j = 0; j < NB; j++) {
      uint64_t t = (uint64_t)a[i] * b[j] + out[i + j] + carry;
      out[i + j] = (uint32_t)t;
      carry = t >> 32;
    }
    out[i + NB] = (uint32_t)carry;
  }
}

// s -= m if s >= m (8 words), branch-free.
__device__ __forceinline__ void sub_if_geq(uint32_t (&s)[8], const uint32_t (&m)[8]) {
  uint32_t d[8];
  uint32_t borrow = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    uint64_t t = (uint64_t)s[i] - m[i] - borrow;
    d[i] = (uint32_t)t;
    borrow = (uint32_t)(t >> 63);
  }
#pragma unroll
  for (int i = 0; i < 8; i++) s[i] = borrow ? s[i] : d[i];
}

// acc -= x (8-word two's complement, x given in NX words).
template <int NX>
__device__ __forceinline__ void sub_words(uint32_t (&acc)[8], const uint32_t (&x)[NX]) {
  uint32_t borrow = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    uint64_t t = (uint64_t)acc[i] - (i < NX ? x[i] : 0u) - borrow;
    acc[i] = (uint32_t)t;
    borrow = (uint32_t)(t >> 63);
  }
}

// Magnitude (4 words, < 2^127) with the sign in bit 127; *bad if |k| >= 2^127.
__device__ __forceinline__ void sign_magnitude(const uint32_t (&k)[8], uint32_t (&o)[4], bool& bad) {
  const uint32_t neg = k[7] >> 31;
  uint32_t m[8];
  uint32_t carry = neg;  // two's-complement negation: ~k + 1 when negative
#pragma unroll
  for (int i = 0; i < 8; i++) {
    uint64_t t = (uint64_t)(neg ? ~k[i] : k[i]) + carry;
    m[i] = (uint32_t)t;
    carry = (uint32_t)(t >> 32);
  }
  bad = bad || (m[4] | m[5] | m[6] | m[7]) != 0 || (m[3] >> 31) != 0;
  o[0] = m[0];
  o[1] = m[1];
  o[2] = m[2];
  o[3] = m[3] | (neg << 31);
}

// s 2^-256 mod r for any 256-bit s: the scalar of a Montgomery-form F_r element (s = x 2^256
// mod r, how a prover's field code keeps scalars). Word-serial Montgomery reduction: eight
// steps of t = (t + m r) / 2^32 with m = t_0 (-r^-1) mod 2^32, then one subtraction of r
// ((s + M r) / 2^256 < 1 + r).
__device__ __forceinline__ void fr_from_mont(uint32_t (&s)[8]) {
  const uint32_t r[8] = {0xf0000001u, 0x43e1f593u, 0x79b97091u, 0x2833e848u,
                         0x8181585du, 0xb85045b6u, 0xe131a029u, 0x30644e72u};
  const uint32_t rinv = 0xefffffffu;  // -r^-1 mod 2^32
  uint32_t t[9];
#pragma unroll
  for (int i = 0; i < 8; i++) t[i] = s[i];
  t[8] = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t m = t[0] * rinv;
    uint64_t acc = (uint64_t)m * r[0] + t[0];  // low word becomes 0
    uint32_t cy = (uint32_t)(acc >> 32);
#pragma unroll
    for (int j = 1; j < 8; j++) {
      acc = (uint64_t)m * r[j] + t[j] + cy;
      t[j - 1] = (uint32_t)acc;
      cy = (uint32_t)(acc >> 32);
    }
    acc = (uint64_t)t[8] + cy;
    t[7] = (uint32_t)acc;
    t[8] = (uint32_t)(acc >> 32);
  }
  uint32_t d[8], borrow = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) d[i] = __builtin_subc(t[i], r[i], borrow, &borrow);
  // t <= r: keep t when it is below r (borrow), else t - r (= 0)
#pragma unroll
  for (int i = 0; i < 8; i++) s[i] = borrow ? t[i] : d[i];
}

// s (any 256-bit integer) -> (k1, k2) with s = k1 + k2 lambda (mod r), each as four
// words of magnitude with its sign in bit 127.
__device__ __forceinline__ void glv_split(const uint32_t (&s_in)[8], uint32_t (&k1)[4],
                                          uint32_t (&k2)[4], bool& bad) {
  const uint32_t R1[8] = {0xf0000001u, 0x43e1f593u, 0x79b97091u, 0x2833e848u,
                          0x8181585du, 0xb85045b6u, 0xe131a029u, 0x30644e72u};
  const uint32_t R2[8] = {0xe0000002u, 0x87c3eb27u, 0xf372e122u, 0x5067d090u,
                          0x0302b0bau, 0x70a08b6du, 0xc2634053u, 0x60c89ce5u};
  const uint32_t R4[8] = {0xc0000004u, 0x0f87d64fu, 0xe6e5c245u, 0xa0cfa121u,
                          0x06056174u, 0xe14116dau, 0x84c680a6u, 0xc19139cbu};
  const uint32_t G1[5] = {0x00ff6565u, 0x5398fd03u, 0xa773d2d2u, 0x4ccef014u, 0x00000002u};
  const uint32_t G2[3] = {0xc7e0b3d7u, 0xd91d232eu, 0x00000002u};
  const uint32_t A1[4] = {0x7d4f1128u, 0x8211bbebu, 0xeeb859fcu, 0x6f4d8248u};
  const uint32_t A2[2] = {0x94d213e3u, 0x89d32568u};
  const uint32_t NB1[2] = {0x94d213e3u, 0x89d32568u};  // -b1
  const uint32_t B2[4] = {0x1221250bu, 0x0be4e154u, 0xeeb859fdu, 0x6f4d8248u};

  uint32_t s[8];
#pragma unroll
  for (int i = 0; i < 8; i++) s[i] = s_in[i];
  sub_if_geq(s, R4);  // s < 2^256 < 6 r
  sub_if_geq(s, R2);
  sub_if_geq(s, R1);  // now s < r

  // c = (s g + 2^255) >> 256, rounding to nearest
  uint32_t p1[13], p2[11];
  mul_words(s, G1, p1);
  mul_words(s, G2, p2);
  {
    uint64_t t = (uint64_t)p1[7] + 0x80000000u;
    p1[7] = (uint32_t)t;
    uint32_t cy = (uint32_t)(t >> 32);
#pragma unroll
    for (int i = 8; i < 13; i++) {
      t = (uint64_t)p1[i] + cy;
      p1[i] = (uint32_t)t;
      cy = (uint32_t)(t >> 32);
    }
    t = (uint64_t)p2[7] + 0x80000000u;
    p2[7] = (uint32_t)t;
    cy = (uint32_t)(t >> 32);
#pragma unroll
    for (int i = 8; i < 11; i++) {
      t = (uint64_t)p2[i] + cy;
      p2[i] = (uint32_t)t;
      cy = (uint32_t)(t >> 32);
    }
  }
  // s < 2^254, g1 < 2^130, g2 < 2^66: c1 fits 4 words, c2 fits 2
  const uint32_t c1[4] = {p1[8], p1[9], p1[10], p1[11]};
  const uint32_t c2[2] = {p2[8], p2[9]};

  // k1 = s - c1 a1 - c2 a2
  uint32_t t8[8], t4[4];
  mul_words(c1, A1, t8);
  mul_words(c2, A2, t4);
  uint32_t k[8];
#pragma unroll
  for (int i = 0; i < 8; i++) k[i] = s[i];
  sub_words(k, t8);
  sub_words(k, t4);
  sign_magnitude(k, k1, bad);

  // k2 = c1 (-b1) - c2 b2
  uint32_t u1[6], u2[6];
  mul_words(c1, NB1, u1);
  mul_words(c2, B2, u2);
#pragma unroll
  for (int i = 0; i < 8; i++) k[i] = i < 6 ? u1[i] : 0u;
  sub_words(k, u2);
  sign_magnitude(k, k2, bad);
}

}  // namespace msmk
