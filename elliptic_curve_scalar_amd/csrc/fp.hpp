// BN254 base field F_p on gfx950: 256-bit Montgomery arithmetic on 32-bit limbs.
//
// The multi-scalar multiplication of aztec-packages PR #23738 / #23736 / #23520
// ("bb/msm") spends its accumulate time in Montgomery products and a field
// inversion per batch (PR #23520, "Measurements": compute-bound on the inverse and
// the Montgomery products). This header is that arithmetic for CDNA4:
//
//   * an element is eight little-endian 32-bit limbs holding x * 2^256 mod p
//     (Montgomery form, R = 2^256), the same bytes as the library's interchange
//     format, always fully reduced (< p) between operations;
//   * the product is coarsely integrated operand scanning with 32x32->64
//     multiply-adds (v_mad_u64_u32 on gfx950, issued at half the rate of plain 32-bit
//     ALU ops); p < 2^254 keeps every partial sum inside 288 bits and the result
//     before the final subtraction below 2p;
//   * Fermat's x^(p-2) (fp_inv_fermat) is here; the inverse the kernels use is the
//     binary GCD of bingcd.hpp (Fermat remains its fallback).
//
// Everything is branch-free except where noted, so a wavefront never diverges on
// field values.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msmk {

struct fp {
  uint32_t v[8];
};

// p = 0x30644e72e131a029b85045b68181585d97816a916871ca8d3c208c16d87cfd47 (EIP-196).
#define MSM_P0 0xd87cfd47u
#define MSM_P1 0x3c208c16u
#define MSM_P2 0x6871ca8du
#define MSM_P3 0x97816a91u
#define MSM_P4 0x8181585du
#define MSM_P5 0xb85045b6u
#define MSM_P6 0xe131a029u
#define MSM_P7 0x30644e72u
// -p^{-1} mod 2^32
#define MSM_PINV 0xe4866389u

__device__ __forceinline__ uint32_t p_limb(int i) {
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

__device__ __forceinline__ fp fp_zero() {
  fp r;
#pragma unroll
  for (int i = 0; i < 8; i++) r.v[i] = 0;
  return r;
}

// 2^256 mod p: the Montgomery form of 1.
__device__ __forceinline__ fp fp_one() {
  fp r;
  r.v[0] = 0xc58f0d9du; r.v[1] = 0xd35d438du; r.v[2] = 0xf5c70b3du; r.v[3] = 0x0a78eb28u;
  r.v[4] = 0x7879462cu; r.v[5] = 0x666ea36fu; r.v[6] = 0x9a07df2fu; r.v[7] = 0x0e0a77c1u;
  return r;
}

// 2^512 mod p: multiplying by it converts a plain integer into Montgomery form.
__device__ __forceinline__ fp fp_r2() {
  fp r;
  r.v[0] = 0x538afa89u; r.v[1] = 0xf32cfc5bu; r.v[2] = 0xd44501fbu; r.v[3] = 0xb5e71911u;
  r.v[4] = 0x0a417ff6u; r.v[5] = 0x47ab1effu; r.v[6] = 0xcab8351fu; r.v[7] = 0x06d89f71u;
  return r;
}

__device__ __forceinline__ bool fp_is_zero(const fp& a) {
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) x |= a.v[i];
  return x == 0;
}

__device__ __forceinline__ bool fp_eq(const fp& a, const fp& b) {
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) x |= a.v[i] ^ b.v[i];
  return x == 0;
}

// a < p (a canonical element).
__device__ __forceinline__ bool fp_is_reduced(const fp& a) {
  uint32_t borrow = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) (void)__builtin_subc(a.v[i], p_limb(i), borrow, &borrow);
  return borrow != 0;
}

// r = t - p if t >= p else t, for t < 2^256 given as 8 limbs.
__device__ __forceinline__ fp fp_reduce_once(const fp& t) {
  // 32-bit borrow chain (clang's subtract-with-borrow builtin, v_sub_co / v_subb_co):
  // uint64_t arithmetic here compiles to 64-bit adds of widened operands
  fp d;
  uint32_t borrow = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) d.v[i] = __builtin_subc(t.v[i], p_limb(i), borrow, &borrow);
  fp r;
#pragma unroll
  for (int i = 0; i < 8; i++) r.v[i] = borrow ? t.v[i] : d.v[i];
  return r;
}

__device__ __forceinline__ fp fp_add(const fp& a, const fp& b) {
  fp s;
  uint32_t carry = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) s.v[i] = __builtin_addc(a.v[i], b.v[i], carry, &carry);
  // a, b < p < 2^254: the sum is below 2^255, so no carry leaves limb 7.
  return fp_reduce_once(s);
}

__device__ __forceinline__ fp fp_sub(const fp& a, const fp& b) {
  fp d;
  uint32_t borrow = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) d.v[i] = __builtin_subc(a.v[i], b.v[i], borrow, &borrow);
  // a < b: add p back (masked, branch-free)
  const uint32_t mask = 0u - borrow;
  uint32_t carry = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) d.v[i] = __builtin_addc(d.v[i], p_limb(i) & mask, carry, &carry);
  return d;
}

__device__ __forceinline__ fp fp_neg(const fp& a) { return fp_sub(fp_zero(), a); }

__device__ __forceinline__ fp fp_dbl(const fp& a) { return fp_add(a, a); }

// a / 2 mod p: (a + p) / 2 for odd a, a / 2 for even a (a + p < 2p < 2^255, so the
// sum fits the eight limbs).
__device__ __forceinline__ fp fp_half(const fp& a) {
  const uint32_t mask = 0u - (a.v[0] & 1u);
  fp s;
  uint32_t carry = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) s.v[i] = __builtin_addc(a.v[i], p_limb(i) & mask, carry, &carry);
  fp r;
#pragma unroll
  for (int i = 0; i < 7; i++) r.v[i] = (s.v[i] >> 1) | (s.v[i + 1] << 31);
  r.v[7] = s.v[7] >> 1;
  return r;
}

// Montgomery product a * b * 2^-256 mod p, coarsely integrated operand scanning on
// 32-bit limbs.
// 64-bit value kept whole through code generation: the empty asm stops the compiler
// from re-associating a * b + (t + c) into (a * b + t) + c, which costs two 64-bit
// adds and the register moves that widen t and c, where the form below costs one
// 32-bit add and the select of its carry.
__device__ __forceinline__ uint64_t fp_opaque(uint64_t x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm("" : "+v"(x));
#endif
  return x;
}

// t + c (both 32-bit) as a 64-bit multiply-add addend.
__device__ __forceinline__ uint64_t fp_add33(uint32_t t, uint32_t c) {
  const uint32_t lo = t + c;
  const uint32_t hi = lo < c ? 1u : 0u;
  return fp_opaque(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ fp fp_mul_cios(const fp& a, const fp& b) {
  uint32_t t[9];
#pragma unroll
  for (int j = 0; j < 9; j++) t[j] = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    // t += a * b_i: each step is (hi, lo) = a_j b_i + (t_j + carry), which fits 64 bits
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint64_t s = (uint64_t)a.v[j] * b.v[i] + (i == 0 ? fp_opaque(c) : fp_add33(t[j], c));
      t[j] = (uint32_t)s;
      c = (uint32_t)(s >> 32);
    }
    uint64_t top = (uint64_t)t[8] + c;
    t[8] = (uint32_t)top;
    // with p < 2^254 the running value stays below 2p * 2^32, so no word above t[8]
    const uint32_t m = t[0] * MSM_PINV;
    const uint64_t s0 = (uint64_t)m * p_limb(0) + fp_opaque(t[0]);
    c = (uint32_t)(s0 >> 32);
#pragma unroll
    for (int j = 1; j < 8; j++) {
      const uint64_t s = (uint64_t)m * p_limb(j) + fp_add33(t[j], c);
      t[j - 1] = (uint32_t)s;
      c = (uint32_t)(s >> 32);
    }
    top = (uint64_t)t[8] + c;
    t[7] = (uint32_t)top;
    t[8] = (uint32_t)(top >> 32);
  }
  fp r;
#pragma unroll
  for (int j = 0; j < 8; j++) r.v[j] = t[j];
  // inputs < p give t < 2p < 2^255, so t[8] == 0
  return fp_reduce_once(r);
}

// Montgomery square a^2 * 2^-256 mod p by separated operand scanning: the 28 products
// a_i a_j (i < j) once, the 512-bit sum doubled by a one-bit shift, the 8 squares a_i^2
// added, then the word-serial Montgomery reduction (8 rounds of t += m p 2^(32 i),
// m = t_i (-p^-1) mod 2^32): 108 multiply-adds against 136 for the product.
__device__ __forceinline__ fp fp_sqr_sos(const fp& a) {
  uint32_t t[16];
#pragma unroll
  for (int k = 0; k < 16; k++) t[k] = 0;
  // off-diagonal products: row i adds a_i a_j (j > i) at t[i + j]
#pragma unroll
  for (int i = 0; i < 7; i++) {
    uint32_t c = 0;
#pragma unroll
    for (int j = i + 1; j < 8; j++) {
      const uint64_t s = (uint64_t)a.v[i] * a.v[j] + fp_add33(t[i + j], c);
      t[i + j] = (uint32_t)s;
      c = (uint32_t)(s >> 32);
    }
    t[i + 8] = c;
  }
  // double (the top bit of t[14] moves into t[15], which is still 0)
#pragma unroll
  for (int k = 15; k > 0; k--) t[k] = __builtin_amdgcn_alignbit(t[k], t[k - 1], 31);
  t[0] = 0;
  // the squares a_i^2 at t[2i], t[2i + 1]
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint64_t s = (uint64_t)a.v[i] * a.v[i] + fp_add33(t[2 * i], c);
    t[2 * i] = (uint32_t)s;
    const uint64_t u = (uint64_t)t[2 * i + 1] + (uint32_t)(s >> 32);
    t[2 * i + 1] = (uint32_t)u;
    c = (uint32_t)(u >> 32);
  }
  // reduction: after round i, t[0..i] are 0 and the value is unchanged mod p; the carry
  // out of t[i + 8] is deferred to round i + 1, whose last add lands on t[i + 9]
  uint32_t cc = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t m = t[i] * MSM_PINV;
    uint32_t c2 = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint64_t s = (uint64_t)m * p_limb(j) + fp_add33(t[i + j], c2);
      t[i + j] = (uint32_t)s;
      c2 = (uint32_t)(s >> 32);
    }
    const uint64_t u = (uint64_t)t[i + 8] + c2 + cc;
    t[i + 8] = (uint32_t)u;
    cc = (uint32_t)(u >> 32);
  }
  // (a^2 + M p) / 2^256 < (p^2 + 2^256 p) / 2^256 < 2p < 2^255: no carry is left in cc
  fp r;
#pragma unroll
  for (int j = 0; j < 8; j++) r.v[j] = t[8 + j];
  return fp_reduce_once(r);
}

// Montgomery product a * b * 2^-256 mod p; inputs and output fully reduced.
__device__ __forceinline__ fp fp_mul(const fp& a, const fp& b) { return fp_mul_cios(a, b); }
__device__ __forceinline__ fp fp_sqr(const fp& a) { return fp_sqr_sos(a); }

// Small constant c (< 2^32) in Montgomery form.
__device__ __forceinline__ fp fp_from_u32(uint32_t c) {
  fp x = fp_zero();
  x.v[0] = c;
  return fp_mul(x, fp_r2());
}

// x^(p-2) mod p, the inverse of a non-zero x (0 maps to 0): left-to-right binary
// square-and-multiply. The exponent is the same for every lane, so the multiply
// branch is uniform across the wavefront. (The library inverts with the binary GCD
// of bingcd.hpp, which falls back to this form for x = 0.)
__device__ __forceinline__ fp fp_inv_fermat(const fp& x) {
  const uint32_t e[8] = {MSM_P0 - 2u, MSM_P1, MSM_P2, MSM_P3, MSM_P4, MSM_P5, MSM_P6, MSM_P7};
  fp acc = x;  // the exponent's top bit (bit 253) is set
  for (int bit = 252; bit >= 0; bit--) {
    acc = fp_sqr(acc);
    if ((e[bit >> 5] >> (bit & 31)) & 1u) acc = fp_mul(acc, x);
  }
  return acc;
}

}  // namespace msmk
