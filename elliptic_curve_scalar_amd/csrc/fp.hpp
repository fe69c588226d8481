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
//     ALU ops), each row's multiply-adds independent of each other and its carries in
//     one add-with-carry chain; p < 2^254 keeps every partial sum inside 288 bits and
//     the result before the final subtraction below 2p;
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
// 32-bit limbs. Each row (t += a b_i, then t = (t + m p) / 2^32 with m = t_0 (-p^-1) mod
// 2^32) is eight independent multiply-adds s_j = x_j y + t_j (each below 2^64) and one
// carry chain t_j = lo(s_j) + hi(s_(j-1)) + carry: the products of a row do not wait for
// each other, and the chain of the row overlaps the next row's products. The word t_8
// rides in the high half of the last addend (s_7 = x_7 y + t_7 + 2^32 t_8), which stays
// below 2^64 because a_7 and p_7 are below 2^30, so the chain needs no ninth step. Bounds:
// t < 2p before each product row, so t + a b_i < 2^287 (t_8 < 2^31) and after each
// reduction row t < 2p again (t_8 = 0).
__device__ __forceinline__ fp fp_mul_cios(const fp& a, const fp& b) {
  uint32_t t[9];
#pragma unroll
  for (int j = 0; j < 9; j++) t[j] = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    uint64_t s[8];
#pragma unroll
    for (int j = 0; j < 7; j++) s[j] = (uint64_t)a.v[j] * b.v[i] + t[j];
    s[7] = (uint64_t)a.v[7] * b.v[i] + (((uint64_t)t[8] << 32) | t[7]);
    uint32_t c = 0;
    t[0] = (uint32_t)s[0];
#pragma unroll
    for (int j = 1; j < 8; j++) t[j] = __builtin_addc((uint32_t)s[j], (uint32_t)(s[j - 1] >> 32), c, &c);
    t[8] = (uint32_t)(s[7] >> 32) + c;
    const uint32_t m = t[0] * MSM_PINV;
#pragma unroll
    for (int j = 0; j < 7; j++) s[j] = (uint64_t)m * p_limb(j) + t[j];
    s[7] = (uint64_t)m * p_limb(7) + (((uint64_t)t[8] << 32) | t[7]);
    c = 0;  // lo(s_0) = 0 by the choice of m: the row drops it
#pragma unroll
    for (int j = 1; j < 8; j++) t[j - 1] = __builtin_addc((uint32_t)s[j], (uint32_t)(s[j - 1] >> 32), c, &c);
    t[7] = (uint32_t)(s[7] >> 32) + c;
    t[8] = 0;
  }
  fp r;
#pragma unroll
  for (int j = 0; j < 8; j++) r.v[j] = t[j];
  return fp_reduce_once(r);  // t < 2p
}

// Montgomery square a^2 * 2^-256 mod p by separated operand scanning: the 28 products
// a_i a_j (i < j) once, the 512-bit sum doubled by a one-bit shift, the 8 squares a_i^2
// added, then the word-serial Montgomery reduction (8 rounds of t += m p 2^(32 i),
// m = t_i (-p^-1) mod 2^32): 108 multiply-adds against 136 for the product. Every row is
// independent multiply-adds and one carry chain, as in fp_mul_cios. The carry out of a
// reduction round's top word (t_(i+8)) belongs to word i + 9, which is the high half of
// the next round's last addend (m p_7 < 2^62 leaves room for it); after the last round
// it is 0, since (a^2 + M p) / 2^256 < 2p < 2^255.
__device__ __forceinline__ fp fp_sqr_sos(const fp& a) {
  uint32_t t[16];
#pragma unroll
  for (int k = 0; k < 16; k++) t[k] = 0;
  // off-diagonal products: row i adds a_i a_j (j > i) at t[i + j]; t[i + 8] is still 0
#pragma unroll
  for (int i = 0; i < 7; i++) {
    uint64_t s[8];
#pragma unroll
    for (int j = i + 1; j < 8; j++) s[j] = (uint64_t)a.v[i] * a.v[j] + t[i + j];
    uint32_t c = 0;
    t[2 * i + 1] = (uint32_t)s[i + 1];
#pragma unroll
    for (int j = i + 2; j < 8; j++) t[i + j] = __builtin_addc((uint32_t)s[j], (uint32_t)(s[j - 1] >> 32), c, &c);
    t[i + 8] = (uint32_t)(s[7] >> 32) + c;
  }
  // double (the top bit of t[14] moves into t[15], which is still 0)
#pragma unroll
  for (int k = 15; k > 0; k--) t[k] = __builtin_amdgcn_alignbit(t[k], t[k - 1], 31);
  t[0] = 0;
  // the squares a_i^2 at t[2i], t[2i + 1]: one chain over the sixteen words
  {
    uint64_t s[8];
#pragma unroll
    for (int i = 0; i < 8; i++) s[i] = (uint64_t)a.v[i] * a.v[i] + t[2 * i];
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      t[2 * i] = __builtin_addc((uint32_t)s[i], 0u, c, &c);
      t[2 * i + 1] = __builtin_addc(t[2 * i + 1], (uint32_t)(s[i] >> 32), c, &c);
    }
  }
  // reduction: after round i, t[0..i] are 0 and the value is unchanged mod p
  uint32_t cc = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t m = t[i] * MSM_PINV;
    uint64_t s[8];
#pragma unroll
    for (int j = 0; j < 7; j++) s[j] = (uint64_t)m * p_limb(j) + t[i + j];
    s[7] = (uint64_t)m * p_limb(7) + (((uint64_t)cc << 32) | t[i + 7]);
    uint32_t c = 0;
#pragma unroll
    for (int j = 1; j < 8; j++) t[i + j] = __builtin_addc((uint32_t)s[j], (uint32_t)(s[j - 1] >> 32), c, &c);
    t[i + 8] = __builtin_addc(t[i + 8], (uint32_t)(s[7] >> 32), c, &c);
    cc = c;
  }
  fp r;
#pragma unroll
  for (int j = 0; j < 8; j++) r.v[j] = t[8 + j];
  return fp_reduce_once(r);
}

// Montgomery product a * b * 2^-256 mod p; inputs and output fully reduced.
__device__ __forceinline__ fp fp_mul(const fp& a, const fp& b) { return fp_mul_cios(a, b); }
__device__ __forceinline__ fp fp_sqr(const fp& a) { return fp_sqr_sos(a); }

// The same as calls, one copy of each in the code object: for kernels that would inline
// hundreds of them into one body (the stream walker's batches at large S), where the
// register coalescer's compile time grows without bound on the inlined form.
__device__ __noinline__ fp fp_mul_call(const fp& a, const fp& b) { return fp_mul_cios(a, b); }
__device__ __noinline__ fp fp_sqr_call(const fp& a) { return fp_sqr_sos(a); }

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
