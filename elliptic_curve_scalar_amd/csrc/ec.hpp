// BN254 G1 (y^2 = x^3 + 3 over F_p, prime order r) point arithmetic on gfx950.
//
// Two coordinate systems, chosen per phase of the bucket MSM:
//   * affine (x, y) for the bucket accumulate, where S additions share one field
//     inversion (Montgomery's trick; aztec-packages PR #23738 "TL;DR" and PR #23736
//     "Goal & lever": inversion cost per add = |inversion| / S). The batched adder
//     lives in batch_add.hpp; this header gives the point types and codecs.
//   * XYZZ (X, Y, ZZ, ZZZ) with x = X/ZZ, y = Y/ZZZ, ZZ^3 = ZZZ^2, for the running
//     sum and the window combine, which need no inversion. Formulas are the
//     Explicit-Formulas Database's "xyzz" set for short Weierstrass curves with
//     a = 0: madd-2008-s, add-2008-s, dbl-2008-s-1, mdbl-2008-s-1.
//
// The point at infinity is (0, 0) in affine storage (not on the curve, since
// 0 != 0^3 + 3) and ZZ = ZZZ = 0 in XYZZ.
#pragma once
#include "bingcd.hpp"

namespace msmk {

// Interchange layout: x then y, eight little-endian 32-bit words each, Montgomery
// form, fully reduced. 64 bytes, loaded and stored as four 16-byte vectors.
struct g1a {
  uint32_t w[16];
};

struct aff {
  fp x, y;
};

struct xyzz {
  fp X, Y, ZZ, ZZZ;
};

__device__ __forceinline__ aff aff_load(const g1a* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 a = q[0], b = q[1], c = q[2], d = q[3];
  aff r;
  r.x.v[0] = a.x; r.x.v[1] = a.y; r.x.v[2] = a.z; r.x.v[3] = a.w;
  r.x.v[4] = b.x; r.x.v[5] = b.y; r.x.v[6] = b.z; r.x.v[7] = b.w;
  r.y.v[0] = c.x; r.y.v[1] = c.y; r.y.v[2] = c.z; r.y.v[3] = c.w;
  r.y.v[4] = d.x; r.y.v[5] = d.y; r.y.v[6] = d.z; r.y.v[7] = d.w;
  return r;
}

__device__ __forceinline__ fp fp_load_x(const g1a* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 a = q[0], b = q[1];
  fp r;
  r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
  return r;
}

__device__ __forceinline__ void aff_store(g1a* p, const aff& a) {
  uint4* q = reinterpret_cast<uint4*>(p);
  q[0] = make_uint4(a.x.v[0], a.x.v[1], a.x.v[2], a.x.v[3]);
  q[1] = make_uint4(a.x.v[4], a.x.v[5], a.x.v[6], a.x.v[7]);
  q[2] = make_uint4(a.y.v[0], a.y.v[1], a.y.v[2], a.y.v[3]);
  q[3] = make_uint4(a.y.v[4], a.y.v[5], a.y.v[6], a.y.v[7]);
}

__device__ __forceinline__ bool aff_is_inf(const aff& a) { return fp_is_zero(a.x) && fp_is_zero(a.y); }

__device__ __forceinline__ aff aff_inf() {
  aff r;
  r.x = fp_zero();
  r.y = fp_zero();
  return r;
}

// Coordinates below p, and y^2 = x^3 + 3 (both sides in Montgomery form), or the
// infinity encoding (0, 0).
__device__ __forceinline__ bool aff_valid(const aff& a) {
  if (aff_is_inf(a)) return true;
  if (!fp_is_reduced(a.x) || !fp_is_reduced(a.y)) return false;
  const fp one = fp_one();
  const fp b = fp_add(fp_add(one, one), one);  // 3 in Montgomery form
  return fp_eq(fp_sqr(a.y), fp_add(fp_mul(fp_sqr(a.x), a.x), b));
}

__device__ __forceinline__ xyzz xyzz_inf() {
  xyzz r;
  r.X = fp_zero();
  r.Y = fp_zero();
  r.ZZ = fp_zero();
  r.ZZZ = fp_zero();
  return r;
}

__device__ __forceinline__ bool xyzz_is_inf(const xyzz& p) { return fp_is_zero(p.ZZ); }

__device__ __forceinline__ xyzz xyzz_from_aff(const aff& a) {
  if (aff_is_inf(a)) return xyzz_inf();
  xyzz r;
  r.X = a.x;
  r.Y = a.y;
  r.ZZ = fp_one();
  r.ZZZ = fp_one();
  return r;
}

// 2 * (x, y) for an affine point (mdbl-2008-s-1).
__device__ __forceinline__ xyzz xyzz_dbl_aff(const aff& a) {
  if (aff_is_inf(a)) return xyzz_inf();
  fp U = fp_dbl(a.y);
  fp V = fp_sqr(U);
  fp W = fp_mul(U, V);
  fp S = fp_mul(a.x, V);
  fp xx = fp_sqr(a.x);
  fp M = fp_add(fp_dbl(xx), xx);
  xyzz r;
  r.X = fp_sub(fp_sub(fp_sqr(M), S), S);
  r.Y = fp_sub(fp_mul(M, fp_sub(S, r.X)), fp_mul(W, a.y));
  r.ZZ = V;
  r.ZZZ = W;
  return r;
}

// 2P (dbl-2008-s-1 with a = 0). Infinity and Y = 0 both give ZZ3 = 0.
__device__ __forceinline__ xyzz xyzz_dbl(const xyzz& p) {
  fp U = fp_dbl(p.Y);
  fp V = fp_sqr(U);
  fp W = fp_mul(U, V);
  fp S = fp_mul(p.X, V);
  fp xx = fp_sqr(p.X);
  fp M = fp_add(fp_dbl(xx), xx);
  xyzz r;
  r.X = fp_sub(fp_sub(fp_sqr(M), S), S);
  r.Y = fp_sub(fp_mul(M, fp_sub(S, r.X)), fp_mul(W, p.Y));
  r.ZZ = fp_mul(V, p.ZZ);
  r.ZZZ = fp_mul(W, p.ZZZ);
  return r;
}

// P + Q with Q affine (madd-2008-s), every special case handled.
__device__ __forceinline__ xyzz xyzz_add_aff(const xyzz& p, const aff& q) {
  if (aff_is_inf(q)) return p;
  if (xyzz_is_inf(p)) return xyzz_from_aff(q);
  fp U2 = fp_mul(q.x, p.ZZ);
  fp S2 = fp_mul(q.y, p.ZZZ);
  fp P = fp_sub(U2, p.X);
  fp R = fp_sub(S2, p.Y);
  if (fp_is_zero(P)) {
    if (fp_is_zero(R)) return xyzz_dbl_aff(q);  // same point
    return xyzz_inf();                          // P + (-P)
  }
  fp PP = fp_sqr(P);
  fp PPP = fp_mul(P, PP);
  fp Q = fp_mul(p.X, PP);
  xyzz r;
  r.X = fp_sub(fp_sub(fp_sub(fp_sqr(R), PPP), Q), Q);
  r.Y = fp_sub(fp_mul(R, fp_sub(Q, r.X)), fp_mul(p.Y, PPP));
  r.ZZ = fp_mul(p.ZZ, PP);
  r.ZZZ = fp_mul(p.ZZZ, PPP);
  return r;
}

// P + Q for two affine points, XYZZ result (mmadd-2008-s: 4M + 2S); every special
// case handled.
__device__ __forceinline__ xyzz xyzz_add_aa(const aff& p, const aff& q) {
  if (aff_is_inf(q)) return xyzz_from_aff(p);
  if (aff_is_inf(p)) return xyzz_from_aff(q);
  const fp P = fp_sub(q.x, p.x);
  const fp R = fp_sub(q.y, p.y);
  if (fp_is_zero(P)) {
    if (fp_is_zero(R)) return xyzz_dbl_aff(p);
    return xyzz_inf();
  }
  const fp PP = fp_sqr(P);
  const fp PPP = fp_mul(P, PP);
  const fp Q = fp_mul(p.x, PP);
  xyzz r;
  r.X = fp_sub(fp_sub(fp_sub(fp_sqr(R), PPP), Q), Q);
  r.Y = fp_sub(fp_mul(R, fp_sub(Q, r.X)), fp_mul(p.y, PPP));
  r.ZZ = PP;
  r.ZZZ = PPP;
  return r;
}

// P + Q, both XYZZ (add-2008-s), every special case handled.
__device__ __forceinline__ xyzz xyzz_add(const xyzz& p, const xyzz& q) {
  if (xyzz_is_inf(q)) return p;
  if (xyzz_is_inf(p)) return q;
  fp U1 = fp_mul(p.X, q.ZZ);
  fp U2 = fp_mul(q.X, p.ZZ);
  fp S1 = fp_mul(p.Y, q.ZZZ);
  fp S2 = fp_mul(q.Y, p.ZZZ);
  fp P = fp_sub(U2, U1);
  fp R = fp_sub(S2, S1);
  if (fp_is_zero(P)) {
    if (fp_is_zero(R)) return xyzz_dbl(p);
    return xyzz_inf();
  }
  fp PP = fp_sqr(P);
  fp PPP = fp_mul(P, PP);
  fp Q = fp_mul(U1, PP);
  xyzz r;
  r.X = fp_sub(fp_sub(fp_sub(fp_sqr(R), PPP), Q), Q);
  r.Y = fp_sub(fp_mul(R, fp_sub(Q, r.X)), fp_mul(S1, PPP));
  r.ZZ = fp_mul(fp_mul(p.ZZ, q.ZZ), PP);
  r.ZZZ = fp_mul(fp_mul(p.ZZZ, q.ZZZ), PPP);
  return r;
}

// k * P for a small non-negative k (MSB-first double-and-add).
__device__ __forceinline__ xyzz xyzz_mul_small(const xyzz& p, uint32_t k) {
  xyzz acc = xyzz_inf();
  if (k == 0) return acc;
  int top = 31 - __clz(k);
  acc = p;
  for (int b = top - 1; b >= 0; b--) {
    acc = xyzz_dbl(acc);
    if ((k >> b) & 1u) acc = xyzz_add(acc, p);
  }
  return acc;
}

// XYZZ -> affine with one inversion: 1/ZZ = ZZZ * t, 1/ZZZ = ZZ * t, t = (ZZ ZZZ)^-1.
__device__ __forceinline__ aff xyzz_to_aff(const xyzz& p) {
  if (xyzz_is_inf(p)) return aff_inf();
  fp t = fp_inv(fp_mul(p.ZZ, p.ZZZ));
  aff r;
  r.x = fp_mul(p.X, fp_mul(p.ZZZ, t));
  r.y = fp_mul(p.Y, fp_mul(p.ZZ, t));
  return r;
}

}  // namespace msmk
