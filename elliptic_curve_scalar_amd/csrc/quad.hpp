// XYZZ point arithmetic shared by the four lanes of a quad.
//
// The running sum, the per-window trees and the deep pair-tree levels have too
// little parallel work to fill the chip, so their time is the latency of one lane's
// chain of additions. An XYZZ addition (add-2008-s) has 12 field products but only 4
// dependent rounds of at most 4 independent products each, and a doubling
// (dbl-2008-s-1) 9 products in 3 rounds. Here the four lanes of a quad hold the same
// points; in each round lane k computes product k and a DPP quad_perm broadcast hands
// every result to all four lanes. A step then costs 3-4 product latencies instead of
// 9-14, at about 1.4x the total lane work, which pays only where lanes are idle.
//
// All four lanes of a quad see the same values, so every branch below is uniform
// within the quad (quads of one wavefront may still diverge from each other).
#pragma once
#include "ec.hpp"

namespace msmk {

// Lane K of this lane's quad, for every word of v (v_mov_b32 with DPP quad_perm).
template <int K>
__device__ __forceinline__ fp quad_from(const fp& v) {
  constexpr int ctrl = K | (K << 2) | (K << 4) | (K << 6);
  fp r;
#pragma unroll
  for (int i = 0; i < 8; i++)
    r.v[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v.v[i], ctrl, 0xf, 0xf, false);
  return r;
}

// Operand for this lane: a0 on quad lane 0, a1 on 1, ... Written as bit selects on the
// two bits of q: a chain of q == k tests is turned by the compiler into a lookup table
// in private memory (a scratch store and a lane-indexed load per word).
__device__ __forceinline__ fp quad_pick(int q, const fp& a0, const fp& a1, const fp& a2,
                                        const fp& a3) {
  const uint32_t m0 = 0u - ((uint32_t)q & 1u), m1 = 0u - (((uint32_t)q >> 1) & 1u);
  fp r;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t lo = (a1.v[i] & m0) | (a0.v[i] & ~m0);
    const uint32_t hi = (a3.v[i] & m0) | (a2.v[i] & ~m0);
    r.v[i] = (hi & m1) | (lo & ~m1);
  }
  return r;
}

__device__ __forceinline__ xyzz quad_dbl(const xyzz& p, int q) {
  const fp U = fp_dbl(p.Y);
  const fp x = quad_pick(q, U, p.X, U, p.X);
  fp r = fp_sqr(x);                                   // V = U^2, XX = X^2
  const fp V = quad_from<0>(r), XX = quad_from<1>(r);
  const fp M = fp_add(fp_dbl(XX), XX);
  r = fp_mul(quad_pick(q, U, p.X, M, V), quad_pick(q, V, V, M, p.ZZ));  // W, S, M^2, ZZ3
  const fp W = quad_from<0>(r), S = quad_from<1>(r), MM = quad_from<2>(r);
  xyzz o;
  o.ZZ = quad_from<3>(r);
  o.X = fp_sub(fp_sub(MM, S), S);
  r = fp_mul(quad_pick(q, W, W, M, W), quad_pick(q, p.ZZZ, p.Y, fp_sub(S, o.X), p.ZZZ));
  o.ZZZ = quad_from<0>(r);                            // ZZZ3 = W ZZZ
  o.Y = fp_sub(quad_from<2>(r), quad_from<1>(r));     // M (S - X3) - W Y
  return o;
}

// ---- runs of doublings with one round of lookahead --------------------------------
// A run keeps (X, U = 2Y, M = 3X^2) and a factor z; the XYZZ point it stands for is
// (X, U / 2, ZZ0 z^2, ZZZ0 z^3), with ZZ0, ZZZ0 those of the run's input. With a = 0, the
// doubling dbl-2008-s-1 written in U reads
//   V = U^2,  S = X V,  X' = M^2 - 2 S,
//   U' = 2 M (S - X') - V^2 = 6 (M X) V - 2 M M^2 - V^2,  z' = z U,
// its ZZ' = V ZZ and ZZZ' = U V ZZZ being folded into z. M X and M^2 need only X, which
// the previous step knows a round before its U', so those products start early: two
// doublings take five rounds of at most four products, against six for two quad_dbl.
// ZZ and ZZZ never enter the recurrence, so a run on the point at infinity (ZZ0 = 0)
// stays at infinity.
struct dchain {
  fp X, U, M, z;
};

__device__ __forceinline__ fp fp_triple(const fp& a) { return fp_add(fp_dbl(a), a); }

// Start a run on p. The one product (X^2) is the same on every lane: no broadcast.
__device__ __forceinline__ dchain quad_chain_begin(const xyzz& p) {
  dchain c;
  c.X = p.X;
  c.U = fp_dbl(p.Y);
  c.M = fp_triple(fp_sqr(p.X));
  c.z = fp_one();
  return c;
}

// Two doublings in five rounds.
__device__ __forceinline__ void quad_chain_dbl2(dchain& c, int q) {
  // round A: V = U^2, M X, M^2, z U
  fp r = fp_mul(quad_pick(q, c.U, c.M, c.M, c.z), quad_pick(q, c.U, c.X, c.M, c.U));
  const fp V = quad_from<0>(r), MX = quad_from<1>(r), MM = quad_from<2>(r), z1 = quad_from<3>(r);
  // round B: X V, (M X) V, M M^2, V^2
  r = fp_mul(quad_pick(q, c.X, MX, c.M, V), quad_pick(q, V, V, MM, V));
  const fp XV = quad_from<0>(r), MXV = quad_from<1>(r), M3 = quad_from<2>(r), VV = quad_from<3>(r);
  const fp X1 = fp_sub(MM, fp_dbl(XV));
  const fp U1 = fp_sub(fp_dbl(fp_sub(fp_triple(MXV), M3)), VV);
  // round C: X1^2, V1 = U1^2, z1 U1 (lane 3 repeats lane 0)
  r = fp_mul(quad_pick(q, X1, U1, z1, X1), quad_pick(q, X1, U1, U1, X1));
  const fp M1 = fp_triple(quad_from<0>(r)), V1 = quad_from<1>(r);
  c.z = quad_from<2>(r);
  // round D: M1 X1, M1^2, X1 V1, V1^2
  r = fp_mul(quad_pick(q, M1, M1, X1, V1), quad_pick(q, X1, M1, V1, V1));
  const fp M1X1 = quad_from<0>(r), MM1 = quad_from<1>(r), X1V1 = quad_from<2>(r), VV1 = quad_from<3>(r);
  c.X = fp_sub(MM1, fp_dbl(X1V1));
  // round E: (M1 X1) V1, M1 M1^2, X2^2 (lane 3 repeats lane 2)
  r = fp_mul(quad_pick(q, M1X1, M1, c.X, c.X), quad_pick(q, V1, MM1, c.X, c.X));
  c.U = fp_sub(fp_dbl(fp_sub(fp_triple(quad_from<0>(r)), quad_from<1>(r))), VV1);
  c.M = fp_triple(quad_from<2>(r));
}

// One doubling in three rounds (the last one, X'^2, the same on every lane).
__device__ __forceinline__ void quad_chain_dbl1(dchain& c, int q) {
  fp r = fp_mul(quad_pick(q, c.U, c.M, c.M, c.z), quad_pick(q, c.U, c.X, c.M, c.U));
  const fp V = quad_from<0>(r), MX = quad_from<1>(r), MM = quad_from<2>(r);
  c.z = quad_from<3>(r);
  r = fp_mul(quad_pick(q, c.X, MX, c.M, V), quad_pick(q, V, V, MM, V));
  const fp XV = quad_from<0>(r), MXV = quad_from<1>(r), M3 = quad_from<2>(r), VV = quad_from<3>(r);
  c.X = fp_sub(MM, fp_dbl(XV));
  c.U = fp_sub(fp_dbl(fp_sub(fp_triple(MXV), M3)), VV);
  c.M = fp_triple(fp_sqr(c.X));
}

// The XYZZ point a run stands for, given its input's ZZ0 and ZZZ0: two rounds.
__device__ __forceinline__ xyzz quad_chain_end(const dchain& c, const fp& ZZ0, const fp& ZZZ0, int q) {
  fp r = fp_mul(c.z, quad_pick(q, c.z, ZZZ0, c.z, ZZZ0));  // z^2, z ZZZ0
  const fp zz = quad_from<0>(r), zZZZ = quad_from<1>(r);
  r = fp_mul(quad_pick(q, ZZ0, zZZZ, ZZ0, zZZZ), zz);  // ZZ0 z^2, ZZZ0 z^3
  xyzz o;
  o.X = c.X;
  o.Y = fp_half(c.U);
  o.ZZ = quad_from<0>(r);
  o.ZZZ = quad_from<1>(r);
  return o;
}

// 2^n p by runs of two doublings.
__device__ __forceinline__ xyzz quad_dbl_n(const xyzz& p, uint32_t n, int q) {
  if (n == 0) return p;
  dchain c = quad_chain_begin(p);
  for (uint32_t i = 0; i < n / 2; i++) quad_chain_dbl2(c, q);
  if (n & 1u) quad_chain_dbl1(c, q);
  return quad_chain_end(c, p.ZZ, p.ZZZ, q);
}

// One exit: with several return statements the compiler passes the result through
// private memory.
__device__ __forceinline__ xyzz quad_add(const xyzz& p, const xyzz& s, int q) {
  xyzz o;
  if (xyzz_is_inf(s)) {
    o = p;
  } else if (xyzz_is_inf(p)) {
    o = s;
  } else {
    fp r = fp_mul(quad_pick(q, p.X, s.X, p.Y, s.Y), quad_pick(q, s.ZZ, p.ZZ, s.ZZZ, p.ZZZ));
    const fp U1 = quad_from<0>(r), U2 = quad_from<1>(r);  // U1 = X1 ZZ2, U2 = X2 ZZ1
    const fp S1 = quad_from<2>(r), S2 = quad_from<3>(r);  // S1 = Y1 ZZZ2, S2 = Y2 ZZZ1
    const fp P = fp_sub(U2, U1), R = fp_sub(S2, S1);
    if (fp_is_zero(P)) {
      if (fp_is_zero(R)) o = quad_dbl(p, q);
      else o = xyzz_inf();
    } else {
      r = fp_mul(quad_pick(q, p.ZZ, p.ZZZ, P, R), quad_pick(q, s.ZZ, s.ZZZ, P, R));
      const fp ZZ12 = quad_from<0>(r), ZZZ12 = quad_from<1>(r);
      const fp PP = quad_from<2>(r), RR = quad_from<3>(r);
      r = fp_mul(quad_pick(q, P, U1, ZZ12, P), PP);         // PPP, Q = U1 PP, ZZ3
      const fp PPP = quad_from<0>(r), Qv = quad_from<1>(r);
      o.ZZ = quad_from<2>(r);
      o.X = fp_sub(fp_sub(fp_sub(RR, PPP), Qv), Qv);
      r = fp_mul(quad_pick(q, ZZZ12, S1, R, ZZZ12), quad_pick(q, PPP, PPP, fp_sub(Qv, o.X), PPP));
      o.ZZZ = quad_from<0>(r);
      o.Y = fp_sub(quad_from<2>(r), quad_from<1>(r));       // R (Q - X3) - S1 PPP
    }
  }
  return o;
}

// P + Q for two affine points (mmadd-2008-s), quad-cooperative: 3 rounds.
__device__ __forceinline__ xyzz quad_add_aa(const aff& p, const aff& s, int q) {
  xyzz o;
  if (aff_is_inf(s)) {
    o = xyzz_from_aff(p);
  } else if (aff_is_inf(p)) {
    o = xyzz_from_aff(s);
  } else {
    const fp P = fp_sub(s.x, p.x), R = fp_sub(s.y, p.y);
    if (fp_is_zero(P)) {
      if (fp_is_zero(R)) o = quad_dbl(xyzz_from_aff(p), q);
      else o = xyzz_inf();
    } else {
      fp r = fp_mul(quad_pick(q, P, R, P, R), quad_pick(q, P, R, P, R));  // PP, RR
      const fp PP = quad_from<0>(r), RR = quad_from<1>(r);
      r = fp_mul(quad_pick(q, P, p.x, P, p.x), PP);                        // PPP, Q
      const fp PPP = quad_from<0>(r), Qv = quad_from<1>(r);
      o.X = fp_sub(fp_sub(fp_sub(RR, PPP), Qv), Qv);
      r = fp_mul(quad_pick(q, R, p.y, R, p.y), quad_pick(q, fp_sub(Qv, o.X), PPP, fp_sub(Qv, o.X), PPP));
      o.Y = fp_sub(quad_from<0>(r), quad_from<1>(r));                      // R (Q - X3) - Y1 PPP
      o.ZZ = PP;
      o.ZZZ = PPP;
    }
  }
  return o;
}

// k * P for a small non-negative k (MSB-first double-and-add), quad-cooperative.
__device__ __forceinline__ xyzz quad_mul_small(const xyzz& p, uint32_t k, int q) {
  xyzz acc = xyzz_inf();
  if (k != 0) {
    const int top = 31 - __clz(k);
    acc = p;
    for (int b = top - 1; b >= 0; b--) {
      acc = quad_dbl(acc, q);
      if ((k >> b) & 1u) acc = quad_add(acc, p, q);
    }
  }
  return acc;
}

}  // namespace msmk
