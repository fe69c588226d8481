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

__device__ __forceinline__ xyzz quad_add(const xyzz& p, const xyzz& s, int q) {
  if (xyzz_is_inf(s)) return p;
  if (xyzz_is_inf(p)) return s;
  fp r = fp_mul(quad_pick(q, p.X, s.X, p.Y, s.Y), quad_pick(q, s.ZZ, p.ZZ, s.ZZZ, p.ZZZ));
  const fp U1 = quad_from<0>(r), U2 = quad_from<1>(r);  // U1 = X1 ZZ2, U2 = X2 ZZ1
  const fp S1 = quad_from<2>(r), S2 = quad_from<3>(r);  // S1 = Y1 ZZZ2, S2 = Y2 ZZZ1
  const fp P = fp_sub(U2, U1), R = fp_sub(S2, S1);
  if (fp_is_zero(P)) {
    if (fp_is_zero(R)) return quad_dbl(p, q);
    return xyzz_inf();
  }
  r = fp_mul(quad_pick(q, p.ZZ, p.ZZZ, P, R), quad_pick(q, s.ZZ, s.ZZZ, P, R));
  const fp ZZ12 = quad_from<0>(r), ZZZ12 = quad_from<1>(r);
  const fp PP = quad_from<2>(r), RR = quad_from<3>(r);
  r = fp_mul(quad_pick(q, P, U1, ZZ12, P), PP);         // PPP, Q = U1 PP, ZZ3
  const fp PPP = quad_from<0>(r), Qv = quad_from<1>(r);
  xyzz o;
  o.ZZ = quad_from<2>(r);
  o.X = fp_sub(fp_sub(fp_sub(RR, PPP), Qv), Qv);
  r = fp_mul(quad_pick(q, ZZZ12, S1, R, ZZZ12), quad_pick(q, PPP, PPP, fp_sub(Qv, o.X), PPP));
  o.ZZZ = quad_from<0>(r);
  o.Y = fp_sub(quad_from<2>(r), quad_from<1>(r));       // R (Q - X3) - S1 PPP
  return o;
}

// P + Q for two affine points (mmadd-2008-s), quad-cooperative: 3 rounds.
__device__ __forceinline__ xyzz quad_add_aa(const aff& p, const aff& s, int q) {
  if (aff_is_inf(s)) return xyzz_from_aff(p);
  if (aff_is_inf(p)) return xyzz_from_aff(s);
  const fp P = fp_sub(s.x, p.x), R = fp_sub(s.y, p.y);
  if (fp_is_zero(P)) {
    if (fp_is_zero(R)) return quad_dbl(xyzz_from_aff(p), q);
    return xyzz_inf();
  }
  fp r = fp_mul(quad_pick(q, P, R, P, R), quad_pick(q, P, R, P, R));  // PP, RR
  const fp PP = quad_from<0>(r), RR = quad_from<1>(r);
  r = fp_mul(quad_pick(q, P, p.x, P, p.x), PP);                        // PPP, Q
  const fp PPP = quad_from<0>(r), Qv = quad_from<1>(r);
  xyzz o;
  o.X = fp_sub(fp_sub(fp_sub(RR, PPP), Qv), Qv);
  r = fp_mul(quad_pick(q, R, p.y, R, p.y), quad_pick(q, fp_sub(Qv, o.X), PPP, fp_sub(Qv, o.X), PPP));
  o.Y = fp_sub(quad_from<0>(r), quad_from<1>(r));                      // R (Q - X3) - Y1 PPP
  o.ZZ = PP;
  o.ZZZ = PPP;
  return o;
}

// k * P for a small non-negative k (MSB-first double-and-add), quad-cooperative.
__device__ __forceinline__ xyzz quad_mul_small(const xyzz& p, uint32_t k, int q) {
  if (k == 0) return xyzz_inf();
  const int top = 31 - __clz(k);
  xyzz acc = p;
  for (int b = top - 1; b >= 0; b--) {
    acc = quad_dbl(acc, q);
    if ((k >> b) & 1u) acc = quad_add(acc, p, q);
  }
  return acc;
}

}  // namespace msmk
