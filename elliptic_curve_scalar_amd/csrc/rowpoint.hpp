// XYZZ points in row form (rowfp.hpp), for the window combine's few long chains.
//
// One wavefront holds one point: each coordinate is one word per lane (lane l of every row
// holds word l of X, Y, ZZ and ZZZ), and values stay in the lazy form [0, 3p) between
// operations. An addition is four rounds of at most four products with every round's
// products on the four rows at once, so a lone wavefront's chain of additions (a plane's
// terms, the joins of the planes) runs at four row products per addition instead of four
// whole products per lane in the quad form (quad.hpp). The formulas are those of quad.hpp
// (add-2008-s and dbl-2008-s-1 in XYZZ coordinates, a = 0), so the fully reduced results
// are the same field elements.
//
// Every function here must be called with the whole wavefront active (ballots, DPP).
#pragma once
#include "kern_util.hpp"
#include "rowchain.hpp"

namespace msmk {

struct rxyzz {
  uint32_t X, Y, ZZ, ZZZ;
};

// The point at infinity: ZZ = 0 (all coordinates 0, like xyzz_inf).
__device__ __forceinline__ rxyzz rxyzz_inf() { return rxyzz{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ bool rxyzz_is_inf(const rxyzz& a, row_consts& k) {
  return row_all_zero(row_canon(a.ZZ, k));
}

__device__ __forceinline__ rxyzz rxyzz_canon(const rxyzz& a, row_consts& k) {
  return rxyzz{row_canon(a.X, k), row_canon(a.Y, k), row_canon(a.ZZ, k), row_canon(a.ZZZ, k)};
}

// Loads and stores of the 32-word point layout (xyzz_st): lanes 0..7 of each row read word
// l of every coordinate, the other lanes hold 0; a store writes from row 0.
__device__ __forceinline__ rxyzz rxyzz_load(const xyzz_st* p) {
  const uint32_t l = __lane_id() & 15u;
  rxyzz r = rxyzz_inf();
  if (l < 8u) {
    r.X = p->w[l];
    r.Y = p->w[8 + l];
    r.ZZ = p->w[16 + l];
    r.ZZZ = p->w[24 + l];
  }
  return r;
}

// The same for a point that another block has just written (after the fence that
// preceded its counter's atomic): device-scope loads that bypass this CU's cache.
__device__ __forceinline__ rxyzz rxyzz_load_coherent(const xyzz_st* p) {
  const uint32_t l = __lane_id() & 15u;
  rxyzz r = rxyzz_inf();
  if (l < 8u) {
    r.X = __hip_atomic_load(&p->w[l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    r.Y = __hip_atomic_load(&p->w[8 + l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    r.ZZ = __hip_atomic_load(&p->w[16 + l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    r.ZZZ = __hip_atomic_load(&p->w[24 + l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return r;
}

// Fully reduced store (every lane calls it; lanes 0..7 write).
__device__ __forceinline__ void rxyzz_store(xyzz_st* p, const rxyzz& a, row_consts& k) {
  const rxyzz c = rxyzz_canon(a, k);
  const uint32_t lane = __lane_id();
  if (lane < 8u) {
    p->w[lane] = c.X;
    p->w[8 + lane] = c.Y;
    p->w[16 + lane] = c.ZZ;
    p->w[24 + lane] = c.ZZZ;
  }
}

// The same layout in LDS (32 words; lazy values kept as they are).
__device__ __forceinline__ void rxyzz_to_lds(uint32_t* s, const rxyzz& a) {
  const uint32_t lane = __lane_id();
  if (lane < 8u) {
    s[lane] = a.X;
    s[8 + lane] = a.Y;
    s[16 + lane] = a.ZZ;
    s[24 + lane] = a.ZZZ;
  }
}

__device__ __forceinline__ rxyzz rxyzz_from_lds(const uint32_t* s) {
  const uint32_t l = __lane_id() & 15u;
  rxyzz r = rxyzz_inf();
  if (l < 8u) {
    r.X = s[l];
    r.Y = s[8 + l];
    r.ZZ = s[16 + l];
    r.ZZZ = s[24 + l];
  }
  return r;
}

// The point as per-lane field elements (every lane holds all eight words of each
// coordinate, read from lanes 0..7 of its row), fully reduced. The values stay in vector
// registers: in scalar registers the binary-GCD inverse that follows would run its steps
// on the scalar unit, which issues them no faster and needs more of them.
__device__ __forceinline__ xyzz rxyzz_to_fp(const rxyzz& a, row_consts& k) {
  const rxyzz c = rxyzz_canon(a, k);
  xyzz r;
  r.X = row_to_fp(c.X);
  r.Y = row_to_fp(c.Y);
  r.ZZ = row_to_fp(c.ZZ);
  r.ZZZ = row_to_fp(c.ZZZ);
  return r;
}

// 2a (dbl-2008-s-1, three rounds): U = 2Y, V = U^2, W = U V, S = X V, M = 3 X^2,
// X3 = M^2 - 2S, Y3 = M (S - X3) - W Y, ZZ3 = V ZZ, ZZZ3 = W ZZZ.
__device__ __forceinline__ rxyzz rxyzz_dbl(const rxyzz& a, row_consts& k) {
  const uint32_t U = row_lin_2a(a.Y, k);
  row4 r = row_round(k, U, a.X, U, a.X, U, a.X, U, a.X);  // V = U^2, X^2 (rows 2, 3 repeat)
  const uint32_t V = r.r0, M = row_lin_3a(r.r1, k);
  r = row_round(k, U, a.X, M, V, V, V, M, a.ZZ);  // W, S, M^2, ZZ3
  const uint32_t W = r.r0, S = r.r1;
  rxyzz o;
  o.ZZ = r.r3;
  o.X = row_lin_a_2b(r.r2, S, k);
  r = row_round(k, W, W, M, W, a.ZZZ, a.Y, row_lin_a_b(S, o.X, k), a.ZZZ);  // ZZZ3, W Y, M (S - X3)
  o.ZZZ = r.r0;
  o.Y = row_lin_a_b(r.r2, r.r1, k);
  return o;
}

// a + b (add-2008-s, four rounds) for every input: infinity on either side, a = b (the
// doubling) and a = -b (infinity). The branches depend only on the point, which the
// whole wavefront holds: no divergence.
//   U1 = X1 ZZ2, U2 = X2 ZZ1, S1 = Y1 ZZZ2, S2 = Y2 ZZZ1, P = U2 - U1, R = S2 - S1,
//   PP = P^2, PPP = P PP, Q = U1 PP, X3 = R^2 - PPP - 2Q, Y3 = R (Q - X3) - S1 PPP,
//   ZZ3 = ZZ1 ZZ2 PP, ZZZ3 = ZZZ1 ZZZ2 PPP.
// One exit: with several return statements the compiler passes the result through
// private memory.
__device__ __forceinline__ rxyzz rxyzz_add(const rxyzz& a, const rxyzz& b, row_consts& k) {
  rxyzz o;
  if (rxyzz_is_inf(b, k)) {
    o = a;
  } else if (rxyzz_is_inf(a, k)) {
    o = b;
  } else {
    row4 r = row_round(k, a.X, b.X, a.Y, b.Y, b.ZZ, a.ZZ, b.ZZZ, a.ZZZ);
    const uint32_t U1 = r.r0, S1 = r.r2;
    const uint32_t P = row_lin_a_b(r.r1, U1, k), R = row_lin_a_b(r.r3, S1, k);
    if (row_all_zero(row_canon(P, k))) {
      if (row_all_zero(row_canon(R, k))) o = rxyzz_dbl(a, k);
      else o = rxyzz_inf();
    } else {
      r = row_round(k, a.ZZ, a.ZZZ, P, R, b.ZZ, b.ZZZ, P, R);  // ZZ1 ZZ2, ZZZ1 ZZZ2, PP, RR
      const uint32_t ZZ12 = r.r0, ZZZ12 = r.r1, PP = r.r2, RR = r.r3;
      r = row_round(k, P, U1, ZZ12, P, PP, PP, PP, PP);  // PPP, Q, ZZ3 (row 3 repeats row 0)
      const uint32_t PPP = r.r0, Q = r.r1;
      o.ZZ = r.r2;
      o.X = row_lin_a_b_2c(RR, PPP, Q, k);
      r = row_round(k, ZZZ12, R, S1, ZZZ12, PPP, row_lin_a_b(Q, o.X, k), PPP, PPP);
      o.ZZZ = r.r0;
      o.Y = row_lin_a_b(r.r1, r.r2, k);  // R (Q - X3) - S1 PPP
    }
  }
  return o;
}

// 2^n a by a run of doublings (rowchain.hpp) on (X, U = 2Y, M = 3 X^2) with the factor z
// from 1; then Y = U / 2, ZZ = ZZ0 z^2 and ZZZ = ZZZ0 z^3 (two rounds). A run on the point
// at infinity stays there (ZZ0 = 0).
__device__ __forceinline__ rxyzz rxyzz_dbl_n(const rxyzz& a, uint32_t n, row_consts& k) {
  rxyzz o = a;
  if (n != 0) {
    rchain c;
    c.X = a.X;
    c.U = row_lin_2a(a.Y, k);
    c.M = row_lin_3a(row_mul_lazy(a.X, a.X, k), k);  // every row computes X^2
    c.z = row_from_fp(fp_one());
    for (uint32_t i = 0; i < n / 2; i++) row_chain_dbl2(c, k);
    if (n & 1u) row_chain_dbl1(c, k);
    row4 r = row_round(k, c.z, c.z, c.z, c.z, c.z, a.ZZZ, c.z, a.ZZZ);  // z^2, z ZZZ0
    const uint32_t zz = r.r0;
    r = row_round(k, a.ZZ, r.r1, a.ZZ, r.r1, zz, zz, zz, zz);  // ZZ0 z^2, ZZZ0 z^3
    o.X = c.X;
    o.Y = row_half(c.U, k);
    o.ZZ = r.r0;
    o.ZZZ = r.r1;
  }
  return o;
}

}  // namespace msmk
