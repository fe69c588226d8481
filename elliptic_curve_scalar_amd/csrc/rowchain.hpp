// Runs of doublings on one wavefront in row form (rowfp.hpp): the same recurrence as the
// quad runs of quad.hpp, with each round's (at most) four products on the four rows of the
// wavefront instead of the four lanes of a quad, and every field value one word per lane.
//
// A run keeps (X, U = 2Y, M = 3X^2) and a factor z; the XYZZ point it stands for is
// (X, U / 2, ZZ0 z^2, ZZZ0 z^3). Two doublings take five rounds (dbl-2008-s-1 with a = 0
// written in U, with M X and M^2 started a round early; quad.hpp states the algebra).
#pragma once
#include "rowfp.hpp"

namespace msmk {

struct rchain {
  uint32_t X, U, M, z;
};

// One round: row r computes a_r b_r (lazy product); every row gets all four results.
__device__ __forceinline__ row4 row_round(row_consts& k, uint32_t a0, uint32_t a1, uint32_t a2,
                                          uint32_t a3, uint32_t b0, uint32_t b1, uint32_t b2,
                                          uint32_t b3) {
  return row_gather(row_mul_lazy(row_pick(k, a0, a1, a2, a3), row_pick(k, b0, b1, b2, b3), k));
}

// Two doublings in five rounds. Values stay in the lazy form [0, 3p); the field
// combinations between rounds are one linear combination each (rowfp.hpp):
//   X' = M^2 - 2 X V,  U' = 6 (M X) V - 2 M M^2 - V^2,  M' = 3 X'^2.
__device__ __forceinline__ void row_chain_dbl2(rchain& c, row_consts& k) {
  // round A: V = U^2, M X, M^2, z U
  row4 r = row_round(k, c.U, c.M, c.M, c.z, c.U, c.X, c.M, c.U);
  const uint32_t V = r.r0, MX = r.r1, MM = r.r2, z1 = r.r3;
  // round B: X V, (M X) V, M M^2, V^2
  r = row_round(k, c.X, MX, c.M, V, V, V, MM, V);
  const uint32_t XV = r.r0, MXV = r.r1, M3 = r.r2, VV = r.r3;
  const uint32_t X1 = row_lin_a_2b(MM, XV, k);
  const uint32_t U1 = row_lin_6a_2b_c(MXV, M3, VV, k);
  // round C: X1^2, V1 = U1^2, z1 U1 (row 3 repeats row 0)
  r = row_round(k, X1, U1, z1, X1, X1, U1, U1, X1);
  const uint32_t M1 = row_lin_3a(r.r0, k), V1 = r.r1;
  c.z = r.r2;
  // round D: M1 X1, M1^2, X1 V1, V1^2
  r = row_round(k, M1, M1, X1, V1, X1, M1, V1, V1);
  const uint32_t M1X1 = r.r0, MM1 = r.r1, X1V1 = r.r2, VV1 = r.r3;
  c.X = row_lin_a_2b(MM1, X1V1, k);
  // round E: (M1 X1) V1, M1 M1^2, X2^2 (row 3 repeats row 2)
  r = row_round(k, M1X1, M1, c.X, c.X, V1, MM1, c.X, c.X);
  c.U = row_lin_6a_2b_c(r.r0, r.r1, VV1, k);
  c.M = row_lin_3a(r.r2, k);
}

__device__ __forceinline__ void row_chain_dbl1(rchain& c, row_consts& k) {
  row4 r = row_round(k, c.U, c.M, c.M, c.z, c.U, c.X, c.M, c.U);
  const uint32_t V = r.r0, MX = r.r1, MM = r.r2;
  c.z = r.r3;
  r = row_round(k, c.X, MX, c.M, V, V, V, MM, V);
  const uint32_t XV = r.r0, MXV = r.r1, M3 = r.r2, VV = r.r3;
  c.X = row_lin_a_2b(MM, XV, k);
  c.U = row_lin_6a_2b_c(MXV, M3, VV, k);
  c.M = row_lin_3a(row_mul_lazy(c.X, c.X, k), k);  // every row computes X'^2
}

}  // namespace msmk
