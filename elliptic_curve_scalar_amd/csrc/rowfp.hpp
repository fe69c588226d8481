// F_p arithmetic spread over the 16 lanes of a DPP row, for one wavefront's chains.
//
// The window combine's runs of doublings are a single wavefront's dependent chain of
// Montgomery products, and a lone wavefront issues at most one instruction per 4 cycles (8
// for a 64-bit-result multiply-add): the chain is as long as the instructions one lane
// executes, whatever the other lanes do. The quad form (quad.hpp) spreads a round's four
// products over four lanes but leaves each product whole in one lane (about 450
// instructions). Here each product is spread over one row of 16 lanes, and the four rows of
// the wavefront compute a round's four products at once.
//
// Row form: lane l of a row (l = lane mod 16) holds word l of an element for l < 8 (eight
// little-endian 32-bit words, Montgomery form with R = 2^256, fully reduced) and 0 for
// l >= 8. A product a b R^-1 mod p is separated operand scanning in three passes, lane l
// summing column l of each:
//   T = a b                     (16 columns),
//   m = (T mod 2^256) n' mod 2^256,   n' = -p^-1 mod 2^256   (columns 0..7),
//   U = T + m p                 (U = 0 mod 2^256, U / 2^256 < 2p),
// each pass followed by one carry resolution across the row, and the result is U / 2^256
// (lanes 8..15 moved down to 0..7) less p when it is not below p. Every column sums at
// most eight 32 x 16-bit products per half (one operand split into 16-bit halves), so
// the 64-bit multiply-add accumulators never overflow and need no carry instructions.
//
// Carry resolution: a row's words w_l with carry bits h_l (carry out of lane l) give the
// generate mask G = {l : h_l} and the propagate mask P = {l : w_l = 2^32 - 1}; the carry
// into each lane is ((G << 1) + P) xor P, one 64-bit scalar addition for the four rows
// (the lane-0 and lane-15 bits are masked so that no carry crosses rows). Lanes read their
// bit of the mask back with an inverse ballot.
//
// Every function here must be called with the whole wavefront active (ballots).
#pragma once
#include "fp.hpp"

namespace msmk {

template <int I>
struct row_ic {
  static constexpr int value = I;
};

template <int I, int N, class F>
__device__ __forceinline__ void row_for(F&& f) {
  if constexpr (I < N) {
    f(row_ic<I>{});
    row_for<I + 1, N>(f);
  }
}

// Lane I of this lane's row, on every lane of the row (DPP row_newbcast).
template <int I>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150 + I, 0xf, 0xf, false);
}

// Lane l - I of this lane's row, 0 for l < I (DPP row_shr, bound_ctrl: zero fill).
template <int I>
__device__ __forceinline__ uint32_t row_shr(uint32_t x) {
  if constexpr (I == 0) {
    return x;
  } else {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x110 + I, 0xf, 0xf, true);
  }
}

// Lane l + I of this lane's row, 0 for l + I >= 16 (DPP row_shl, zero fill).
template <int I>
__device__ __forceinline__ uint32_t row_shl(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x100 + I, 0xf, 0xf, true);
}

__device__ __forceinline__ bool row_lane_bit(uint64_t mask) {
  return __builtin_amdgcn_inverse_ballot_w64(mask);
}

// Lane masks of a < b and a == b (v_cmp straight into a scalar register pair).
__device__ __forceinline__ uint64_t row_lt(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_uicmp(a, b, 36);  // unsigned less-than
}
__device__ __forceinline__ uint64_t row_eq(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_uicmp(a, b, 32);  // equal
}

// Lane masks of the four rows of a wavefront.
constexpr uint64_t ROW_L0 = 0x0001000100010001ull;     // lane 0 of each row
constexpr uint64_t ROW_L7 = 0x0080008000800080ull;     // lane 7
constexpr uint64_t ROW_L15 = 0x8000800080008000ull;    // lane 15
constexpr uint64_t ROW_LO8 = 0x00ff00ff00ff00ffull;    // lanes 0..7
constexpr uint64_t ROW_LO7 = 0x007f007f007f007full;    // lanes 0..6

// Per-lane constants of the row arithmetic: for lane l and shift i, the 16-bit halves of
// word l - i of p and of n' (0 where l - i is outside 0..7), and word l of p (0 for l >= 8).
struct row_consts {
  uint32_t pl[8], ph[8], nl[8], nh[8];
  uint32_t plo;
  uint32_t m0, m1;  // all ones where bit 0 / bit 1 of the row index is set
  // lanes 0..7 (0 above): words of 6 p - (2^256 - 1), 11 p - 2 (2^256 - 1),
  // 16 p - 3 (2^256 - 1) and 2^256 - p, and a mask of all ones
  uint32_t c1, c2, c3, negp, lo8;
};

// p and n' = -p^-1 mod 2^256, each between eight zero words on either side so that word
// l - i is entry 8 + l - i for every l in 0..15 and i in 0..7.
__device__ const uint32_t kRowP[24] = {
    0, 0, 0, 0, 0, 0, 0, 0,
    MSM_P0, MSM_P1, MSM_P2, MSM_P3, MSM_P4, MSM_P5, MSM_P6, MSM_P7,
    0, 0, 0, 0, 0, 0, 0, 0};
__device__ const uint32_t kRowNp[24] = {
    0, 0, 0, 0, 0, 0, 0, 0,
    0xe4866389u, 0x87d20782u, 0x1eca6ac9u, 0x9ede7d65u,
    0x1833da80u, 0xd8afcbd0u, 0x91888c6bu, 0xf57a22b7u,
    0, 0, 0, 0, 0, 0, 0, 0};

// Offsets of the linear combinations (row_lin_* below) and 2^256 - p, then eight zero
// words, so that lane l reads entry l.
__device__ const uint32_t kRowC1[16] = {
    0x12edefabu, 0x68c34889u, 0x72aabf4fu, 0x8d087f68u,
    0x09081231u, 0x51e1a247u, 0x4729c0fau, 0x2259d6b1u, 0, 0, 0, 0, 0, 0, 0, 0};
__device__ const uint32_t kRowC2[16] = {
    0x4d5ee20fu, 0x956604fbu, 0x7ce3b411u, 0x828f943fu,
    0x908ecc05u, 0xeb72fed7u, 0xad21e1cau, 0x144f5eefu, 0, 0, 0, 0, 0, 0, 0, 0};
__device__ const uint32_t kRowC3[16] = {
    0x87cfd473u, 0xc208c16du, 0x871ca8d3u, 0x7816a916u,
    0x181585d9u, 0x85045b68u, 0x131a029bu, 0x0644e72eu, 0, 0, 0, 0, 0, 0, 0, 0};
__device__ const uint32_t kRowNegP[16] = {
    0x278302b9u, 0xc3df73e9u, 0x978e3572u, 0x687e956eu,
    0x7e7ea7a2u, 0x47afba49u, 0x1ece5fd6u, 0xcf9bb18du, 0, 0, 0, 0, 0, 0, 0, 0};

__device__ __forceinline__ row_consts row_consts_load() {
  const uint32_t lane = __lane_id(), l = lane & 15u;
  row_consts k;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const uint32_t pw = kRowP[8 + l - i], nw = kRowNp[8 + l - i];
    k.pl[i] = pw & 0xffffu;
    k.ph[i] = pw >> 16;
    k.nl[i] = nw & 0xffffu;
    k.nh[i] = nw >> 16;
  }
  k.plo = kRowP[8 + l] * (l < 8 ? 1u : 0u);
  k.m0 = ((lane >> 4) & 1u) ? 0xffffffffu : 0u;
  k.m1 = ((lane >> 5) & 1u) ? 0xffffffffu : 0u;
  k.c1 = kRowC1[l];
  k.c2 = kRowC2[l];
  k.c3 = kRowC3[l];
  k.negp = kRowNegP[l];
  k.lo8 = l < 8 ? 0xffffffffu : 0u;
  return k;
}

// Marks the constants as redefined here (no instruction): the optimizer would otherwise
// hoist their 64-bit widening out of the loops that use them, and a product by a widened
// value that arrives from another block takes three multiply-adds instead of one.
__device__ __forceinline__ void row_consts_here(row_consts& k) {
  asm volatile("" : "+v"(k.pl[0]), "+v"(k.pl[1]), "+v"(k.pl[2]), "+v"(k.pl[3]), "+v"(k.pl[4]),
               "+v"(k.pl[5]), "+v"(k.pl[6]), "+v"(k.pl[7]), "+v"(k.ph[0]), "+v"(k.ph[1]),
               "+v"(k.ph[2]), "+v"(k.ph[3]), "+v"(k.ph[4]), "+v"(k.ph[5]), "+v"(k.ph[6]),
               "+v"(k.ph[7]), "+v"(k.negp));
  asm volatile("" : "+v"(k.nl[0]), "+v"(k.nl[1]), "+v"(k.nl[2]), "+v"(k.nl[3]), "+v"(k.nl[4]),
               "+v"(k.nl[5]), "+v"(k.nl[6]), "+v"(k.nl[7]), "+v"(k.nh[0]), "+v"(k.nh[1]),
               "+v"(k.nh[2]), "+v"(k.nh[3]), "+v"(k.nh[4]), "+v"(k.nh[5]), "+v"(k.nh[6]),
               "+v"(k.nh[7]));
}

// Words w_l plus the carries that reach them: G holds the lanes with a carry out. No
// carry leaves lane 15 (callers guarantee it by the value's bound).
__device__ __forceinline__ uint32_t row_carry16(uint32_t w, uint64_t G) {
  const uint64_t P = row_eq(w, 0xffffffffu) & ~ROW_L15;
  const uint64_t C = (((G << 1) & ~ROW_L0) + P) ^ P;
  return w + (row_lane_bit(C) ? 1u : 0u);
}

// Column l holds SL_l + 2^16 SH_l (SL, SH < 2^52): the row's value sum_l col_l 2^(32 l) as
// words, lane l word l. A column is c0 + 2^32 c1 + 2^64 c2 (c2 <= 8); lane l adds c0_l,
// c1_(l-1) and c2_(l-2) (carry g <= 2), then g_(l-1) (carry h <= 1), then the rippled
// carries.
__device__ __forceinline__ uint32_t row_columns(uint64_t SL, uint64_t SH) {
  // opaque to the optimizer: otherwise it may fold SL + 2^16 SH back into the sums as one
  // 64 x 32-bit product per term (three multiply-adds per term instead of two)
  asm("" : "+v"(SL), "+v"(SH));
  const uint64_t x = SL + (SH << 16);
  const uint32_t c2 = (uint32_t)(SH >> 48) + (x < SL ? 1u : 0u);
  const uint32_t c0 = (uint32_t)x, c1s = row_shr<1>((uint32_t)(x >> 32)), c2s = row_shr<2>(c2);
  const uint32_t t1 = c0 + c1s;
  const uint32_t t2 = t1 + c2s;
  const uint32_t g = (t1 < c1s ? 1u : 0u) + (t2 < c2s ? 1u : 0u);
  const uint32_t gs = row_shr<1>(g);
  const uint32_t w = t2 + gs;
  return row_carry16(w, row_lt(w, gs));
}

// s - p if s >= p, for s < 2p in lanes 0..7 (0 in lanes 8..15).
__device__ __forceinline__ uint32_t row_sub_p_if_ge(uint32_t s, row_consts& k) {
  const uint32_t d = s - k.plo;
  const uint64_t G = row_lt(s, k.plo) & ROW_LO8;
  const uint64_t Pf = row_eq(d, 0u) & ROW_LO8;
  const uint64_t P = Pf & ROW_LO7;
  const uint64_t C = ((((G << 1) & ~ROW_L0) + P) ^ P) & ROW_LO8;  // borrow into each lane
  const uint64_t x = ((G | (Pf & C)) & ROW_L7) >> 7;             // rows with s < p
  const uint64_t keep = (x << 16) - x;
  const uint32_t dd = d - (row_lane_bit(C) ? 1u : 0u);
  return row_lane_bit(keep) ? s : dd;
}

// a + b mod p.
__device__ __forceinline__ uint32_t row_add(uint32_t a, uint32_t b, row_consts& k) {
  const uint32_t s = a + b;
  // a + b < 2p < 2^255: no carry leaves lane 7, and lanes 8..15 stay 0
  return row_sub_p_if_ge(row_carry16(s, row_lt(s, b)), k);
}

__device__ __forceinline__ uint32_t row_dbl(uint32_t a, row_consts& k) { return row_add(a, a, k); }
__device__ __forceinline__ uint32_t row_triple(uint32_t a, row_consts& k) {
  return row_add(row_add(a, a, k), a, k);
}

// a - b mod p.
__device__ __forceinline__ uint32_t row_sub(uint32_t a, uint32_t b, row_consts& k) {
  uint32_t d = a - b;
  const uint64_t G = row_lt(a, b) & ROW_LO8;
  const uint64_t Pf = row_eq(d, 0u) & ROW_LO8;
  const uint64_t P = Pf & ROW_LO7;
  const uint64_t C = ((((G << 1) & ~ROW_L0) + P) ^ P) & ROW_LO8;
  const uint64_t x = ((G | (Pf & C)) & ROW_L7) >> 7;  // rows with a < b
  const uint64_t neg = (x << 16) - x;
  d -= row_lane_bit(C) ? 1u : 0u;
  // a < b: d = a - b + 2^256 in lanes 0..7; add p, dropping the carry out of lane 7
  const uint32_t pa = row_lane_bit(neg) ? k.plo : 0u;
  const uint32_t e = d + pa;
  const uint64_t G2 = row_lt(e, pa) & ROW_LO8;
  const uint64_t P2 = row_eq(e, 0xffffffffu) & ROW_LO7;
  const uint64_t C2 = ((((G2 << 1) & ~ROW_L0) + P2) ^ P2) & ROW_LO8;
  return e + (row_lane_bit(C2) ? 1u : 0u);
}

// Montgomery product without the final subtraction: U / 2^256 for a, b < 3p, which is
// below 9 p^2 / 2^256 + p < 2.71 p (p < 0.19 * 2^256), so the lazy form [0, 3p) is closed
// under it. With a, b < p it is below 2p.
__device__ __forceinline__ uint32_t row_mul_lazy(uint32_t a, uint32_t b, row_consts& k);

// Montgomery product a b 2^-256 mod p of two row-form elements.
__device__ __forceinline__ uint32_t row_mul(uint32_t a, uint32_t b, row_consts& k) {
  return row_sub_p_if_ge(row_mul_lazy(a, b, k), k);
}

__device__ __forceinline__ uint32_t row_mul_lazy(uint32_t a, uint32_t b, row_consts& k) {
  row_consts_here(k);
  const uint32_t bl = b & 0xffffu, bh = b >> 16;
  uint64_t SL = 0, SH = 0;
  row_for<0, 8>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const uint32_t ai = row_bcast<i>(a);
    SL += (uint64_t)ai * row_shr<i>(bl);
    SH += (uint64_t)ai * row_shr<i>(bh);
  });
  const uint32_t T = row_columns(SL, SH);
  SL = 0;
  SH = 0;
  row_for<0, 8>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const uint32_t ti = row_bcast<i>(T);
    SL += (uint64_t)ti * k.nl[i];
    SH += (uint64_t)ti * k.nh[i];
  });
  const uint32_t m = row_columns(SL, SH);  // lanes 0..7: m; lanes 8..15 are never read
  SL = T;
  SH = 0;
  row_for<0, 8>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const uint32_t mi = row_bcast<i>(m);
    SL += (uint64_t)mi * k.pl[i];
    SH += (uint64_t)mi * k.ph[i];
  });
  const uint32_t U = row_columns(SL, SH);  // lanes 0..7: 0; lanes 8..15: U / 2^256
  return row_shl<8>(U);
}

// ---- linear combinations in the lazy form [0, 3p) ---------------------------------------
// A small combination of lazy elements, ka a - kb b - kc c, is formed per lane as the column
// ka a_l + kb ~b_l + kc ~c_l + C_l, where ~ is the word-wise complement (2^32 - 1 - w) and
// C = K p - (kb + kc)(2^256 - 1) >= 0 makes the whole value V = ka a - kb b - kc c + K p
// non-negative and below 2^259 (lanes 0..8). Then q ~ V / p is estimated from V's top 64 bits
// and V - q p (formed as V + q (2^256 - p) mod 2^256) is the result. The estimate is never
// above floor(V / p) and at most 2 below it, so the result lies in [0, 3p).

// Words (lanes 0..8) of sum_l x_l 2^(32 l), x_l < 2^38 given in lanes 0..7.
__device__ __forceinline__ uint32_t row_resolve(uint64_t x) {
  const uint32_t c1s = row_shr<1>((uint32_t)(x >> 32));
  const uint32_t w = (uint32_t)x + c1s;
  return row_carry16(w, row_lt(w, c1s));
}

// V - q p in [0, 3p) for V < 2^259 in lanes 0..8 with V = r (mod p). q = floor of
// (V >> 224) times a float just below 1 / (p_7 + 1) (p_7 = p >> 224): the float error
// (below 2^-21 relative) is smaller than the factor's margin (2^-18), so q <= V / p, and
// q is at least floor(V / p) - 2 because V / p < 35.
__device__ __forceinline__ uint32_t row_reduce_q(uint32_t V, row_consts& k) {
  const float top = (float)row_bcast<8>(V) * 0x1.52917cp+2f + (float)row_bcast<7>(V) * 0x1.52917cp-30f;
  const uint32_t q = (uint32_t)top;
  const uint64_t y = (uint64_t)q * k.negp + (V & k.lo8);
  return row_resolve(y) & k.lo8;  // mod 2^256: what reaches lane 8 is dropped
}

// a - 2b, b < 3p, via 11 p - 2 (2^256 - 1).
__device__ __forceinline__ uint32_t row_lin_a_2b(uint32_t a, uint32_t b, row_consts& k) {
  const uint64_t x = (uint64_t)(~b & k.lo8) * 2u + a + k.c2;
  return row_reduce_q(row_resolve(x), k);
}

// 6a - 2b - c, via 16 p - 3 (2^256 - 1).
__device__ __forceinline__ uint32_t row_lin_6a_2b_c(uint32_t a, uint32_t b, uint32_t c,
                                                    row_consts& k) {
  const uint64_t x = (uint64_t)a * 6u + (uint64_t)(~b & k.lo8) * 2u + (~c & k.lo8) + k.c3;
  return row_reduce_q(row_resolve(x), k);
}

// 3a.
__device__ __forceinline__ uint32_t row_lin_3a(uint32_t a, row_consts& k) {
  return row_reduce_q(row_resolve((uint64_t)a * 3u), k);
}

// 2a.
__device__ __forceinline__ uint32_t row_lin_2a(uint32_t a, row_consts& k) {
  return row_reduce_q(row_resolve((uint64_t)a * 2u), k);
}

// a - b, via 6 p - (2^256 - 1).
__device__ __forceinline__ uint32_t row_lin_a_b(uint32_t a, uint32_t b, row_consts& k) {
  const uint64_t x = (uint64_t)(~b & k.lo8) + a + k.c1;
  return row_reduce_q(row_resolve(x), k);
}

// a - b - 2c, via 16 p - 3 (2^256 - 1).
__device__ __forceinline__ uint32_t row_lin_a_b_2c(uint32_t a, uint32_t b, uint32_t c,
                                                   row_consts& k) {
  const uint64_t x = (uint64_t)(~b & k.lo8) + (uint64_t)(~c & k.lo8) * 2u + a + k.c3;
  return row_reduce_q(row_resolve(x), k);
}

// a / 2 mod p in [0, 2p) for a < 3p: (a + p) / 2 when a is odd, a / 2 when even.
__device__ __forceinline__ uint32_t row_half(uint32_t a, row_consts& k) {
  const uint32_t add = (row_bcast<0>(a) & 1u) ? k.plo : 0u;
  uint32_t s = a + add;
  s = row_carry16(s, row_lt(s, add));  // a + p < 4p < 2^256: no carry leaves lane 7
  return (s >> 1) | (row_shl<1>(s) << 31);
}

// True when the element is 0 on every row (all four rows hold the same fully reduced
// element, or the whole wavefront tests one element).
__device__ __forceinline__ bool row_all_zero(uint32_t a) { return row_eq(a, 0u) == ~0ull; }

// The fully reduced element of a lazy one (< 3p).
__device__ __forceinline__ uint32_t row_canon(uint32_t a, row_consts& k) {
  return row_sub_p_if_ge(row_sub_p_if_ge(a, k), k);
}

// Operand of this row: a0 on row 0, a1 on row 1, ...
__device__ __forceinline__ uint32_t row_pick(row_consts& k, uint32_t a0, uint32_t a1,
                                             uint32_t a2, uint32_t a3) {
  const uint32_t lo = (a1 & k.m0) | (a0 & ~k.m0), hi = (a3 & k.m0) | (a2 & ~k.m0);
  return (hi & k.m1) | (lo & ~k.m1);
}

// Row r's value of x on every row: r0 from row 0, ..., r3 from row 3.
struct row4 {
  uint32_t r0, r1, r2, r3;
};

__device__ __forceinline__ row4 row_gather(uint32_t x) {
  // permlane16_swap exchanges the odd rows of its first operand with the even rows of its
  // second; permlane32_swap the upper half of the first with the lower half of the second
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);  // [0 0 2 2], [1 1 3 3]
  const auto b = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);  // [0 0 0 0], [2 2 2 2]
  const auto c = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);  // [1 1 1 1], [3 3 3 3]
  return row4{b[0], c[0], b[1], c[1]};
}

// Conversions between the per-lane form (every lane holds all eight words) and row form.
__device__ __forceinline__ uint32_t row_from_fp(const fp& a) {
  const uint32_t l = __lane_id() & 15u;
  const uint32_t s0 = (l & 1u) ? 0xffffffffu : 0u, s1 = (l & 2u) ? 0xffffffffu : 0u,
                 s2 = (l & 4u) ? 0xffffffffu : 0u;
  const uint32_t w01 = (a.v[1] & s0) | (a.v[0] & ~s0), w23 = (a.v[3] & s0) | (a.v[2] & ~s0);
  const uint32_t w45 = (a.v[5] & s0) | (a.v[4] & ~s0), w67 = (a.v[7] & s0) | (a.v[6] & ~s0);
  const uint32_t w03 = (w23 & s1) | (w01 & ~s1), w47 = (w67 & s1) | (w45 & ~s1);
  const uint32_t w = (w47 & s2) | (w03 & ~s2);
  return l < 8u ? w : 0u;
}

__device__ __forceinline__ fp row_to_fp(uint32_t w) {
  fp r;
  row_for<0, 8>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    r.v[i] = row_bcast<i>(w);
  });
  return r;
}

}  // namespace msmk
