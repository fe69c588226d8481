// S affine additions that share one field inversion (Montgomery's trick).
//
// aztec-packages PR #23738 ("TL;DR") and PR #23736 ("Goal & lever") describe the
// bucket accumulate as S affine adds per batch with one inversion, so the
// inversion costs |inversion| / S per add. PR #23520 ("Summary") gives the three
// passes over the S slots: a forward pass that stores each slot's prefix product,
// one inversion, and a backward pass that peels one slot's inverse off the running
// inverse at a time. This is that batch for one gfx950 lane:
//
//   forward:  d_s = denominator of slot s, pref_s = d_0 * ... * d_s
//   invert:   inv = pref_{S-1}^{-1}
//   backward: for s = S-1 .. 0:  1/d_s = inv * pref_{s-1} (inv itself for s = 0),
//             then inv = inv * d_s; lambda = numerator_s / d_s; finish the add.
//
// Slot state is pref_s (8 words per slot), optionally d_s, and the operands' element
// indices; operands are re-read in the backward pass instead of being held. Where the
// prefix products live (private memory or LDS) is the Store policy below.
//
// Special cases (the pages only report that x-collisions break an affine add,
// PR #23736 "Correctness-harness fix"; the handling below is this library's):
//   A = inf -> B;  B = inf -> A;  x_A != x_B -> chord, d = x_B - x_A;
//   A == B -> tangent, d = 2 y_A, numerator 3 x_A^2;  A == -B -> inf.
// Every special slot uses d = 1, so the batch product is never zero (BN254 G1 has
// no point with y = 0).
#pragma once
#include "ec.hpp"

namespace msmk {

enum : int { ADD_CHORD = 0, ADD_A_INF = 1, ADD_B_INF = 2, ADD_TANGENT = 3, ADD_CANCEL = 4 };

__device__ __forceinline__ int add_case(const aff& A, const aff& B) {
  if (aff_is_inf(A)) return ADD_A_INF;
  if (aff_is_inf(B)) return ADD_B_INF;
  if (!fp_eq(A.x, B.x)) return ADD_CHORD;
  return fp_eq(A.y, B.y) ? ADD_TANGENT : ADD_CANCEL;
}

__device__ __forceinline__ fp add_denominator(const aff& A, const aff& B, int cs) {
  if (cs == ADD_CHORD) return fp_sub(B.x, A.x);
  if (cs == ADD_TANGENT) return fp_dbl(A.y);
  return fp_one();
}

// Product and square of a batch: inline, or as calls (OUTLINE, fp_mul_call).
template <bool OUTLINE>
__device__ __forceinline__ fp bmul(const fp& a, const fp& b) {
  if constexpr (OUTLINE) return fp_mul_call(a, b);
  else return fp_mul(a, b);
}
template <bool OUTLINE>
__device__ __forceinline__ fp bsqr(const fp& a) {
  if constexpr (OUTLINE) return fp_sqr_call(a);
  else return fp_sqr(a);
}

// Finish slot s once 1/d is known.
template <bool OUTLINE = false>
__device__ __forceinline__ aff add_finish(const aff& A, const aff& B, int cs, const fp& inv_d) {
  if (cs == ADD_A_INF) return B;
  if (cs == ADD_B_INF) return A;
  if (cs == ADD_CANCEL) return aff_inf();
  fp num;
  if (cs == ADD_CHORD) {
    num = fp_sub(B.y, A.y);
  } else {
    fp xx = bsqr<OUTLINE>(A.x);
    num = fp_add(fp_dbl(xx), xx);
  }
  fp lam = bmul<OUTLINE>(num, inv_d);
  aff r;
  r.x = fp_sub(fp_sub(bsqr<OUTLINE>(lam), A.x), B.x);
  r.y = fp_sub(bmul<OUTLINE>(lam, fp_sub(A.x, r.x)), A.y);
  return r;
}

// Where a batch keeps its slot state: the prefix products pref_s and, with DX (the
// cached-denominator option of PR #23520 "Summary"), each slot's denominator d_s so the
// backward pass need not form it again.
//   PrefPrivate: per-lane arrays, which the compiler places in private memory (scratch)
//                because the slot loops are too large to unroll;
//   PrefLds:     the block's LDS, word w of slot s of lane l at base[(8 s + w) lanes + l]
//                (lanes = threads per block), so the 64 lanes of a wavefront touch 64
//                consecutive words of one row: no bank conflicts.
template <int S, bool DX>
struct PrefPrivate {
  fp pref[S];
  fp dx[S];
  __device__ __forceinline__ fp get(int s) const { return pref[s]; }
  __device__ __forceinline__ void set(int s, const fp& v) { pref[s] = v; }
  __device__ __forceinline__ fp get_dx(int s) const { return dx[s]; }
  __device__ __forceinline__ void set_dx(int s, const fp& v) { dx[s] = v; }
};

template <int S>
struct PrefPrivate<S, false> {
  fp pref[S];
  __device__ __forceinline__ fp get(int s) const { return pref[s]; }
  __device__ __forceinline__ void set(int s, const fp& v) { pref[s] = v; }
  __device__ __forceinline__ fp get_dx(int) const { return fp_zero(); }  // not used
  __device__ __forceinline__ void set_dx(int, const fp&) {}
};

template <int S, bool DX>
struct PrefLds {
  uint32_t* base;  // the block's LDS: (DX ? 2 : 1) * 8 S words per lane
  uint32_t lanes, lane;
  __device__ __forceinline__ fp ld(int row) const {
    fp r;
#pragma unroll
    for (int w = 0; w < 8; w++) r.v[w] = base[(size_t)(8 * row + w) * lanes + lane];
    return r;
  }
  __device__ __forceinline__ void st(int row, const fp& v) const {
#pragma unroll
    for (int w = 0; w < 8; w++) base[(size_t)(8 * row + w) * lanes + lane] = v.v[w];
  }
  __device__ __forceinline__ fp get(int s) const { return ld(s); }
  __device__ __forceinline__ void set(int s, const fp& v) { st(s, v); }
  __device__ __forceinline__ fp get_dx(int s) const { return ld(S + s); }
  __device__ __forceinline__ void set_dx(int s, const fp& v) { st(S + s, v); }
};

// LDS bytes per lane of a PrefLds store.
constexpr uint32_t pref_lds_bytes(int S, bool DX) { return (DX ? 2u : 1u) * 32u * (uint32_t)S; }

// Src supplies: fp ax(int s), fp bx(int s) (x-coordinates only), aff a(int s),
// aff b(int s) (whole points), void put(int s, const aff&). Slots s >= cnt are idle
// (d = 1, nothing stored). The forward pass reads only the x-coordinates unless an x
// is 0 or the two x agree (infinity, tangent, cancel), which then loads the whole
// points.
template <int S, bool DX, bool OUTLINE = false, class Store, class Src>
__device__ __forceinline__ void batch_affine_add(Src& src, int cnt, Store& st) {
  fp acc = fp_one();
#pragma unroll
  for (int s = 0; s < S; s++) {
    if (s < cnt) {
      const fp xa = src.ax(s), xb = src.bx(s);
      fp d;
      if (!fp_eq(xa, xb) && !fp_is_zero(xa) && !fp_is_zero(xb)) {
        d = fp_sub(xb, xa);  // chord, the common case
      } else {
        const aff A = src.a(s), B = src.b(s);
        d = add_denominator(A, B, add_case(A, B));
      }
      if (DX) st.set_dx(s, d);
      acc = (s == 0) ? d : bmul<OUTLINE>(acc, d);
    }
    st.set(s, acc);
  }
  fp inv = fp_inv(acc);
#pragma unroll
  for (int s = S - 1; s >= 0; s--) {
    if (s < cnt) {
      const fp inv_d = (s > 0) ? bmul<OUTLINE>(inv, st.get(s - 1)) : inv;
      const aff A = src.a(s), B = src.b(s);
      const int cs = add_case(A, B);
      inv = bmul<OUTLINE>(inv, DX ? st.get_dx(s) : add_denominator(A, B, cs));
      src.put(s, add_finish<OUTLINE>(A, B, cs, inv_d));
    }
  }
}

// The same batch with checkpointed slot state: only the last prefix of every group of G
// slots is stored (S / G of them, in a store of that many rows), and the backward pass
// rebuilds a group's other prefixes, and its denominators, in registers from the
// previous group's checkpoint before peeling the group's inverses: G - 1 more products
// and G more denominators per group, for G times less stored state. The group's
// operands are re-read in the backward pass as in the plain batch.
template <int S, int G, class Store, class Src>
__device__ __forceinline__ void batch_affine_add_ckpt(Src& src, int cnt, Store& st) {
  static_assert(S % G == 0, "groups must tile the slots");
  auto denom = [&](int s) -> fp {
    const fp xa = src.ax(s), xb = src.bx(s);
    if (!fp_eq(xa, xb) && !fp_is_zero(xa) && !fp_is_zero(xb)) return fp_sub(xb, xa);
    const aff A = src.a(s), B = src.b(s);
    return add_denominator(A, B, add_case(A, B));
  };
  fp acc = fp_one();
#pragma unroll
  for (int s = 0; s < S; s++) {
    if (s < cnt) {
      const fp d = denom(s);
      acc = (s == 0) ? d : fp_mul(acc, d);
    }
    if (s % G == G - 1) st.set(s / G, acc);
  }
  fp inv = fp_inv(acc);
  static_assert(G == 4, "the group's registers are written out for four slots");
  for (int g = S / G - 1; g >= 0; g--) {
    if (G * g >= cnt) continue;
    const int s0 = G * g;
    // the group's denominators d0..d3 and prefixes p0..p2 (pref of slots s0 .. s0 + 2),
    // named registers: the compiler will not unroll a loop this large, and an indexed
    // array would go to private memory
    const fp base = (g > 0) ? st.get(g - 1) : fp_one();
    const fp d0 = denom(s0);
    const fp d1 = (s0 + 1 < cnt) ? denom(s0 + 1) : fp_one();
    const fp d2 = (s0 + 2 < cnt) ? denom(s0 + 2) : fp_one();
    const fp d3 = (s0 + 3 < cnt) ? denom(s0 + 3) : fp_one();
    const fp p0 = (g > 0) ? fp_mul(base, d0) : d0;
    const fp p1 = fp_mul(p0, d1);
    const fp p2 = fp_mul(p1, d2);
    auto peel = [&](int s, const fp& prev, const fp& d, bool first) {
      if (s < cnt) {
        const fp inv_d = first ? inv : fp_mul(inv, prev);
        const aff A = src.a(s), B = src.b(s);
        const int cs = add_case(A, B);
        inv = fp_mul(inv, d);
        src.put(s, add_finish(A, B, cs, inv_d));
      }
    };
    peel(s0 + 3, p2, d3, false);
    peel(s0 + 2, p1, d2, false);
    peel(s0 + 1, p0, d1, false);
    peel(s0, base, d0, g == 0);
  }
}

// The batch with its slot state in private memory.
template <int S, bool OUTLINE = false, class Src>
__device__ __forceinline__ void batch_affine_add(Src& src, int cnt) {
  PrefPrivate<S, false> st;
  batch_affine_add<S, false, OUTLINE>(src, cnt, st);
}

}  // namespace msmk
