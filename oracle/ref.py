"""Exact Python-integer reference for BN254 G1 arithmetic and multi-scalar multiplication.

TEST INFRASTRUCTURE ONLY. Nothing in the product package imports this module; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may.

What the pages fix (aztec-packages PR #23738 / #23736 / #23520, "bb/msm"): the
quantity is the multi-scalar multiplication Q = sum_i s_i * P_i over the curve
barretenberg uses, and a GPU result counts as correct when it is on the curve and
bit-identical to an independent implementation (PR #23736, "Correctness-harness fix"
and the real-hardware table). The pages never name the curve; BN254 / alt_bn128 is
the curve barretenberg uses, with constants from Ethereum's EIP-196.

Everything here is written with Python's arbitrary-precision ``int`` so that each
formula reads like the textbook one:

* field F_p with p the BN254 base-field prime; inverse by Fermat, x^(p-2);
* the short Weierstrass curve y^2 = x^3 + 3 in affine coordinates, the point at
  infinity written ``None``; addition by the chord-and-tangent rule;
* k*P by MSB-first double-and-add; Q by summing the per-term products, or by the
  closed form (sum_i s_i r_i mod r) * G when every P_i = r_i * G (linearity).

Montgomery form: the interchange format stores a coordinate x as x * 2^256 mod p in
eight little-endian 32-bit words; ``to_mont`` / ``from_mont`` convert.
"""
from __future__ import annotations

# EIP-196 (alt_bn128): base-field prime, group order, curve constant and generator.
P = 0x30644E72E131A029B85045B68181585D97816A916871CA8D3C208C16D87CFD47
R = 0x30644E72E131A029B85045B68181585D2833E84879B9709143E1F593F0000001
B = 3
G = (1, 2)
MONT_R = 1 << 256  # Montgomery radix used by the interchange format

INF = None  # the point at infinity


# ----------------------------------------------------------------------------- field
def fp_inv(a: int) -> int:
    """Inverse in F_p by Fermat's little theorem; a must be non-zero mod p."""
    a %= P
    if a == 0:
        raise ZeroDivisionError("inverse of 0 in F_p")
    return pow(a, P - 2, P)


def to_mont(x: int) -> int:
    return (x * MONT_R) % P


def from_mont(xm: int) -> int:
    return (xm * pow(MONT_R, -1, P)) % P


# ----------------------------------------------------------------------------- curve
def on_curve(pt) -> bool:
    if pt is None:
        return True
    x, y = pt
    if not (0 <= x < P and 0 <= y < P):
        return False
    return (y * y - x * x * x - B) % P == 0


def neg(pt):
    if pt is None:
        return None
    x, y = pt
    return (x, (-y) % P)


def add(p1, p2):
    """Chord-and-tangent addition on y^2 = x^3 + 3 (affine, all special cases)."""
    if p1 is None:
        return p2
    if p2 is None:
        return p1
    x1, y1 = p1
    x2, y2 = p2
    if x1 == x2:
        if (y1 + y2) % P == 0:
            return None  # P + (-P), which also covers y = 0 (absent on this curve)
        lam = (3 * x1 * x1) * fp_inv(2 * y1) % P  # tangent slope (curve a = 0)
    else:
        lam = (y2 - y1) * fp_inv(x2 - x1) % P  # chord slope
    x3 = (lam * lam - x1 - x2) % P
    y3 = (lam * (x1 - x3) - y1) % P
    return (x3, y3)


def dbl(pt):
    return add(pt, pt)


def scalar_mul(k: int, pt):
    """k * pt by MSB-first double-and-add; k is any non-negative integer."""
    if k < 0:
        raise ValueError("negative scalar")
    acc = None
    for bit in bin(k)[2:] if k else "":
        acc = dbl(acc)
        if bit == "1":
            acc = add(acc, pt)
    return acc


def repeated_add(k: int, pt):
    """k * pt as pt + pt + ... + pt (k terms): brute force for small k."""
    acc = None
    for _ in range(k):
        acc = add(acc, pt)
    return acc


# ----------------------------------------------------------------------------- MSM
def msm_naive(points, scalars):
    """Q = sum_i s_i * P_i, each term by double-and-add (the definition written out)."""
    acc = None
    for pt, s in zip(points, scalars):
        acc = add(acc, scalar_mul(s, pt))
    return acc


def msm_brute(points, scalars):
    """Q = sum_i s_i * P_i by repeated addition; only for tiny scalars."""
    acc = None
    for pt, s in zip(points, scalars):
        acc = add(acc, repeated_add(s, pt))
    return acc


def msm_linear(dlogs, scalars):
    """Closed form for P_i = r_i * G: Q = (sum_i s_i * r_i mod R) * G."""
    t = 0
    for r_i, s in zip(dlogs, scalars):
        t += int(r_i) * int(s)
    return scalar_mul(t % R, G)


def window_digits(s: int, c: int, nwin: int):
    """Unsigned c-bit windows from the least significant bit: s = sum_j d_j 2^(c j)."""
    mask = (1 << c) - 1
    return [(s >> (c * j)) & mask for j in range(nwin)]


def num_windows(c: int) -> int:
    """Number of c-bit windows covering a 254-bit scalar."""
    return -(-254 // c)


def msm_pippenger(points, scalars, c: int):
    """Bucket method, written plainly: per window, buckets by digit, running sum,
    then Horner over the windows. Used only as a cross-check on small inputs."""
    nwin = num_windows(c)
    windows = []
    for j in range(nwin):
        buckets = [None] * (1 << c)
        for pt, s in zip(points, scalars):
            d = (s >> (c * j)) & ((1 << c) - 1)
            if d:
                buckets[d] = add(buckets[d], pt)
        run = None
        total = None
        for b in range((1 << c) - 1, 0, -1):
            run = add(run, buckets[b])
            total = add(total, run)
        windows.append(total)
    q = None
    for j in range(nwin - 1, -1, -1):
        for _ in range(c):
            q = dbl(q)
        q = add(q, windows[j])
    return q


# ----------------------------------------------------------------------------- codec
def int_to_words(x: int, nwords: int = 8):
    return [(x >> (32 * i)) & 0xFFFFFFFF for i in range(nwords)]


def words_to_int(words) -> int:
    v = 0
    for i, w in enumerate(words):
        v |= int(w) << (32 * i)
    return v


def encode_point(pt):
    """Affine point -> 16 little-endian u32 words (x then y, Montgomery form);
    the point at infinity is all zeros."""
    if pt is None:
        return [0] * 16
    x, y = pt
    return int_to_words(to_mont(x)) + int_to_words(to_mont(y))


def decode_point(words):
    w = [int(v) for v in words]
    xm, ym = words_to_int(w[:8]), words_to_int(w[8:16])
    if xm == 0 and ym == 0:
        return None
    return (from_mont(xm), from_mont(ym))
