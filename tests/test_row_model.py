"""A lane-exact model, on Python integers, of the row-form field arithmetic (rowfp.hpp):
a product spread over the 16 lanes of a row by separated operand scanning (T = a b,
m = T n' mod 2^256, U = T + m p, result U / 2^256 less p when not below p), with one
carry resolution per pass done by lane masks ((G << 1) + P) xor P on the wavefront's 64
lanes. Checked against a * b * 2^-256 mod p, a + b and a - b mod p on random values and on
the words that make carries ripple the whole row; and the header's table of
n' = -p^-1 mod 2^256 against its definition.

The model follows the kernel's steps (what each lane holds after each step) but shares no
code with it; it pins the algorithm, its bounds (no accumulator overflows, no carry leaves
a row) and the carry-resolution formula.
"""
import os
import random
import re

from oracle import ref

P = ref.P
R = 1 << 256
M32 = (1 << 32) - 1
M64 = (1 << 64) - 1
NP = (-pow(P, -1, R)) % R
ROW_L0, ROW_L7, ROW_L15 = 0x0001000100010001, 0x0080008000800080, 0x8000800080008000
ROW_LO8, ROW_LO7 = 0x00FF00FF00FF00FF, 0x007F007F007F007F
HERE = os.path.dirname(os.path.abspath(__file__))
ROWFP = os.path.join(HERE, "..", "elliptic_curve_scalar_amd", "csrc", "rowfp.hpp")


def word(x, i):
    return (x >> (32 * i)) & M32 if 0 <= i < 8 else 0


# ---- lane operations (a wavefront is a list of 64 values) ----------------------------
def shr(v, k):   # lane l of each row takes lane l - k of its row, 0 below
    return [v[i - k] if (i & 15) >= k else 0 for i in range(64)]


def shl(v, k):   # lane l takes lane l + k, 0 at and above 16 - k
    return [v[i + k] if (i & 15) + k < 16 else 0 for i in range(64)]


def bcast(v, k):  # lane k of each row, on the whole row
    return [v[(i & ~15) + k] for i in range(64)]


def ballot(pred):
    return sum(1 << i for i, b in enumerate(pred) if b)


def lane_bit(mask):
    return [(mask >> i) & 1 for i in range(64)]


def carry16(w, h):
    G, Pm = ballot(h), ballot(x == M32 for x in w) & ~ROW_L15 & M64
    C = ((((G << 1) & ~ROW_L0 & M64) + Pm) ^ Pm) & M64
    return [(x + b) & M32 for x, b in zip(w, lane_bit(C))]


def columns(SL, SH):
    assert all(x < 1 << 52 for x in SL + SH)   # the multiply-add accumulators never wrap
    x = [(a + ((b << 16) & M64)) & M64 for a, b in zip(SL, SH)]
    c2 = [(b >> 48) + (1 if xx < a else 0) for a, b, xx in zip(SL, SH, x)]
    c0 = [xx & M32 for xx in x]
    c1s, c2s = shr([xx >> 32 for xx in x], 1), shr(c2, 2)
    t1 = [(a + b) & M32 for a, b in zip(c0, c1s)]
    t2 = [(a + b) & M32 for a, b in zip(t1, c2s)]
    g = [(1 if a < b else 0) + (1 if c < d else 0) for a, b, c, d in zip(t1, c1s, t2, c2s)]
    gs = shr(g, 1)
    w = [(a + b) & M32 for a, b in zip(t2, gs)]
    return carry16(w, [a < b for a, b in zip(w, gs)])


def sub_p_if_ge(s, plo):
    d = [(a - b) & M32 for a, b in zip(s, plo)]
    G = ballot(a < b for a, b in zip(s, plo)) & ROW_LO8
    Pf = ballot(x == 0 for x in d) & ROW_LO8
    Pm = Pf & ROW_LO7
    C = ((((G << 1) & ~ROW_L0 & M64) + Pm) ^ Pm) & ROW_LO8
    x = ((G | (Pf & C)) & ROW_L7) >> 7
    keep = ((x << 16) - x) & M64
    dd = [(a - b) & M32 for a, b in zip(d, lane_bit(C))]
    return [a if k else b for a, b, k in zip(s, dd, lane_bit(keep))]


def consts():
    lanes = range(64)
    pl = [[word(P, (i & 15) - k) & 0xFFFF for i in lanes] for k in range(8)]
    ph = [[word(P, (i & 15) - k) >> 16 for i in lanes] for k in range(8)]
    nl = [[word(NP, (i & 15) - k) & 0xFFFF for i in lanes] for k in range(8)]
    nh = [[word(NP, (i & 15) - k) >> 16 for i in lanes] for k in range(8)]
    plo = [word(P, i & 15) if (i & 15) < 8 else 0 for i in lanes]
    return pl, ph, nl, nh, plo


K = consts()


def row_mul(a, b):
    pl, ph, nl, nh, plo = K
    bl, bh = [x & 0xFFFF for x in b], [x >> 16 for x in b]
    SL, SH = [0] * 64, [0] * 64
    for i in range(8):
        ai = bcast(a, i)
        SL = [s + x * y for s, x, y in zip(SL, ai, shr(bl, i))]
        SH = [s + x * y for s, x, y in zip(SH, ai, shr(bh, i))]
    T = columns(SL, SH)
    SL, SH = [0] * 64, [0] * 64
    for i in range(8):
        ti = bcast(T, i)
        SL = [s + x * y for s, x, y in zip(SL, ti, nl[i])]
        SH = [s + x * y for s, x, y in zip(SH, ti, nh[i])]
    m = columns(SL, SH)
    SL, SH = list(T), [0] * 64
    for i in range(8):
        mi = bcast(m, i)
        SL = [s + x * y for s, x, y in zip(SL, mi, pl[i])]
        SH = [s + x * y for s, x, y in zip(SH, mi, ph[i])]
    U = columns(SL, SH)
    for r in range(4):
        assert U[16 * r: 16 * r + 8] == [0] * 8  # U = 0 mod 2^256
    return sub_p_if_ge(shl(U, 8), plo)


# ---- lazy form [0, 3p) and linear combinations -----------------------------------------
C1 = 6 * P - (R - 1)
C2 = 11 * P - 2 * (R - 1)
C3 = 16 * P - 3 * (R - 1)
NEGP = R - P
P7 = P >> 224


def lane_words(x):
    return [word(x, i & 15) if (i & 15) < 8 else 0 for i in range(64)]


def row_mul_lazy(a, b):
    pl, ph, nl, nh, plo = K
    bl, bh = [x & 0xFFFF for x in b], [x >> 16 for x in b]
    SL, SH = [0] * 64, [0] * 64
    for i in range(8):
        ai = bcast(a, i)
        SL = [s + x * y for s, x, y in zip(SL, ai, shr(bl, i))]
        SH = [s + x * y for s, x, y in zip(SH, ai, shr(bh, i))]
    T = columns(SL, SH)
    SL, SH = [0] * 64, [0] * 64
    for i in range(8):
        ti = bcast(T, i)
        SL = [s + x * y for s, x, y in zip(SL, ti, nl[i])]
        SH = [s + x * y for s, x, y in zip(SH, ti, nh[i])]
    m = columns(SL, SH)
    SL, SH = list(T), [0] * 64
    for i in range(8):
        mi = bcast(m, i)
        SL = [s + x * y for s, x, y in zip(SL, mi, pl[i])]
        SH = [s + x * y for s, x, y in zip(SH, mi, ph[i])]
    return shl(columns(SL, SH), 8)


def resolve(x):
    assert all(v < 1 << 38 for v in x)  # c0 + c1 of the lane below carries at most 1
    c1s = shr([v >> 32 for v in x], 1)
    w = [((v & M32) + c) & M32 for v, c in zip(x, c1s)]
    return carry16(w, [u < c for u, c in zip(w, c1s)])


def reduce_q(V, q_shift=0):
    """V - q p with q estimated from V's top 64 bits (the kernel's float estimate is never
    above floor((V >> 224) / (p_7 + 1)) and at most one below it; q_shift = 1 takes that
    lower end)."""
    lo8 = lane_words(R - 1)
    out = []
    for r in range(4):
        top = (V[16 * r + 8] << 32) | V[16 * r + 7]
        q = max(0, top // (P7 + 1) - q_shift)
        out += [q] * 16
    y = [q * n + (v & m) for q, n, v, m in zip(out, lane_words(NEGP), V, lo8)]
    return [w & m for w, m in zip(resolve(y), lo8)]


def lin_a_2b(a, b, q_shift=0):
    lo8 = lane_words(R - 1)
    x = [2 * ((~v & M32) & m) + u + c for u, v, m, c in zip(a, b, lo8, lane_words(C2))]
    return reduce_q(resolve(x), q_shift)


def lin_6a_2b_c(a, b, c, q_shift=0):
    lo8 = lane_words(R - 1)
    x = [6 * u + 2 * ((~v & M32) & m) + ((~w & M32) & m) + k
         for u, v, w, m, k in zip(a, b, c, lo8, lane_words(C3))]
    return reduce_q(resolve(x), q_shift)


def lin_3a(a, q_shift=0):
    return reduce_q(resolve([3 * u for u in a]), q_shift)


def lin_2a(a, q_shift=0):
    return reduce_q(resolve([2 * u for u in a]), q_shift)


def lin_a_b(a, b, q_shift=0):
    lo8 = lane_words(R - 1)
    x = [((~v & M32) & m) + u + c for u, v, m, c in zip(a, b, lo8, lane_words(C1))]
    return reduce_q(resolve(x), q_shift)


def lin_a_b_2c(a, b, c, q_shift=0):
    lo8 = lane_words(R - 1)
    x = [((~v & M32) & m) + 2 * ((~w & M32) & m) + u + k
         for u, v, w, m, k in zip(a, b, c, lo8, lane_words(C3))]
    return reduce_q(resolve(x), q_shift)


def row_half(a):
    """The kernel's a / 2 mod p: add p (lane l word l) when lane 0's word is odd, carry,
    then shift the row right by one bit (lane l takes bit 0 of lane l + 1 as its bit 31)."""
    plo = K[4]
    out = []
    for r in range(4):
        row = a[16 * r:16 * r + 16]
        add = plo[16 * r:16 * r + 16] if row[0] & 1 else [0] * 16
        s = [(x + y) & M32 for x, y in zip(row, add)]
        s = carry16(s + [0] * 48, [x < y for x, y in zip(s, add)] + [False] * 48)[:16]
        out += [(s[l] >> 1) | (((s[l + 1] if l < 15 else 0) << 31) & M32) for l in range(16)]
    return out


def row_add(a, b):
    s = [(x + y) & M32 for x, y in zip(a, b)]
    return sub_p_if_ge(carry16(s, [x < y for x, y in zip(s, b)]), K[4])


def row_sub(a, b):
    plo = K[4]
    d = [(x - y) & M32 for x, y in zip(a, b)]
    G = ballot(x < y for x, y in zip(a, b)) & ROW_LO8
    Pf = ballot(x == 0 for x in d) & ROW_LO8
    Pm = Pf & ROW_LO7
    C = ((((G << 1) & ~ROW_L0 & M64) + Pm) ^ Pm) & ROW_LO8
    x = ((G | (Pf & C)) & ROW_L7) >> 7
    neg = ((x << 16) - x) & M64
    d = [(u - v) & M32 for u, v in zip(d, lane_bit(C))]
    pa = [q if n else 0 for q, n in zip(plo, lane_bit(neg))]
    e = [(u + v) & M32 for u, v in zip(d, pa)]
    G2 = ballot(u < v for u, v in zip(e, pa)) & ROW_LO8
    P2 = ballot(u == M32 for u in e) & ROW_LO7
    C2 = ((((G2 << 1) & ~ROW_L0 & M64) + P2) ^ P2) & ROW_LO8
    return [(u + v) & M32 for u, v in zip(e, lane_bit(C2))]


# ---- packing: four elements, one per row ----------------------------------------------
def pack(xs):
    return [word(xs[i >> 4], i & 15) if (i & 15) < 8 else 0 for i in range(64)]


def unpack(v):
    for r in range(4):
        assert v[16 * r + 8: 16 * r + 16] == [0] * 8  # lanes 8..15 stay 0
    return [sum(v[16 * r + i] << (32 * i) for i in range(8)) for r in range(4)]


def _values(rng, n):
    edge = [0, 1, 2, P - 1, P - 2, (P - 1) // 2, (P + 1) // 2, R % P, (R * R) % P,
            (1 << 224) - 1, (1 << 253) % P, P - (1 << 32), (1 << 32) - 1]
    return edge + [rng.randrange(P) for _ in range(n)]


def test_n_prime_table_is_minus_p_inverse():
    src = open(ROWFP).read()
    body = src[src.index("kRowNp[24]"):]
    body = body[:body.index("};")]
    words = [int(w, 16) for w in re.findall(r"0x([0-9a-f]+)u", body)]
    assert len(words) == 8
    assert sum(w << (32 * i) for i, w in enumerate(words)) == NP
    assert (NP * P) % R == R - 1


def test_row_product_matches_montgomery_product():
    rng = random.Random(5)
    vals = _values(rng, 120)
    rinv = pow(R, -1, P)
    pairs = [(a, b) for a in vals[:13] for b in vals[:13]]
    pairs += [(rng.choice(vals), rng.choice(vals)) for _ in range(200)]
    for k in range(0, len(pairs), 4):
        chunk = (pairs[k:k + 4] + [(0, 0)] * 4)[:4]
        got = unpack(row_mul(pack([a for a, _ in chunk]), pack([b for _, b in chunk])))
        assert got == [a * b * rinv % P for a, b in chunk]


def test_row_add_sub_match_field_ops():
    rng = random.Random(6)
    vals = _values(rng, 60)
    pairs = [(a, b) for a in vals[:13] for b in vals[:13]]
    pairs += [(rng.choice(vals), rng.choice(vals)) for _ in range(100)]
    for k in range(0, len(pairs), 4):
        chunk = (pairs[k:k + 4] + [(0, 0)] * 4)[:4]
        A, B = pack([a for a, _ in chunk]), pack([b for _, b in chunk])
        assert unpack(row_add(A, B)) == [(a + b) % P for a, b in chunk]
        assert unpack(row_sub(A, B)) == [(a - b) % P for a, b in chunk]


def test_carry_resolution_ripples_a_whole_row():
    # w = 2^32 - 1 everywhere except a generated carry at lane 0: the carry ripples through
    # lanes 1..15, lane 15 does not pass it on, and the next row is untouched
    w = [M32] * 64
    h = [False] * 64
    h[0] = True
    w[0] = 5
    out = carry16(w, h)
    assert out[0] == 5 and out[1:16] == [0] * 15
    assert out[16:] == [M32] * 48


def test_lazy_form_closed_under_products_and_combinations():
    rng = random.Random(8)
    rinv = pow(R, -1, P)
    lazy = [0, 1, P - 1, P, P + 1, 2 * P - 1, 2 * P, 3 * P - 1, 3 * P - 2, 2 * P + (1 << 200)]
    lazy += [rng.randrange(3 * P) for _ in range(60)]
    for k in range(0, 64, 4):
        xs, ys, zs = lazy[k:k + 4], lazy[k + 4:k + 8], lazy[k + 8:k + 12]
        if len(zs) < 4:
            break
        A, B, Cv = pack(xs), pack(ys), pack(zs)
        got = unpack(row_mul_lazy(A, B))
        for g, x, y in zip(got, xs, ys):
            assert g < 3 * P and g % P == x * y * rinv % P
        for sh in (0, 1):
            for g, x, y in zip(unpack(lin_a_2b(A, B, sh)), xs, ys):
                assert g < 3 * P and g % P == (x - 2 * y) % P
            for g, x, y, z in zip(unpack(lin_6a_2b_c(A, B, Cv, sh)), xs, ys, zs):
                assert g < 3 * P and g % P == (6 * x - 2 * y - z) % P
            for g, x in zip(unpack(lin_3a(A, sh)), xs):
                assert g < 3 * P and g % P == 3 * x % P
            for g, x in zip(unpack(lin_2a(A, sh)), xs):
                assert g < 3 * P and g % P == 2 * x % P
            for g, x, y in zip(unpack(lin_a_b(A, B, sh)), xs, ys):
                assert g < 3 * P and g % P == (x - y) % P
            for g, x, y, z in zip(unpack(lin_a_b_2c(A, B, Cv, sh)), xs, ys, zs):
                assert g < 3 * P and g % P == (x - y - 2 * z) % P
        half = pow(2, -1, P)
        for g, x in zip(unpack(row_half(A)), xs):
            assert g < 2 * P and g % P == x * half % P


def test_lazy_offsets_and_estimate_bounds():
    assert C1 >= 0 and C2 >= 0 and C3 >= 0
    assert C1 == 6 * P - (R - 1) and C2 == 11 * P - 2 * (R - 1) and C3 == 16 * P - 3 * (R - 1)
    # the largest combination stays below 2^259 (lanes 0..8) and below 35 p
    assert 6 * 3 * P + 2 * (R - 1) + (R - 1) + C3 < min(1 << 259, 35 * P)
    # the kernel's float factor is below 1 / (p_7 + 1) by more than the float error (2^-21)
    f = float.fromhex("0x1.52917cp-30")
    assert f * (P7 + 1) < 1 - 2 ** -19
    assert f * (P7 + 1) > 1 - 2 ** -17
    assert float.fromhex("0x1.52917cp+2") == f * 2 ** 32
    src = open(ROWFP).read()
    for name, val in (("kRowC1", C1), ("kRowC2", C2), ("kRowC3", C3), ("kRowNegP", NEGP)):
        body = src[src.index(name + "[16]"):]
        body = body[:body.index("};")]
        ws = [int(w, 16) for w in re.findall(r"0x([0-9a-f]+)u", body)]
        assert sum(w << (32 * i) for i, w in enumerate(ws)) == val, name
