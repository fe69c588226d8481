"""Word-exact models of the per-lane Montgomery product and square of fp.hpp
(fp_mul_cios, fp_sqr_sos) and of the binary-GCD inverse's linear combination (bingcd.hpp,
bg_comb): each row's 32 x 32 -> 64-bit multiply-adds with their addends, then one
add-with-carry chain, with the top word carried in the high half of the row's last addend.
The models assert every bound the kernels rely on (no multiply-add above 2^64, no carry
lost) and check the results against the plain integer definitions on edge and random
values."""
import random

from oracle import ref

P = ref.P
R = 1 << 256
M32 = (1 << 32) - 1
PINV = (-pow(P, -1, 1 << 32)) % (1 << 32)
PL = [(P >> (32 * i)) & M32 for i in range(8)]


def words(x):
    return [(x >> (32 * i)) & M32 for i in range(8)]


def mad(x, y, addend):
    s = x * y + addend
    assert s < 1 << 64
    return s


def addc(x, y, c):
    s = x + y + c
    return s & M32, s >> 32


def reduce_once(t):
    v = sum(w << (32 * i) for i, w in enumerate(t))
    assert v < 2 * P
    return v - P if v >= P else v


def mul_model(a, b):
    A, B = words(a), words(b)
    assert A[7] < 1 << 30
    t = [0] * 9
    for i in range(8):
        s = [mad(A[j], B[i], t[j]) for j in range(7)] + [mad(A[7], B[i], (t[8] << 32) | t[7])]
        c = 0
        t[0] = s[0] & M32
        for j in range(1, 8):
            t[j], c = addc(s[j] & M32, s[j - 1] >> 32, c)
        t[8] = (s[7] >> 32) + c
        assert t[8] < 1 << 31
        m = (t[0] * PINV) & M32
        s = [mad(m, PL[j], t[j]) for j in range(7)] + [mad(m, PL[7], (t[8] << 32) | t[7])]
        assert s[0] & M32 == 0
        c = 0
        for j in range(1, 8):
            t[j - 1], c = addc(s[j] & M32, s[j - 1] >> 32, c)
        t[7] = (s[7] >> 32) + c
        assert t[7] <= M32
        t[8] = 0
    return reduce_once(t[:8])


def sqr_model(a):
    A = words(a)
    t = [0] * 16
    for i in range(7):
        s = {j: mad(A[i], A[j], t[i + j]) for j in range(i + 1, 8)}
        c = 0
        t[2 * i + 1] = s[i + 1] & M32
        for j in range(i + 2, 8):
            t[i + j], c = addc(s[j] & M32, s[j - 1] >> 32, c)
        assert t[i + 8] == 0
        t[i + 8] = (s[7] >> 32) + c
        assert t[i + 8] <= M32
    assert t[15] == 0
    for k in range(15, 0, -1):
        t[k] = ((t[k] << 1) | (t[k - 1] >> 31)) & M32
    t[0] = 0
    s = [mad(A[i], A[i], t[2 * i]) for i in range(8)]
    c = 0
    for i in range(8):
        t[2 * i], c = addc(s[i] & M32, 0, c)
        t[2 * i + 1], c = addc(t[2 * i + 1], s[i] >> 32, c)
    assert c == 0 and sum(w << (32 * k) for k, w in enumerate(t)) == a * a
    cc = 0
    for i in range(8):
        m = (t[i] * PINV) & M32
        s = [mad(m, PL[j], t[i + j]) for j in range(7)] + [mad(m, PL[7], (cc << 32) | t[i + 7])]
        assert s[0] & M32 == 0
        c = 0
        for j in range(1, 8):
            t[i + j], c = addc(s[j] & M32, s[j - 1] >> 32, c)
        t[i + 8], c = addc(t[i + 8], s[7] >> 32, c)
        cc = c
    assert cc == 0
    return reduce_once(t[8:])


def _values(rng, n):
    edge = [0, 1, 2, P - 1, P - 2, (P - 1) // 2, (P + 1) // 2, R % P, (R * R) % P,
            (1 << 224) - 1, (1 << 253) % P, P - (1 << 32), (1 << 32) - 1, (M32 << 224) % P,
            P - (M32 << 192)]
    assert all(0 <= v < P for v in edge)  # the kernels take fully reduced inputs
    return edge + [rng.randrange(P) for _ in range(n)]


def test_product_model_matches_montgomery_product():
    rng = random.Random(21)
    rinv = pow(R, -1, P)
    xs = _values(rng, 300)
    ys = _values(rng, 300)
    for x in xs:
        for y in (ys[:15] + [rng.choice(ys)]):
            assert mul_model(x, y) == x * y * rinv % P


def test_square_model_matches_montgomery_square():
    rng = random.Random(22)
    rinv = pow(R, -1, P)
    for x in _values(rng, 2000):
        assert sqr_model(x) == x * x * rinv % P


def test_models_catch_a_dropped_top_word():
    """The top word carried in the high half of the last addend matters: dropping it (a
    plausible slip) changes the product for most inputs."""
    rng = random.Random(23)
    rinv = pow(R, -1, P)

    def mul_dropped(a, b):
        A, B = words(a), words(b)
        t = [0] * 9
        for i in range(8):
            s = [A[j] * B[i] + t[j] for j in range(8)]  # t[8] left out of s[7]
            c = 0
            t[0] = s[0] & M32
            for j in range(1, 8):
                t[j], c = addc(s[j] & M32, s[j - 1] >> 32, c)
            t[8] = (s[7] >> 32) + c
            m = (t[0] * PINV) & M32
            s = [m * PL[j] + t[j] for j in range(8)]
            c = 0
            for j in range(1, 8):
                t[j - 1], c = addc(s[j] & M32, s[j - 1] >> 32, c)
            t[7] = ((s[7] >> 32) + c) & M32
            t[8] = 0
        v = sum(w << (32 * k) for k, w in enumerate(t[:8]))
        return v % P

    wrong = 0
    for _ in range(50):
        x, y = rng.randrange(P), rng.randrange(P)
        wrong += mul_dropped(x, y) != x * y * rinv % P
    assert wrong > 40


def comb_model(x, y, f, g, k, kp):
    """bingcd.hpp's bg_comb before its final subtraction: word i's products summed into one
    64-bit value (f, g offset by 2^30), then one add-with-carry chain over the words."""
    fo, go = f + (1 << 30), g + (1 << 30)
    assert 0 <= fo <= 1 << 31 and 0 <= go <= 1 << 31
    X, Y = words(x), words(y)
    s = [mad(X[i], fo, 0) + Y[i] * go + (k * PL[i] if kp else 0) for i in range(8)]
    assert all(v < 1 << 64 for v in s)
    t, c = [s[0] & M32], 0
    for i in range(1, 8):
        w, c = addc(s[i] & M32, s[i - 1] >> 32, c)
        t.append(w)
    top = (s[7] >> 32) + c
    assert top <= M32
    return sum(w << (32 * i) for i, w in enumerate(t + [top]))


def test_inverse_combination_model():
    rng = random.Random(24)
    for _ in range(3000):
        x, y = rng.randrange(1 << 254), rng.randrange(1 << 254)
        f = rng.randrange(-(1 << 30), (1 << 30) + 1)
        lim = (1 << 30) - abs(f)
        g = rng.randrange(-lim, lim + 1)
        k, kp = rng.randrange(1 << 30), rng.random() < 0.5
        want = x * (f + (1 << 30)) + y * (g + (1 << 30)) + (k * P if kp else 0)
        assert comb_model(x, y, f, g, k, kp) == want
    # extremes of the factors
    for f, g in ((1 << 30, 0), (0, 1 << 30), (-(1 << 30), 0), (0, -(1 << 30)), (1 << 29, -(1 << 29))):
        x = y = (1 << 254) - 1
        assert comb_model(x, y, f, g, (1 << 30) - 1, True) == \
            x * (f + (1 << 30)) + y * (g + (1 << 30)) + ((1 << 30) - 1) * P
