"""Models, on exact Python integers, of arithmetic rearrangements inside the HIP kernels,
each checked against the plain definition it replaces:

* the top-window spread (msm_kernels.hip, window_spread / digit_slot): with 127-bit
  half-scalar magnitudes the top window's digit never exceeds 2^(127 - c (W - 1)), so
  spreading each digit over 2^(c W - 128) slots stays inside the window's 2^(c-1) slots;
* the running-sum segments with that spread (rsum_segment): R adds T at every slot that
  is a multiple of f, and a segment's share is R + ceil(lo / f) T, which must equal the
  weighted sum sum_b (floor(b / f) + 1) B_b over the segment;
* the runs of doublings with lookahead (quad.hpp, quad_dbl_n): the (X, U = 2Y, M = 3X^2, z)
  recurrence against repeated XYZZ doubling (dbl-2008-s-1) on curve points, odd and even
  run lengths, and the point at infinity;
* the bucket lookup (bucket_of / bisect_le): the bracket around a guess, then bisection,
  against a plain search on even and skewed pair offsets.
"""
import bisect
import random

from oracle import ref

P = ref.P


# ---- top-window spread ---------------------------------------------------------------
def _num_windows(c):
    return (128 + c - 1) // c


def _signed_digits(k, c, nwin):
    """Signed c-bit digits of k (carry run up from window 0), as in the device recoding."""
    half, carry, out = 1 << (c - 1), 0, []
    for j in range(nwin):
        raw = ((k >> (c * j)) & ((1 << c) - 1)) + carry
        neg = j + 1 < nwin and raw > half
        carry = 1 if neg else 0
        out.append(raw - (1 << c) if neg else raw)
    return out


def test_top_window_spread_fits_every_c():
    rng = random.Random(11)
    for c in range(1, 17):
        nwin = _num_windows(c)
        top = 1 << (127 - c * (nwin - 1))  # largest top digit
        f = 1 << (c * nwin - 128)          # slots per top digit
        assert top * f <= 1 << (c - 1), c
        ks = [(1 << 127) - 1, 0, 1] + [rng.getrandbits(127) for _ in range(300)]
        for k in ks:
            d = _signed_digits(k, c, nwin)
            assert sum(v << (c * j) for j, v in enumerate(d)) == k
            assert 0 <= d[-1] <= top
            if d[-1]:
                for i in range(f):  # every slot the digit can take
                    assert (d[-1] - 1) * f + i < 1 << (c - 1)


# ---- running-sum segments ------------------------------------------------------------
def _segment_share(B, lo, hi, f):
    T = R = 0
    for b in range(hi - 1, lo - 1, -1):
        T += B[b]
        if b % f == 0:
            R += T
    return R + (-(-lo // f)) * T


def test_segment_shares_sum_to_weighted_bucket_sum():
    rng = random.Random(12)
    for _ in range(400):
        f = 1 << rng.randrange(0, 8)
        nb = 1 << rng.randrange(1, 12)
        seg = (1 << rng.randrange(0, 9)) if rng.random() < 0.7 else rng.randrange(1, 40)
        B = [rng.randrange(1 << 20) for _ in range(nb)]
        want = sum((b // f + 1) * B[b] for b in range(nb))
        got = sum(_segment_share(B, lo, min(nb, lo + seg), f) for lo in range(0, nb, seg))
        assert got == want, (f, nb, seg)


def test_segment_share_catches_a_wrong_weight():
    # a planted mistake (floor instead of ceil) must show up
    B = [3, 5, 7, 11, 13, 17, 19, 23]
    lo, hi, f = 1, 3, 4
    T = sum(B[lo:hi])
    wrong = _segment_share(B, lo, hi, f) - (-(-lo // f)) * T + (lo // f) * T
    assert wrong != sum((b // f + 1) * B[b] for b in range(lo, hi))


# ---- doubling runs -------------------------------------------------------------------
def _xyzz_dbl(pt):
    X, Y, ZZ, ZZZ = pt
    U = 2 * Y % P
    V = U * U % P
    W = U * V % P
    S = X * V % P
    M = 3 * X * X % P
    X3 = (M * M - 2 * S) % P
    return X3, (M * (S - X3) - W * Y) % P, V * ZZ % P, W * ZZZ % P


def _run(pt, n):
    """quad_dbl_n on integers: two doublings per step, then one if n is odd."""
    if n == 0:
        return pt
    X, Y, ZZ0, ZZZ0 = pt
    X, U, z = X, 2 * Y % P, 1
    M = 3 * X * X % P
    for _ in range(n // 2):
        V, MX, MM, z = U * U % P, M * X % P, M * M % P, z * U % P
        XV, MXV, M3, VV = X * V % P, MX * V % P, M * MM % P, V * V % P
        X1 = (MM - 2 * XV) % P
        U1 = (2 * (3 * MXV - M3) - VV) % P
        M1, V1, z = 3 * X1 * X1 % P, U1 * U1 % P, z * U1 % P
        M1X1, MM1, X1V1, VV1 = M1 * X1 % P, M1 * M1 % P, X1 * V1 % P, V1 * V1 % P
        X = (MM1 - 2 * X1V1) % P
        U = (2 * (3 * (M1X1 * V1 % P) - M1 * MM1 % P) - VV1) % P
        M = 3 * X * X % P
    if n & 1:
        V, MX, MM, z = U * U % P, M * X % P, M * M % P, z * U % P
        XV, MXV, M3, VV = X * V % P, MX * V % P, M * MM % P, V * V % P
        X = (MM - 2 * XV) % P
        U = (2 * (3 * MXV - M3) - VV) % P
        M = 3 * X * X % P
    zz = z * z % P
    return X, U * pow(2, -1, P) % P, ZZ0 * zz % P, ZZZ0 * zz * z % P


def _affine(pt):
    X, Y, ZZ, ZZZ = pt
    if ZZ == 0:
        return None
    return X * pow(ZZ, -1, P) % P, Y * pow(ZZZ, -1, P) % P


def test_doubling_runs_match_repeated_doubling():
    rng = random.Random(13)
    for _ in range(12):
        k = rng.randrange(1, ref.R)
        x, y = ref.scalar_mul(k, ref.G)
        t = rng.randrange(1, P)
        pt = (x * t * t % P, y * t * t * t % P, t * t % P, t * t * t % P)
        for n in (0, 1, 2, 3, 12, 13, 26, 117):
            want = pt
            for _ in range(n):
                want = _xyzz_dbl(want)
            got = _run(pt, n)
            assert _affine(got) == _affine(want) == ref.scalar_mul((k << n) % ref.R, ref.G), n
            assert got[2] ** 3 % P == got[3] ** 2 % P  # ZZ^3 = ZZZ^2 still holds


def test_doubling_run_keeps_infinity():
    assert _run((1, 1, 0, 0), 5)[2:] == (0, 0)


# ---- bucket lookup -------------------------------------------------------------------
GUESS_SPAN = 128


def _bisect_le(a, lo, hi, x):
    while hi - lo > 1:
        mid = lo + (hi - lo) // 2
        if a[mid] <= x:
            lo = mid
        else:
            hi = mid
    return lo


def _bucket_of(a, n, x, g):
    g = min(g, n - 1)
    lo, hi = max(g - GUESS_SPAN, 0), min(g + GUESS_SPAN, n)
    if not (a[lo] <= x < a[hi]):
        lo, hi = 0, n
    return _bisect_le(a, lo, hi, x)


def test_bucket_lookup_matches_plain_search():
    rng = random.Random(14)
    for skew in (False, True):
        for _ in range(20):
            K = rng.randrange(1, 5000)
            pairs = [rng.randrange(0, 6) for _ in range(K)]
            if skew:
                pairs[rng.randrange(K)] += 20000
            a = [0]
            for v in pairs:
                a.append(a[-1] + v)
            total = a[-1]
            if total == 0:
                continue
            for p in [0, total - 1] + [rng.randrange(total) for _ in range(200)]:
                want = bisect.bisect_right(a, p, 0, K) - 1  # last k < K with a[k] <= p
                assert _bucket_of(a, K, p, p * K // total) == want
