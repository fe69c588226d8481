"""Models, on exact Python integers, of arithmetic rearrangements inside the HIP kernels,
each checked against the plain definition it replaces:

* the top-window spread (kern_util.hpp, window_spread; k_sort.hip, digit_slot): with 127-bit
  half-scalar magnitudes the top window's digit never exceeds 2^(127 - c (W - 1)), so
  spreading each digit over 2^(c W - 128) slots stays inside the window's 2^(c-1) slots;
* the bucket reduction by planes (msm_api.hip: make_planes; k_reduce.hip: k_seg_sums,
  k_plane_sums, with_bit):
  segment running sums plus bit planes of the segment weights, each plane doubled by its
  exponent and formed from shared group sums (A_hi, B_lo), must add up to
  sum_j 2^(c j) sum_b (floor(b / f_j) + 1) B_{j,b} for every c;
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


# ---- bucket reduction by planes -------------------------------------------------------
def _seg_log2(c):
    return 3 if c >= 15 else 2


def _planes(c, nwin):
    """make_planes (msm_api.hip): (exponent, window, selector) of every plane, in order
    of decreasing exponent, plus the segment count and log2 segment length."""
    lam = _seg_log2(c)
    slots = 1 << (c - 1)
    nseg = slots >> lam if slots > (1 << lam) else 1
    lgseg = (nseg - 1).bit_length()
    out = []
    for j in range(nwin):
        phi = c * nwin - 128 if j + 1 == nwin else 0
        out.append((c * j, j, 0))
        for beta in range(lgseg):
            if beta + lam < phi:
                continue
            out.append((c * j + beta + lam - phi, j, beta + 1))
    out.sort(key=lambda e: -e[0])
    return out, nseg, lam


def _with_bit(t, beta):
    """with_bit (k_reduce.hip): the t-th index whose bit beta is set."""
    return ((t >> beta) << (beta + 1)) | (1 << beta) | (t & ((1 << beta) - 1))


def _seg_sums(B, lo, hi, f):
    """k_seg_sums: T and P = R + T of one segment, R by a running sum from the top."""
    T = R = 0
    for b in range(hi - 1, lo - 1, -1):
        T += B[b]
        if b > lo and b % f == 0:
            R += T
    return T, R + T


def _reduce_by_planes(buckets, c, nwin, mistake=None):
    planes, nseg, lam = _planes(c, nwin)
    slots = 1 << (c - 1)
    T, Pv = {}, {}
    for j in range(nwin):
        f = 1 << (c * nwin - 128) if j + 1 == nwin else 1
        for s in range(nseg):
            lo, hi = s << lam, min(slots, (s + 1) << lam)
            T[j, s], Pv[j, s] = _seg_sums(buckets[j], lo, hi, f)
    # k_plane_sums: per window the (R + T) group sums of 2^pg segments, A_hi = sum over lo of
    # T_s and B_lo = sum over hi of T_s, s = hi 2^lb + lo
    lgseg = (nseg - 1).bit_length()
    hb = lgseg // 2
    lb = lgseg - hb
    pg = 6 if nseg >= 2048 else 5
    np_ = (nseg + (1 << pg) - 1) >> pg
    assert max(np_, 1 << (lb - 1) if lb else 1, 1 << (hb - 1) if hb else 1) <= 64  # chain terms
    assert max(1 << pg, 1 << lb, 1 << hb) <= 64  # group sizes of k_plane_sums
    G = {}
    for j in range(nwin):
        for r in range(np_):
            G[j, r] = sum(Pv[j, s] for s in range((r << pg), min((r + 1) << pg, nseg)))
        for hi in range(1 << hb):
            G[j, np_ + hi] = sum(T[j, (hi << lb) + lo] for lo in range(1 << lb))
        for lo in range(1 << lb):
            G[j, np_ + (1 << hb) + lo] = sum(T[j, (hi << lb) + lo] for hi in range(1 << hb))
    # k_plane_chain: each plane's terms among its window's group sums
    total = 0
    for e, j, sel in planes:
        if sel == 0:
            terms = list(range(np_))
        elif sel - 1 < lb:
            beta = sel - 1 + (1 if mistake == "selector" else 0)
            terms = [np_ + (1 << hb) + _with_bit(t, beta) % (1 << lb) for t in range(1 << (lb - 1))]
        else:
            beta = sel - 1 - lb
            terms = [np_ + _with_bit(t, beta) for t in range(1 << (hb - 1))]
        v = sum(G[j, r] for r in terms)
        total += v << (e + (1 if mistake == "exponent" and sel == 1 else 0))
    return total, planes


def test_plane_reduction_equals_weighted_window_sum():
    """Every c: the planes' doubled sums add up to sum_j 2^(c j) sum_b w_b B_{j,b}, with
    w_b = floor(b / f_j) + 1, for random integers standing in for the bucket sums."""
    rng = random.Random(12)
    for c in range(1, 17):
        nwin = _num_windows(c)
        for trial in range(3):
            buckets = [[rng.randrange(1 << 40) for _ in range(1 << (c - 1))] for _ in range(nwin)]
            want = 0
            for j in range(nwin):
                f = 1 << (c * nwin - 128) if j + 1 == nwin else 1
                want += sum((b // f + 1) * B for b, B in enumerate(buckets[j])) << (c * j)
            got, planes = _reduce_by_planes(buckets, c, nwin)
            assert got == want, (c, trial)
        # table limits the kernels rely on: exponent below 128 in 8 bits, at most 160
        # planes (10 groups of 16), segment selector and window in their fields
        assert max(e for e, _, _ in planes) <= 127
        assert len(planes) <= 160
        assert all(j < 256 and sel < 256 for _, j, sel in planes)
        assert [e for e, _, _ in planes] == sorted((e for e, _, _ in planes), reverse=True)


def test_bench_plane_exponents_follow_the_table():
    """bench.py prices the combine kernel from the planes' exponents; they must be the
    reduction's own."""
    import bench
    for c in range(1, 17):
        planes, _, _ = _planes(c, _num_windows(c))
        assert sorted(bench.plane_exponents(c)) == sorted(e for e, _, _ in planes), c


def test_plane_reduction_catches_planted_mistakes():
    rng = random.Random(13)
    c, nwin = 13, _num_windows(13)
    buckets = [[rng.randrange(1 << 40) for _ in range(1 << (c - 1))] for _ in range(nwin)]
    good, _ = _reduce_by_planes(buckets, c, nwin)
    for mistake in ("exponent", "selector"):
        assert _reduce_by_planes(buckets, c, nwin, mistake)[0] != good, mistake


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
