"""Pins for the C oracle (oracle/oracle.c): field ops against Python ints, curve ops
against the Python chord-and-tangent reference, Pippenger against brute force at
n <= 16 for every window width, and against the linearity closed form
sum_i s_i (r_i G) = (sum_i s_i r_i mod r) G at larger n."""
import random

import numpy as np
import pytest

import oracle
from oracle import ref
from elliptic_curve_scalar_amd import workloads as wl

P = ref.P


def _limbs64(vals):
    return np.array([[(v >> (64 * i)) & 0xFFFFFFFFFFFFFFFF for i in range(4)] for v in vals],
                    dtype=np.uint64)


def _ints64(arr):
    return [sum(int(row[i]) << (64 * i) for i in range(4)) for row in arr]


EDGE = [0, 1, 2, P - 1, P - 2, (1 << 256) % P, (1 << 255) % P, P // 2, P // 3]


def test_field_ops_match_python():
    rng = random.Random(1)
    xs = EDGE + [rng.randrange(P) for _ in range(300)]
    ys = list(reversed(EDGE)) + [rng.randrange(P) for _ in range(300)]
    a, b = _limbs64(xs), _limbs64(ys)
    rinv = pow(1 << 256, -1, P)
    assert _ints64(oracle.fp_op(oracle.FP_MUL, a, b)) == [x * y * rinv % P for x, y in zip(xs, ys)]
    assert _ints64(oracle.fp_op(oracle.FP_SQR, a)) == [x * x * rinv % P for x in xs]
    assert _ints64(oracle.fp_op(oracle.FP_ADD, a, b)) == [(x + y) % P for x, y in zip(xs, ys)]
    assert _ints64(oracle.fp_op(oracle.FP_SUB, a, b)) == [(x - y) % P for x, y in zip(xs, ys)]
    assert _ints64(oracle.fp_op(oracle.FP_TO_MONT, a)) == [x * (1 << 256) % P for x in xs]
    assert _ints64(oracle.fp_op(oracle.FP_FROM_MONT, a)) == [x * rinv % P for x in xs]
    # inverse of a Montgomery-form value xR is x^{-1} R, i.e. (xR)^{-1} R^2
    inv = _ints64(oracle.fp_op(oracle.FP_INV, a))
    for x, got in zip(xs, inv):
        if x == 0:
            assert got == 0
        else:
            assert got * x % P == (1 << 512) % P


def _rand_pt(rng):
    return ref.scalar_mul(rng.randrange(1, ref.R), ref.G)


def _enc(pt):
    return np.array(ref.encode_point(pt), dtype=np.uint32)


def test_point_add_matches_python():
    rng = random.Random(2)
    for _ in range(20):
        p1, p2 = _rand_pt(rng), _rand_pt(rng)
        for a, b in ((p1, p2), (p1, p1), (p1, ref.neg(p1)), (None, p2), (p1, None), (None, None)):
            got = ref.decode_point(oracle.g1_add(_enc(a), _enc(b)))
            assert got == ref.add(a, b)


def test_on_curve_check():
    assert oracle.on_curve(_enc(ref.G))
    assert oracle.on_curve(np.zeros(16, np.uint32))       # infinity encoding
    bad = _enc(ref.G).copy()
    bad[8] ^= 1
    assert not oracle.on_curve(bad)


def test_scalar_mul_matches_python():
    rng = random.Random(3)
    g = _enc(ref.G)
    ks = [0, 1, 2, 3, ref.R - 1, ref.R, ref.R + 1, (1 << 256) - 1] + [rng.randrange(1 << 256) for _ in range(10)]
    for k in ks:
        got = ref.decode_point(oracle.g1_scalar_mul(g, wl.from_ints([k])[0]))
        assert got == ref.scalar_mul(k, ref.G)


def test_fixed_base_points_match_double_and_add():
    rng = random.Random(4)
    ks = [0, 1, 2, 255, 256, 257, ref.R - 1] + [rng.randrange(1, ref.R) for _ in range(40)]
    pts = oracle.g1_from_scalars(wl.from_ints(ks), threads=4)
    for k, row in zip(ks, pts):
        assert ref.decode_point(row) == ref.scalar_mul(k, ref.G)


def _points_for(dl_ints):
    return oracle.g1_from_scalars(wl.from_ints(dl_ints), threads=4)


def test_naive_msm_matches_python():
    rng = random.Random(5)
    for n in (1, 2, 4, 7):
        dl = [rng.randrange(1, ref.R) for _ in range(n)]
        sc = [rng.randrange(ref.R) for _ in range(n)]
        got = oracle.msm_naive(_points_for(dl), wl.from_ints(sc))
        assert ref.decode_point(got) == ref.msm_linear(dl, sc)


def test_pippenger_matches_brute_force_all_c():
    """n <= 16 with small scalars: brute-force repeated addition is the reference."""
    rng = random.Random(6)
    for n in (1, 3, 16):
        dl = [rng.randrange(1, ref.R) for _ in range(n)]
        pts_i = [ref.scalar_mul(r, ref.G) for r in dl]
        sc = [rng.randrange(0, 1 << 9) for _ in range(n)]
        want = ref.msm_brute(pts_i, sc)
        pts = _points_for(dl)
        for c in range(1, 17):
            got = oracle.msm_pippenger(pts, wl.from_ints(sc), c, threads=4)
            assert ref.decode_point(got) == want, (n, c)


def test_pippenger_full_scalars_all_c():
    rng = random.Random(7)
    n = 16
    dl = [rng.randrange(1, ref.R) for _ in range(n)]
    sc = [rng.randrange(ref.R) for _ in range(n)]
    want = ref.msm_linear(dl, sc)
    pts, s = _points_for(dl), wl.from_ints(sc)
    assert ref.decode_point(oracle.msm_naive(pts, s)) == want
    for c in range(1, 17):
        assert ref.decode_point(oracle.msm_pippenger(pts, s, c, threads=8)) == want, c


@pytest.mark.parametrize("name,n", [("n256_c8", 256), ("n65536_c13", 2048),
                                    ("n262144_c13_edge", 4096), ("n1048576_c16", 1024),
                                    ("n4194304_c16_skew", 2048)])
def test_pippenger_linearity_on_workloads(name, n):
    w = wl.generate(name, n=n)
    pts = oracle.g1_from_scalars(w["dlogs"], threads=8)
    got = oracle.msm_pippenger(pts, w["scalars"], w["c"], threads=8)
    want = ref.msm_linear(wl.to_ints(w["dlogs"]), wl.to_ints(w["scalars"]))
    assert ref.decode_point(got) == want
    assert oracle.on_curve(got)


def test_window_and_bucket_sums_shadow_scalars():
    """Intermediate pins: B_{j,b} = (sum_{d_j(s_i) = b} r_i) G and
    W_j = (sum_i d_j(s_i) r_i) G, since every P_i = r_i G. The expected points come
    from the fixed-base routine, itself pinned to double-and-add above."""
    w = wl.generate("n256_c8", n=64)
    c = 6
    dl, sc = wl.to_ints(w["dlogs"]), wl.to_ints(w["scalars"])
    pts = oracle.g1_from_scalars(w["dlogs"], threads=4)
    out, wins, bks = oracle.msm_pippenger(pts, w["scalars"], c, threads=4, windows=True, buckets=True)
    nwin = ref.num_windows(c)
    digs = [ref.window_digits(s, c, nwin) for s in sc]
    wk = [sum(d[j] * r for d, r in zip(digs, dl)) % ref.R for j in range(nwin)]
    bk = [sum(r for d, r in zip(digs, dl) if d[j] == b) % ref.R
          for j in range(nwin) for b in range(1 << c)]
    assert np.array_equal(wins, oracle.g1_from_scalars(wl.from_ints(wk), threads=4))
    want_b = oracle.g1_from_scalars(wl.from_ints(bk), threads=4).reshape(nwin, 1 << c, 16)
    want_b[:, 0] = 0  # bucket 0 is never filled
    assert np.array_equal(bks, want_b)
    # and a few of them against the Python double-and-add directly
    for j, b in ((0, 1), (nwin - 1, 3), (nwin // 2, (1 << c) - 1)):
        assert ref.decode_point(bks[j, b]) == ref.scalar_mul(bk[j * (1 << c) + b], ref.G)


def test_msm_edge_cases():
    rng = random.Random(8)
    dl = [rng.randrange(1, ref.R) for _ in range(6)]
    pts = _points_for(dl)
    inf = np.zeros((1, 16), np.uint32)
    neg = _points_for([ref.R - dl[0]])
    cases = [
        (pts[:1], [0], None),
        (pts[:1], [1], ref.scalar_mul(dl[0], ref.G)),
        (pts[:1], [ref.R - 1], ref.neg(ref.scalar_mul(dl[0], ref.G))),
        (np.vstack([pts[:1], neg]), [99, 99], None),                       # P, -P cancel
        (np.vstack([pts[:1], pts[:1]]), [5, 5], ref.scalar_mul(10 * dl[0] % ref.R, ref.G)),
        (np.vstack([inf, pts[1:2]]), [7, 3], ref.scalar_mul(3 * dl[1] % ref.R, ref.G)),
        (pts, [1] * 6, ref.scalar_mul(sum(dl) % ref.R, ref.G)),
        (pts[:0], [], None),
    ]
    for p_, s_, want in cases:
        s_arr = wl.from_ints(s_) if s_ else np.zeros((0, 8), np.uint32)
        for c in (1, 8, 13, 16):
            assert ref.decode_point(oracle.msm_pippenger(p_, s_arr, c, threads=2)) == want


def test_range_and_point_errors():
    pts = _points_for([5])
    # c = 15 gives W = 17 windows covering 255 bits; bit 255 set is out of range.
    with pytest.raises(oracle.OracleError) as e:
        oracle.msm_pippenger(pts, wl.from_ints([1 << 255]), 15)
    assert e.value.code == oracle.ORACLE_ERR_RANGE
    # scalars in [r, 2^(W c)) are integer multiples: (r + 3) P = 3 P
    got = oracle.msm_pippenger(pts, wl.from_ints([ref.R + 3]), 13)
    assert ref.decode_point(got) == ref.scalar_mul(15, ref.G)
    bad = pts.copy()
    bad[0, 8] ^= 1
    with pytest.raises(oracle.OracleError) as e:
        oracle.msm_pippenger(bad, wl.from_ints([1]), 8)
    assert e.value.code == oracle.ORACLE_ERR_POINT
    with pytest.raises(oracle.OracleError):
        oracle.msm_pippenger(pts, wl.from_ints([1]), 17)


def test_arithmetic_progression_set():
    """The degenerate set the pages warn about still has a unique sum."""
    dl = wl.arithmetic_progression(32, a=12345, d=777)
    sc = wl.from_ints([random.Random(9).randrange(ref.R) for _ in range(32)])
    pts = oracle.g1_from_scalars(dl, threads=4)
    want = ref.msm_linear(wl.to_ints(dl), wl.to_ints(sc))
    for c in (4, 8, 13):
        assert ref.decode_point(oracle.msm_pippenger(pts, sc, c, threads=4)) == want
