"""GPU row-form arithmetic (rowfp.hpp, rowchain.hpp, rowpoint.hpp) against Python integers
and the chord-and-tangent reference: the product, sum and difference spread over the 16
lanes of a DPP row; 2^d P by runs of doublings in row form (which must also equal the quad
runs bit for bit: both compute the same recurrence in canonical field elements); the
row-form point addition and doubling with every special case; and the affine conversion
that ends the window combine."""
import random

import numpy as np
import pytest

from oracle import ref
from elliptic_curve_scalar_amd import workloads as wl

from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu
P = ref.P
R = 1 << 256

# values whose words make carries and borrows run across the whole row
EDGE = [0, 1, 2, 3, P - 1, P - 2, R % P, (R * R) % P, P // 2, P // 2 + 1, (1 << 224) - 1,
        (1 << 32) - 1, 1 << 32, (1 << 253) - 1, P - (1 << 32), P - (1 << 224),
        ((1 << 256) - 1) % P, (0xFFFFFFFF << 32) % P]


@pytest.mark.parametrize("op", [0, 1, 2])
def test_row_field_ops_match_python(op):
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(300 + op)
    n = 4099  # 1025 wavefronts of four elements, the last one with a single live row
    pairs = [(a, b) for a in EDGE for b in EDGE]
    pairs += [(rng.randrange(P), rng.randrange(P)) for _ in range(n - len(pairs))]
    xs, ys = [a for a, _ in pairs], [b for _, b in pairs]
    say("row op", op, "n", n)
    got = wl.to_ints(to_host(M.test_row(op, to_dev(wl.from_ints(xs)), to_dev(wl.from_ints(ys)))))
    rinv = pow(R, -1, P)
    if op == 0:
        want = [x * y * rinv % P for x, y in pairs]
    elif op == 1:
        want = [(x + y) % P for x, y in pairs]
    else:
        want = [(x - y) % P for x, y in pairs]
    assert got == want


def _xyzz_words(pts, rng):
    """Affine points -> XYZZ (X, Y, ZZ, ZZZ) = (x l^2, y l^3, l^2, l^3) with a random l, in
    Montgomery form, 32 words each; infinity -> all zeros."""
    rows = []
    for pt in pts:
        if pt is None:
            rows.append([0] * 4)
            continue
        x, y = pt
        lam = rng.randrange(1, P)
        zz, zzz = lam * lam % P, lam * lam * lam % P
        rows.append([ref.to_mont(v) for v in (x * zz % P, y * zzz % P, zz, zzz)])
    out = np.zeros((len(rows), 32), dtype=np.uint32)
    for i, r in enumerate(rows):
        out[i] = wl.from_ints(r).reshape(-1)
    return out


def _affine(words):
    X, Y, ZZ, ZZZ = [ref.from_mont(v) for v in wl.to_ints(words.reshape(4, 8))]
    if ZZ == 0:
        return None
    return X * pow(ZZ, -1, P) % P, Y * pow(ZZZ, -1, P) % P


@pytest.mark.parametrize("d", [0, 1, 2, 3, 7, 20, 126, 127])
def test_row_doubling_runs(d):
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(400 + d)
    pts = [ref.scalar_mul(rng.randrange(1, ref.R), ref.G) for _ in range(6)] + [None, ref.G]
    a = to_dev(_xyzz_words(pts, rng))
    say("row doubling run d", d, "points", len(pts))
    got = to_host(M.test_row(3, a, None, d))
    quad = to_host(M.test_row(4, a, None, d))
    assert np.array_equal(got, quad)
    for i, pt in enumerate(pts):
        assert _affine(got[i]) == ref.scalar_mul(1 << d, pt), (d, i)


def test_row_latency_probe_matches_per_lane_chain():
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(7)
    xs = [rng.randrange(P) for _ in range(4)]
    ys = [rng.randrange(P) for _ in range(4)]
    a, b = to_dev(wl.from_ints(xs)), to_dev(wl.from_ints(ys))
    say("row latency probe")
    row = wl.to_ints(to_host(M.test_row(5, a, b, 50)))
    lane = wl.to_ints(to_host(M.test_row(6, a, b, 50)))
    rinv = pow(R, -1, P)
    want = []
    for x, y in zip(xs, ys):
        for _ in range(50):
            x = x * y * rinv % P
        want.append(x)
    assert row == want and lane == want


def _point_cases(rng):
    """Pairs (a, b) of affine points (None = infinity) with every special case of the XYZZ
    addition: infinity on either or both sides, a = b (the doubling branch), a = -b, and
    random pairs."""
    pts = [ref.scalar_mul(rng.randrange(1, ref.R), ref.G) for _ in range(40)]
    pairs = [(None, None), (None, pts[0]), (pts[1], None), (pts[2], pts[2]), (ref.G, ref.G),
             (pts[3], ref.neg(pts[3])), (ref.G, ref.neg(ref.G)), (pts[4], ref.dbl(pts[4]))]
    pairs += [(pts[i], pts[i + 1]) for i in range(5, 39)]
    return pairs


def _check_xyzz_invariant(words):
    X, Y, ZZ, ZZZ = [ref.from_mont(v) for v in wl.to_ints(words.reshape(4, 8))]
    assert max(X, Y, ZZ, ZZZ) < P
    assert ZZ ** 3 % P == ZZZ ** 2 % P  # ZZ = Z^2, ZZZ = Z^3 for some Z


def test_row_point_addition_every_case():
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(500)
    pairs = _point_cases(rng)
    # each side gets its own random scaling, so a = b arrives in different coordinates
    a = to_dev(_xyzz_words([x for x, _ in pairs], rng))
    b = to_dev(_xyzz_words([y for _, y in pairs], rng))
    say("row point add, pairs", len(pairs))
    got = to_host(M.test_row(7, a, b))
    for i, (x, y) in enumerate(pairs):
        _check_xyzz_invariant(got[i])
        assert _affine(got[i]) == ref.add(x, y), i


def test_row_point_doubling():
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(501)
    pts = [None, ref.G] + [ref.scalar_mul(rng.randrange(1, ref.R), ref.G) for _ in range(30)]
    a = to_dev(_xyzz_words(pts, rng))
    say("row point doubling, points", len(pts))
    got = to_host(M.test_row(8, a))
    for i, pt in enumerate(pts):
        _check_xyzz_invariant(got[i])
        assert _affine(got[i]) == ref.dbl(pt), i


def test_uniform_affine_conversion():
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(502)
    pts = [None, ref.G, ref.neg(ref.G)] + [ref.scalar_mul(rng.randrange(1, ref.R), ref.G)
                                           for _ in range(29)]
    a = to_dev(_xyzz_words(pts, rng))
    say("uniform affine conversion, points", len(pts))
    got = to_host(M.test_row(9, a))
    for i, pt in enumerate(pts):
        x, y = [ref.from_mont(v) for v in wl.to_ints(got[i].reshape(2, 8))]
        assert (None if (x, y) == (0, 0) else (x, y)) == pt, i
