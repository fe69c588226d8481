"""Pins for the Python-integer oracle (oracle/ref.py) against what mathematics fixes:
primality of the published constants, the group order, brute force, and the group
law's homomorphism k -> k*G. Mutation tests show each pin catches a planted mistake."""
import os
import random

import pytest

from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_params():
    vals = {}
    with open(os.path.join(GOLDEN, "bn254_params.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = (t.strip() for t in line.split("="))
                vals[k] = int(v)
    return vals


def _is_probable_prime(n, rounds=32):
    if n < 2:
        return False
    small = [2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37]
    for q in small:
        if n % q == 0:
            return n == q
    d, s = n - 1, 0
    while d % 2 == 0:
        d //= 2
        s += 1
    rng = random.Random(12345)
    for _ in range(rounds):
        a = rng.randrange(2, n - 1)
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(s - 1):
            x = x * x % n
            if x == n - 1:
                break
        else:
            return False
    return True


def test_constants_match_eip196():
    g = _golden_params()
    assert ref.P == g["p"] and ref.R == g["r"] and ref.B == g["b"]
    assert ref.G == (g["Gx"], g["Gy"])


def test_constants_are_prime():
    assert _is_probable_prime(ref.P)
    assert _is_probable_prime(ref.R)
    assert not _is_probable_prime(ref.P + 2)  # the test itself can say "no"
    assert ref.P.bit_length() == 254 and ref.R.bit_length() == 254
    assert ref.P % 4 == 3


def test_generator_on_curve_and_order():
    assert ref.on_curve(ref.G)
    assert ref.scalar_mul(ref.R, ref.G) is None           # r * G = infinity (#E = r)
    assert ref.scalar_mul(ref.R - 1, ref.G) == (1, ref.P - 2)  # (r-1) G = -G
    assert ref.scalar_mul(ref.R + 5, ref.G) == ref.scalar_mul(5, ref.G)


def test_doubling_closed_form():
    # 2G by the tangent at (1, 2): lambda = 3 x^2 / (2 y) = 3/4, written out by hand.
    lam = 3 * pow(4, -1, ref.P) % ref.P
    x3 = (lam * lam - 2) % ref.P
    y3 = (lam * (1 - x3) - 2) % ref.P
    assert ref.dbl(ref.G) == (x3, y3)
    assert ref.on_curve((x3, y3))


def test_scalar_mul_equals_repeated_addition():
    for k in list(range(0, 40)) + [255, 256, 511, 1000, 1023, 1024]:
        assert ref.scalar_mul(k, ref.G) == ref.repeated_add(k, ref.G)


def _rand_point(rng):
    return ref.scalar_mul(rng.randrange(1, ref.R), ref.G)


def test_group_law():
    rng = random.Random(7)
    for _ in range(6):
        a, b = rng.randrange(1, ref.R), rng.randrange(1, ref.R)
        pa, pb = ref.scalar_mul(a, ref.G), ref.scalar_mul(b, ref.G)
        assert ref.on_curve(pa) and ref.on_curve(pb)
        assert ref.add(pa, pb) == ref.scalar_mul((a + b) % ref.R, ref.G)   # homomorphism
        assert ref.add(pa, pb) == ref.add(pb, pa)
        assert ref.scalar_mul(a, pb) == ref.scalar_mul(a * b % ref.R, ref.G)
        pc = _rand_point(rng)
        assert ref.add(ref.add(pa, pb), pc) == ref.add(pa, ref.add(pb, pc))
        assert ref.add(pa, ref.neg(pa)) is None
        assert ref.add(pa, None) == pa and ref.add(None, pa) == pa
        assert ref.dbl(pa) == ref.scalar_mul(2 * a % ref.R, ref.G)


def test_msm_brute_naive_linear_pippenger_agree():
    rng = random.Random(11)
    for n in (1, 2, 3, 5, 8):
        dl = [rng.randrange(1, ref.R) for _ in range(n)]
        pts = [ref.scalar_mul(r, ref.G) for r in dl]
        small = [rng.randrange(0, 60) for _ in range(n)]
        brute = ref.msm_brute(pts, small)
        assert brute == ref.msm_naive(pts, small)
        assert brute == ref.msm_linear(dl, small)
        big = [rng.randrange(0, ref.R) for _ in range(n)]
        lin = ref.msm_linear(dl, big)
        assert ref.msm_naive(pts, big) == lin
        for c in (1, 5):
            assert ref.msm_pippenger(pts, big, c) == lin


def test_msm_special_cases():
    rng = random.Random(5)
    p1 = _rand_point(rng)
    assert ref.msm_naive([p1], [0]) is None
    assert ref.msm_naive([p1], [1]) == p1
    assert ref.msm_naive([p1], [ref.R - 1]) == ref.neg(p1)
    assert ref.msm_naive([p1, ref.neg(p1)], [77, 77]) is None
    assert ref.msm_naive([None, p1], [5, 1]) == p1


def test_codec_roundtrip():
    rng = random.Random(3)
    for _ in range(5):
        pt = _rand_point(rng)
        assert ref.decode_point(ref.encode_point(pt)) == pt
    assert ref.encode_point(None) == [0] * 16
    assert ref.decode_point([0] * 16) is None
    assert ref.to_mont(1) == (1 << 256) % ref.P


# --------------------------------------------------------------------------- mutations
def _mutant_add(kind):
    def add(p1, p2):
        if p1 is None:
            return p2
        if p2 is None:
            return p1
        x1, y1 = p1
        x2, y2 = p2
        if x1 == x2:
            if (y1 + y2) % ref.P == 0:
                return None
            k = 2 if kind == "tangent_coeff" else 3
            lam = (k * x1 * x1) * ref.fp_inv(2 * y1) % ref.P
        else:
            lam = (y2 - y1) * ref.fp_inv(x2 - x1) % ref.P
        x3 = (lam * lam - x1 - (0 if kind == "drop_x2" else x2)) % ref.P
        y3 = (lam * (x1 - x3) + (y1 if kind == "sign_y" else -y1)) % ref.P
        return (x3, y3)
    return add


@pytest.mark.parametrize("kind", ["tangent_coeff", "drop_x2", "sign_y"])
def test_pins_catch_planted_mistakes(monkeypatch, kind):
    """Each planted mistake in the addition law must break the order pin or the
    homomorphism pin (the pins are not tautologies)."""
    monkeypatch.setattr(ref, "add", _mutant_add(kind))
    order_ok = ref.scalar_mul(ref.R, ref.G) is None
    a, b = 123456789, 987654321
    hom_ok = ref.add(ref.scalar_mul(a, ref.G), ref.scalar_mul(b, ref.G)) == ref.scalar_mul(a + b, ref.G)
    brute_ok = ref.scalar_mul(37, ref.G) == ref.repeated_add(37, ref.G)
    assert not (order_ok and hom_ok and brute_ok)
