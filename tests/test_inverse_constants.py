"""Pins for the constants of the binary-GCD field inverse in the HIP source
(csrc/bingcd.hpp), checked against what p fixes:

* -p^-1 mod 2^30, which makes the exact division by 2^30 mod p clear the low bits;
* the start value u = R^2 mod p (R = 2^256, fp_r2 in fp.hpp): started from (y, p, C, 0)
  the steps end with v = C / y, so with y = x R the result is x^-1 R, the Montgomery
  form of the inverse, with no product afterwards;
* the batch shape: 30 steps a batch keep |f| + |g| <= 2^30 inside int32;
* a big-integer model of the batches (64-bit stand-ins, factors applied to the full
  values) reaches b = 1 with u, v giving the inverse, within the shipped batch count
  for random and structured inputs (inputs it does not cover take the Fermat path).
"""
import random
import os
import re

from oracle import ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "elliptic_curve_scalar_amd", "csrc", "bingcd.hpp")).read()


def _define(name):
    return int(re.search(r"#define %s (0x[0-9a-fA-F]+|\d+)u?" % name, SRC).group(1), 0)


def test_npinv30():
    k = _define("BG_NPINV30")
    assert k < (1 << 30)
    assert (ref.P * k + 1) % (1 << 30) == 0


def test_start_constant_is_r_squared():
    fp_src = open(os.path.join(ROOT, "elliptic_curve_scalar_amd", "csrc", "fp.hpp")).read()
    body = fp_src[fp_src.index("fp fp_r2()"):]
    body = body[:body.index("}")]
    words = dict((int(i), int(v, 16)) for i, v in re.findall(r"r\.v\[(\d)\] = 0x([0-9a-f]+)u", body))
    assert sorted(words) == list(range(8))
    R = 1 << 256
    assert sum(words[i] << (32 * i) for i in range(8)) == R * R % ref.P
    assert "u[i] = r2.v[i]" in SRC  # the inverse starts from it


def test_start_constant_scales_the_result():
    """Started from (y, p, C, 0) the batches end with v = C / y: with C = R^2 and
    y = x R that is x^-1 R; a wrong start (C = 1, the plain inverse) is caught."""
    R = 1 << 256
    rng = random.Random(79)
    batches = _define("BG_BATCHES")
    for _ in range(40):
        x = rng.randrange(1, ref.P)
        y = x * R % ref.P
        ok, v = _bingcd(y, batches, start=R * R % ref.P)
        assert ok and v == pow(x, -1, ref.P) * R % ref.P
        C = rng.randrange(1, ref.P)
        assert _bingcd(y, batches, start=C)[1] == C * pow(y, -1, ref.P) % ref.P
    x = 987654321
    assert _bingcd(x * R % ref.P, batches, start=1)[1] != pow(x, -1, ref.P) * R % ref.P


def test_batch_shape():
    steps, batches = _define("BG_STEPS"), _define("BG_BATCHES")
    assert steps <= 30  # |f| + |g| <= 2^steps must fit a signed 32-bit factor
    assert 10 <= batches <= 18


def _approx(a, b):
    """64-bit stand-ins: low 30 bits exact under the top 34 bits of max(a, b)."""
    n = max(a.bit_length(), b.bit_length())
    if n <= 64:
        return a, b
    sh = n - 34
    m34 = (1 << 34) - 1
    lo = (1 << 30) - 1
    return (((a >> sh) & m34) << 30) | (a & lo), (((b >> sh) & m34) << 30) | (b & lo)


def _batch(xa, xb, steps):
    f0, g0, f1, g1 = 1, 0, 0, 1
    for _ in range(steps):
        if xa & 1:
            if xa < xb:
                xa, xb, f0, g0, f1, g1 = xb, xa, f1, g1, f0, g0
            xa -= xb
            f0, g0 = f0 - f1, g0 - g1
        xa >>= 1
        f1, g1 = 2 * f1, 2 * g1
    return f0, g0, f1, g1


def _bingcd(y, batches, steps=30, start=1):
    """The batches of the device inverse on Python integers, from (a, b, u, v) =
    (y, p, start, 0); returns (converged, v)."""
    P = ref.P
    a, b, u, v = y, P, start, 0
    inv2k = pow(2, -steps, P)
    for _ in range(batches):
        f0, g0, f1, g1 = _batch(*_approx(a, b), steps)
        na, nb = f0 * a + g0 * b, f1 * a + g1 * b
        assert na % (1 << steps) == 0 and nb % (1 << steps) == 0
        if na < 0:
            na, f0, g0 = -na, -f0, -g0
        if nb < 0:
            nb, f1, g1 = -nb, -f1, -g1
        a, b = na >> steps, nb >> steps
        u, v = (f0 * u + g0 * v) * inv2k % P, (f1 * u + g1 * v) * inv2k % P
        assert abs(f0) + abs(g0) <= 1 << steps and abs(f1) + abs(g1) <= 1 << steps
    return b == 1, v


def test_batched_binary_gcd_model():
    batches = _define("BG_BATCHES")
    rng = random.Random(77)
    ys = [rng.randrange(1, ref.P) for _ in range(400)]
    ys += [1, 2, 3, ref.P - 1, ref.P - 2, (ref.P + 1) // 2] + [1 << k for k in range(0, 254, 7)]
    ys += [ref.P - (1 << k) for k in range(1, 254, 11)] + [(1 << k) - 1 for k in range(2, 254, 13)]
    for y in ys:
        ok, v = _bingcd(y, batches)
        assert ok, y  # every sampled input converges within the shipped batch count
        assert v * y % ref.P == 1
    # y = 0 never converges: the device takes the Fermat path (0 -> 0)
    assert not _bingcd(0, batches)[0]


def test_batches_after_convergence_leave_v_unchanged():
    """The device stops once every lane has a = 0: a later batch only halves a (factors
    (1, 0) and (0, 2^30)), so b and v, the inverse, must come out of it unchanged."""
    P = ref.P
    rng = random.Random(78)
    inv2k = pow(2, -30, P)
    for y in [rng.randrange(1, P) for _ in range(60)] + [1, 2, P - 1]:
        a, b, u, v = y, P, 1, 0
        stopped = None
        for it in range(18):
            f0, g0, f1, g1 = _batch(*_approx(a, b), 30)
            na, nb = f0 * a + g0 * b, f1 * a + g1 * b
            if na < 0:
                na, f0, g0 = -na, -f0, -g0
            if nb < 0:
                nb, f1, g1 = -nb, -f1, -g1
            if a == 0:
                assert (f0, g0, f1, g1) == (1, 0, 0, 1 << 30)
            a, b = na >> 30, nb >> 30
            u, v = (f0 * u + g0 * v) * inv2k % P, (f1 * u + g1 * v) * inv2k % P
            if stopped is None and a == 0:
                stopped = (it, b, v)
            elif stopped is not None:
                assert (b, v) == stopped[1:]  # unchanged by every later batch
        assert stopped is not None and stopped[0] < _define("BG_BATCHES")
        assert stopped[1] == 1 and stopped[2] * y % P == 1
