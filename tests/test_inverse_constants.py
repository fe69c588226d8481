"""Pins for the constants of the binary-GCD field inverse in the HIP source
(csrc/bingcd.hpp), checked against what p fixes:

* -p^-1 mod 2^30, which makes the exact division by 2^30 mod p clear the low bits;
* R^3 mod p (R = 2^256), which turns the integer inverse of the Montgomery form x R
  into the Montgomery form x^-1 R of the inverse;
* the batch shape: 30 steps a batch keep |f| + |g| <= 2^30 inside int32, and the
  batch count covers the 2 len(p) - 1 steps the exact binary GCD needs.
"""
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


def test_r_cubed():
    words = dict((int(i), int(v, 16)) for i, v in re.findall(r"c\.v\[(\d)\] = 0x([0-9a-f]+)u", SRC))
    assert sorted(words) == list(range(8))
    val = sum(words[i] << (32 * i) for i in range(8))
    R = 1 << 256
    assert val == R ** 3 % ref.P
    # mont(X^-1, R^3) = X^-1 R^2 = x^-1 R for X = x R
    x = 123456789
    X = x * R % ref.P
    assert pow(X, -1, ref.P) * val * pow(R, -1, ref.P) % ref.P == pow(x, -1, ref.P) * R % ref.P


def test_batch_shape():
    steps, batches = _define("BG_STEPS"), _define("BG_BATCHES")
    assert steps <= 30  # |f| + |g| <= 2^steps must fit a signed 32-bit factor
    assert steps * batches >= 2 * ref.P.bit_length() - 1
