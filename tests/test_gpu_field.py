"""GPU field and point arithmetic against the oracle: F_p operations against Python
integers, the batched-affine adder against the chord-and-tangent rule, and the
fixed-base generator against the oracle's fixed-base points."""
import random

import numpy as np
import pytest

import oracle
from oracle import ref
from elliptic_curve_scalar_amd import workloads as wl

from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu
P = ref.P


def _words(vals):
    return wl.from_ints(vals)


EDGE = [0, 1, 2, 3, P - 1, P - 2, (1 << 256) % P, (1 << 255) % P, P // 2, P // 2 + 1, P // 3,
        (1 << 224) - 1, (1 << 32) - 1, (1 << 32), 0xFFFFFFFF << 224 & ((1 << 254) - 1)]
EDGE = [e % P for e in EDGE]


@pytest.mark.parametrize("op", [0, 1, 2, 3, 4, 5, 6])
def test_fp_ops_match_python(op):
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(100 + op)
    n = 4099  # several blocks and a ragged tail
    edge = EDGE
    if op == 4:  # the binary-GCD inverse: powers of two and their neighbours, tiny values
        edge = EDGE + [1 << k for k in range(254)] + [P - (1 << k) for k in range(254)] + \
            [(1 << k) - 1 for k in range(2, 254)] + list(range(4, 64))
    xs = edge + [rng.randrange(P) for _ in range(n - len(edge))]
    ys = list(reversed(edge)) + [rng.randrange(P) for _ in range(n - len(edge))]
    say("fp op", op, "n", n)
    got = wl.to_ints(to_host(M.test_fp(op, to_dev(_words(xs)), to_dev(_words(ys)))))
    rinv = pow(1 << 256, -1, P)
    if op == 0:
        want = [x * y * rinv % P for x, y in zip(xs, ys)]
    elif op == 1:
        want = [(x + y) % P for x, y in zip(xs, ys)]
    elif op == 2:
        want = [(x - y) % P for x, y in zip(xs, ys)]
    elif op == 3:
        want = [x * x * rinv % P for x in xs]
    elif op == 4:  # (xR)^-1 R^2 = x^-1 R
        want = [0 if x == 0 else pow(x, P - 2, P) * (1 << 512) % P for x in xs]
    elif op == 5:
        want = [x * (1 << 256) % P for x in xs]
    else:
        want = [x * rinv % P for x in xs]
    assert got == want


def test_named_field_hooks():
    """msm_test_fp_{mul, sqr, add, sub, inv} against Python integers."""
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(17)
    xs = EDGE + [rng.randrange(P) for _ in range(777)]
    ys = list(reversed(EDGE)) + [rng.randrange(P) for _ in range(777)]
    a, b = to_dev(_words(xs)), to_dev(_words(ys))
    rinv = pow(1 << 256, -1, P)
    want = {"mul": [x * y * rinv % P for x, y in zip(xs, ys)],
            "sqr": [x * x * rinv % P for x in xs],
            "add": [(x + y) % P for x, y in zip(xs, ys)],
            "sub": [(x - y) % P for x, y in zip(xs, ys)],
            "inv": [0 if x == 0 else pow(x, P - 2, P) * (1 << 512) % P for x in xs]}
    for name, w in want.items():
        say("named hook", name, "n", len(xs))
        got = wl.to_ints(to_host(M.test_fp_named(name, a, b if name not in ("sqr", "inv") else None)))
        assert got == w, name


@pytest.mark.parametrize("op", [7, 8])
def test_inverse_parts(op):
    """Fermat's inverse alone (op 7) and the binary-GCD inverse with no special case for
    0 (op 8): its fallback must map 0 to 0 and every other input to the inverse."""
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(300 + op)
    xs = [0, 1, 2, P - 1, P - 2] + [1 << k for k in range(0, 254, 7)] + \
        [P - (1 << k) for k in range(1, 254, 11)] + [rng.randrange(1, P) for _ in range(300)]
    say("fp op", op, "n", len(xs))
    got = wl.to_ints(to_host(M.test_fp(op, to_dev(_words(xs)))))
    assert got == [0 if x == 0 else pow(x, P - 2, P) * (1 << 512) % P for x in xs]


def _rand_dlogs(rng, n):
    return [rng.randrange(1, ref.R) for _ in range(n)]


def test_generator_matches_oracle():
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(7)
    ks = [0, 1, 2, 3, ref.R - 1, ref.R, ref.R + 1, (1 << 256) - 1] + _rand_dlogs(rng, 1025)
    say("g1_from_scalars n", len(ks))
    got = to_host(M.g1_from_scalars(to_dev(_words(ks))))
    want = oracle.g1_from_scalars(_words(ks))
    assert np.array_equal(got, want)
    assert ref.decode_point(got[0]) is None
    assert ref.decode_point(got[1]) == ref.G


@pytest.mark.parametrize("S", [4, 8, 16, 32])
def test_batched_affine_add_all_cases(S):
    """Every slot position sees every special case; slot 0 and slot S-1 included."""
    from elliptic_curve_scalar_amd import msm as M
    rng = random.Random(S)
    dl = _rand_dlogs(rng, 64)
    pts = oracle.g1_from_scalars(_words(dl))
    inf = np.zeros(16, np.uint32)
    negs = oracle.g1_from_scalars(_words([ref.R - d for d in dl]))
    A, B, kinds = [], [], []
    for i in range(8 * S + 3):  # ragged tail: the last lane has 3 live slots
        k = rng.randrange(6) if i % S not in (0, S - 1) else (i // S) % 6
        a, b = pts[rng.randrange(64)], pts[rng.randrange(64)]
        j = rng.randrange(64)
        if k == 1:
            a = inf
        elif k == 2:
            b = inf
        elif k == 3:
            a, b = pts[j], pts[j]
        elif k == 4:
            a, b = pts[j], negs[j]
        elif k == 5:
            a, b = inf, inf
        A.append(a)
        B.append(b)
        kinds.append(k)
    A, B = np.array(A), np.array(B)
    say("batched_add S", S, "n", len(A))
    got = to_host(M.test_batched_add(to_dev(A), to_dev(B), S))
    for i in range(len(A)):
        want = ref.add(ref.decode_point(A[i]), ref.decode_point(B[i]))
        assert ref.decode_point(got[i]) == want, (i, kinds[i])
    assert set(kinds) == set(range(6))
