"""Oracle for the BN254 G1 multi-scalar multiplication.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product package, which must not
fall back to it.

Two independent parts:

* ``oracle.ref`` - exact Python-integer arithmetic (chord-and-tangent affine adds,
  double-and-add, the linearity closed form); slow, for small cases and closed forms;
* ``oracle.oracle.c`` - a plain C Pippenger on 4 x 64-bit limbs with Jacobian
  points, compiled with gcc into ``oracle/_build/liboracle.so`` and wrapped here.

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``
(primality of the constants, the group order, brute force on tiny inputs, Python
``int`` arithmetic, and the linearity identity).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")

ORACLE_OK = 0
ORACLE_ERR_ARG = -1
ORACLE_ERR_RANGE = -4
ORACLE_ERR_POINT = -5

_lib = None


def build() -> str:
    """Compile oracle.c with gcc (always recompiles)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    """Load the compiled oracle, building it only if nothing is built yet."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ORACLE_LIB") or LIB_PATH  # another build (the sanitizer test's)
    if path == LIB_PATH and not os.path.exists(LIB_PATH):
        build()
    L = ctypes.CDLL(path)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    I = ctypes.c_int
    sig = {
        "oracle_fp_op": (I, [I, P, P, P, S]),
        "oracle_g1_on_curve": (I, [P]),
        "oracle_g1_scalar_mul": (I, [P, P, P]),
        "oracle_g1_add": (I, [P, P, P]),
        "oracle_g1_from_scalars": (I, [P, S, P, I]),
        "oracle_threads_default": (I, []),
        "oracle_msm_naive": (I, [P, P, S, P]),
        "oracle_msm_pippenger": (I, [P, P, S, I, I, P]),
        "oracle_msm_pippenger_ex": (I, [P, P, S, I, I, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u32(a, cols):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint32))
    return a.reshape(-1, cols)


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle error {code}")
        self.code = code


def _check(rc):
    if rc != ORACLE_OK:
        raise OracleError(rc)


FP_MUL, FP_ADD, FP_SUB, FP_SQR, FP_INV, FP_TO_MONT, FP_FROM_MONT = range(7)


def fp_op(op: int, a, b=None):
    """Batched F_p operation on [n, 4] uint64 Montgomery-form inputs."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint64).reshape(-1, 4))
    bb = None if b is None else np.ascontiguousarray(np.asarray(b, dtype=np.uint64).reshape(-1, 4))
    out = np.zeros_like(a)
    _check(lib().oracle_fp_op(op, _ptr(a), _ptr(bb), _ptr(out), a.shape[0]))
    return out


def on_curve(pt_words) -> bool:
    p = _u32(pt_words, 16)
    return bool(lib().oracle_g1_on_curve(_ptr(p)))


def g1_add(p1, p2):
    a, b = _u32(p1, 16), _u32(p2, 16)
    out = np.zeros(16, dtype=np.uint32)
    _check(lib().oracle_g1_add(_ptr(a), _ptr(b), _ptr(out)))
    return out


def g1_scalar_mul(pt_words, k_words):
    p, k = _u32(pt_words, 16), _u32(k_words, 8)
    out = np.zeros(16, dtype=np.uint32)
    _check(lib().oracle_g1_scalar_mul(_ptr(p), _ptr(k), _ptr(out)))
    return out


def g1_from_scalars(k_words, threads: int = 0):
    """[n, 8] u32 scalars k_i -> [n, 16] u32 affine Montgomery points k_i * G."""
    k = _u32(k_words, 8)
    out = np.zeros((k.shape[0], 16), dtype=np.uint32)
    _check(lib().oracle_g1_from_scalars(_ptr(k), k.shape[0], _ptr(out), threads))
    return out


def threads_default() -> int:
    return int(lib().oracle_threads_default())


def msm_naive(points, scalars):
    p, s = _u32(points, 16), _u32(scalars, 8)
    out = np.zeros(16, dtype=np.uint32)
    _check(lib().oracle_msm_naive(_ptr(p), _ptr(s), p.shape[0], _ptr(out)))
    return out


def num_windows(c: int) -> int:
    return -(-254 // c)


def msm_pippenger(points, scalars, c: int, threads: int = 0, windows=False, buckets=False):
    """Plain Pippenger. Returns the output words, or (out, window_sums, bucket_sums)
    when either extra is requested (arrays of affine interchange points)."""
    p, s = _u32(points, 16), _u32(scalars, 8)
    n = p.shape[0]
    out = np.zeros(16, dtype=np.uint32)
    nwin = num_windows(c)
    wout = np.zeros((nwin, 16), dtype=np.uint32) if windows else None
    bout = np.zeros((nwin, 1 << c, 16), dtype=np.uint32) if buckets else None
    _check(lib().oracle_msm_pippenger_ex(_ptr(p), _ptr(s), n, c, threads, _ptr(out),
                                         _ptr(wout), _ptr(bout)))
    if windows or buckets:
        return out, wout, bout
    return out
