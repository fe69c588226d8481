"""Run by tests/test_host_sanitize.py in a subprocess with a sanitizer runtime preloaded
(not a test module): exercises the host code of a sanitizer build and exits non-zero on
the first mismatch; the sanitizers abort on the first error they find.

  python sanitize_driver.py oracle          the oracle build named by ORACLE_LIB
  python sanitize_driver.py libmsm LIB REF  the host code of libmsm build LIB (argument
                                            checks, workspace plans) against build REF
"""
import ctypes
import os
import random
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))


def check_oracle():
    import numpy as np

    import oracle
    from oracle import ref

    rng = random.Random(3)
    # field ops against Python integers
    xs = [0, 1, ref.P - 1] + [rng.randrange(ref.P) for _ in range(61)]
    ys = [rng.randrange(ref.P) for _ in xs]
    to4 = lambda v: [(v >> (64 * i)) & (2 ** 64 - 1) for i in range(4)]
    a = np.array([to4(x) for x in xs], dtype=np.uint64)
    b = np.array([to4(y) for y in ys], dtype=np.uint64)
    got = oracle.fp_op(oracle.FP_MUL, a, b)
    rinv = pow(1 << 256, -1, ref.P)
    for row, x, y in zip(got, xs, ys):
        assert sum(int(w) << (64 * i) for i, w in enumerate(row)) == x * y * rinv % ref.P
    # Pippenger against the closed form, every c, with the oracle's threads
    dl = [rng.randrange(1, ref.R) for _ in range(40)]
    sc = [rng.randrange(ref.R) for _ in range(40)] + [0, ref.R - 1]
    dl += [5, 7]
    pts = oracle.g1_from_scalars(np.array([ref.int_to_words(d) for d in dl], dtype=np.uint32))
    words = np.array([ref.int_to_words(s) for s in sc], dtype=np.uint32)
    want = ref.msm_linear(dl, sc)
    for c in (1, 4, 8, 13, 16):
        assert ref.decode_point(oracle.msm_pippenger(pts, words, c)) == want, c
    print("ok oracle")


def check_libmsm(path, ref_path):
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    libs = []
    for p in (path, ref_path):
        L = ctypes.CDLL(p)
        L.msm_workspace_bytes.restype = S
        L.msm_workspace_bytes.argtypes = [S, I, I]
        L.msm_run.restype = I
        L.msm_run.argtypes = [P, P, P, S, I, I, I, I, P, S, P, P]
        L.msm_run_noalloc.restype = I
        L.msm_run_noalloc.argtypes = [P, P, P, S, I, I, I, I, P, P]
        L.msm_last_error.restype = ctypes.c_char_p
        for name in ("msm_ctx_set_affine_levels", "msm_ctx_set_walker_state",
                     "msm_ctx_set_prefix_store", "msm_ctx_set_scalar_form", "msm_ctx_set_timing"):
            getattr(L, name).restype = I
            getattr(L, name).argtypes = [P, I]
        L.msm_test_row.restype = I
        L.msm_test_row.argtypes = [I, P, P, P, S, ctypes.c_uint32, P]
        L.msm_test_fp.restype = I
        L.msm_test_fp.argtypes = [I, P, P, P, S, P]
        libs.append(L)
    L, R = libs
    # workspace plans: every c and S over a range of n, identical to the plain build
    for n in (0, 1, 2, 3, 255, 256, 4097, 65536, 262144, 1 << 20, 1 << 22, 1 << 26):
        for c in range(1, 17):
            for s in (4, 8, 16, 32):
                assert L.msm_workspace_bytes(n, c, s) == R.msm_workspace_bytes(n, c, s), (n, c, s)
    assert L.msm_workspace_bytes(16, 0, 8) == 0 and L.msm_workspace_bytes(16, 17, 8) == 0
    # argument checks that return before any HIP call (a dummy context is never touched)
    ctx, p, out = P(4096), P(512), P(256)
    need = L.msm_workspace_bytes(16, 13, 8)
    cases = [
        (ctx, p, p, 16, 13, 5, 0, 0, None, 0, None, out),
        (ctx, p, p, 16, 13, 8, 2, 0, None, 0, None, out),
        (ctx, p, p, 16, 13, 8, 0, 2, None, 0, None, out),
        (ctx, p, p, 16, 0, 8, 0, 0, None, 0, None, out),
        (ctx, p, p, 16, 13, 8, 0, 0, None, 0, None, None),
        (ctx, P(520), p, 16, 13, 8, 0, 0, None, 0, None, out),
        (ctx, p, p, 16, 13, 8, 0, 0, P(1 << 20), need - 1, None, out),
        (None, p, p, 16, 13, 8, 0, 0, None, 0, None, out),
    ]
    for args in cases:
        assert L.msm_run(*args) == -1, args
        assert len(L.msm_last_error()) > 0
    assert L.msm_run_noalloc(None, p, p, 16, 13, 8, 0, 0, None, out) == -1
    assert L.msm_run_noalloc(ctx, p, p, 16, 17, 8, 0, 0, None, out) == -1
    for name, bad in (("msm_ctx_set_affine_levels", 33), ("msm_ctx_set_walker_state", 2),
                      ("msm_ctx_set_prefix_store", 5), ("msm_ctx_set_scalar_form", 2),
                      ("msm_ctx_set_timing", 3)):
        assert getattr(L, name)(None, 0) == -1 and getattr(L, name)(ctx, bad) == -1, name
    assert L.msm_test_row(10, p, p, p, 4, 0, None) == -1
    assert L.msm_test_row(7, p, None, p, 4, 0, None) == -1
    assert L.msm_test_fp(9, p, p, p, 4, None) == -1
    print("ok libmsm")


if __name__ == "__main__":
    if sys.argv[1] == "oracle":
        check_oracle()
    else:
        check_libmsm(sys.argv[2], sys.argv[3])
