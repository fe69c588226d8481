"""msm_run_noalloc (the entry point that allocates nothing; its workspace is a fixed
device array built into the library) against msm_run through the C ABI, bit-exact:
two calls in a row on one context, the second with a smaller input, and the size
limit reported as an ordinary argument error."""
import ctypes

import numpy as np
import pytest

import oracle
from elliptic_curve_scalar_amd import workloads as wl

from gpu_util import DEV, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_noalloc_matches_msm_run():
    import torch
    from elliptic_curve_scalar_amd import msm as M
    L = M.lib()
    ctx = M.Context(0)
    try:
        stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
        for name, n, c, S in (("n65536_c13", 8000, 13, 8), ("n256_c8", 3001, 8, 4)):
            w = wl.generate(name, n=n)
            assert M.workspace_bytes(n, c, S) <= M.MSM_NOALLOC_MAX_BYTES
            pts = to_dev(oracle.g1_from_scalars(w["dlogs"]))
            sc = to_dev(w["scalars"])
            say("msm_run n", n, "c", c, "S", S)
            want = to_host(ctx.run(pts, sc, c, S))
            out = torch.zeros(16, dtype=torch.uint32, device=DEV)
            say("msm_run_noalloc n", n, "c", c, "S", S)
            rc = L.msm_run_noalloc(ctx._h, ctypes.c_void_p(pts.data_ptr()),
                                   ctypes.c_void_p(sc.data_ptr()), n, c, S, 0, 0, stream,
                                   ctypes.c_void_p(out.data_ptr()))
            assert rc == M.MSM_OK, L.msm_last_error()
            got = to_host(out)
            assert np.array_equal(got, want), (n, c, S)
            assert np.array_equal(got, oracle.msm_pippenger(oracle.g1_from_scalars(w["dlogs"]),
                                                            w["scalars"], c))
        # beyond the fixed workspace: an argument error, nothing launched
        big = 1 << 16
        assert M.workspace_bytes(big, 13) > M.MSM_NOALLOC_MAX_BYTES
        rc = L.msm_run_noalloc(ctx._h, ctypes.c_void_p(256), ctypes.c_void_p(256), big, 13, 8, 0,
                               0, stream, ctypes.c_void_p(256))
        assert rc == M.MSM_ERR_ARG and b"MSM_NOALLOC_MAX_BYTES" in L.msm_last_error()
    finally:
        torch.cuda.synchronize()
        ctx.close()
