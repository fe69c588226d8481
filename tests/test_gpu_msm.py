"""End-to-end MSM parity on the GPU through the C ABI, bit-exact against the oracle:

* every workload recipe at reduced sizes (several tiles, ragged n);
* the full-size workloads, against the oracle's Pippenger on the oracle's own points
  and against the linearity closed form (sum_i s_i r_i mod r) * G;
* knob invariance: the same bits for every S and several c;
* edge cases: n = 0, 1, 2, all-zero scalars, {P, P}, {P, -P}, infinity inputs,
  the arithmetic-progression point set, one giant bucket, and scalars over the
  whole 256-bit range.
"""
import random

import numpy as np
import pytest

import oracle
from oracle import ref
from elliptic_curve_scalar_amd import workloads as wl

from gpu_util import DEV, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _msm():
    from elliptic_curve_scalar_amd import msm as M
    return M


def _gpu_msm(pts, sc, c, S=8, sched=0):
    M = _msm()
    return to_host(M.msm(to_dev(pts), to_dev(sc), c, S, sched=sched))


@pytest.mark.parametrize("name,n", [("n256_c8", 256), ("n256_c8", 1000), ("n65536_c13", 4097),
                                    ("n262144_c13_edge", 6000), ("n1048576_c16", 3001),
                                    ("n4194304_c16_skew", 5000)])
def test_reduced_sizes_bit_exact(name, n):
    w = wl.generate(name, n=n)
    pts = oracle.g1_from_scalars(w["dlogs"])
    want = oracle.msm_pippenger(pts, w["scalars"], w["c"])
    for S in (w["S"],):
        say(name, "n", n, "c", w["c"], "S", S)
        got = _gpu_msm(pts, w["scalars"], w["c"], S)
        assert np.array_equal(got, want)
    assert ref.decode_point(want) == ref.msm_linear(wl.to_ints(w["dlogs"]), wl.to_ints(w["scalars"]))


@pytest.mark.parametrize("name", ["n256_c8", "n65536_c13", "n262144_c13_edge", "n1048576_c16",
                                  "n4194304_c16_skew"])
def test_full_size_workloads(name):
    """Full-size inputs: GPU-generated points must equal the oracle's, and the GPU MSM
    must equal the oracle's Pippenger and the closed form."""
    M = _msm()
    w = wl.generate(name)
    say(name, "generate points n", w["n"])
    k = to_dev(w["dlogs"])
    pts_gpu = M.g1_from_scalars(k)
    pts = oracle.g1_from_scalars(w["dlogs"])
    assert np.array_equal(to_host(pts_gpu), pts)
    sweep = wl.CONFIGS[name].get("S_sweep", (w["S"],))
    want = oracle.msm_pippenger(pts, w["scalars"], w["c"])
    sc = to_dev(w["scalars"])
    for S in sweep:
        say(name, "msm c", w["c"], "S", S)
        got = to_host(M.msm(pts_gpu, sc, w["c"], S))
        assert np.array_equal(got, want), S
    if w["n"] <= (1 << 20):
        lin = ref.msm_linear(wl.to_ints(w["dlogs"]), wl.to_ints(w["scalars"]))
        assert ref.decode_point(want) == lin


def test_knob_invariance():
    """Same inputs, every S, several c and both schedules: one answer (the sum is
    unique)."""
    w = wl.generate("n65536_c13", n=3000)
    pts = oracle.g1_from_scalars(w["dlogs"])
    want = oracle.msm_pippenger(pts, w["scalars"], 13)
    for sched in (0, 1):
        for c in (1, 5, 8, 11, 13, 16):
            for S in (4, 8, 16, 32):
                say("knobs sched", sched, "c", c, "S", S)
                assert np.array_equal(_gpu_msm(pts, w["scalars"], c, S, sched), want), (sched, c, S)


def test_prefix_store_placements():
    """The level kernel's slot state in private memory or LDS, with or without cached
    denominators, every S: the same bits, including the edge-case mix."""
    M = _msm()
    ctx = M.Context(0)
    try:
        for name, n in (("n65536_c13", 4000), ("n262144_c13_edge", 5000)):
            w = wl.generate(name, n=n)
            pts = oracle.g1_from_scalars(w["dlogs"])
            want = oracle.msm_pippenger(pts, w["scalars"], 13)
            for store in (0, 1, 2, 3, 4):
                ctx.set_prefix_store(store)
                for S in (4, 8, 16, 32):
                    say("prefix store", store, name, "S", S)
                    got = to_host(ctx.run(to_dev(pts), to_dev(w["scalars"]), 13, S))
                    assert np.array_equal(got, want), (name, store, S)
        with pytest.raises(M.MsmError):
            ctx.set_prefix_store(5)
    finally:
        ctx.close()


@pytest.mark.parametrize("device_state", [1, 0])
def test_walker_schedules(device_state):
    """The stream walker, slot state on the device or private, against the oracle: every
    S on uniform inputs, the edge-case mix, a giant bucket split over many chunks (the
    pair passes over partial sums) and all-equal points (every add a doubling)."""
    M = _msm()
    ctx = M.Context(0)
    try:
        ctx.set_walker_state(device_state)
        cases = []
        w = wl.generate("n65536_c13", n=5000)
        cases.append(("uniform", oracle.g1_from_scalars(w["dlogs"]), w["scalars"], 13))
        w = wl.generate("n262144_c13_edge", n=6000)
        cases.append(("edge", oracle.g1_from_scalars(w["dlogs"]), w["scalars"], 13))
        w = wl.generate("n65536_c13", n=6000)
        sc = w["scalars"].copy()
        sc[::2] = wl.from_ints([ref.R - 1])[0]
        cases.append(("giant", oracle.g1_from_scalars(w["dlogs"]), sc, 13))
        cases.append(("equal", np.repeat(_pts([987654321]), 700, axis=0),
                      wl.from_ints([ref.R - 5] * 700), 13))
        w = wl.generate("n4194304_c16_skew", n=5000)
        cases.append(("skew", oracle.g1_from_scalars(w["dlogs"]), w["scalars"], 16))
        for name, pts, sc, c in cases:
            want = oracle.msm_pippenger(pts, sc, c)
            for S in (4, 8, 16, 32):
                say("walker", name, "state", device_state, "c", c, "S", S)
                got = to_host(ctx.run(to_dev(pts), to_dev(sc), c, S, sched=1))
                assert np.array_equal(got, want), (name, S)
    finally:
        ctx.close()


@pytest.mark.parametrize("name", ["n65536_c13", "n1048576_c16", "n4194304_c16_skew"])
def test_walker_full_size(name):
    """The stream walker at full size (the S sweep at n = 2^20), against the oracle."""
    M = _msm()
    w = wl.generate(name)
    say("walker full size", name, "generate points n", w["n"])
    pts_gpu = M.g1_from_scalars(to_dev(w["dlogs"]))
    pts = oracle.g1_from_scalars(w["dlogs"])
    want = oracle.msm_pippenger(pts, w["scalars"], w["c"])
    sc = to_dev(w["scalars"])
    for S in wl.CONFIGS[name].get("S_sweep", (w["S"],)):
        say("walker full size", name, "c", w["c"], "S", S)
        assert np.array_equal(to_host(M.msm(pts_gpu, sc, w["c"], S, sched=1)), want), S


def test_pair_tree_schedule_invariance():
    """Batched-affine levels vs XYZZ levels: every split gives the same bits."""
    from elliptic_curve_scalar_amd import msm as M
    w = wl.generate("n262144_c13_edge", n=8000)
    pts = oracle.g1_from_scalars(w["dlogs"])
    want = oracle.msm_pippenger(pts, w["scalars"], 13)
    ctx = M.Context(0)
    try:
        for levels in (-1, 0, 1, 2, 5):
            ctx.set_affine_levels(levels)
            for S in (4, 32):
                say("affine levels", levels, "S", S)
                got = to_host(ctx.run(to_dev(pts), to_dev(w["scalars"]), 13, S))
                assert np.array_equal(got, want), (levels, S)
    finally:
        ctx.close()


def test_sync_entry_point():
    M = _msm()
    w = wl.generate("n256_c8")
    pts = oracle.g1_from_scalars(w["dlogs"])
    say("msm() sync n 256")
    got = M.msm_sync(to_dev(pts), to_dev(w["scalars"]), 8)
    assert got == list(oracle.msm_pippenger(pts, w["scalars"], 8))


def _pts(dl):
    return oracle.g1_from_scalars(wl.from_ints(dl))


def test_edge_cases():
    rng = random.Random(99)
    dl = [rng.randrange(1, ref.R) for _ in range(8)]
    pts = _pts(dl)
    negp = _pts([ref.R - dl[0]])
    inf = np.zeros((1, 16), np.uint32)
    cases = {
        "n1": (pts[:1], [12345]),
        "n2": (pts[:2], [ref.R - 1, 1]),
        "zero_scalars": (pts, [0] * 8),
        "dup_pair": (np.vstack([pts[:1], pts[:1]]), [77, 77]),
        "neg_pair": (np.vstack([pts[:1], negp]), [77, 77]),
        "p_p_m2p": (np.vstack([pts[:1], pts[:1], _pts([(ref.R - 2 * dl[0]) % ref.R])]), [5, 5, 5]),
        "inf_inputs": (np.vstack([inf, pts[:2], inf]), [3, 4, 5, 6]),
        "all_ones": (pts, [1] * 8),
        "r_minus_1": (pts, [ref.R - 1] * 8),
        "high_scalar": (pts[:2], [ref.R + 7, (1 << 254) - 1]),
    }
    for name, (p, s) in cases.items():
        sc = wl.from_ints(s)
        want = oracle.msm_pippenger(p, sc, 13)
        for c, S in ((13, 8), (4, 4), (16, 32)):
            say("edge", name, "c", c, "S", S)
            assert np.array_equal(_gpu_msm(p, sc, c, S), want), (name, c, S)


def test_empty_input():
    M = _msm()
    import torch
    say("n = 0")
    out = M.msm(torch.zeros((0, 16), dtype=torch.uint32, device=DEV),
                torch.zeros((0, 8), dtype=torch.uint32, device=DEV), 13)
    assert not to_host(out).any()


def test_equal_points_equal_scalars():
    """Every pair-tree add is a doubling: n copies of one point with one scalar."""
    dl = [123456789]
    p = np.repeat(_pts(dl), 1000, axis=0)
    sc = wl.from_ints([ref.R - 3] * 1000)
    want = oracle.msm_pippenger(p, sc, 13)
    say("all equal n 1000")
    assert np.array_equal(_gpu_msm(p, sc, 13, 8), want)


def test_arithmetic_progression_points():
    """The point set the pages report breaks affine partial sums (PR #23736)."""
    dl = wl.arithmetic_progression(4096, a=1234567, d=89)
    pts = oracle.g1_from_scalars(dl)
    sc = wl.generate("n65536_c13", n=4096)["scalars"]
    want = oracle.msm_pippenger(pts, sc, 13)
    for S in (4, 8, 32):
        say("AP set S", S)
        assert np.array_equal(_gpu_msm(pts, sc, 13, S), want)
    assert ref.decode_point(want) == ref.msm_linear(wl.to_ints(dl), wl.to_ints(sc))


def test_giant_bucket():
    """One bucket per window holds ~half of all entries (deep pair-tree)."""
    w = wl.generate("n65536_c13", n=6000)
    sc = w["scalars"].copy()
    sc[::2] = wl.from_ints([ref.R - 1])[0]
    pts = oracle.g1_from_scalars(w["dlogs"])
    want = oracle.msm_pippenger(pts, sc, 13)
    say("giant bucket n 6000")
    assert np.array_equal(_gpu_msm(pts, sc, 13, 8), want)


def test_full_range_scalars():
    """Every 256-bit scalar is accepted: the split reduces it mod r first. Expected
    values come from the oracle's unsigned Pippenger at c = 16 (16 windows cover all
    256 bits, so it adds s P for the integer s) and the closed form."""
    rng = random.Random(5)
    dl = [rng.randrange(1, ref.R) for _ in range(40)]
    ints = [(1 << 256) - 1, 1 << 255, ref.R, 2 * ref.R, 5 * ref.R + 3, (1 << 254) + 1,
            ref.R - 1, 0] + [rng.getrandbits(256) for _ in range(32)]
    pts = _pts(dl)
    sc = wl.from_ints(ints)
    want = oracle.msm_pippenger(pts, sc, 16)
    assert ref.decode_point(want) == ref.msm_linear(dl, [s % ref.R for s in ints])
    for c, S in ((1, 4), (8, 8), (13, 8), (16, 32)):
        say("full-range scalars c", c, "S", S)
        assert np.array_equal(_gpu_msm(pts, sc, c, S), want), (c, S)


def test_montgomery_form_scalars():
    """With MSM_SCALARS_MONTGOMERY each scalar word vector s is read as x 2^256 mod r and
    the result is sum x_i P_i, x_i = s_i 2^-256 mod r, for any 256-bit s_i (reduced or
    not). Expected values: the oracle's Pippenger on the integers x_i and the closed form."""
    M = _msm()
    rng = random.Random(17)
    dl = [rng.randrange(1, ref.R) for _ in range(300)]
    pts = _pts(dl)
    mont = [0, 1, ref.R - 1, ref.R, (1 << 256) - 1, (1 << 256) % ref.R] + \
        [rng.getrandbits(256) for _ in range(294)]
    rinv = pow(1 << 256, -1, ref.R)
    xs = [m * rinv % ref.R for m in mont]
    want = oracle.msm_pippenger(pts, wl.from_ints(xs), 13)
    assert ref.decode_point(want) == ref.msm_linear(dl, xs)
    ctx = M.Context(DEV)
    try:
        ctx.set_scalar_form(M.MSM_SCALARS_MONTGOMERY)
        for c, S in ((8, 8), (13, 8), (16, 16)):
            say("montgomery-form scalars c", c, "S", S)
            got = to_host(ctx.run(to_dev(pts), to_dev(wl.from_ints(mont)), c, S))
            assert np.array_equal(got, want), (c, S)
        ctx.set_scalar_form(M.MSM_SCALARS_INTEGER)  # back to integers: the same words mean s_i
        got = to_host(ctx.run(to_dev(pts), to_dev(wl.from_ints(xs)), 13, 8))
        assert np.array_equal(got, want)
    finally:
        ctx.close()


def test_timing_levels():
    """Level 1 times only the batched-affine kernels, level 2 every phase, 0 nothing;
    the result does not depend on the level."""
    M = _msm()
    w = wl.generate("n65536_c13", n=4000)
    pts = oracle.g1_from_scalars(w["dlogs"])
    want = oracle.msm_pippenger(pts, w["scalars"], 13)
    ctx = M.Context(0)
    try:
        for level in (0, 1, 2):
            say("timing level", level)
            ctx.set_timing(level)
            got = to_host(ctx.run(to_dev(pts), to_dev(w["scalars"]), 13, 8))
            assert np.array_equal(got, want)
            tm = ctx.timing_read()
            assert tm["runs"] == (1 if level else 0)
            assert (tm["level_kernel_ms"] > 0) == (level >= 1)
            assert (tm["sort_ms"] > 0) == (level == 2)
            assert (tm["final_ms"] > 0) == (level >= 1)
        with pytest.raises(M.MsmError):
            ctx.set_timing(3)
    finally:
        ctx.close()


def test_verify_flags_off_curve_points():
    """verify = 1: a good input gives the right point and MSM_OK; one point off the
    curve, or with a coordinate not reduced below p, gives MSM_ERR_OFF_CURVE (the
    pages' failure signal, PR #23736 "Correctness-harness fix") as an ordinary error."""
    M = _msm()
    w = wl.generate("n65536_c13", n=2000)
    pts = oracle.g1_from_scalars(w["dlogs"])
    want = oracle.msm_pippenger(pts, w["scalars"], 13)
    say("verify good input")
    got = to_host(M.msm(to_dev(pts), to_dev(w["scalars"]), 13, 8, verify=True))
    assert np.array_equal(got, want)
    bad = pts.copy()
    y = wl.to_ints(bad[777:778, 8:16])[0]
    bad[777, 8:16] = wl.from_ints([(y + 1) % ref.P])[0]          # y + 1: off the curve
    unreduced = pts.copy()
    x = wl.to_ints(unreduced[5:6, 0:8])[0]
    unreduced[5, 0:8] = wl.from_ints([x + ref.P])[0] if x + ref.P < (1 << 256) else unreduced[5, 0:8]
    for name, p in (("off-curve y", bad), ("x + p", unreduced)):
        say("verify", name)
        with pytest.raises(M.MsmError) as ei:
            M.msm(to_dev(p), to_dev(w["scalars"]), 13, 8, verify=True)
        assert ei.value.code == M.MSM_ERR_OFF_CURVE, name
    # the context stays usable after the error
    say("verify after error")
    assert np.array_equal(to_host(M.msm(to_dev(pts), to_dev(w["scalars"]), 13, 8)), want)


def test_two_streams_growing_n():
    """One context used alternately from two streams with growing n: every run sees
    its own workspace contents (the context orders its calls across streams)."""
    import torch
    M = _msm()
    ctx = M.Context(0)
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    try:
        outs = []
        for k, n in enumerate((500, 1200, 3000, 7000)):
            w = wl.generate("n65536_c13", n=n)
            pts = oracle.g1_from_scalars(w["dlogs"])
            s = s1 if k % 2 == 0 else s2
            with torch.cuda.stream(s):
                dp, ds = to_dev(pts), to_dev(w["scalars"])
                say("two streams n", n, "stream", k % 2)
                out = ctx.run(dp, ds, 13, 8, stream=s)
            outs.append((out, oracle.msm_pippenger(pts, w["scalars"], 13)))
        torch.cuda.synchronize()
        for out, want in outs:
            assert np.array_equal(out.cpu().numpy().astype(np.uint32), want)
    finally:
        torch.cuda.synchronize()
        ctx.close()


def test_alternating_shapes_one_context():
    """Shapes that alternate on one context (the layout plan is kept per shape, the
    workspace only grows): every run matches the oracle."""
    M = _msm()
    ctx = M.Context(0)
    try:
        for n, c in ((3000, 13), (700, 13), (3000, 13), (700, 9), (3000, 13)):
            w = wl.generate("n65536_c13", n=n)
            pts = oracle.g1_from_scalars(w["dlogs"])
            say("alternating shapes n", n, "c", c)
            out = ctx.run(to_dev(pts), to_dev(w["scalars"]), c, 8)
            assert np.array_equal(to_host(out), oracle.msm_pippenger(pts, w["scalars"], c)), (n, c)
    finally:
        ctx.close()
