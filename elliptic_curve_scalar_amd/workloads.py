"""Seeded synthetic workloads for the BN254 G1 MSM.

This module draws random integers only: the discrete logs r_i of the input points
(P_i = r_i * G) and the scalars s_i. It holds no field or curve arithmetic; each side
(the GPU library through its ``msm_g1_from_scalars`` entry point, the oracle through
its own fixed-base code) turns r_i into points by itself.

Random source: SplitMix64 (Steele, Lea and Flood, 2014) used as a counter-based
generator, word k of stream ``seed`` being mix(seed + (k + 1) * 0x9E3779B97F4A7C15).
A 254-bit draw takes four consecutive words as little-endian limbs, masks the top
limb to 62 bits and is accepted when below the group order r (rejection sampling).

Workloads (the pages measure n = 2^16 independent random points, PR #23736 "Change",
and the pair-tree accumulate at n = 2^16, c = 13, S = 8, PR #23520 "Measurements";
the larger shapes stretch the same recipe):

=====================  =======  ===  ==============  =========================================
name                   n        c    S               scalars
=====================  =======  ===  ==============  =========================================
n256_c8                2^8      8    8               uniform in [0, r)
n65536_c13             2^16     13   8               uniform in [0, r)
n262144_c13_edge       2^18     13   8               90% uniform; 0, 1, r-1, duplicate and
                                                     negated point pairs (see ``_edge``)
n1048576_c16           2^20     16   4, 8, 16, 32    uniform in [0, r)
n4194304_c16_skew      2^22     16   8               50% uniform in [0, 2^64), 50% in [0, r)
=====================  =======  ===  ==============  =========================================

The pages warn that points on an arithmetic progression make partial sums collide
in x (PR #23736, "Correctness-harness fix"); every workload therefore uses
independent points, and ``arithmetic_progression`` builds that degenerate set for a
separate test.
"""
from __future__ import annotations

import numpy as np

GROUP_ORDER = 0x30644E72E131A029B85045B68181585D2833E84879B9709143E1F593F0000001
_R64 = [(GROUP_ORDER >> (64 * i)) & 0xFFFFFFFFFFFFFFFF for i in range(4)]
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

CONFIGS = {
    "n256_c8": dict(n=1 << 8, c=8, S=8, point_seed=1001, scalar_seed=2001, kind="uniform"),
    "n65536_c13": dict(n=1 << 16, c=13, S=8, point_seed=1002, scalar_seed=2002, kind="uniform"),
    "n262144_c13_edge": dict(n=1 << 18, c=13, S=8, point_seed=1003, scalar_seed=2003,
                             kind="edge", layout_seed=3003),
    "n1048576_c16": dict(n=1 << 20, c=16, S=8, S_sweep=(4, 8, 16, 32), point_seed=1004,
                         scalar_seed=2004, kind="uniform"),
    "n4194304_c16_skew": dict(n=1 << 22, c=16, S=8, point_seed=1005, scalar_seed=2005,
                              kind="skew", coin_seed=3005),
}


def splitmix64(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Words start .. start+count-1 of the SplitMix64 stream ``seed`` (uint64)."""
    with np.errstate(over="ignore"):
        k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _below_r(l: np.ndarray) -> np.ndarray:
    """Row-wise test limbs < r for [m, 4] uint64 little-endian limbs."""
    r = [np.uint64(v) for v in _R64]
    lt = l[:, 0] < r[0]
    for i in (1, 2, 3):
        lt = (l[:, i] < r[i]) | ((l[:, i] == r[i]) & lt)
    return lt


def uniform_mod_r(seed: int, n: int, nonzero: bool = False) -> np.ndarray:
    """n integers uniform in [0, r) (or [1, r)) as [n, 4] uint64 limbs."""
    out = np.zeros((n, 4), dtype=np.uint64)
    have, cand = 0, 0
    top_mask = np.uint64((1 << 62) - 1)
    while have < n:
        m = max(1024, int((n - have) * 1.4) + 64)
        w = splitmix64(seed, 4 * m, start=4 * cand).reshape(m, 4)
        w[:, 3] &= top_mask
        ok = _below_r(w)
        if nonzero:
            ok &= (w != 0).any(axis=1)
        acc = w[ok]
        take = min(n - have, acc.shape[0])
        out[have:have + take] = acc[:take]
        have += take
        cand += m
    return out


def to_u32(limbs64: np.ndarray) -> np.ndarray:
    """[n, 4] uint64 limbs -> [n, 8] uint32 little-endian words."""
    return np.ascontiguousarray(limbs64, dtype=np.uint64).view(np.uint32).reshape(-1, 8).copy()


def to_ints(words32: np.ndarray):
    """[n, 8] uint32 words -> list of Python ints."""
    w = np.asarray(words32, dtype=np.uint32).reshape(-1, 8)
    l = w.astype(np.uint64)
    out = []
    for row in l:
        v = 0
        for i in range(7, -1, -1):
            v = (v << 32) | int(row[i])
        out.append(v)
    return out


def from_ints(values) -> np.ndarray:
    """Python ints (< 2^256) -> [n, 8] uint32 words."""
    vals = list(values)
    out = np.zeros((len(vals), 8), dtype=np.uint32)
    for i, v in enumerate(vals):
        for j in range(8):
            out[i, j] = (v >> (32 * j)) & 0xFFFFFFFF
    return out


def _neg_mod_r(limbs: np.ndarray) -> np.ndarray:
    """r - x for x in [1, r) as [m, 4] uint64 limbs (integer subtraction with borrow)."""
    out = np.zeros_like(limbs)
    borrow = np.zeros(limbs.shape[0], dtype=np.uint64)
    with np.errstate(over="ignore"):
        for i in range(4):
            ri = np.uint64(_R64[i])
            d = ri - limbs[:, i] - borrow
            nb = (limbs[:, i] > ri) | ((limbs[:, i] == ri) & (borrow == 1))
            out[:, i] = d
            borrow = nb.astype(np.uint64)
    return out


def _edge(cfg, n, dlogs, scalars):
    """Edge-case composition: the n indices form n/2 aligned pairs (2k, 2k+1); a
    seeded shuffle gives 2% of the pairs to each of five categories - scalar 0,
    scalar 1, scalar r-1, a duplicated point (P_{2k+1} = P_{2k}, equal scalars),
    a negated point (P_{2k+1} = -P_{2k}, equal scalars) - and leaves the other 90%
    uniform. Returns the per-pair category array."""
    npairs = n // 2
    per = (npairs * 2) // 100
    cat = np.zeros(npairs, dtype=np.int8)
    for k in range(5):
        cat[k * per:(k + 1) * per] = k + 1
    keys = splitmix64(cfg["layout_seed"], npairs)
    cat = cat[np.argsort(keys, kind="stable")]
    idx0 = 2 * np.arange(npairs)
    for k, val in ((1, 0), (2, 1), (3, GROUP_ORDER - 1)):
        sel = idx0[cat == k]
        v = np.array([(val >> (64 * i)) & 0xFFFFFFFFFFFFFFFF for i in range(4)], dtype=np.uint64)
        scalars[sel] = v
        scalars[sel + 1] = v
    dup = idx0[cat == 4]
    dlogs[dup + 1] = dlogs[dup]
    scalars[dup + 1] = scalars[dup]
    ng = idx0[cat == 5]
    dlogs[ng + 1] = _neg_mod_r(dlogs[ng])
    scalars[ng + 1] = scalars[ng]
    return cat


def generate(name: str, n: int | None = None):
    """Return dict(dlogs=[n,8] u32, scalars=[n,8] u32, c, S, name, n) for a workload.
    ``n`` overrides the size (same recipe, same seeds) for reduced-size tests."""
    cfg = dict(CONFIGS[name])
    n = cfg["n"] if n is None else int(n)
    dlogs = uniform_mod_r(cfg["point_seed"], n, nonzero=True)
    scal = uniform_mod_r(cfg["scalar_seed"], n)
    extra = {}
    if cfg["kind"] == "edge":
        if n % 2:
            raise ValueError("edge workload needs an even n")
        extra["pair_category"] = _edge(cfg, n, dlogs, scal)
    elif cfg["kind"] == "skew":
        coin = (splitmix64(cfg["coin_seed"], n) & np.uint64(1)).astype(bool)
        small = splitmix64(cfg["scalar_seed"] ^ 0x5EED5EED, n)
        scal[coin] = 0
        scal[coin, 0] = small[coin]
        extra["small"] = coin
    out = dict(name=name, n=n, c=cfg["c"], S=cfg["S"], dlogs=to_u32(dlogs), scalars=to_u32(scal))
    out.update(extra)
    return out


def arithmetic_progression(n: int, a: int, d: int):
    """Discrete logs r_i = a + i*d mod r: the degenerate point set (linear relation
    between the points) that the pages report makes affine partial sums collide."""
    return from_ints([(a + i * d) % GROUP_ORDER for i in range(n)])
