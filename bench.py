#!/usr/bin/env python3
"""Benchmark of the BN254 G1 multi-scalar multiplication on one MI355X.

One step = one whole MSM (decompose + sort, accumulate, bucket reduction, window
combine) over the n = 2^16, c = 13, S = 8 workload: independent random points
P_i = r_i * G and uniform scalars below r, the shape of the pages' measurements
(aztec-packages PR #23738 "Real-hardware data", PR #23520 "Measurements"). Inputs are
generated on the device before timing and stay resident.

Prints one JSON line: throughput in points/s (value), latency per MSM, the accumulate
kernel against the integer multiply-add roofline (roofline), the largest kernel of the
step against the same peak (roofline_largest), and the CPU oracle timed on this host's
cores on the same workload (cpu_baseline).

Other modes (one JSON line each, not the benchmark line):
  --probe-latency  latency of one wavefront's product and doubling chains, row form
                   against the per-lane and quad forms (msm_test_row);
  --probe-rates    sustained issue rates of the instruction classes the field code is
                   made of (msm_test_issue_rate), which set the integer roofline's peak;
  --cpu-table      the oracle on every workload, all host cores and one core.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MSM latency ms and points/sec at n=2^16,c=13; achieved int-VALU % of peak"

CLOCK_HZ = 2.4e9  # MI355X peak engine clock
N_CU = 256
# Peak rate of 32x32->64-bit multiply-adds (v_mad_u64_u32): 256 CUs x 4 SIMDs x 16
# lanes per clock x 2.4 GHz = 39.3 T/s; the 64-bit-result multiply issues at half the
# lane rate of plain 32-bit ALU ops (--probe-rates measures both classes).
PEAK_MAD_PER_S = N_CU * 4 * 16 * CLOCK_HZ
MAD_PER_MUL = 8 * 8 * 2 + 8          # CIOS Montgomery product on 8 x 32-bit limbs
MAD_PER_ADD = 6 * MAD_PER_MUL        # batched affine add: 5 products + 1 square
# The inverse that runs (Pornin's binary GCD in batches of 30 steps): each batch applies
# its factors to a, b (8 words x 2 multiply-adds each) and to u, v (8 words x 3, the third
# for the multiple of p), 80 multiply-adds; a wavefront runs until its slowest lane has
# converged, 13 batches for random inputs (the host model of the batches gives 13 in 97%
# of 64-lane waves, 14 otherwise). No product converts the result (the run starts from
# R^2 mod p).
INV_BATCHES = 13
MAD_PER_INV = INV_BATCHES * (2 * 16 + 2 * 24)
# A doubling in a run of the window combine (dbl-2008-s-1 written in U = 2Y with its ZZ,
# ZZZ updates folded into one factor): V, M X, M^2, z U, X V, (M X) V, M M^2, V^2, X'^2.
MAD_PER_DBL = 9 * MAD_PER_MUL


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the HIP sources: hardware counters taken on another build do not apply."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "elliptic_curve_scalar_amd", "csrc", "*"))):
        if f.endswith((".hip", ".hpp")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def counter_record(kind: str, workload: str, S: int, affine_levels: int, src: str):
    """A hardware-counter figure for the batched-affine kernel from the committed
    summaries under profiles/: kind "traffic" (HBM bytes per launch from rocprofv3
    FETCH_SIZE and WRITE_SIZE, scaled by a copy of known size) or "valu" (int-VALU
    issue %). None when no entry matches this workload, S, schedule and kernel source."""
    name = {"traffic": "k_level_hbm_traffic.md", "valu": "k_level_valu_counters.md"}[kind]
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if not line.startswith(kind + ": "):
                continue
            rec = json.loads(line[len(kind) + 2:])
            if (rec["workload"], rec["S"], rec["affine_levels"], rec["src"]) == (
                    workload, S, affine_levels, src):
                return rec
    return None


def plane_exponents(c: int) -> list[int]:
    """Exponents of the reduction's planes (the doubling-run lengths of the window
    combine), by the rule of make_planes in the library's host plan."""
    nwin = (128 + c - 1) // c
    lam = 3 if c >= 15 else 2
    slots = 1 << (c - 1)
    nseg = slots >> lam if slots > (1 << lam) else 1
    lgseg = (nseg - 1).bit_length()
    out = []
    for j in range(nwin):
        phi = c * nwin - 128 if j + 1 == nwin else 0
        out.append(c * j)
        out += [c * j + beta + lam - phi for beta in range(lgseg) if beta + lam >= phi]
    return out


def probe_rates(args) -> int:
    """Sustained issue rates of v_mad_u64_u32, v_add_u32 and the add-with-carry chain,
    from the msm_test_issue_rate hook timed with events over 8 waves per SIMD."""
    import torch

    from elliptic_curve_scalar_amd import msm as M

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    blocks = N_CU * 4 * 8 // 4          # 8 wavefronts per SIMD, 4 per 256-lane block
    iters = 4096
    out = torch.empty(blocks * 256, dtype=torch.uint32, device=dev)
    names = {0: "v_mad_u64_u32", 1: "v_add_u32", 2: "v_add_co_u32 / v_addc_co_u32"}
    res = {}
    for op in (0, 1, 2):
        M.test_issue_rate(op, blocks, iters, out)  # warm-up
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(5):
            ev0.record()
            M.test_issue_rate(op, blocks, iters, out)
            ev1.record()
            torch.cuda.synchronize()
            times.append(ev0.elapsed_time(ev1) * 1e-3)
        t = min(times)
        lane_ops = blocks * 256 * iters * 16
        per_cu_clk = lane_ops / t / CLOCK_HZ / N_CU
        res[names[op]] = {"lane_ops_per_s": lane_ops / t, "lane_ops_per_cu_per_clock": per_cu_clk,
                          "wave64_cycles_per_instr": 64 / (per_cu_clk / 4), "kernel_ms": t * 1e3}
        log(f"[probe] {names[op]}: {per_cu_clk:.1f} lane-ops/CU/clock, {t * 1e3:.3f} ms")
    print(json.dumps({"probe": "issue rates", "clock_hz_assumed": CLOCK_HZ, "cus": N_CU,
                      "waves_per_simd": 8, "rounds": iters, "chains_per_lane": 16,
                      "rates": res}), flush=True)
    return 0


def probe_latency(args) -> int:
    """Latency of one wavefront's dependent chains, from the msm_test_row hooks timed with
    events: a chain of 2000 Montgomery products in row form (one product per row of 16
    lanes, op 5) and with the per-lane product (op 6), and a run of 2000 doublings of one
    point in row form (op 3) and in the quad form (op 4)."""
    import random

    import torch

    from elliptic_curve_scalar_amd import msm as M
    from elliptic_curve_scalar_amd import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    P = 0x30644E72E131A029B85045B68181585D97816A916871CA8D3C208C16D87CFD47
    rng = random.Random(11)
    a = torch.from_numpy(wl.from_ints([rng.randrange(P) for _ in range(4)])).to(dev)
    b = torch.from_numpy(wl.from_ints([rng.randrange(P) for _ in range(4)])).to(dev)
    # one XYZZ point (X, Y, ZZ, ZZZ) = (x, y, 1, 1) in Montgomery form: the generator (1, 2)
    R = 1 << 256
    pt = torch.from_numpy(wl.from_ints([R % P, 2 * R % P, R % P, R % P]).reshape(1, 32)).to(dev)
    D = 2000

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = None
        for _ in range(5):
            ev0.record()
            fn()
            ev1.record()
            torch.cuda.synchronize()
            t = ev0.elapsed_time(ev1) * 1e3 / D  # us per step
            best = t if best is None else min(best, t)
        return best

    res = {
        "row_product_us": timed(lambda: M.test_row(5, a, b, D)),
        "lane_product_us": timed(lambda: M.test_row(6, a, b, D)),
        "row_doubling_us": timed(lambda: M.test_row(3, pt, None, D)),
        "quad_doubling_us": timed(lambda: M.test_row(4, pt, None, D)),
    }
    for k, v in res.items():
        log(f"[latency] {k}: {v:.3f}")
    print(json.dumps({"probe": "chain latency", "steps": D, **res}), flush=True)
    return 0


def cpu_table(args) -> int:
    """The oracle's Pippenger on every workload at the workload's c, with every host core
    (one thread per window, up to the cores there are) and with one core."""
    import oracle
    from elliptic_curve_scalar_amd import workloads as wl

    nproc = os.cpu_count() or 1
    for name in ("n256_c8", "n65536_c13", "n262144_c13_edge", "n1048576_c16", "n4194304_c16_skew"):
        w = wl.generate(name)
        t0 = time.perf_counter()
        pts = oracle.g1_from_scalars(w["dlogs"])
        gen_s = time.perf_counter() - t0
        row = {"cpu_table": name, "n": w["n"], "c": w["c"], "nproc": nproc,
               "point_generation_s": gen_s}
        for threads in (min(oracle.num_windows(w["c"]), oracle.threads_default()), 1):
            reps = 3 if w["n"] <= (1 << 20) else 1
            times = []
            for _ in range(reps):
                ts = time.perf_counter()
                oracle.msm_pippenger(pts, w["scalars"], w["c"], threads=threads)
                times.append(time.perf_counter() - ts)
            key = "one_core" if threads == 1 else "all_cores"
            row[key] = {"threads": threads, "ms": statistics.median(times) * 1e3, "reps": reps}
            log(f"[cpu] {name} threads={threads}: {statistics.median(times) * 1e3:.1f} ms")
        print(json.dumps(row), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="n65536_c13")
    ap.add_argument("--S", type=int, default=None, help="override the workload's S")
    ap.add_argument("--affine-levels", type=int, default=None,
                    help="pair-tree levels done with batched affine adds (-1: all)")
    ap.add_argument("--sched", type=int, default=0,
                    help="accumulate schedule: 0 pair tree, 1 stream walker")
    ap.add_argument("--walker-state", type=int, default=1,
                    help="stream walker slot state: 1 device buffer, 0 private memory")
    ap.add_argument("--prefix-store", type=int, default=0,
                    help="pair-tree level slot state: 0 private, 1 LDS, +2 cached "
                         "denominators, 4 checkpointed")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0,
                    help="CPU seconds for the oracle baseline (0 disables it)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB on the device once: "
                         "a kernel of known traffic for scaling hardware byte counters")
    ap.add_argument("--probe-latency", action="store_true",
                    help="latency of one wavefront's product and doubling chains (row vs per-lane)")
    ap.add_argument("--probe-rates", action="store_true",
                    help="measure instruction issue rates instead of the MSM")
    ap.add_argument("--cpu-table", action="store_true",
                    help="time the CPU oracle on every workload instead of the MSM")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2
    if args.probe_rates:
        return probe_rates(args)
    if args.probe_latency:
        return probe_latency(args)
    if args.cpu_table:
        return cpu_table(args)

    import numpy as np
    import torch

    from elliptic_curve_scalar_amd import msm as M
    from elliptic_curve_scalar_amd import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = wl.generate(args.workload)
    n, c = w["n"], w["c"]
    S = args.S or w["S"]
    log(f"[bench] workload {args.workload} n={n} c={c} S={S} sched={args.sched}")
    k = torch.from_numpy(w["dlogs"]).to(dev)
    scalars = torch.from_numpy(w["scalars"]).to(dev)
    points = M.g1_from_scalars(k)
    torch.cuda.synchronize()
    del k

    ctx = M.context(dev)
    if args.affine_levels is not None:
        ctx.set_affine_levels(args.affine_levels)
    ctx.set_walker_state(args.walker_state)
    ctx.set_prefix_store(args.prefix_store)
    out = torch.empty(16, dtype=torch.uint32, device=dev)
    for _ in range(args.warmup):
        ctx.run(points, scalars, c, S, out=out, sched=args.sched)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup})")

    # The timed steps bracket the accumulate kernel and the combine kernel with events
    # (timing level 1, both on the stream they run on); the per-phase breakdown comes from
    # separate, untimed steps afterwards (level 2).
    ctx.set_timing(1)
    ctx.timing_read()
    lat = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ts = time.perf_counter()
        ctx.run(points, scalars, c, S, out=out, sched=args.sched)
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - ts) * 1e3)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tm = ctx.timing_read()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ctx.set_timing(2)
    for _ in range(3):
        ctx.run(points, scalars, c, S, out=out, sched=args.sched)
    torch.cuda.synchronize()
    tm_phases = ctx.timing_read()
    ctx.set_timing(0)
    gpu_out = out.cpu().numpy().astype(np.uint32)
    if args.copy_mb > 0:
        src = torch.ones(args.copy_mb << 18, dtype=torch.int32, device=dev)
        dst = src.clone()
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    runs = max(1, tm["runs"])
    launches = max(1, tm["level_launches"])
    mads = tm["level_pairs"] * MAD_PER_ADD + tm["level_lanes"] * MAD_PER_INV
    level_s = tm["level_kernel_ms"] * 1e-3
    achieved = mads / level_s if level_s > 0 else 0.0
    al = args.affine_levels if args.affine_levels is not None else 1
    src = kernel_source_hash()
    tr = counter_record("traffic", args.workload, S, al, src) if args.sched == 0 else None
    vu = counter_record("valu", args.workload, S, al, src) if args.sched == 0 else None
    kname = f"k_level<{S}> (pair-tree level 0, batched affine)" if args.sched == 0 else \
        f"k_walk<{S}> (stream walker, batched affine)"
    roofline = {
        "bound": "alu",
        "kernel": kname,
        "achieved": achieved / 1e12,
        "peak": PEAK_MAD_PER_S / 1e12,
        "unit": "TOP/s",
        "op": "32x32->64-bit multiply-add (algorithmic count: 816 per add, "
              f"{MAD_PER_INV} per inversion)",
        "frac": achieved / PEAK_MAD_PER_S,
        "traffic": tr["bytes_per_launch"] if tr else None,
        "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
        "int_valu_pct": vu["int_valu_pct"] if vu else None,
        "launches_per_step": tm["level_launches"] / runs,
        "avg_launch_ms": tm["level_kernel_ms"] / launches,
        "algorithmic_ops_per_launch": mads / launches,
    }
    # the combine kernel: one run of doublings per plane, a wavefront each (latency-bound)
    exps = plane_exponents(c)
    fin_s = tm["final_ms"] * 1e-3 / runs
    fin_mads = sum(exps) * MAD_PER_DBL
    roofline_largest = {
        "bound": "alu",
        "kernel": "k_plane_chain (window combine: a run of doublings per plane, then the "
                  "planes' sum and the conversion to affine)",
        "achieved": (fin_mads / fin_s / 1e12) if fin_s > 0 else 0.0,
        "peak": PEAK_MAD_PER_S / 1e12,
        "unit": "TOP/s",
        "frac": (fin_mads / fin_s / PEAK_MAD_PER_S) if fin_s > 0 else 0.0,
        "traffic": None,
        "avg_launch_ms": fin_s * 1e3,
        "algorithmic_ops_per_launch": fin_mads,
        "critical_path": {"doublings": max(exps), "planes": len(exps),
                          "us_per_doubling_if_all": (fin_s * 1e6 / max(exps)) if exps else None},
    }
    # per-phase times (events around every phase, from 3 untimed steps)
    phases = {kk: tm_phases[kk] / max(1, tm_phases["runs"])
              for kk in ("sort_ms", "accumulate_ms", "level_kernel_ms", "xyzz_level_ms",
                         "reduce_ms", "final_ms")}

    cpu = None
    verified = None
    if args.cpu_budget_s > 0:
        import oracle
        pts_host = oracle.g1_from_scalars(w["dlogs"])
        nthreads = min(oracle.num_windows(c), oracle.threads_default())
        times = []
        t_start = time.perf_counter()
        want = None
        while True:
            ts = time.perf_counter()
            want = oracle.msm_pippenger(pts_host, w["scalars"], c, threads=nthreads)
            times.append(time.perf_counter() - ts)
            if time.perf_counter() - t_start > args.cpu_budget_s or len(times) >= 50:
                break
        med = statistics.median(times)
        verified = bool(np.array_equal(gpu_out, want))
        cpu = {"value": n / med, "unit": "points/s", "cores": nthreads,
               "cores_available": os.cpu_count(), "kind": "oracle",
               "sample": f"the full workload (n={n}, c={c}) run {len(times)} times, one "
                         f"thread per window up to the host's cores; median "
                         f"{med * 1e3:.1f} ms per MSM",
               "ms_per_msm": med * 1e3}
        log(f"[bench] oracle: {med * 1e3:.1f} ms/MSM on {nthreads} threads; verified={verified}")

    rec = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": f"BN254 G1 MSM, n={n}, c={c}, S={S}, independent random points "
                               f"r_i*G, scalars uniform in [0, r) ({args.workload})",
                   "n": n, "c": c, "S": S, "sched": ["pair_tree", "walker"][args.sched],
                   "prefix_store": args.prefix_store, "walker_state": args.walker_state},
        "latency_ms": {"median": statistics.median(lat), "min": min(lat)},
        "phases_ms_per_step": phases,
        "roofline": roofline,
        "roofline_largest": roofline_largest,
        "cpu_baseline": cpu,
        "verified_vs_oracle": verified,
        "workspace_bytes": M.workspace_bytes(n, c, S),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
