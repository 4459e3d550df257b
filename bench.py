#!/usr/bin/env python3
"""Benchmark of the Periodic Row-wise Muon optimizer step on one MI355X.

One step is a full optimizer step of the whole parameter set (momentum, the
branch direction - NS5 on refresh steps, gamma * RowNorm otherwise - and the
weight update; plus AdamW on the per-block bias vectors).  Throughput is
optimizer steps/s averaged over whole K-cycles (the cycle average of paper
Eq. (9) in the PaperDaily post on "Scaling Muon for Diffusion Transformers").

Inputs are seeded synthetic DiT-shaped weights and bf16 gradients, resident
in HBM before the timed region.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import workloads  # noqa: E402

METRIC = "optimizer steps/s (K=3 cycle avg); NS5 MFMA %peak; RowNorm HBM GB/s"
PEAK_BF16 = 2.5e15        # dense bf16 MFMA, FLOP/s
PEAK_F32 = 157.3e12       # dense fp32 MFMA, FLOP/s
PEAK_HBM = 8.0e12         # bytes/s
ROWNORM_BYTES = 18        # per element: read G bf16 2 + M 4 + W 4, write M 4 + W 4


def ns5_class_flops(shapes, iters=5):
    """Algorithmic flops per refresh step, per kernel class.

    Per matrix and iteration (r short side, c long side): symmetric Gram
    r^2 c, symmetric A^2 r^3, product 2 r^2 c.
    """
    g = p = x = 0.0
    for m, n in shapes:
        r, c = min(m, n), max(m, n)
        g += r * r * c
        p += float(r) ** 3
        x += 2.0 * r * r * c
    return {"ns_gram": iters * g, "ns_poly": iters * p, "ns_product": (iters - 1) * x,
            "ns_product_last": x}


def ns5_class_bytes(shapes, es=2, lo=False):
    """Minimal HBM bytes per launch-set of each NS5 product class: every
    operand read once and every result written once (es = workspace bytes
    per value).  Gram: read X, write A; poly: read A, write B; product: read
    B and X, write X; last product: read B, X and W (fp32), write W.  With X's
    bf16 remainder (lo) the product also reads and rewrites it, and the last
    product reads it."""
    g = p = x = xl = 0.0
    for m, n in shapes:
        r, c = min(m, n), max(m, n)
        g += es * (r * c + r * r)
        p += es * 2 * r * r
        x += es * (r * r + 2 * r * c) + (4 * r * c if lo else 0)
        xl += es * (r * r + r * c) + 8 * r * c + (2 * r * c if lo else 0)
    return {"ns_gram": g, "ns_poly": p, "ns_product": x, "ns_product_last": xl}


def cnt_per(name: str, cfg) -> int:
    """Launch-sets of a class per refresh step (one per Newton-Schulz round;
    the last product runs once)."""
    if name == "ns_product_last":
        return 1
    return cfg.ns_iters - 1 if name == "ns_product" else cfg.ns_iters


KERNEL_SOURCES = {"ns_": "kernels_ns5.hip", "rownorm_": "kernels_rownorm.hip",
                  "adamw": "kernels_misc.hip"}


def source_digest(kernel: str) -> str:
    """sha256 over the device source of `kernel` (the .hip file that holds it
    and the header of structures it shares with the planner), so that counter
    figures taken on other code are not reported.  Host code (the launch
    planner) is left out: the counters follow the kernels."""
    import hashlib
    d = os.path.join(HERE, "matrix_aware_optimizer_periodic_amd", "csrc")
    src = next(f for p, f in KERNEL_SOURCES.items() if kernel.startswith(p))
    h = hashlib.sha256()
    for f in (src, "muon_internal.h"):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str, as_profiled: bool):
    """HBM bytes per launch of `kernel` from its committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE passes, scaled by a plain copy), or
    None when there is none, it was taken on other sources, or this run's
    launches differ from the profiled ones (`as_profiled` false: another NS5
    precision or workspace cap than the defaults the summaries were taken
    with)."""
    path = os.path.join(HERE, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not as_profiled or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def rownorm_class_bytes(shapes, gbytes, single_pass=True):
    """Algorithmic bytes per RowNorm step per kernel class (long-axis mode).

    Tall matrices with even n and at most 32768 rows take the single-pass
    kernel when it is enabled (read G, M, W; write M, W), the others the two
    passes (G, M -> M, then M, W -> W)."""
    rows = cols1 = cols2 = tall = 0
    for m, n in shapes:
        e = m * n
        if m > n:
            if single_pass and n % 2 == 0 and m <= 32768:
                tall += (gbytes + 16) * e
            else:
                cols1 += (gbytes + 8) * e      # read G, M; write M
                cols2 += 12 * e                # read M, W; write W
        else:
            rows += (gbytes + 16) * e
    return {"rownorm_rows": rows, "rownorm_cols1": cols1, "rownorm_cols2": cols2,
            "rownorm_tall": tall}


def cpu_baseline(wl, cfg_over, flop_budget=1.2e13):
    """The fp64 oracle as it stands, timed on one K-cycle of a sample of the
    set, then scaled to the whole set per branch.

    The sample is the first block's matrices, taken in the order proj, qkv,
    fc1, fc2, adaLN while their NS5 flops stay within ``flop_budget`` (on
    DiT-15B: proj and qkv, one wide and one tall matrix; on DiT-1.3B the
    whole block; a single-matrix set as it is).  Refresh steps (and MuonBP
    block steps) are scaled by algorithmic NS5 flops, RowNorm steps by
    elements, and the cycle average is paper Eq. (9)'s:
    K / (t_refresh + (K - 1) t_other)."""
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    ocfg = oracle.OracleConfig(**cfg_over)
    all_shapes = [(m, n) for _, m, n in wl.shapes]
    if wl.d:
        block = [(lab, m, n) for lab, m, n in wl.shapes[:len(workloads.dit_block_shapes(wl.d))]]
        order = {"proj": 0, "qkv": 1, "fc1": 2, "fc2": 3, "adaln": 4}
        block.sort(key=lambda x: order.get(x[0].split(".")[-1], 9))
        idx, shapes, f = [], [], 0.0
        for k, (lab, m, n) in enumerate(block):
            fk = sum(ns5_class_flops([(m, n)], ocfg.ns_iters).values())
            if shapes and f + fk > flop_budget:
                break
            idx.append(k)
            shapes.append((m, n))
            f += fk
        labels = [block[k][0].split(".")[-1] for k in idx]
    else:
        shapes, labels = list(all_shapes), [lab for lab, _, _ in wl.shapes]
    W = [workloads.host_weight0(0, i, s).astype(np.float64) for i, s in enumerate(shapes)]
    M = [np.zeros(s) for s in shapes]
    G = [workloads.host_grad(0, 0, i, s, wl.grad_std, wl.grad_dtype) for i, s in enumerate(shapes)]
    K = ocfg.K if ocfg.bp_blocks == 0 else ocfg.bp_period

    def one_step(t):
        t0 = time.perf_counter()
        for i in range(len(shapes)):
            W[i], M[i], _ = oracle.muon_matrix_step(W[i], M[i], G[i], t, ocfg)
        return time.perf_counter() - t0

    # one K-cycle (repeated while under a second, for the single small matrix)
    per_branch, t, t_start = {}, 0, time.perf_counter()
    while t < K or time.perf_counter() - t_start < 1.0:
        per_branch.setdefault(oracle.branch(t, ocfg), []).append(one_step(t))
        t += 1
    sample_seconds = time.perf_counter() - t_start

    def ns_flops(shp):
        return sum(ns5_class_flops(shp, ocfg.ns_iters).values())

    def blocks_of(shp):
        return [(m, n // ocfg.bp_blocks) for m, n in shp for _ in range(ocfg.bp_blocks)]

    scale = {oracle.BRANCH_NS5: ns_flops(all_shapes) / ns_flops(shapes),
             oracle.BRANCH_ROWNORM: sum(m * n for m, n in all_shapes) / sum(m * n for m, n in shapes)}
    if ocfg.bp_blocks:
        scale[oracle.BRANCH_BLOCK_NS5] = ns_flops(blocks_of(all_shapes)) / ns_flops(blocks_of(shapes))
    t_branch = {b: float(np.mean(v)) * scale[b] for b, v in per_branch.items()}
    other = oracle.BRANCH_BLOCK_NS5 if ocfg.bp_blocks else oracle.BRANCH_ROWNORM
    cycle_s = t_branch[oracle.BRANCH_NS5] + (K - 1) * t_branch.get(other, 0.0)
    names = {0: "rownorm", 1: "ns5", 2: "block_ns5"}
    exact = all(abs(v - 1.0) < 1e-12 for v in scale.values())
    out = {"value": K / cycle_s, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
           "cpu": cpu_model, "blas": blas, "numpy": np.__version__,
           "sample": (f"{len(shapes)} of {len(all_shapes)} matrices ({', '.join(labels)} of one "
                      f"block), {t} steps (t=0..{t - 1}); per-step times "
                      + ("of the whole set" if exact else
                         "extrapolated to the whole set by NS5 flops (refresh steps) and "
                         "elements (RowNorm steps)")
                      + f"; Eq. (9) cycle average over K={K}"),
           "branch_s": {names[b]: v for b, v in t_branch.items()},
           "sample_seconds": sample_seconds}
    if not wl.blocks:
        # the single-matrix set is small enough to time on one core as well
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                dt1 = sum(one_step(k) for k in range(K))
            out["value_1core"] = K / dt1
        except Exception:
            pass
    return out


def copy_calibration(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling HBM counters."""
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "reps": reps}))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=12)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dit-15b", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--ns-precision", choices=["bf16", "bf16-comp", "f32"], default="bf16",
                    help="NS5 products: bf16 MFMA; bf16 with X's rounding remainder in the a X "
                         "term; fp32 MFMA")
    ap.add_argument("--K", type=int, default=None, help="refresh period (default 3)")
    ap.add_argument("--no-adamw", action="store_true", help="leave out the bias vectors")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-flop-budget", type=float, default=1.2e13,
                    help="NS5 flops of the oracle's sample of matrices")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--ws-gib", type=float, default=None, help="NS5 workspace cap (GiB)")
    ap.add_argument("--tall-two-pass", action="store_true",
                    help="tall RowNorm in two passes instead of one")
    ap.add_argument("--print-digest", default="", metavar="KERNEL",
                    help="only print the device-source digest that keys KERNEL's counters")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the optimizer step is measured on one "
              "MI355X at the full per-GPU matrix shapes; --gpus must be 1", file=sys.stderr)
        return 2

    import torch
    import matrix_aware_optimizer_periodic_amd as mm

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return 0
    if args.print_digest:
        print(source_digest(args.print_digest))
        return 0

    wl = workloads.WORKLOADS[args.workload]
    over = dict(wl.overrides)
    if args.K is not None:
        over["K"] = args.K
    over["ns_precision"] = {"bf16": mm.MUON_NS_BF16, "bf16-comp": mm.MUON_NS_BF16_COMP,
                            "f32": mm.MUON_NS_F32}[args.ns_precision]
    if args.tall_two_pass:
        over["tall_single_pass"] = 0
    if args.ws_gib is not None:
        over["ns_workspace_max"] = int(args.ws_gib * 2 ** 30)
    # the committed counter summaries were taken with these defaults
    as_profiled = args.ns_precision == "bf16" and args.ws_gib is None and not args.tall_two_pass
    cfg = mm.muon_config_default(**over)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    shapes = [(m, n) for _, m, n in wl.shapes]
    gdt = torch.bfloat16 if wl.grad_dtype == "bf16" else torch.float32
    params, grads = [], []
    for i, s in enumerate(shapes):
        params.append(workloads.device_normal_(torch.empty(s, device=dev), 0.02,
                                               workloads.seed_for(0, 0, i, 2)))
        grads.append(workloads.device_normal_(torch.empty(s, dtype=gdt, device=dev),
                                              wl.grad_std, workloads.seed_for(0, 0, i, 1)))
    kinds = [mm.MUON_KIND_MATRIX] * len(shapes)
    n_bias = 0
    bias_elems = 0
    if not args.no_adamw and wl.d:
        for b in range(wl.blocks):
            for j, L in enumerate(workloads.dit_bias_sizes(wl.d)):
                params.append(workloads.device_normal_(torch.empty(L, device=dev), 0.02,
                                                       workloads.seed_for(0, b, j, 3)))
                grads.append(workloads.device_normal_(torch.empty(L, dtype=gdt, device=dev),
                                                      wl.grad_std, workloads.seed_for(0, b, j, 4)))
                kinds.append(mm.MUON_KIND_ADAMW)
                n_bias += 1
                bias_elems += L
    stream = torch.cuda.current_stream(dev)
    sess = mm.MuonSession(params, grads, kinds=kinds, cfg=cfg, stream=stream)
    torch.cuda.synchronize()

    K = cfg.K if cfg.bp_blocks == 0 else cfg.bp_period
    for t in range(args.warmup):
        sess.step(t)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` optimizer steps, events on the step stream.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(args.steps):
        starts[k].record(stream)
        sess.step(args.warmup + k)
    starts[args.steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = [starts[k].elapsed_time(starts[k + 1]) for k in range(args.steps)]
    total_ms = sum(step_ms)
    # Raises if a cross-workgroup wait of the single-pass tall RowNorm kernel
    # gave up in any step so far (those steps' weights would be wrong).
    sess.sync()

    # Per-kernel durations: the same steps again (same branch sequence, K | t0),
    # with the library's own HIP event pairs around every launch on its stream.
    kt = {}
    kt_branch = {}
    if not args.no_kernel_timing:
        t1 = args.warmup + args.steps
        t1 += (-(t1 - args.warmup)) % K
        mm.muon_timing_read(sess.ctx)          # clear
        mm.muon_timing_enable(sess.ctx, True)
        kt_branch = {}
        for k in range(args.steps):
            sess.step(t1 + k)
            torch.cuda.synchronize()
            rec = mm.muon_timing_read(sess.ctx)
            acc = kt_branch.setdefault(sess.branch(t1 + k), {})
            for name, (ms, cnt) in rec.items():
                a = acc.get(name, (0.0, 0))
                acc[name] = (a[0] + ms, a[1] + cnt)
        mm.muon_timing_enable(sess.ctx, False)
        sess.sync()
        for acc in kt_branch.values():
            for name, (ms, cnt) in acc.items():
                a = kt.get(name, (0.0, 0))
                kt[name] = (a[0] + ms, a[1] + cnt)

    branches = [sess.branch(args.warmup + k) for k in range(args.steps)]
    by_branch = {}
    for b, ms in zip(branches, step_ms):
        by_branch.setdefault(b, []).append(ms)
    names = {0: "rownorm", 1: "ns5", 2: "block_ns5"}
    branch_ms = {names[b]: float(np.mean(v)) for b, v in by_branch.items()}
    n_refresh = branches.count(mm.MUON_BRANCH_NS5)

    # ---- NS5 and RowNorm figures -------------------------------------------
    peak_mm = PEAK_F32 if args.ns_precision == "f32" else PEAK_BF16
    fl = ns5_class_flops(shapes, cfg.ns_iters)
    f_refresh = sum(fl.values())
    # MuonBP block steps orthogonalise bp_blocks column blocks of each matrix
    blk_shapes = [(m, n // cfg.bp_blocks) for m, n in shapes for _ in range(cfg.bp_blocks)] \
        if cfg.bp_blocks else []
    flb = ns5_class_flops(blk_shapes, cfg.ns_iters) if blk_shapes else {}
    f_block = sum(flb.values())
    n_block = branches.count(mm.MUON_BRANCH_BLOCK_NS5)
    ns5 = None
    if "ns5" in branch_ms:
        tf = f_refresh / (branch_ms["ns5"] * 1e-3)
        ns5 = {"step_ms": branch_ms["ns5"], "tflops": tf / 1e12, "frac": tf / peak_mm,
               "flops_alg": f_refresh}
    block_ns5 = None
    if "block_ns5" in branch_ms:
        tf = f_block / (branch_ms["block_ns5"] * 1e-3)
        block_ns5 = {"step_ms": branch_ms["block_ns5"], "tflops": tf / 1e12, "frac": tf / peak_mm,
                     "flops_alg": f_block}
    elems = sum(m * n for m, n in shapes)
    gbytes = 2 if gdt == torch.bfloat16 else 4
    rown = None
    if "rownorm" in branch_ms:
        bps = (gbytes + 16) * elems / (branch_ms["rownorm"] * 1e-3)
        rown = {"step_ms": branch_ms["rownorm"], "gbps": bps / 1e9, "frac": bps / PEAK_HBM,
                "bytes_alg": (gbytes + 16) * elems}

    roofline = None
    kernels = {}
    if kt:
        nb = rownorm_class_bytes(shapes, gbytes, bool(cfg.tall_single_pass))
        nsb = ns5_class_bytes(shapes, 4 if args.ns_precision == "f32" else 2,
                              lo=args.ns_precision == "bf16-comp")
        n_rn = branches.count(mm.MUON_BRANCH_ROWNORM)
        for name, (ms, cnt) in kt.items():
            if cnt == 0:
                continue
            rec = {"total_ms": ms, "launches": cnt, "avg_ms": ms / cnt}
            if name in fl and (n_refresh or n_block):
                per = (fl[name] * n_refresh + flb.get(name, 0.0) * n_block) / cnt
                rec.update(bound="mfma", work_per_launch=per, achieved=per / (ms / cnt * 1e-3) / 1e12,
                           unit="TFLOP/s", peak=peak_mm / 1e12)
                if not n_block:
                    rec["min_bytes_per_launch"] = nsb[name] * n_refresh * cnt_per(name, cfg) / cnt
            elif name in nb and n_rn:
                per = nb[name] * n_rn / cnt
                rec.update(bound="hbm", work_per_launch=per, achieved=per / (ms / cnt * 1e-3) / 1e9,
                           unit="GB/s", peak=PEAK_HBM / 1e9)
            if "achieved" in rec:
                rec["frac"] = rec["achieved"] / rec["peak"]
            kernels[name] = rec
        dom = max((k for k in kernels if "achieved" in kernels[k]),
                  key=lambda k: kernels[k]["total_ms"], default=None)
        if dom:
            r = kernels[dom]
            roofline = {"kernel": dom, "bound": r["bound"], "achieved": r["achieved"],
                        "peak": r["peak"], "unit": r["unit"], "frac": r["frac"],
                        "traffic": measured_traffic(dom, wl.name, as_profiled),
                        "avg_launch_ms": r["avg_ms"],
                        "work_per_launch": r["work_per_launch"]}
            if "min_bytes_per_launch" in r:
                roofline["min_bytes_per_launch"] = r["min_bytes_per_launch"]

    cpu = None
    if not args.no_cpu_baseline:
        ocfg = {k: v for k, v in over.items() if k in ("K", "bp_blocks", "bp_period", "bp_lr_ratio")}
        cpu = cpu_baseline(wl, ocfg, args.cpu_flop_budget)

    # Paper Eq. (9): one refresh and K - 1 other steps per cycle, from the
    # mean time of each branch over the timed steps, so that a timed window
    # that does not start or end on a cycle boundary still gives the cycle
    # average.  Without every branch in the window: the plain mean.
    other = mm.MUON_BRANCH_BLOCK_NS5 if cfg.bp_blocks else mm.MUON_BRANCH_ROWNORM
    if K == 1 and "ns5" in branch_ms:
        cycle_ms, value_kind = branch_ms["ns5"], "every step refreshes (K = 1)"
    elif "ns5" in branch_ms and names[other] in branch_ms:
        cycle_ms = (branch_ms["ns5"] + (K - 1) * branch_ms[names[other]]) / K
        value_kind = f"Eq. (9) cycle average: (t_ns5 + {K - 1} t_{names[other]}) / {K}"
    else:
        cycle_ms, value_kind = total_ms / args.steps, "mean over the timed steps (not a whole cycle)"
    value = 1e3 / cycle_ms
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": cycle_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.ns_precision == "f32" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "d": wl.d, "blocks": wl.blocks, "matrices": len(shapes),
            "matrix_elements": elems, "grad_dtype": wl.grad_dtype, "state_dtype": "f32",
            "K": cfg.K, "gamma": round(cfg.gamma, 6), "lr": round(cfg.lr, 6),
            "beta": round(cfg.beta, 6), "eps_row": cfg.eps_row,
            "ns_iters": cfg.ns_iters, "ns_coeffs": [round(cfg.ns_a, 6), round(cfg.ns_b, 6),
                                                    round(cfg.ns_c, 6)],
            "ns_eps": cfg.ns_eps, "ns_prenorm": "X / (||X||_F + ns_eps)",
            "ns_precision": args.ns_precision, "rownorm_axis": "long" if cfg.rownorm_axis == 0 else "rows",
            "tall_rownorm": "single-pass" if cfg.tall_single_pass else "two-pass",
            "bp_blocks": cfg.bp_blocks, "adamw_tensors": n_bias, "adamw_elements": bias_elems,
            "ns_workspace_max": int(cfg.ns_workspace_max), "state_bytes": sess.state_bytes,
        },
        "value_kind": value_kind,
        "timed_total_ms": total_ms,
        "branch_ms": branch_ms,
        "ns5": ns5,
        "block_ns5": block_ns5,
        "rownorm": rown,
        "roofline": roofline,
        "kernels": kernels,
        "kernel_ms_by_branch": {names[b]: {k: round(v[0] / max(1, branches.count(b)), 4)
                                           for k, v in acc.items() if v[1]}
                                for b, acc in kt_branch.items()},
        "cpu_baseline": cpu,
        "wall_s": wall,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out))
    sess.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
