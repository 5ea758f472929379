"""Benchmark: exact epsilon self-join on one MI355X.

One step is one complete self-join of the workload with its points already
resident in HBM: build_index, count_pass, plan_batches, and fill_pass of
every batch (pairs written to device memory).  The default workload is the
largest single-GPU one: N = 10,000,000 points, d = 18, 70% in 500 Gaussian
clusters (sigma = 0.01) and 30% uniform background, epsilon giving a mean of
256 neighbours per point.

Printed JSON (one line): throughput in distance evaluations computed per
second over the whole join (the candidates the count pass produced, minus
those the block box test settled without a distance), the refinement
kernel's roofline position (its duration measured with HIP events on the
stream it runs on), and the CPU oracle timed on a bounded sample of the same
workload.  The sample rows are also compared with the GPU's, and the pairs
whose binary64 squared distance lies within 1e-6 eps^2 of eps^2 counted.

    python bench.py [--steps K] [--warmup W] [--workload c2] [--no-cpu]
                    [--mode semijoin [--nq NQ]]

``--mode semijoin`` joins a separate query set (the workload's cluster
structure, rows from another seed; RT-HiSS Sec. II-A) against the points.
``--mode knn`` finds the exact k nearest neighbours of every point (RT-HiSS
Sec. VI, growing similarity searches from the workload's epsilon); its line
reports queries per second instead.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ε-self-join time + candidate dist evals/s and % of HBM/FP32 roofline, 1 GPU"
FP32_PEAK_TFLOPS = 157.3   # MI355X published fp32 vector peak (256 CUs, 2.4 GHz)
BAND_REL = 1e-6            # threshold band reported beside the result
FP16_PEAK_TFLOPS = 2500.0  # MI355X published dense fp16 matrix peak
INT8_PEAK_TOPS = 5000.0    # MI355X published dense int8 matrix peak
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def load_eps(name):
    with open(os.path.join(ROOT, "tests", "golden", "eps_configs.json")) as f:
        return json.load(f)[name]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--budget-frac", type=float, default=0.0,
                    help="batch budget as a fraction of the total mask (0 = free memory)")
    ap.add_argument("--refine", type=int, default=0, help="0 auto, 1 direct, 2 fp32 MFMA, 3 split-fp16 MFMA")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--mode", choices=("selfjoin", "semijoin", "knn"), default="selfjoin",
                    help="semijoin: a separate query set from the workload's structure; "
                         "knn: exact k nearest neighbours of every point")
    ap.add_argument("--k", type=int, default=0, help="kNN: neighbours per query (0 = the workload's k)")
    ap.add_argument("--eps0-scale", type=float, default=1.0,
                    help="kNN: first radius as a multiple of the workload's epsilon")
    ap.add_argument("--growth", type=float, default=0.0, help="kNN: radius factor (0 = estimated)")
    ap.add_argument("--grid-reach", type=int, default=1, choices=(1, 2),
                    help="2: cells of width eps/2 and a 5x5x5 stencil (fewer candidates)")
    ap.add_argument("--no-block-prune", action="store_true",
                    help="switch off the MFMA kernel's query-block/candidate-group box test")
    ap.add_argument("--nq", type=int, default=0, help="semi-join query rows (0 = as many as points)")
    ap.add_argument("--cell-order", type=int, default=0, choices=(0, 1, 2, 3),
                    help="order of the rows within a cell (0 = the library's choice)")
    ap.add_argument("--filter-bits", type=int, default=0, choices=(0, 8, 16),
                    help="operands of the 64-dimension filter above 64 dimensions: 8 = int8, 16 = fp16 "
                         "high halves, 0 = library default (8)")
    ap.add_argument("--mfma-products", type=int, default=0, choices=(0, 1, 3),
                    help="split-fp16 form above 64 dimensions: products per slab (0 = the library's choice)")
    ap.add_argument("--no-host", action="store_true",
                    help="skip the timing of the join delivered to pinned host memory")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1"}))
        log("bench.py: only --gpus 1 is supported (single-GPU self-join; no sharding in this build)")
        sys.exit(2)

    import numpy as np
    import torch
    import exact_range_similarity_amd as ersj
    from workloads import CONFIGS, make_config, make_queries, x_digest

    spec = CONFIGS[args.workload]
    rec = load_eps(args.workload)
    eps = float.fromhex(rec["eps"])
    t0 = time.time()
    X = make_config(args.workload)
    if x_digest(X) != rec["x_sha256"]:
        raise SystemExit("generated points differ from the ones epsilon was calibrated on")
    log(f"[bench] {args.workload}: n={X.shape[0]} d={X.shape[1]} eps={eps!r} "
        f"(generated in {time.time() - t0:.1f}s)")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    xt = torch.from_numpy(X).to(dev)
    semi = args.mode == "semijoin"
    Q, qt = X, None
    if semi:
        nq = args.nq if args.nq > 0 else X.shape[0]
        Q = make_queries(args.workload, nq, spec.seed + 1000, X.shape[0])
        qt = torch.from_numpy(Q).to(dev)
        log(f"[bench] semi-join: {nq} queries from the workload's structure (seed {spec.seed + 1000})")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if args.mode == "knn":
        run_knn(args, spec, rec, eps, X, xt, stream)
        return

    budget = 0
    if args.budget_frac > 0:
        h = ersj.build_index(xt, eps)
        if semi:
            ersj.set_queries(h, qt)
        ersj.count_pass(h)
        budget = int(ersj.get_stats(h)["total_mask_words"] * 8 * args.budget_frac)
        h.free()

    def step(timing):
        opts = ersj.default_options(timing=int(timing), refine_kernel=args.refine,
                                    grid_reach=args.grid_reach,
                                    block_prune=-1 if args.no_block_prune else 0,
                                mfma_products=args.mfma_products, cell_order=args.cell_order,
                                filter_bits=args.filter_bits)
        h = ersj.build_index(xt, eps, opts, stream)
        if semi:
            ersj.set_queries(h, qt, stream)
        ersj.count_pass(h, stream)
        nb = ersj.plan_batches(h, budget, stream)
        npairs = 0
        for part in ersj.iter_batches(h, nb, stream):
            npairs += part.shape[0]
            del part
        st = ersj.get_stats(h)
        h.free()
        return npairs, st

    for w in range(args.warmup):
        npairs, st = step(False)
        log(f"[bench] warmup {w}: pairs={npairs} batches={st['n_batches']}")

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    stats = []
    for k in range(args.steps):
        npairs, st = step(True)
        stats.append(st)
        log(f"[bench] step {k}: refine {st['refine_ms']:.2f} ms, pairs {npairs}")
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_start) / args.steps

    st = stats[-1]
    cand = st["total_candidates"]
    d = X.shape[1]
    launches = sum(s["refine_launches"] for s in stats)
    refine_ms = sum(s["refine_ms"] for s in stats)
    refined = sum(s["refined_candidates"] for s in stats)
    skipped = sum(s["skipped_candidates"] for s in stats)
    # comparisons the kernel computed: the block box test decides the rest
    # without a distance, so they carry no flops
    evaluated = refined - skipped
    avg_launch_ms = refine_ms / max(1, launches)
    kern = st["refine_kernel"]
    mfma = kern in (ersj.REFINE_MFMA, ersj.REFINE_MFMA16)
    f16 = kern == ersj.REFINE_MFMA16
    prods = st["mfma_products"]  # fp16 products per slab of the split form (1 or 3)
    # algorithmic flops per computed candidate: 2d + 3 for the expanded
    # form (a d-term dot product and the combination with the two norms),
    # 3d for the direct form (difference, square, sum per dimension); the
    # split-fp16 form executes one or three fp16 products per dimension but is
    # priced, like the others, by the work the distance needs
    # comparisons the d > 64 kernel settled from its first 64 dimensions
    # (the squared distance over them already exceeds the band) are priced
    # at 2 * 64 + 3 flops, the work that decided them
    partial = sum(s["partial_candidates"] for s in stats)
    per_cand = (2.0 * d + 3.0) if mfma else 3.0 * d
    flops_per_launch = (per_cand * (evaluated - partial) + (2.0 * 64 + 3.0) * partial) / max(1, launches)
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
    # against the peak of the dtype the contraction runs in; with the int8
    # filter (above 64 dimensions) the settled comparisons are priced at the
    # int8 peak and the refined ones at the fp16 peak: the peak is the work's
    # flops over the time the two parts take at their peaks
    i8 = f16 and st.get("filter_bits", 0) == 8 and st["last_filtered"]
    peak = FP16_PEAK_TFLOPS if f16 else FP32_PEAK_TFLOPS
    if i8 and launches:
        t_peak = ((2.0 * 64 + 3.0) * partial / (INT8_PEAK_TOPS * 1e12) +
                  per_cand * (evaluated - partial) / (FP16_PEAK_TFLOPS * 1e12)) / launches
        peak = flops_per_launch / t_peak / 1e12
    fp32_equiv = achieved
    # algorithmic HBM bytes of a launch: its result mask written once, and
    # the candidate and query rows read once (dimension-blocked, d padded to
    # a multiple of four)
    dpad = (d + 3) // 4 * 4
    mask_bytes = 8.0 * st["total_mask_words"] / max(1, st["n_batches"])
    hbm_bytes = mask_bytes + 4.0 * dpad * (X.shape[0] + (Q.shape[0] if semi else 0))
    hbm_gbs = hbm_bytes / (avg_launch_ms * 1e-3) / 1e9
    # the kernel that ran: the split-fp16 form on the whole-tile kernel up to
    # 64 dimensions and on prepared operands above; the fp32 MFMA form; the
    # direct form
    nb = (d + 3) // 4
    # above 64 dimensions the filter hands live blocks to the run kernel
    # (high halves, up to 24 slabs of 16 dimensions) or the block kernel
    nsl = 2 * (((nb + 3) // 4 + 1) // 2)
    second = "k_refine_g16_runs" if prods == 1 and nsl <= 24 else "k_refine_g16_blocks"
    kname = ("k_refine_m16" if nb <= 16 else
             f"k_filter16+{second}" if st["last_filtered"] else "k_refine_g16") if f16 else \
        "k_refine_mfma" if mfma else "k_refine_direct"
    traffic = None
    tname = ("filter16_" + second.split("_")[-1]) if "+" in kname else kname[2:]
    tfile = os.path.join(ROOT, "profiles", f"{tname}_{args.workload}_traffic.json")
    if os.path.exists(tfile):
        import hashlib
        with open(tfile) as f:
            trec = json.load(f)
        with open(os.path.join(ROOT, trec["source"]), "rb") as f:
            cur = hashlib.sha256(f.read()).hexdigest()
        if cur == trec["source_sha256"] and trec["workload"] == args.workload and not budget and not semi \
                and trec.get("mfma_products", prods) == prods \
                and trec.get("filter_bits", st.get("filter_bits", 0)) == st.get("filter_bits", 0) \
                and args.cell_order == 0 and args.grid_reach == 1 and not args.no_block_prune:
            traffic = trec["hbm_bytes_per_launch"]
    phases = {k: sum(s[k] for s in stats) / args.steps
              for k in ("build_ms", "count_ms", "plan_ms", "refine_ms", "recheck_ms", "expand_ms")}

    out = {
        "metric": METRIC,
        "value": evaluated / args.steps / wall,
        "unit": "candidate dist evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": (("i8/i32+" if i8 else "") + (f"f16x{prods}/f32" if prods > 1 else "f16/f32")) if f16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{args.workload}: {spec.desc}; eps for a mean of {spec.k} neighbours/point"
                         + (f"; semi-join of {Q.shape[0]} queries drawn from the same structure"
                            if semi else "")),
            "mode": args.mode, "n_queries": int(Q.shape[0]),
            "n": int(X.shape[0]), "d": int(d), "eps": rec["eps"], "k": spec.k, "seed": spec.seed,
            "batches": st["n_batches"], "budget_bytes": budget, "grid_reach": args.grid_reach,
            "block_prune": not args.no_block_prune,
            "refine_kernel": {1: "direct", 2: "mfma", 3: "mfma16"}.get(kern, "?"),
            "mfma_products": prods,
            "filter_bits": st.get("filter_bits", 0),
        },
        "join_wall_s": wall,
        "result_pairs": npairs,
        "result_pairs_per_s": npairs / wall,
        "value_note": "distance evaluations computed per second of whole-join wall time; the count pass's "
                      "candidates minus those the block box test settled without a distance",
        "candidates": cand,
        "candidates_per_s": cand / wall,
        "candidate_fraction_of_n2": cand / float(X.shape[0]) ** 2,
        "evaluated_fraction": evaluated / max(1, refined),
        "partial_fraction": partial / max(1, evaluated),
        "cells": st["cells"],
        "grid": st["grid"],
        "boundary_pairs": st["last_boundary_pairs"],
        "recheck_in": st["last_recheck_in"],
        "phase_ms": phases,
        "roofline": {
            "bound": "mfma" if mfma else "alu",
            "kernel": kname,
            "mfma_dtype": (("int8 filter over 64 dimensions (exact int32 sums), then " if i8 else "") +
                           ("f16 (hi/lo split), f32 accumulate" if prods == 3 else
                            "f16 (high halves; binary64 re-check of the wider band), f32 accumulate"))
                          if f16 else "f32" if mfma else None,
            "peak_note": ("settled comparisons at the int8 peak (5.0 POP/s), refined ones at the fp16 peak "
                          "(2.5 PFLOP/s), combined by time") if i8 else None,
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "flops_per_candidate": per_cand,
            "fp32_equivalent": {"achieved": fp32_equiv, "peak": FP32_PEAK_TFLOPS,
                                "frac": fp32_equiv / FP32_PEAK_TFLOPS} if f16 else None,
            "hbm": {"achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": hbm_gbs / HBM_PEAK_GBS,
                    "algorithmic_bytes_per_launch": hbm_bytes},
            "traffic": traffic,
            "flops_per_launch": flops_per_launch,
            "avg_launch_ms": avg_launch_ms,
            "launches": launches,
        },
    }

    if not args.no_host:
        # The same join with every batch delivered to pinned host memory
        # (fill_pass_host: batch b's copy overlaps batch b+1's refinement).
        # Reported beside the device-resident figure, never as `value`.
        host_buf = torch.empty((npairs + 1024, 2), dtype=torch.int32, pin_memory=True)

        def host_step():
            h = ersj.build_index(xt, eps, ersj.default_options(refine_kernel=args.refine), stream)
            if semi:
                ersj.set_queries(h, qt, stream)
            ersj.count_pass(h, stream)
            nb = ersj.plan_batches(h, budget, stream)
            got = ersj.join_to_host(h, nb, host_buf, stream)
            h.free()
            return got.shape[0], nb

        host_step()
        torch.cuda.synchronize()
        t0h = time.perf_counter()
        for _ in range(args.steps):
            hp, hnb = host_step()
        torch.cuda.synchronize()
        hwall = (time.perf_counter() - t0h) / args.steps
        out["host_delivery"] = {
            "ms_per_step": hwall * 1e3, "pairs": hp, "batches": hnb,
            "pair_bytes_per_s": hp * 8 / hwall,
            "note": "join + copy of every pair into pinned host memory; PCIe/xGMI-inclusive, not `value`",
        }
        log(f"[bench] host delivery: {hwall * 1e3:.1f} ms per step ({hnb} batches)")

    if args.copy_calib:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device copies done")

    if not args.no_cpu:
        import oracle
        def cpu_rows(rows):
            if semi:
                return oracle.semijoin_rows(Q, X, eps, rows)
            return oracle.join_rows(X, eps, rows)

        rows_probe = 4 * oracle.threads()
        t = time.perf_counter()
        cpu_rows(np.arange(rows_probe))
        per_row = (time.perf_counter() - t) / rows_probe
        nrows = int(max(rows_probe, min(Q.shape[0], args.cpu_seconds / max(per_row, 1e-9))))
        log(f"[bench] cpu oracle: {nrows} rows (~{per_row * nrows:.0f}s)")
        t = time.perf_counter()
        colptr, cols = cpu_rows(np.arange(nrows))
        dt = time.perf_counter() - t
        evals = nrows * X.shape[0]
        out["cpu_baseline"] = {
            "value": evals / dt, "unit": "candidate dist evals/s", "cores": oracle.threads(),
            "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{'query ' if semi else ''}rows 0..{nrows - 1} of {args.workload} against all "
                      f"{X.shape[0]} points (brute force, binary64, every pair evaluated), {dt:.1f}s",
            "sample_pairs": int(colptr[-1]),
            "full_join_s_extrapolated": dt * Q.shape[0] / nrows,
        }
        # the GPU's pairs of the same rows, from one more (untimed) join
        mism = sample_mismatches(args, ersj, xt, qt, eps, budget, stream, nrows, colptr, cols)
        band = None if semi else oracle.band_count(X, eps, BAND_REL, np.arange(nrows))
        out["threshold_band"] = {
            "rel": BAND_REL, "sample_rows": nrows,
            "oracle_band_pairs": band,
            "gpu_pairs_differing_from_oracle": mism,
            "note": "pairs of the sample rows with |D64 - fl(eps^2)| <= 1e-6 fl(eps^2) (binary64), and GPU pairs "
                    "of those rows that differ from the oracle's after the binary64 re-check",
        }
    print(json.dumps(out), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def sample_mismatches(args, ersj, xt, qt, eps, budget, stream, nrows, colptr, cols):
    """Pairs of query rows 0..nrows-1 in which one more GPU join (default
    options of the timed run) differs from the oracle's neighbour lists."""
    import numpy as np
    import torch
    opts = ersj.default_options(refine_kernel=args.refine, grid_reach=args.grid_reach,
                                block_prune=-1 if args.no_block_prune else 0,
                                mfma_products=args.mfma_products, cell_order=args.cell_order,
                                filter_bits=args.filter_bits)
    h = ersj.build_index(xt, eps, opts, stream)
    if qt is not None:
        ersj.set_queries(h, qt, stream)
    ersj.count_pass(h, stream)
    nb = ersj.plan_batches(h, budget, stream)
    keep = []
    for part in ersj.iter_batches(h, nb, stream):
        for s0 in range(0, part.shape[0], 1 << 27):  # torch indexing stays below 2^31 elements
            blk = part[s0:s0 + (1 << 27)]
            q = blk[:, 0].to(torch.int64) & 0xffffffff
            sel = q < nrows
            if bool(sel.any()):
                x = blk[:, 1].to(torch.int64)[sel] & 0xffffffff
                keep.append(((q[sel] << 32) | x).cpu())
        del part
    h.free()
    got = np.sort(torch.cat(keep).numpy()) if keep else np.zeros(0, dtype=np.int64)
    counts = np.diff(colptr).astype(np.int64)
    rows = np.repeat(np.arange(nrows, dtype=np.int64), counts)
    want = np.sort((rows << 32) | cols.astype(np.int64))
    return int(np.setxor1d(got, want).size)


def run_knn(args, spec, rec, eps, X, xt, stream):
    """One step = exact kNN of every point (ersj_knn) from eps0 = scale * eps."""
    import numpy as np
    import torch
    import exact_range_similarity_amd as ersj

    k = args.k if args.k > 0 else spec.k
    eps0 = eps * args.eps0_scale
    opts = ersj.default_options(timing=1, refine_kernel=args.refine, grid_reach=args.grid_reach,
                                block_prune=-1 if args.no_block_prune else 0,
                                mfma_products=args.mfma_products, cell_order=args.cell_order,
                                filter_bits=args.filter_bits)
    ids = None
    for w in range(args.warmup):
        ids, _, info = ersj.knn(xt, k, eps0, growth=args.growth, options=opts, stream=stream)
        log(f"[bench] knn warmup {w}: rounds {info['rounds']} queries {info['queries']}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    infos = []
    for step in range(args.steps):
        ids, dist, info = ersj.knn(xt, k, eps0, growth=args.growth, options=opts, stream=stream)
        infos.append(info)
        log(f"[bench] knn step {step}: rounds {info['rounds']} refine {info['refine_ms']:.2f} ms "
            f"select {info['select_ms']:.2f} ms")
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    info = infos[-1]
    n, d = X.shape
    refine_ms = sum(i["refine_ms"] for i in infos)
    launches = sum(i["refine_launches"] for i in infos)
    computed = sum(i["computed_candidates"] for i in infos)
    kern = info["refine_kernel"]
    mfma = kern in (ersj.REFINE_MFMA, ersj.REFINE_MFMA16)
    f16 = kern == ersj.REFINE_MFMA16
    # products per slab of the split form: three up to 64 dimensions, above
    # them the option's choice (high halves alone by default)
    prods = 3 if (d + 3) // 4 <= 16 or args.mfma_products == 3 else 1
    per_cand = (2.0 * d + 3.0) if mfma else 3.0 * d
    avg_launch_ms = refine_ms / max(1, launches)
    flops_per_launch = per_cand * computed / max(1, launches)
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
    peak = FP16_PEAK_TFLOPS if f16 else FP32_PEAK_TFLOPS
    phases = {key: sum(i[key] for i in infos) / args.steps
              for key in ("index_ms", "refine_ms", "recheck_ms", "select_ms")}
    out = {
        "metric": f"exact kNN queries/s (k={k}), 1 GPU",
        "value": n / wall,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": (f"f16x{prods}/f32" if prods > 1 else "f16/f32") if f16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {spec.desc}; exact kNN of every point, k={k}, first "
                               f"radius {args.eps0_scale} x the workload's eps",
                   "mode": "knn", "n": int(n), "d": int(d), "k": int(k), "eps0": eps0.hex(),
                   "growth": args.growth, "grid_reach": args.grid_reach,
                   "block_prune": not args.no_block_prune},
        "rounds": info["rounds"],
        "queries_per_round": info["queries"],
        "eps_per_round": info["eps"],
        "dim_estimate": info["dim_estimate"],
        "candidates": info["total_candidates"],
        "phase_ms": phases,
        "roofline": {
            "bound": "mfma" if mfma else "alu",
            "kernel": (("k_refine_m16" if (d + 3) // 4 <= 16 else "k_refine_g16") if f16
                       else "k_refine_mfma" if mfma else "k_refine_direct"),
            "mfma_dtype": (("int8 filter over 64 dimensions (exact int32 sums), then " if i8 else "") +
                           ("f16 (hi/lo split), f32 accumulate" if prods == 3 else
                            "f16 (high halves; binary64 re-check of the wider band), f32 accumulate"))
                          if f16 else "f32" if mfma else None,
            "peak_note": ("settled comparisons at the int8 peak (5.0 POP/s), refined ones at the fp16 peak "
                          "(2.5 PFLOP/s), combined by time") if i8 else None,
            "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": None,
            "flops_per_launch": flops_per_launch, "avg_launch_ms": avg_launch_ms, "launches": launches,
        },
    }
    if not args.no_cpu:
        import oracle
        probe = 2 * oracle.threads()
        t = time.perf_counter()
        oracle.knn(X, k, np.arange(probe))
        per_row = (time.perf_counter() - t) / probe
        nrows = int(max(probe, min(n, args.cpu_seconds / max(per_row, 1e-9))))
        t = time.perf_counter()
        want, _ = oracle.knn(X, k, np.arange(nrows))
        dt = time.perf_counter() - t
        got = ids[:nrows].cpu().numpy().view(np.uint32)
        out["cpu_baseline"] = {
            "value": nrows / dt, "unit": "queries/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"rows 0..{nrows - 1} of {args.workload}: every point ranked (brute force, "
                      f"binary64, sort), {dt:.1f}s",
            "sample_matches_gpu": bool(np.array_equal(got, want)),
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
