#!/usr/bin/env python3
"""Routed tokens/s of the fused low-rank MoE router on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload headline]

A step is one full routing call (more_route_lowrank: sweep-order/weight packing
kernel + the fused router kernel) over one batch of synthetic tokens already
resident in HBM.  Prints ONE JSON line:
  value          routed tokens/s = N / mean step time
  roofline       the routing call alone (weights packed once: the projection
                 kernel streaming X, then the routing kernel), timed with HIP
                 events on its stream: algorithmic bytes (X + outputs +
                 weights) per call over its mean duration, against the 8 TB/s
                 HBM peak
  pct_roofline   roofline time / step time, roofline time = max(X bytes / 8 TB/s,
                 2N(hr + rM) / 2.5 PFLOP/s)
  cpu_baseline   the fp64 oracle on a bounded sample of the same tokens, timed
                 on the host cores (one thread on the first 4096 tokens, then
                 every thread; the CPU model is named)
  parity         the parity rule applied to the GPU routing call's results over
                 the oracle's sample (all N tokens when it fits the CPU budget):
                 gap-clear mismatches (0 expected) and the full rule
  fullrank       the fused full-rank (standard) router on the same tokens
  balance        the training forward with balancing statistics
                 (more_lowrank_balance_packed: routing with the full-softmax
                 normaliser, then the second sweep for psum, the dispatch
                 counts, L_bal and H_norm) on the same tokens, HIP-event timed
  backward       the backward pass (more_lowrank_backward_packed, Alg. 3) on
                 the same tokens with the routing call's selection, seeded
                 incoming gradients and the balancing call's lse, HIP-event
                 timed, against its HBM bound (read X once, write X_grad)
  dispatch       the expert dispatch (more_dispatch_sort: the N x k indices
                 the routing call returned -> expert-sorted slots + offsets),
                 HIP-event timed, algorithmic bytes (read N k indices, write
                 N k experts + N k slots + M + 1 offsets) against 8 TB/s
  sharded        experts cut into --shards shards (default 8): one shard's
                 routing call at the full N (one GPU's share of the routing)
                 and more_topk_merge over all N tokens' shard lists, HIP-event
                 timed, the merge against 8 TB/s over its algorithmic bytes,
                 plus the count of tokens whose merged selection differs
                 from the unsharded call
  configs        the routing call (weights packed once) on the other
                 workloads: prefill at h = 512 with both gates, r = 16, 64
                 and 128 at the headline's shape, the many-expert prefill
                 (N = 65536, h = 4096, M = 65536, r = 64, k = 16, full
                 softmax) and its decode (N = 256); HIP-event timed, against
                 the roofline max(algorithmic bytes / 8 TB/s, 2N(hr + rM) /
                 2.5 PFLOP/s).  Tokens are generated on the device (seeded
                 Gaussian rows, RMS-normalised, bf16: the same recipe); the
                 r = 16/64/128 legs reuse the headline's tokens
  context        published B200 figures of the paper (other hardware)
Only one GPU is supported: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
# the kernels one routing call of the headline workload runs (rocprofv3 names)
ROUTER_KERNELS = ("more::proj_kernel<2, 16, false, 3>", "more::route_kernel<8, false, 2, 8, false>")
KERNEL_NAME = " + ".join(ROUTER_KERNELS)
# the many-expert decode call takes the split-M form (K-part projection,
# one wave per (block, expert shard), merge of the shard lists)
DECODE_KERNELS = ("more::splitm_proj_kernel<4>", "more::splitm_route_kernel<16, true, 4>",
                  "more::merge_wave_kernel<16, true>")


def kernel_label(cfg):
    """Kernels of the timed routing call, by name where the workload fixes them."""
    if cfg.name == "headline":
        return KERNEL_NAME
    if cfg.name == "many_experts_decode":
        return " + ".join(DECODE_KERNELS)
    return "routing call (projection and routing kernels)"
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published (no sparsity)
# v_exp_f32 rate: 256 CUs x 4 SIMDs x 16 lanes per cycle at half rate (one wave64
# exp per 8 cycles, measured against v_fma_f32 at one per 4), 2.4 GHz
EXP_PEAK_PER_S = 256 * 4 * 16 / 2 * 2.4e9
BALANCE_KERNELS = ("more::proj_kernel<2, 16, false, 3>", "more::route_kernel<8, false, 2, 8, true>",
                   "more::psum_kernel<2, 8, 8>", "more::count_kernel", "more::colsum_kernel",
                   "more::stats_kernel")
CONTEXT = {
    "source": "MoRE: Scaling mixture of experts with hardware-aware low-rank routing (B200, bf16)",
    "note": "other hardware and other shapes; no figure is published at this workload",
    "router_alone_ms_EPa_h512_r64_k4_N262144": {"M2048": 1.68, "M8192": 6.09, "M16384": 11.95,
                                                "table": "Table 10(a)"},
    "standard_router_ms_same_setting": {"M2048": 8.20, "M8192": 27.90, "M16384": 45.30},
    "fused_vs_unfused_lowrank_speedup_h2048_M4096_r16_k4": {"B2": 1.4, "B256": 6.3, "figure": "Fig. 24"},
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-fullrank", action="store_true")
    ap.add_argument("--no-balance", action="store_true")
    ap.add_argument("--no-dispatch", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-sharded", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--configs-only", action="store_true", help="only the other workloads' legs")
    ap.add_argument("--shards", type=int, default=8)
    ap.add_argument("--fullrank-steps", type=int, default=3)
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, "
                         "both with --calib-copy) into profiles/traffic_<workload>.json and exit")
    ap.add_argument("--counters-from", nargs="+", metavar="PMC_DIR",
                    help="turn rocprofv3 --pmc runs of this script with SQ counters (SQ_BUSY_CYCLES, "
                         "SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_*) into profiles/counters_<workload>.json and exit")
    ap.add_argument("--whole-calls", type=int, default=11,
                    help="with --counters-from: routing-kernel dispatches of whole calls at the start of "
                         "each run (warmup + steps), left out: they include the ready-word polls")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device copy of 256 MiB three times (byte-counter calibration "
                         "for rocprofv3 --pmc runs)")
    return ap.parse_args()


def source_hash():
    """Hash of the HIP sources the routing call is built from: traffic counters
    taken on another version of its kernels are not reported.  The files that
    hold only the balancing, dispatch, backward, full-rank and shard-merge
    kernels are left out."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_router_top_amd", "csrc")
    other = {"k_backward.hip", "more_backward.h", "k_balance.hip", "more_balance.h", "k_sort.hip", "more_sort.h",
             "k_fullrank.hip", "more_fullrank.h", "k_fullrank_tiled.hip", "more_fullrank_tiled.h",
             "k_merge.hip", "more_merge.h"}
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip")) and name not in other:
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_counter(run_dir, counter):
    """Per-dispatch mean of `counter` (KiB) for each router kernel and the copy
    kernel in a rocprofv3 --pmc CSV (rows are per dimension instance; summed
    per dispatch).  "router" is the sum over the kernels of one routing call."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                kind = next((kn for kn in ROUTER_KERNELS if kn in name), None) or (
                    "copy" if "copyBuffer" in name else None)
                if kind:
                    key = (kind, row["Dispatch_Id"])
                    per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for kind in ROUTER_KERNELS + ("copy",):
        vals = [v for (k, _), v in per.items() if k == kind]
        if kind == "copy" and vals:
            # the calibration copies (256 MiB) are the large ones; the runtime
            # also copies the small inputs with the same kernel
            vals = [v for v in vals if v >= 0.5 * max(vals)]
        if not vals:
            raise SystemExit(f"no {kind} dispatches with {counter} in {run_dir}")
        out[kind] = (sum(vals) / len(vals), len(vals))
    out["router"] = (sum(out[kn][0] for kn in ROUTER_KERNELS), min(out[kn][1] for kn in ROUTER_KERNELS))
    return out


def write_traffic(args):
    from rank_router_top_amd import configs as CF
    cfg = CF.ALL[args.workload]
    copy_bytes = 256 << 20
    fetch = read_counter(args.traffic_from[0], "FETCH_SIZE")
    write = read_counter(args.traffic_from[1], "WRITE_SIZE")
    f_fac = copy_bytes / (fetch["copy"][0] * 1024.0)
    w_fac = copy_bytes / (write["copy"][0] * 1024.0)
    fb = fetch["router"][0] * 1024.0 * f_fac
    wb = write["router"][0] * 1024.0 * w_fac
    alg = algorithmic_bytes(cfg, cfg.k, False)
    res = {"workload": cfg.name, "kernel": KERNEL_NAME, "source_hash": source_hash(),
           "bytes_per_launch": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
           "algorithmic_bytes": alg, "traffic_over_algorithmic": (fb + wb) / alg,
           "fetch_factor": f_fac, "write_factor": w_fac,
           "router_dispatches": [fetch["router"][1], write["router"][1]],
           "per_kernel_fetch_bytes": {kn: fetch[kn][0] * 1024.0 * f_fac for kn in ROUTER_KERNELS},
           "per_kernel_write_bytes": {kn: write[kn][0] * 1024.0 * w_fac for kn in ROUTER_KERNELS},
           "copy_bytes": copy_bytes}
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg.name}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))
    return 0


N_SIMD, N_SE = 1024, 32   # MI355X: 256 CUs x 4 SIMDs; 8 XCDs x 4 shader engines


def write_counters(args):
    """Per-dispatch means of the SQ counters of the two routing-call kernels
    (the routing kernel over its packed-weight dispatches only) and what they
    give: the MFMA pipe's busy fraction (busy cycles per SIMD over the SQ's busy
    cycles per shader engine, one clock domain) and the instruction mix."""
    import csv
    import glob
    from rank_router_top_amd import configs as CF
    cfg = CF.ALL[args.workload]
    sums = {}
    for d in args.counters_from:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for fn in files:
            per = {}
            with open(fn) as f:
                for row in csv.DictReader(f):
                    kn = next((k for k in ROUTER_KERNELS if k in row["Kernel_Name"]), None)
                    if kn:
                        key = (kn, row["Counter_Name"], int(row["Dispatch_Id"]))
                        per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
            route_ids = sorted({di for (kn, _, di) in per if kn == ROUTER_KERNELS[1]})
            whole = set(route_ids[:args.whole_calls])
            for (kn, c, di), v in per.items():
                if kn == ROUTER_KERNELS[1] and di in whole:
                    continue
                sums.setdefault((kn, c), []).append(v)
    kernels = {kn: {c: sum(v) / len(v) for (k2, c), v in sums.items() if k2 == kn} for kn in ROUTER_KERNELS}
    derived = {}
    for kn, cs in kernels.items():
        dd = {}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in cs and "SQ_BUSY_CYCLES" in cs:
            dd["mfma_busy_frac"] = (cs["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD) / (cs["SQ_BUSY_CYCLES"] / N_SE)
        if "SQ_ACTIVE_INST_ANY" in cs and "SQ_WAVE_CYCLES" in cs:
            dd["wave_issue_frac"] = cs["SQ_ACTIVE_INST_ANY"] / cs["SQ_WAVE_CYCLES"]
        if "SQ_WAIT_ANY" in cs and "SQ_WAVE_CYCLES" in cs:
            dd["wave_wait_frac"] = cs["SQ_WAIT_ANY"] / cs["SQ_WAVE_CYCLES"]
        derived[kn] = dd
    rk = kernels[ROUTER_KERNELS[1]]
    if cfg.name == "headline" and "SQ_INSTS_VALU" in rk:
        visits = (cfg.N // 32) * (24 + (cfg.M + 31) // 32)   # blocks x (seed + sweep) tile visits
        derived[ROUTER_KERNELS[1]]["per_wave_tile"] = {
            c.replace("SQ_INSTS_", "").lower(): rk[c] / visits for c in
            ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_BRANCH") if c in rk}
        derived[ROUTER_KERNELS[1]]["per_wave_tile"]["valu"] -= derived[ROUTER_KERNELS[1]]["per_wave_tile"].get("mfma", 0)
    res = {"workload": cfg.name, "source_hash": source_hash(), "n_simd": N_SIMD, "n_se": N_SE,
           "kernels": kernels, "derived": derived}
    path = os.path.join(ROOT, "profiles", f"counters_{cfg.name}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(derived))
    return 0


def algorithmic_bytes(cfg, k, with_lse):
    x = cfg.N * cfg.h * 2
    out = cfg.N * k * 8 + (cfg.N * 4 if with_lse else 0)
    if cfg.fullrank:
        w = cfg.h * cfg.M * 2
    else:
        w = (cfg.h * cfg.r + cfg.r * cfg.M) * 2
    w += cfg.M * 4 if cfg.has_bias else 0
    return x + out + w


def roofline_time_s(cfg):
    return max(cfg.x_bytes() / (HBM_PEAK_GBS * 1e9), cfg.flops() / (BF16_PEAK_TFLOPS * 1e12))


def time_events(torch, fn, steps, stream):
    """Mean ms of fn() over `steps` launches, each bracketed by its own events on `stream`."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    with torch.cuda.stream(stream):
        for s, e in ev:
            s.record(stream)
            fn()
            e.record(stream)
    stream.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in ev)
    return sum(ms) / len(ms), ms[len(ms) // 2], ms[len(ms) // 10], ms[(9 * len(ms)) // 10]


def device_tokens(torch, n, h, seed, dev):
    """Seeded Gaussian rows, RMS-normalised, as bf16 on the device."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    x = torch.randn((n, h), generator=g, device=dev, dtype=torch.float32)
    x = x * torch.rsqrt((x * x).mean(dim=1, keepdim=True))
    return x.to(torch.bfloat16)


CONFIG_LEGS = (("prefill_h512", 0), ("prefill_h512", 1), ("rank16", 0), ("rank64", 0), ("rank128", 0),
               ("many_experts_prefill", 1), ("many_experts_decode", 1))


def config_legs(args, torch, R, CF, dev, stream, X_headline):
    """The routing call (packed weights) on the other workloads."""
    out = {}
    X_many = None
    X_h512 = None
    for name, gate in CONFIG_LEGS:
        cfg = CF.ALL[name]
        Xs = None
        if name == "prefill_h512":
            # two token buffers, alternated call by call: one (268 MB) would
            # stay in the 256 MB Infinity Cache between calls
            if X_h512 is None:
                X_h512 = [device_tokens(torch, cfg.N, cfg.h, 1000 + 2 * args.seed + i, dev) for i in range(2)]
            Xs = X_h512
            X = Xs[0]
        elif name == "many_experts_prefill":
            X_many = device_tokens(torch, cfg.N, cfg.h, 2000 + args.seed, dev)
            X = X_many
        elif name == "many_experts_decode":
            X = X_many[:cfg.N] if X_many is not None else device_tokens(torch, cfg.N, cfg.h, 2000 + args.seed, dev)
        else:
            X = X_headline
        R1, R2, b = (R.to_device(a, dev) for a in cfg.weights(args.seed))
        nb = R.workspace_bytes(False, R.MORE_DT_BF16, cfg.N, cfg.h, cfg.r, cfg.M, cfg.k, gate, b is not None)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        R.pack_lowrank(R1, R2, b, ws, stream=stream)
        o = dict(idx=torch.empty((cfg.N, cfg.k), dtype=torch.int32, device=dev),
                 gate=torch.empty((cfg.N, cfg.k), dtype=torch.float32, device=dev),
                 logit=None, lse=torch.empty((cfg.N,), dtype=torch.float32, device=dev) if gate else None)

        turn = [0]

        def call():
            Xc = X if Xs is None else Xs[turn[0] & 1]
            turn[0] += 1
            R.route_lowrank_packed(Xc, cfg.r, cfg.M, cfg.k, gate, ws, out=o, stream=stream)

        for _ in range(3):
            call()
        mean, med, p10, p90 = time_events(torch, call, 20, stream)
        alg = algorithmic_bytes(cfg, cfg.k, gate == 1)
        flops = cfg.flops()
        t_hbm, t_mfma = alg / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
        roof = max(t_hbm, t_mfma)
        key = f"{name}/{'full_softmax' if gate else 'topk_softmax'}"
        out[key] = {"N": cfg.N, "h": cfg.h, "M": cfg.M, "r": cfg.r, "k": cfg.k, "bias": cfg.has_bias,
                    "ms_per_call": mean, "ms_median": med, "ms_p10": p10, "ms_p90": p90,
                    "tokens_per_s": cfg.N / (mean * 1e-3), "algorithmic_bytes": alg,
                    "hbm_gbs": alg / (mean * 1e-3) / 1e9, "mfma_tflops": flops / (mean * 1e-3) / 1e12,
                    "roofline_us": roof * 1e6, "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                    "frac": roof / (mean * 1e-3)}
        log(f"{key}: {mean:.4f} ms (roofline {roof * 1e6:.1f} us, frac {roof / (mean * 1e-3):.3f})")
        del ws
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(args, cfg, gate, X_np, R1_np, R2_np, b_np, ref):
    """The fp64 oracle on the host cores: one thread on the first 4096 tokens
    (per-core rate), then every thread on a sample of about --cpu-seconds of
    work (all N tokens when that fits), and the parity rule applied to the
    GPU routing call's results over that sample."""
    import numpy as np

    import oracle
    from oracle import parity as P
    oracle.build(force=False)
    threads = oracle.max_threads()
    n1 = min(4096, cfg.N)
    t = time.perf_counter()
    oracle.route_lowrank(X_np[:n1], R1_np, R2_np, b_np, cfg.k, gate, nthreads=1)
    one = n1 / (time.perf_counter() - t)
    n = int(min(cfg.N, max(n1, args.cpu_seconds * one * threads)))
    t = time.perf_counter()
    o = oracle.route_lowrank(X_np[:n], R1_np, R2_np, b_np, cfg.k, gate, nthreads=threads)
    dt_cpu = time.perf_counter() - t
    log(f"cpu oracle {n / dt_cpu:.0f} tokens/s on {threads} threads, {one:.0f} tokens/s on one")
    cpu = {"value": n / dt_cpu, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(), "one_thread_tokens_per_s": one, "one_thread_sample": f"first {n1} tokens",
           "sample": f"first {n} of the {cfg.N} tokens, same weights, fp64, {dt_cpu:.1f} s wall"}
    gpu = {key: (None if v is None else v[:n]) for key, v in ref.items()}
    at = oracle.logits_at(X_np[:n], R1_np, R2_np, b_np, gpu["idx"], nthreads=threads)
    par = {"tokens": n, "rule": "gap-clear index sets identical, gates within 1e-3; every index tied to its own "
                                "oracle logit and gate",
           "gap_clear_mismatches": P.mismatches(o, gpu["idx"])}
    try:
        par.update(P.compare(o, gpu, cfg.k, gate == 1, 2e-4, "bench", at))
        par["pass"] = True
    except AssertionError as e:
        par["pass"] = False
        par["failure"] = str(e)[:300]
    par["max_gate_error"] = float(np.max(np.abs(gpu["gate"].astype(np.float64) - o["gate"])))
    log(f"parity over {n} tokens: {par}")
    return cpu, par


def main():
    args = parse()
    if args.traffic_from:
        return write_traffic(args)
    if args.counters_from:
        return write_counters(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this router benchmark runs on exactly one GPU; "
                                   "multi-GPU runs are not supported (token sharding would need no "
                                   "communication, so one GPU's share is the measured kernel)"}))
        return 2
    import numpy as np
    import torch

    from rank_router_top_amd import configs as CF
    from rank_router_top_amd import route as R

    cfg = CF.ALL[args.workload]
    assert not cfg.fullrank
    gate = cfg.gates[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.configs_only:
        Xh = device_tokens(torch, CF.HEADLINE.N, CF.HEADLINE.h, args.seed, dev)
        print(json.dumps({"configs": config_legs(args, torch, R, CF, dev, stream, Xh)}), flush=True)
        return 0

    t0 = time.time()
    log(f"generating {cfg.name}: N={cfg.N} h={cfg.h} M={cfg.M} r={cfg.r} k={cfg.k}")
    X_np = cfg.x_rows(args.seed)
    R1_np, R2_np, b_np = cfg.weights(args.seed)
    X = R.to_device(X_np, dev)
    R1, R2, b = (R.to_device(a, dev) for a in (R1_np, R2_np, b_np))
    log(f"inputs ready in {time.time() - t0:.1f}s")

    dt = R.MORE_DT_BF16
    nb = R.workspace_bytes(False, dt, cfg.N, cfg.h, cfg.r, cfg.M, cfg.k, gate, b is not None)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    out = dict(idx=torch.empty((cfg.N, cfg.k), dtype=torch.int32, device=dev),
               gate=torch.empty((cfg.N, cfg.k), dtype=torch.float32, device=dev),
               logit=None, lse=None)

    def step():
        R.route_lowrank(X, R1, R2, b, cfg.k, gate, out=out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_step = (t_end - t_start) * 1e3 / args.steps
    log(f"step {ms_step:.4f} ms")

    # the routing call alone (weights packed once, as for static weights)
    R.pack_lowrank(R1, R2, b, ws, stream=stream)

    def kernel_only():
        R.route_lowrank_packed(X, cfg.r, cfg.M, cfg.k, gate, ws, out=out, stream=stream)

    for _ in range(3):
        kernel_only()
    k_mean, k_med, k_p10, k_p90 = time_events(torch, kernel_only, max(args.steps, 20), stream)

    def pack_only():
        R.pack_lowrank(R1, R2, b, ws, stream=stream)

    p_mean = time_events(torch, pack_only, 20, stream)[0]
    log(f"routing call mean {k_mean:.4f} ms (p10 {k_p10:.4f}, p90 {k_p90:.4f}); pack {p_mean:.4f} ms")

    # the routing call's results over all N (logits too), for the parity check of the CPU leg
    ref = R.route_lowrank_packed(X, cfg.r, cfg.M, cfg.k, gate, ws, stream=stream)
    torch.cuda.synchronize()
    ref = {key: (None if v is None else v.cpu().numpy()) for key, v in ref.items()}

    alg_bytes = algorithmic_bytes(cfg, cfg.k, False)
    achieved = alg_bytes / (k_mean * 1e-3) / 1e9
    rt = roofline_time_s(cfg)
    # HBM bytes per launch from the committed rocprofv3 counter runs (FETCH_SIZE,
    # WRITE_SIZE, scaled by the same counters on a copy of known size); only
    # when they were taken on the current kernel sources
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{cfg.name}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash():
            traffic = tr.get("bytes_per_launch")
    # MFMA busy fraction and issue / wait fractions of the two kernels from the
    # committed SQ counter runs, under the same condition
    counters = None
    cpath = os.path.join(ROOT, "profiles", f"counters_{cfg.name}.json")
    if os.path.exists(cpath):
        with open(cpath) as f:
            cr = json.load(f)
        if cr.get("source_hash") == source_hash():
            counters = {"source": os.path.relpath(cpath, ROOT), **cr.get("derived", {})}

    result = {
        "metric": f"routed tokens/sec & % roofline, N={cfg.N} h={cfg.h} M={cfg.M} r={cfg.r} k={cfg.k}, 1 GPU",
        "value": cfg.N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy: RMS-normalised Gaussian tokens, Gaussian weights, N(0,0.5) bias)",
        "config": {"workload": cfg.name, "N": cfg.N, "h": cfg.h, "M": cfg.M, "r": cfg.r, "k": cfg.k,
                   "gate": "topk_softmax" if gate == 0 else "full_softmax", "bias": cfg.has_bias,
                   "parallelism": "single GPU"},
        "pct_roofline": rt / (ms_step * 1e-3),
        "roofline_time_us": rt * 1e6,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel_label(cfg), "kernel_ms": k_mean, "kernel_ms_median": k_med,
                     "kernel_ms_p10": k_p10, "kernel_ms_p90": k_p90,
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "mfma_tflops": cfg.flops() / (k_mean * 1e-3) / 1e12,
                     "pack_kernel_ms": p_mean, "counters": counters},
        "context": CONTEXT,
    }

    nbb = 0 if args.no_balance else R.balance_workspace_bytes(dt, cfg.N, cfg.h, cfg.r, cfg.M, cfg.k)
    if nbb > 0:
        wsb = torch.empty(nbb, dtype=torch.uint8, device=dev)
        R.pack_lowrank(R1, R2, b, wsb, stream=stream)
        bout = dict(out, lse=torch.empty((cfg.N,), dtype=torch.float32, device=dev),
                    psum=torch.empty((cfg.M,), dtype=torch.float32, device=dev),
                    counts=torch.empty((cfg.M,), dtype=torch.int32, device=dev),
                    stats=torch.empty((4,), dtype=torch.float32, device=dev))

        def balance_call():
            R.balance_lowrank_packed(X, cfg.r, cfg.M, cfg.k, gate, wsb, out=bout, stream=stream)

        for _ in range(3):
            balance_call()
        b_mean, b_med, b_p10, b_p90 = time_events(torch, balance_call, max(args.steps, 20), stream)
        st = bout["stats"].cpu().tolist()
        log(f"balance call mean {b_mean:.4f} ms (p10 {b_p10:.4f}, p90 {b_p90:.4f}); "
            f"L_bal {st[0]:.6f} H_norm {st[1]:.6f}")
        result["balance"] = {
            "entry": "more_lowrank_balance_packed", "value": cfg.N / (b_mean * 1e-3), "unit": "tokens/s",
            "ms_per_call": b_mean, "ms_median": b_med, "ms_p10": b_p10, "ms_p90": b_p90,
            "extra_ms_over_routing_call": b_mean - k_mean, "kernels": list(BALANCE_KERNELS),
            "L_bal": st[0], "H_norm": st[1],
            "exp_count_per_call": 2 * cfg.N * cfg.M,
            "exp_bound_ms_per_call": 2 * cfg.N * cfg.M / EXP_PEAK_PER_S * 1e3}
        if not args.no_backward:
            nbw = R.backward_workspace_bytes(dt, cfg.N, cfg.h, cfg.r, cfg.M, cfg.k)
            if nbw > 0:
                from rank_router_top_amd import inputs as I
                wsw_b = torch.empty(max(nbw, nbb), dtype=torch.uint8, device=dev)
                R.pack_lowrank(R1, R2, b, wsw_b, stream=stream)
                R.balance_lowrank_packed(X, cfg.r, cfg.M, cfg.k, gate, wsw_b, out=bout, stream=stream)
                tv_np, pb_np = I.make_grads(args.seed, 73, cfg.N, cfg.k, cfg.M)
                tv_t = torch.from_numpy(tv_np).to(dev)
                pb_t = torch.from_numpy(pb_np).to(dev)
                gout = dict(X_grad=torch.empty((cfg.N, cfg.h), dtype=torch.bfloat16, device=dev),
                            R1_grad=torch.empty((cfg.h, cfg.r), dtype=torch.float32, device=dev),
                            R2_grad=torch.empty((cfg.r, cfg.M), dtype=torch.float32, device=dev),
                            bias_grad=torch.empty((cfg.M,), dtype=torch.float32, device=dev))

                def backward_call():
                    R.backward_lowrank_packed(X, R1, R2, bout["idx"], tv_t, pb_t, bout["lse"], wsw_b, out=gout,
                                              stream=stream)

                for _ in range(2):
                    backward_call()
                w_mean, w_med, w_p10, w_p90 = time_events(torch, backward_call, max(args.steps // 2, 10), stream)
                w_bytes = 2 * cfg.N * cfg.h * 2 + (cfg.h * cfg.r + cfg.r * cfg.M) * 2 * 2 + cfg.N * cfg.k * 12
                w_ach = w_bytes / (w_mean * 1e-3) / 1e9
                log(f"backward call mean {w_mean:.4f} ms (p10 {w_p10:.4f}, p90 {w_p90:.4f})")
                result["backward"] = {
                    "entry": "more_lowrank_backward_packed", "value": cfg.N / (w_mean * 1e-3), "unit": "tokens/s",
                    "ms_per_call": w_mean, "ms_median": w_med, "ms_p10": w_p10, "ms_p90": w_p90,
                    "exp_count_per_call": 3 * cfg.N * cfg.M,
                    "mfma_flop_per_call": 2 * cfg.N * (3 * cfg.h * cfg.r + 4 * cfg.M * cfg.r),
                    "roofline": {"bound": "hbm", "achieved": w_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": w_ach / HBM_PEAK_GBS, "algorithmic_bytes_per_call": w_bytes}}
                del wsw_b, gout
        del wsb, bout

    if not args.no_dispatch:
        nk = cfg.N * cfg.k
        dws = torch.empty(max(R.dispatch_workspace_bytes(cfg.N, cfg.k, cfg.M), 1), dtype=torch.uint8, device=dev)
        dout = dict(sorted_expert=torch.empty((nk,), dtype=torch.int32, device=dev),
                    sorted_slot=torch.empty((nk,), dtype=torch.int32, device=dev),
                    offsets=torch.empty((cfg.M + 1,), dtype=torch.int32, device=dev))
        kernel_only()   # the routing call's own indices

        def dispatch_call():
            R.dispatch_sort(out["idx"], cfg.M, out=dout, workspace=dws, stream=stream)

        for _ in range(3):
            dispatch_call()
        d_mean, d_med, d_p10, d_p90 = time_events(torch, dispatch_call, max(args.steps, 20), stream)
        d_bytes = nk * 4 + 2 * nk * 4 + (cfg.M + 1) * 4
        d_ach = d_bytes / (d_mean * 1e-3) / 1e9
        log(f"dispatch call mean {d_mean:.4f} ms (p10 {d_p10:.4f}, p90 {d_p90:.4f})")
        result["dispatch"] = {
            "entry": "more_dispatch_sort", "ms_per_call": d_mean, "ms_median": d_med, "ms_p10": d_p10,
            "ms_p90": d_p90, "entries": nk, "digit_passes": 1 if cfg.M <= 4096 else -(-(cfg.M - 1).bit_length() // 12),
            "roofline": {"bound": "hbm", "achieved": d_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": d_ach / HBM_PEAK_GBS, "algorithmic_bytes_per_call": d_bytes}}
        del dws, dout

    if not args.no_sharded and cfg.M % args.shards == 0 and cfg.M // args.shards >= cfg.k:
        # Experts sharded over G GPUs: each GPU routes all N tokens over its
        # M / G experts (timed here at that real shape), then, after an
        # all-to-all of the candidates, merges N / G tokens' G lists; the
        # merge is timed here over all N tokens' lists.
        G = args.shards
        width = cfg.M // G
        nbs = R.workspace_bytes(False, dt, cfg.N, cfg.h, cfg.r, width, cfg.k, gate, True)
        wss = torch.empty(nbs, dtype=torch.uint8, device=dev)
        cand_l = torch.empty((G, cfg.N, cfg.k), dtype=torch.float32, device=dev)
        cand_i = torch.empty((G, cfg.N, cfg.k), dtype=torch.int32, device=dev)
        for g in range(G):
            R.pack_lowrank(R1, R2[:, g * width:(g + 1) * width].contiguous(),
                           b[g * width:(g + 1) * width].contiguous(), wss, stream=stream)
            so = R.route_lowrank_packed(X, cfg.r, width, cfg.k, gate, wss, stream=stream)
            cand_l[g].copy_(so["logit"])
            cand_i[g].copy_(so["idx"])
        torch.cuda.synchronize()

        def shard_call():   # shard G - 1 is packed in wss
            R.route_lowrank_packed(X, cfg.r, width, cfg.k, gate, wss, out=so, stream=stream)

        def merge_call():
            return R.topk_merge(cand_l, cand_i, None, cfg.M, width, gate, want_logit=False, stream=stream)

        for _ in range(3):
            shard_call()
            mo = merge_call()
        s_mean = time_events(torch, shard_call, max(args.steps, 20), stream)[0]
        m_mean, m_med, m_p10, m_p90 = time_events(torch, merge_call, max(args.steps, 20), stream)
        kernel_only()
        torch.cuda.synchronize()
        mism = int((mo["idx"] != out["idx"]).any(dim=1).sum())
        m_bytes = cfg.N * (G * cfg.k * 8 + cfg.k * 8)
        m_ach = m_bytes / (m_mean * 1e-3) / 1e9
        log(f"sharded: {G} shards of {width} experts, shard call {s_mean:.4f} ms, merge {m_mean:.4f} ms, "
            f"{mism} tokens differ from the unsharded call")
        result["sharded"] = {
            "entry": "more_topk_merge", "shards": G, "shard_width": width,
            "shard_call_ms": s_mean, "merge_ms": m_mean, "merge_ms_p10": m_p10, "merge_ms_p90": m_p90,
            "tokens_differing_from_unsharded": mism,
            "merge_roofline": {"bound": "hbm", "achieved": m_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": m_ach / HBM_PEAK_GBS, "algorithmic_bytes_per_call": m_bytes}}
        del wss, cand_l, cand_i

    if not args.no_fullrank:
        FR = CF.FULLRANK
        n_fr = cfg.N
        W_np, _, bw_np = FR.weights(args.seed)
        W, bw = R.to_device(W_np, dev), R.to_device(bw_np, dev)
        nbw = R.workspace_bytes(True, dt, n_fr, FR.h, 0, FR.M, FR.k, 0, True)
        wsw = torch.empty(nbw, dtype=torch.uint8, device=dev)

        def fr_step():
            R.route_fullrank(X, W, bw, FR.k, 0, out=out, workspace=wsw, stream=stream)

        fr_step()
        torch.cuda.synchronize()
        fr_ms = time_events(torch, fr_step, args.fullrank_steps, stream)[0]
        fr_roof = max(FR.x_bytes() / (HBM_PEAK_GBS * 1e9), FR.flops() / (BF16_PEAK_TFLOPS * 1e12))
        result["fullrank"] = {"value": n_fr / (fr_ms * 1e-3), "unit": "tokens/s", "ms_per_step": fr_ms,
                              "pct_roofline": fr_roof / (fr_ms * 1e-3), "bound": "mfma",
                              "tflops": FR.flops() / (fr_ms * 1e-3) / 1e12, "peak_tflops": BF16_PEAK_TFLOPS}
        log(f"fullrank {fr_ms:.3f} ms")
        del W, wsw

    if not args.no_configs:
        result["configs"] = config_legs(args, torch, R, CF, dev, stream, X)
    if not args.no_cpu:
        result["cpu_baseline"], result["parity"] = cpu_leg(args, cfg, gate, X_np, R1_np, R2_np, b_np, ref)

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = src.numel()

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
