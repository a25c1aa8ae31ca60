"""Benchmark of the Periodic Row-wise Muon step on one MI355X.

One bench step is one Periodic cycle of K = 3 optimizer steps over the whole
layer set: an NS5 refresh step (momentum, Newton-Schulz, Eq. 4 update) followed
by K - 1 RowNorm steps; together they run every stage of the path. The default
workload is the 15B-scale layer set at H = 5120 (both streams: qkv [15360,5120],
proj [5120,5120], MLP [20480,5120] and [5120,20480], modulation [30720,5120];
944 M fp32 elements per state tensor), gradients 1e-3 * Student-t(3), all state
resident in HBM.

Prints ONE JSON line. `value` is the mean time of one Muon optimizer step
averaged over the Periodic cycle (ms, lower is better); `ms_per_step` is the time
of one whole cycle. Also reported: the vanilla (every step NS5) step time, NS5
TFLOP/s, RowNorm GB/s, the dominant kernel against its roofline (per-launch
HIP-event durations recorded by the library on the launch stream), the same step
figures for the other multi-matrix workloads (the H = 2048 DiT block, the 16-matrix
bucket, the H = 3072 MMDiT pair), the attainable ceilings measured in the same run
(the library's streaming copy kernel and its register-only MFMA loop, beside the spec
peaks), and the float64 oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Muon step ms per DiT block set; NS5 MFMA TFLOP/s; RowNorm HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP64_TFLOPS = 78.6     # MI355X dense fp64 MFMA

# The pages' own systems figures, reported beside this benchmark's as context only:
# "Scaling Muon for Diffusion Transformers" (summary page, results paragraph, and the
# abstract page): 256 H100 under FSDP2, optimizer time including communication,
# normalised to the 1.3B AdamW mean step time. Not the same metric or hardware.
PAGES_CONTEXT = {
    "source": "Scaling Muon for Diffusion Transformers, results paragraph and abstract: "
              "256 H100, FSDP2, communication included, normalised units; context, not a target",
    "periodic_optimizer_time_saving_pct": [46.9, 54.3],
    "optimizer_time_15b_normalised": {"vanilla": 2.884, "periodic": 1.317},
    "step_time_15b_normalised": {"vanilla": 6.527, "naive_periodic": 5.685, "periodic": 5.002},
    "logical_comm_gib_per_rank_step_15b": {"vanilla": 28.62, "periodic": 9.54},
}


def ns5_flops_sym(m, n, steps=5):
    """Algorithmic NS5 flops counting only the symmetric halves of X X^T and A A."""
    return steps * (3.0 * m * m * n + 1.0 * m ** 3)


def apply_flops(m, n):
    """The B X product of one iteration: [m, m] x [m, n]."""
    return 2.0 * m * m * n


def measured_traffic(kernel, workload_key):
    """HBM bytes per dispatch of `kernel` from the committed rocprofv3 counter summary
    (a list of names: the first kernel plus the others that run with it, e.g. a split
    stage's fixup).

    The summary records FETCH_SIZE / WRITE_SIZE per dispatch, the copy-kernel
    calibration factors and a hash of the GEMM sources; a changed kernel (or another
    workload) gets None, as counters taken on other code say nothing about it.
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", "hbm_traffic_15b_h5120.json")
    if workload_key != "15b" or not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    h = hashlib.sha256()
    for src in GEMM_SOURCES:
        with open(os.path.join(ROOT, "matrix_orthogonalising_optimizer_02_amd", "csrc", src), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != rec["gemm_source_sha256"]:
        return None
    kernels = [kernel] if isinstance(kernel, str) else list(kernel)
    entries = [rec["kernels"].get(k) for k in kernels]
    if entries[0] is None:
        return None
    return sum(e["hbm_bytes_per_dispatch"] for e in entries if e is not None)


GEMM_SOURCES = ["gemm_kernel.hpp", "k_gemm.hip", "launch.hpp", "common.hpp"]


def summarize_traffic(cal_fetch, cal_write, run_fetch, run_write, out):
    """Write the per-dispatch HBM traffic record that measured_traffic() reads.

    Inputs are rocprofv3 --pmc counter CSVs (run_counter_collection.csv): FETCH_SIZE and
    WRITE_SIZE of a calibration run (a torch copy of 2^28 fp32, 1 GiB read and 1 GiB
    written, dispatched as __amd_rocclr_copyBuffer) and of a benchmark run, each counter
    from its own run. Bytes = counter KiB x 1024 x the copy's calibration factor, averaged
    over each kernel's dispatches. The record carries the hash of the GEMM sources.
    """
    import collections
    import csv
    import hashlib

    def per_kernel(path, counter):
        per_dispatch, names = collections.defaultdict(float), {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                per_dispatch[r["Dispatch_Id"]] += float(r["Counter_Value"])
                names[r["Dispatch_Id"]] = r["Kernel_Name"]
        agg = collections.defaultdict(list)
        for d, v in per_dispatch.items():
            n = names[d]
            if "muon::" not in n and "rocclr_copyBuffer" not in n:
                continue
            short = n.replace("void ", "").split("(")[0]
            agg[short[len("muon::"):] if short.startswith("muon::") else short].append(v)
        return {k: sum(v) / len(v) for k, v in agg.items()}

    cf, cw = per_kernel(cal_fetch, "FETCH_SIZE"), per_kernel(cal_write, "WRITE_SIZE")
    ck = [k for k in cf if "copyBuffer" in k][0]
    gib_kib = 1024.0 * 1024.0
    ff, wf = gib_kib / cf[ck], gib_kib / cw[ck]
    bf, bw = per_kernel(run_fetch, "FETCH_SIZE"), per_kernel(run_write, "WRITE_SIZE")
    h = hashlib.sha256()
    for src in GEMM_SOURCES:
        with open(os.path.join(ROOT, "matrix_orthogonalising_optimizer_02_amd", "csrc", src), "rb") as fh:
            h.update(fh.read())
    rec = {"workload": "15B-scale layer set H=5120 (10 matrices)",
           "calibration": {"kernel": "__amd_rocclr_copyBuffer (torch copy_ of 2^28 fp32 = 1 GiB read + 1 GiB written)",
                           "fetch_kib": cf[ck], "write_kib": cw[ck], "fetch_factor": round(ff, 4),
                           "write_factor": round(wf, 4)},
           "gemm_source_sha256": h.hexdigest(), "gemm_sources": GEMM_SOURCES, "kernels": {}}
    for k in sorted(set(bf) | set(bw)):
        if "copyBuffer" in k:
            continue
        f, w = bf.get(k, 0.0), bw.get(k, 0.0)
        rec["kernels"][k] = {"fetch_kib_per_dispatch": round(f), "write_kib_per_dispatch": round(w),
                             "hbm_bytes_per_dispatch": round((f * ff + w * wf) * 1024)}
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8, help="timed Periodic cycles")
    ap.add_argument("--warmup", type=int, default=2, help="untimed Periodic cycles")
    ap.add_argument("--workload", default="15b", choices=["15b", "mmdit3072", "bucket2048", "dit2048"])
    ap.add_argument("--vanilla-steps", type=int, default=4)
    ap.add_argument("--variant-steps", type=int, default=2,
                    help="timed steps per scale-rule / monitor variant (0: skip)")
    ap.add_argument("--adamw-steps", type=int, default=5,
                    help="timed AdamW steps over the model's AdamW group (0: skip)")
    ap.add_argument("--spectrum-calls", type=int, default=1,
                    help="timed SVD-entropy diagnostic calls over the layer set (0 = skip)")
    ap.add_argument("--shard-degree", type=int, default=8,
                    help="time one GPU's share of the row-sharded RowNorm step at this degree (0 = skip)")
    ap.add_argument("--ns5-batched", type=int, default=1,
                    help="also time ns5_batched over the set in the variants leg (0 = skip)")
    ap.add_argument("--graph-cycles", type=int, default=20,
                    help="eager vs HIP-graph-replayed Periodic cycles on the small workloads (0 = skip)")
    ap.add_argument("--config-cycles", type=int, default=10,
                    help="timed Periodic cycles (and vanilla steps) on each other multi-matrix workload (0 = skip)")
    ap.add_argument("--ceiling-reps", type=int, default=5,
                    help="calls per window of the copy and MFMA-loop ceilings (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-traffic", nargs=5, metavar=("CAL_FETCH", "CAL_WRITE", "RUN_FETCH", "RUN_WRITE", "OUT"),
                    help="write the HBM traffic record from rocprofv3 counter CSVs and exit (no GPU)")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def pick_workload(name):
    from matrix_orthogonalising_optimizer_02_amd import workloads as WL
    return {"15b": WL.LAYER_SET_15B_H5120, "mmdit3072": WL.MMDIT_PAIR_H3072,
            "bucket2048": WL.MIXED_BUCKET_H2048, "dit2048": WL.DIT_BLOCK_H2048}[name]


def cpu_baseline(wl, k):
    """Time the float64 oracle on a sample of the workload's matrices and scale to the set.

    Sample: the median of three refresh steps and of three RowNorm steps of the oracle
    on the smallest matrix (about 11 s of host work), plus one refresh step on a second,
    longer matrix of the set whose size is at most three times the first (about 10 s).
    The refresh time is scaled by the oracle's own flop count (Eq. 2 as written:
    X X^T, A X and A (A X), 8 m^2 n per iteration), at the sampled matrices' combined
    seconds per flop; the RowNorm time by elements. The two matrices' seconds per flop
    are reported, so the scaling can be checked.
    """
    import numpy as np
    from oracle import muon_oracle as O
    from matrix_orthogonalising_optimizer_02_amd import workloads as WL

    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    sizes = [s[0] * s[1] for s in wl.shapes]
    idx = min(range(len(wl.shapes)), key=lambda i: sizes[i])
    shape = wl.shapes[idx]
    hp = O.OracleHParams(period_k=k)

    def oflops(s):
        mm, nn = min(s), max(s)
        return hp.ns_steps * 8.0 * mm * mm * nn

    w, m, g = WL.host_inputs(wl, idx)
    reps = 3  # median of three: about 11 s of host work on the 5120 x 5120 matrix
    t_refs, t_rns = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        O.vanilla_step(w, m, g, hp)
        t_refs.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        O.rownorm_step(w, m, g, hp)
        t_rns.append(time.perf_counter() - t0)
    t_ref, t_rn = sorted(t_refs)[reps // 2], sorted(t_rns)[reps // 2]
    # a second, longer matrix (the largest of at most three times the first one's size)
    second = [i for i in range(len(wl.shapes)) if sizes[idx] < sizes[i] <= 3 * sizes[idx]]
    rates = {f"{shape[0]}x{shape[1]}": t_ref / oflops(shape)}
    t_sum, f_sum = t_ref, oflops(shape)
    second_desc = "no second matrix of at most three times its size"
    if second:
        j = max(second, key=lambda i: sizes[i])
        w2, m2, g2 = WL.host_inputs(wl, j)
        t0 = time.perf_counter()
        O.vanilla_step(w2, m2, g2, hp)
        t2 = time.perf_counter() - t0
        name2 = f"{wl.shapes[j][0]}x{wl.shapes[j][1]}"
        rates[name2] = t2 / oflops(wl.shapes[j])
        t_sum, f_sum = t_sum + t2, f_sum + oflops(wl.shapes[j])
        second_desc = f"one refresh step ({t2:.1f} s) on the {name2} matrix"
    ref_total = t_sum / f_sum * sum(oflops(s) for s in wl.shapes)
    rn_total = t_rn * wl.elements / (shape[0] * shape[1])
    avg_ms = 1e3 * (ref_total + (k - 1) * rn_total) / k
    return {"value": round(avg_ms, 1), "unit": "ms", "cores": int(threads), "kind": "oracle",
            "host": host_info(),
            "sample": f"oracle refresh step ({t_ref:.1f} s) and RowNorm step ({t_rn:.2f} s), medians of {reps} runs on "
                      f"the {shape[0]}x{shape[1]} matrix, and {second_desc}; refresh scaled by the oracle's flops at the "
                      f"sampled matrices' combined rate, RowNorm by elements, to the {len(wl.shapes)}-matrix set; "
                      f"value = mean ms per optimizer step over a K={k} cycle",
            "seconds_per_gflop": {kk: round(v * 1e9, 4) for kk, v in rates.items()},
            "vanilla_step_ms": round(1e3 * ref_total, 1), "rownorm_step_ms": round(1e3 * rn_total, 1)}


def measure_variants(pkg, torch, weights, momenta, grads, ws, k, wl, n, say, ns5_calls=1):
    """Refresh steps under the Eq. 5 and Eq. 6 scale rules and a Periodic cycle with the
    update-RMS monitor, on the same resident state (HIP events around each block)."""
    shapes = [tuple(w.shape) for w in weights]
    rms = torch.zeros(len(weights), dtype=torch.float32, device=weights[0].device)

    def timed(fn):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    res = {}
    hidden = max(max(s) for s in shapes if s[0] == s[1]) if any(s[0] == s[1] for s in shapes) else max(shapes[0])
    hp5 = pkg.default_hparams(period_k=1, scale_mode=pkg.SCALE_HIDDEN, hidden=hidden)
    res["eq5_refresh_step_ms"] = round(timed(lambda: pkg.muon_step(weights, momenta, grads[0], 0, hp5, ws)), 4)
    res["eq5_hidden"] = hidden
    hp6 = pkg.default_hparams(period_k=1, scale_mode=pkg.SCALE_RMS)
    pkg.timing_enable(True)
    res["eq6_refresh_step_ms"] = round(timed(lambda: pkg.muon_step(weights, momenta, grads[0], 0, hp6, ws)), 4)
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    for name, bytes_per_elem in (("rms_finalize", None), ("scaled_update", 12.0), ("apply_final", None)):
        ms_, c = kern[name]
        if c:
            ent = {"avg_ms": round(ms_ / c, 4)}
            if bytes_per_elem:
                ent["algorithmic_gbs"] = round(bytes_per_elem * wl.elements / (ms_ / c * 1e-3) / 1e9, 1)
            res[f"eq6_{name}"] = ent
    hp = pkg.default_hparams(period_k=k)
    hp1 = pkg.default_hparams(period_k=1)
    res["monitored_refresh_step_ms"] = round(timed(
        lambda: pkg.muon_step(weights, momenta, grads[0], 0, hp1, ws, update_rms=rms)), 4)
    res["monitored_rownorm_step_ms"] = round(timed(
        lambda: pkg.muon_step(weights, momenta, grads[1], 1, hp, ws, update_rms=rms)), 4)
    res["unmonitored_rownorm_step_ms"] = round(timed(
        lambda: pkg.muon_step(weights, momenta, grads[1], 1, hp, ws)), 4)
    res["update_rms_last"] = [round(float(x), 5) for x in rms.cpu().tolist()]
    # ns5_batched: O = NS5(M) for the set into separate fp32 outputs (the entry point
    # without momentum or update), NS5 TFLOP/s on the symmetric count
    if ns5_calls > 0:
        outs = [torch.empty_like(m) for m in momenta]
        hp_ns = pkg.default_hparams()
        pkg.ns5_batched(momenta, outs, hp_ns, ws)
        t = timed(lambda: pkg.ns5_batched(momenta, outs, hp_ns, ws))
        flops = sum(ns5_flops_sym(min(s), max(s), hp_ns.ns_steps) for s in shapes)
        res["ns5_batched_ms"] = round(t, 4)
        res["ns5_batched_tflops"] = round(flops / (t * 1e-3) / 1e12, 1)
        del outs
    say(f"variants: {res}")
    return res


def measure_configs(pkg, torch, dev, names, cycles, say):
    """The step figures for the other multi-matrix workloads, in the same run: Periodic
    (K = 3) and vanilla step times, NS5 TFLOP/s and RowNorm GB/s with their roofline
    fractions, from the library's per-launch HIP events. State is freed after each."""
    from matrix_orthogonalising_optimizer_02_amd import workloads as WL
    k = 3
    res = {}
    for name in names:
        wl = pick_workload(name)
        shapes = list(wl.shapes)
        weights = [torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
        momenta = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
        for i, w in enumerate(weights):
            WL.device_fill(w, wl.key, WL.ROLE_W, i, wl.w_std)
        grads = []
        for step in range(k):
            gs = [torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
            for i, g in enumerate(gs):
                WL.device_fill(g, wl.key, WL.ROLE_G, i, wl.g_std, wl.g_dist, step)
            grads.append(gs)
        ws = pkg.make_workspace(shapes, dev)
        hp = pkg.default_hparams(period_k=k)
        hp1 = pkg.default_hparams(period_k=1)
        for s in range(2 * k):  # warm-up: two cycles
            pkg.muon_step(weights, momenta, grads[s % k], s, hp, ws)
        torch.cuda.synchronize()
        pkg.timing_enable(True)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for s in range(cycles * k):
            pkg.muon_step(weights, momenta, grads[s % k], s, hp, ws)
        b.record()
        torch.cuda.synchronize()
        kern = pkg.timing_read()
        pkg.timing_enable(False)
        periodic_ms = a.elapsed_time(b) / (cycles * k)
        a.record()
        for s in range(cycles):
            pkg.muon_step(weights, momenta, grads[s % k], 0, hp1, ws)
        b.record()
        torch.cuda.synchronize()
        vanilla_ms = a.elapsed_time(b) / cycles
        ms = {n_: kern[n_][0] for n_ in kern}
        ns5_ms = (ms["gram"] + ms["poly"] + ms["apply"] + ms["apply_final"]) / cycles
        ns5_tf = sum(ns5_flops_sym(min(s), max(s), hp.ns_steps) for s in shapes) / (ns5_ms * 1e-3) / 1e12
        rn_ms = (ms["rownorm_rows"] + ms["colnorm_partial"] + ms["colnorm_finalize"]
                 + ms["colnorm_apply"]) / (cycles * (k - 1))
        rn_gbs = 20.0 * wl.elements / (rn_ms * 1e-3) / 1e9
        ap_ms = ms["apply"] / max(kern["apply"][1], 1)
        ap_tf = sum(apply_flops(min(s), max(s)) for s in shapes) / (ap_ms * 1e-3) / 1e12
        res[name] = {"workload": wl.name, "matrices": len(shapes), "elements": wl.elements,
                     "muon_step_ms_periodic_avg": round(periodic_ms, 4),
                     "muon_step_ms_vanilla": round(vanilla_ms, 4),
                     "periodic_saving_pct": round(100.0 * (1.0 - periodic_ms / vanilla_ms), 1),
                     "ns5_ms_per_refresh": round(ns5_ms, 4), "ns5_tflops": round(ns5_tf, 1),
                     "ns5_frac_of_bf16_peak": round(ns5_tf / PEAK_BF16_TFLOPS, 4),
                     "apply_tflops": round(ap_tf, 1),
                     "rownorm_step_ms": round(rn_ms, 4), "rownorm_gbs": round(rn_gbs, 1),
                     "rownorm_frac_of_hbm_peak": round(rn_gbs / PEAK_HBM_GBS, 4)}
        say(f"config {name}: {res[name]}")
        del weights, momenta, grads, ws
        torch.cuda.empty_cache()
    return res


def measure_adamw(pkg, torch, dev, wl, n, say):
    """AdamW over the AdamW group of the model whose block the workload is (biases,
    norms, embedders, final layer), 28 bytes per element, HIP events per launch."""
    from matrix_orthogonalising_optimizer_02_amd import hybrid as H
    scale = {5120: "15B", 4096: "9B", 3072: "4B", 2048: "1.3B"}.get(min(min(s) for s in wl.shapes))
    if scale is None:
        return None
    h, depth = H.DIT_SCALES[scale]
    pl = H.dit_parameter_list(h, depth)
    _, adamw_names = H.split_param_groups(pl)
    shapes = dict(pl)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    w = [torch.zeros(shapes[nm], dtype=torch.float32, device=dev) for nm in adamw_names]
    gr = [torch.empty(shapes[nm], dtype=torch.float32, device=dev).normal_(0.0, 1e-3, generator=g) for nm in adamw_names]
    m = [torch.zeros_like(x) for x in w]
    v = [torch.zeros_like(x) for x in w]
    elems = sum(x.numel() for x in w)
    group = pkg.AdamWGroup(w, gr, m, v)
    group.step(0)
    torch.cuda.synchronize()
    pkg.timing_enable(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(n):
        group.step(s + 1)
    b.record()
    torch.cuda.synchronize()
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    step_ms = a.elapsed_time(b) / n
    kms, launches = kern["adamw"]
    mu, ad = H.count_params(pl)
    res = {"model": f"double-stream DiT {scale} (H={h}, {depth} blocks, {(mu + ad) / 1e9:.2f} B parameters)",
           "muon_share": round(mu / (mu + ad), 4), "adamw_tensors": len(w), "adamw_elements": elems,
           "adamw_step_ms": round(step_ms, 4), "adamw_launches_per_step": launches // n,
           "adamw_kernel_gbs": round(28.0 * elems / (kms / n * 1e-3) / 1e9, 1),
           "adamw_step_gbs": round(28.0 * elems / (step_ms * 1e-3) / 1e9, 1)}
    say(f"hybrid: {res}")
    del w, gr, m, v
    return res


def measure_spectrum(pkg, torch, weights, n, say, cpu=True):
    """The SVD-entropy diagnostic over the layer set's weights, fp64 on the device.

    Algorithmic work per matrix (m = min, n = max): the Gram kernel's m (m + 1) n
    flops (upper triangle with the diagonal, 2 flops per product term), and per
    Householder column step j the upper triangle of the trailing block (l = m - j - 1
    rows, l (l + 1) / 2 elements) read and written once, 16 bytes per element (the
    first step only reads: no pending update).
    """
    shapes = [tuple(w.shape) for w in weights]
    ws = pkg.binding.make_svd_entropy_workspace(shapes, weights[0].device)
    ent = torch.empty(len(weights), dtype=torch.float64, device=weights[0].device)
    pkg.svd_entropy(weights, entropy=ent, workspace=ws)  # warm-up
    torch.cuda.synchronize()
    pkg.timing_enable(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        pkg.svd_entropy(weights, entropy=ent, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    call_ms = a.elapsed_time(b) / n
    gram_flops = sum(float(min(s)) * (min(s) + 1) * max(s) for s in shapes)
    pass_bytes = sum(16.0 * (min(s) - 1) * min(s) * (min(s) + 1) / 6.0 - 8.0 * (min(s) - 1) * min(s) / 2.0
                     for s in shapes)
    per = {nm: kern["spec_" + nm] for nm in ("gram", "house", "pass", "reduce", "bisect", "entropy")}
    gram_ms = per["gram"][0] / n
    pass_ms = per["pass"][0] / n
    res = {"call_ms": round(call_ms, 3),
           "entropy": [round(float(x), 6) for x in ent.cpu().tolist()],
           "launches_per_call": sum(c for _, c in per.values()) // n,
           "kernel_ms_per_call": {nm: round(v[0] / n, 3) for nm, v in per.items()},
           "gram": {"bound": "mfma", "dtype": "f64", "achieved": round(gram_flops / (gram_ms * 1e-3) / 1e12, 2),
                    "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(gram_flops / (gram_ms * 1e-3) / 1e12 / PEAK_FP64_TFLOPS, 4)},
           "householder_pass": {"bound": "hbm", "achieved": round(pass_bytes / (pass_ms * 1e-3) / 1e9, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(pass_bytes / (pass_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                "avg_launch_ms": round(per["pass"][0] / max(per["pass"][1], 1), 4)}}
    if cpu:
        res["cpu_oracle"] = spectrum_oracle_time(weights, shapes)
    say(f"spectrum: {res}")
    del ws
    return res


def spectrum_oracle_time(weights, shapes):
    """The float64 oracle (library SVD, singular values only) on the set's smallest
    matrix, scaled to the set by the Golub-Kahan bidiagonalisation count
    4 m^2 n - 4 m^3 / 3 (m = min, n = max); the host's BLAS threads."""
    import numpy as np
    from oracle import spectrum_oracle as SO

    idx = min(range(len(shapes)), key=lambda i: shapes[i][0] * shapes[i][1])
    x = weights[idx].cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    SO.svd_entropy(x)
    t = time.perf_counter() - t0

    def cost(s):
        mm, nn = float(min(s)), float(max(s))
        return 4.0 * mm * mm * nn - 4.0 * mm ** 3 / 3.0

    total = t * sum(cost(s) for s in shapes) / cost(shapes[idx])
    return {"seconds_per_call": round(total, 1), "sample_seconds": round(t, 2),
            "sample": f"oracle SVD entropy of the {shapes[idx][0]}x{shapes[idx][1]} matrix, scaled by "
                      f"4 m^2 n - 4 m^3 / 3 to the {len(shapes)}-matrix set",
            "cores": _blas_threads()}


def host_info():
    """CPU model and BLAS library of the host the oracle ran on."""
    info = {"cpu": None, "blas": None}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        libs = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if libs:
            info["blas"] = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return info


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([d.get("num_threads", 1) for d in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def measure_shard_rownorm(pkg, torch, dev, wl, degree, reps, rn_ms, say):
    """One GPU's share of the RowNorm step with the weights sharded by rows over `degree`
    GPUs: every matrix [A, B] contributes its block [A / degree, B]. Flat blocks take
    rownorm_update (their rows are whole); tall blocks take rownorm_shard_colsq, the
    all-reduce of the column sums (identity here: one GPU), and rownorm_shard_apply."""
    from matrix_orthogonalising_optimizer_02_amd import workloads as WL

    shapes = [(a // degree, b) for a, b in wl.shapes]
    tall = [a > b for a, b in wl.shapes]
    blk = []
    for i, (s, t) in enumerate(zip(shapes, tall)):
        w = torch.empty(s, dtype=torch.float32, device=dev)
        m = torch.zeros(s, dtype=torch.float32, device=dev)
        g = torch.empty(s, dtype=torch.float32, device=dev)
        WL.device_fill(w, wl.key, WL.ROLE_W, i, wl.w_std)
        WL.device_fill(g, wl.key, WL.ROLE_G, i, wl.g_std, wl.g_dist)
        blk.append((w, m, g, t, wl.shapes[i][0]))
    hp = pkg.default_hparams(period_k=3)
    flat = [b for b in blk if not b[3]]
    tl = [b for b in blk if b[3]]
    ws_flat = pkg.make_workspace([tuple(b[0].shape) for b in flat], dev)
    full = [b[4] for b in tl]
    nb = pkg.rownorm_shard_workspace_bytes([tuple(b[0].shape) for b in tl], full)
    ws_tall = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    colsq = [torch.empty(b[0].shape[1], dtype=torch.float32, device=dev) for b in tl]

    def share_step():
        pkg.rownorm_update([b[0] for b in flat], [b[1] for b in flat], [b[2] for b in flat], hp, ws_flat)
        pkg.rownorm_shard_colsq([b[0] for b in tl], [b[1] for b in tl], [b[2] for b in tl], full, colsq, hp, ws_tall)
        pkg.rownorm_shard_apply([b[0] for b in tl], [b[1] for b in tl], full, colsq, hp, ws_tall)  # identity reduce

    def windows(fn, n_windows=5):
        """Median ms per rep over n_windows event windows of `reps` reps each."""
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(n_windows):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / reps)
        return sorted(out)[len(out) // 2]

    # The share is about 0.5 ms of GPU work in five launches; enqueued eagerly from
    # Python, the host's marshalling and validation can take longer than that. The
    # figure is taken from the step captured once as a HIP graph and replayed, which
    # keeps the GPU fed; the eager figure is kept beside it.
    eager_ms = windows(share_step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        share_step()
    torch.cuda.synchronize()
    ms = windows(graph.replay)
    elems = sum(x * y for x, y in shapes)
    res = {"degree": degree, "block_shapes": [list(x) for x in shapes], "elements": elems,
           "share_step_ms": round(ms, 4), "share_gbs": round(20.0 * elems / (ms * 1e-3) / 1e9, 1),
           "eager_share_step_ms": round(eager_ms, 4),
           "unsharded_rownorm_ms_over_degree": round(rn_ms / degree, 4),
           "share_vs_ideal": round((rn_ms / degree) / ms, 3),
           "timing": f"HIP graph of one share step, replayed; median of 5 windows of {reps} replays",
           "note": "tall blocks: column sums, identity all-reduce (one GPU), then the update"}
    say(f"shard: {res}")
    del graph, blk, ws_flat, ws_tall
    return res


def measure_ceilings(pkg, torch, dev, reps, say):
    """The attainable ceilings on this GPU in this run, beside the spec peaks: the
    library's streaming copy kernel over 1 GiB (read + write bytes per second) and its
    register-only bf16 MFMA loop on one block per compute unit; and torch's bf16 GEMM as
    a yardstick. Medians of five event windows."""
    def median_ms(fn, n):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / n)
        return sorted(out)[2]

    n = 1 << 28  # 1 GiB of fp32
    src = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    copy_ms = median_ms(lambda: pkg.ceiling_copy(src, dst), 4 * reps)
    assert torch.equal(src[:4096], dst[:4096]) and torch.equal(src[-4096:], dst[-4096:])
    copy_gbs = 8.0 * n / (copy_ms * 1e-3) / 1e9
    del src, dst
    blocks, iters = 256, 100000
    chk = torch.zeros(4 * blocks, dtype=torch.float32, device=dev)
    flops = pkg.ceiling_mfma(chk, blocks, iters)
    mfma_ms = median_ms(lambda: pkg.ceiling_mfma(chk, blocks, iters), max(1, reps // 2))
    assert bool(torch.isfinite(chk).all())
    mfma_tflops = flops / (mfma_ms * 1e-3) / 1e12
    res = {"copy": {"gbs": round(copy_gbs, 1), "frac_of_spec": round(copy_gbs / PEAK_HBM_GBS, 4),
                    "bytes_per_call": 8 * n, "ms_per_call": round(copy_ms, 4),
                    "kernel": "muon_ceiling_copy: 256 threads, 32 KiB per block, non-temporal"},
           "mfma": {"tflops": round(mfma_tflops, 1), "frac_of_spec": round(mfma_tflops / PEAK_BF16_TFLOPS, 4),
                    "flops_per_call": flops, "ms_per_call": round(mfma_ms, 4),
                    "kernel": "muon_ceiling_mfma: 256 blocks x 4 waves, 16 independent 32x32x16 bf16 MFMA chains "
                              "per wave, operand bits toggling every round as a GEMM's do, no memory traffic"}}
    # the vendor GEMM as a yardstick (torch.matmul, hipBLASLt on this image): bf16
    # operands, fp32 accumulation, bf16 out; 8192^3, and the Apply's largest product
    # (P [5120, 5120] times X [5120, 30720])
    yard = {}
    for name, (mm, kk, nn) in (("8192^3", (8192, 8192, 8192)), ("apply_5120x5120x30720", (5120, 5120, 30720))):
        a = torch.randn(mm, kk, device=dev).to(torch.bfloat16)
        bm = torch.randn(kk, nn, device=dev).to(torch.bfloat16)
        c = torch.empty(mm, nn, device=dev, dtype=torch.bfloat16)
        ms = median_ms(lambda: torch.matmul(a, bm, out=c), max(2, reps))
        tf = 2.0 * mm * kk * nn / (ms * 1e-3) / 1e12
        yard[name] = {"tflops": round(tf, 1), "frac_of_spec": round(tf / PEAK_BF16_TFLOPS, 4), "ms_per_call": round(ms, 4)}
        del a, bm, c
    res["torch_matmul_bf16"] = yard
    say(f"ceilings: {res}")
    return res


def measure_graph(pkg, torch, dev, n, say):
    """Eager Periodic cycles against the same cycle captured once in a HIP graph and
    replayed, on the small workloads where launches dominate (the 128 x 512 matrix and
    the H = 2048 DiT block). Inputs resident; HIP events around n cycles."""
    from matrix_orthogonalising_optimizer_02_amd import workloads as WL

    res = {}
    for wl in (WL.SINGLE_128x512, WL.DIT_BLOCK_H2048):
        shapes = list(wl.shapes)
        w = [torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
        m = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
        g = [[torch.empty(s, dtype=torch.float32, device=dev) for s in shapes] for _ in range(3)]
        for i, t in enumerate(w):
            WL.device_fill(t, wl.key, WL.ROLE_W, i, wl.w_std)
        for j in range(3):
            for i, t in enumerate(g[j]):
                WL.device_fill(t, wl.key, WL.ROLE_G, i, wl.g_std, wl.g_dist, j)
        ws = pkg.make_workspace(shapes, dev)
        hp = pkg.default_hparams(period_k=3)

        def cycle():
            for j in range(3):
                pkg.muon_step(w, m, g[j], j, hp, ws)

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n

        eager = timed(cycle)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            cycle()
        replay = timed(graph.replay)
        res[wl.name] = {"eager_cycle_ms": round(eager, 4), "graph_cycle_ms": round(replay, 4),
                        "speedup": round(eager / replay, 3)}
        del graph, w, m, g, ws
    say(f"graph: {res}")
    return res


def main():
    args = parse()
    if args.summarize_traffic:
        rec = summarize_traffic(*args.summarize_traffic)
        print(json.dumps({k: v["hbm_bytes_per_dispatch"] for k, v in rec["kernels"].items()}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(one GPU's share of the sharded step is what it measures)", file=sys.stderr)
        sys.exit(2)

    import torch
    import matrix_orthogonalising_optimizer_02_amd as pkg
    from matrix_orthogonalising_optimizer_02_amd import workloads as WL

    def say(msg):
        if not args.quiet:
            print(msg, file=sys.stderr, flush=True)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pkg.load_library()
    dev = torch.device("cuda:0")
    wl = pick_workload(args.workload)
    k = 3
    shapes = list(wl.shapes)
    say(f"workload: {wl.name}, {len(shapes)} matrices, {wl.elements / 1e6:.0f} M elements")

    weights = [torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
    momenta = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    for i, w in enumerate(weights):
        WL.device_fill(w, wl.key, WL.ROLE_W, i, wl.w_std)
    grads = []
    for step in range(k):
        gs = [torch.empty(s, dtype=torch.float32, device=dev) for s in shapes]
        for i, g in enumerate(gs):
            WL.device_fill(g, wl.key, WL.ROLE_G, i, wl.g_std, wl.g_dist, step)
        grads.append(gs)
    ws = pkg.make_workspace(shapes, dev)
    torch.cuda.synchronize()
    say(f"inputs resident: workspace {ws.numel() / 2**30:.2f} GiB")

    hp = pkg.default_hparams(period_k=k)
    hp_vanilla = pkg.default_hparams(period_k=1)
    step_counter = [0]

    def cycle():
        for j in range(k):
            pkg.muon_step(weights, momenta, grads[j], step_counter[0], hp, ws)
            step_counter[0] += 1

    for _ in range(args.warmup):
        cycle()
    torch.cuda.synchronize()
    say(f"warmup done ({args.warmup} cycles)")

    # ---- timed region: Periodic cycles, per-kernel events recorded by the library
    pkg.timing_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        cycle()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    cycle_ms = ev0.elapsed_time(ev1) / args.steps
    say(f"periodic: {cycle_ms:.3f} ms per cycle (wall {1e3 * wall / args.steps:.3f} ms)")

    # ---- vanilla steps (NS5 every step) for the Periodic saving
    torch.cuda.synchronize()
    ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev2.record()
    for j in range(args.vanilla_steps):
        pkg.muon_step(weights, momenta, grads[j % k], 0, hp_vanilla, ws)
    ev3.record()
    torch.cuda.synchronize()
    vanilla_ms = ev2.elapsed_time(ev3) / max(args.vanilla_steps, 1)
    say(f"vanilla: {vanilla_ms:.3f} ms per step")

    variants = measure_variants(pkg, torch, weights, momenta, grads, ws, k, wl, args.variant_steps, say,
                                args.ns5_batched) \
        if args.variant_steps > 0 else None
    hybrid = measure_adamw(pkg, torch, dev, wl, args.adamw_steps, say) if args.adamw_steps > 0 else None
    spectrum = measure_spectrum(pkg, torch, weights, args.spectrum_calls, say, not args.no_cpu_baseline) \
        if args.spectrum_calls > 0 else None

    refreshes = args.steps
    rownorm_steps = args.steps * (k - 1)
    ms = {name: kern[name][0] for name in kern}
    cnt = {name: kern[name][1] for name in kern}
    ns5_ms = (ms["gram"] + ms["poly"] + ms["apply"] + ms["apply_final"]) / refreshes
    ns5_flops = sum(ns5_flops_sym(min(s), max(s), hp.ns_steps) for s in shapes)
    ns5_tflops = ns5_flops / (ns5_ms * 1e-3) / 1e12
    rn_ms = (ms["rownorm_rows"] + ms["colnorm_partial"] + ms["colnorm_finalize"] + ms["colnorm_apply"]) / rownorm_steps
    rn_gbs = 20.0 * wl.elements / (rn_ms * 1e-3) / 1e9
    shard = measure_shard_rownorm(pkg, torch, dev, wl, args.shard_degree, 50, rn_ms, say) \
        if args.shard_degree > 1 else None
    graph = measure_graph(pkg, torch, dev, args.graph_cycles, say) if args.graph_cycles > 0 else None
    ceilings = measure_ceilings(pkg, torch, dev, args.ceiling_reps, say) if args.ceiling_reps > 0 else None
    others = [w for w in ("dit2048", "bucket2048", "mmdit3072", "15b") if w != args.workload]
    configs = measure_configs(pkg, torch, dev, others, args.config_cycles, say) if args.config_cycles > 0 else None
    # dominant kernel: the B X product of iterations 1..N-1
    apply_launch_ms = ms["apply"] / max(cnt["apply"], 1)
    apply_launch_flops = sum(apply_flops(min(s), max(s)) for s in shapes)
    apply_tflops = apply_launch_flops / (apply_launch_ms * 1e-3) / 1e12
    kernels = {}
    for name in kern:
        if cnt[name]:
            kernels[name] = {"launches": cnt[name], "avg_ms": round(ms[name] / cnt[name], 4),
                             "total_ms_per_cycle": round(ms[name] / args.steps, 4)}
    for name, fl in (("gram", lambda m, n: m * m * n), ("poly", lambda m, n: 1.0 * m ** 3),
                     ("apply", apply_flops), ("apply_final", apply_flops)):
        if cnt[name]:
            f = sum(fl(min(s), max(s)) for s in shapes)
            kernels[name]["algorithmic_tflops"] = round(f / (ms[name] / cnt[name] * 1e-3) / 1e12, 1)
    elems_flat = sum(a * b for a, b in shapes if a <= b)
    elems_tall = wl.elements - elems_flat
    if cnt["rownorm_rows"]:
        kernels["rownorm_rows"]["algorithmic_gbs"] = round(
            20.0 * elems_flat / (ms["rownorm_rows"] / cnt["rownorm_rows"] * 1e-3) / 1e9, 1)
    if cnt["colnorm_partial"]:
        kernels["colnorm_partial"]["algorithmic_gbs"] = round(
            12.0 * elems_tall / (ms["colnorm_partial"] / cnt["colnorm_partial"] * 1e-3) / 1e9, 1)
        kernels["colnorm_apply"]["algorithmic_gbs"] = round(
            12.0 * elems_tall / (ms["colnorm_apply"] / cnt["colnorm_apply"] * 1e-3) / 1e9, 1)
    if cnt["cast"]:
        # read M, G; write M and bf16 X_c (and the row-major X_r for groups whose Gram
        # runs on 128-wide tiles: fewer than 512 symmetric 256-wide tiles)
        sym_tiles = sum((math.ceil(min(s) / 256)) * (math.ceil(min(s) / 256) + 1) // 2 for s in shapes)
        cast_b = 14.0 if (len(shapes) <= 16 and sym_tiles >= 512) else 16.0
        kernels["cast"]["algorithmic_bytes_per_elem"] = cast_b
        kernels["cast"]["algorithmic_gbs"] = round(
            cast_b * wl.elements / (ms["cast"] / cnt["cast"] * 1e-3) / 1e9, 1)

    out = {
        "metric": METRIC,
        "value": round(cycle_ms / k, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cycle_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "matrices": len(shapes), "elements": wl.elements,
                   "shapes": [list(s) for s in shapes], "period_k": k, "gamma": hp.gamma,
                   "ns_steps": hp.ns_steps, "step": "one Periodic cycle = 1 NS5 refresh + 2 RowNorm steps"},
        "muon_step_ms_periodic_avg": round(cycle_ms / k, 4),
        "muon_step_ms_vanilla": round(vanilla_ms, 4),
        "periodic_saving_pct": round(100.0 * (1.0 - (cycle_ms / k) / vanilla_ms), 1),
        "ns5_ms_per_refresh": round(ns5_ms, 4),
        "ns5_tflops": round(ns5_tflops, 1),
        "ns5_frac_of_bf16_peak": round(ns5_tflops / PEAK_BF16_TFLOPS, 4),
        "rownorm_step_ms": round(rn_ms, 4),
        "rownorm_gbs": round(rn_gbs, 1),
        "rownorm_frac_of_hbm_peak": round(rn_gbs / PEAK_HBM_GBS, 4),
        "pages_context": dict(PAGES_CONTEXT, this_run={
            "periodic_optimizer_time_saving_pct": round(100.0 * (1.0 - (cycle_ms / k) / vanilla_ms), 1),
            "periodic_over_vanilla": round((cycle_ms / k) / vanilla_ms, 4),
            "pages_periodic_over_vanilla_15b": round(1.317 / 2.884, 4),
            "note": "one MI355X, optimizer step only, no communication"}),
        "roofline": {"bound": "mfma", "kernel": "k_ns_gemm<apply> (P X, iterations 1..4; with its tail fixup where split)",
                     "achieved": round(apply_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(apply_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(["k_ns_gemm<2, muon::GemmCfg<256, 256, true, 32, 4>, true>",
                                                  "k_ns_tail_fix<2>"], args.workload),
                     "launch_ms": round(apply_launch_ms, 4), "launch_flops": apply_launch_flops},
        "kernels": kernels,
    }
    if variants is not None:
        out["variants"] = variants
    if hybrid is not None:
        out["hybrid"] = hybrid
    if spectrum is not None:
        out["spectrum"] = spectrum
    if shard is not None:
        out["shard_rownorm"] = shard
    if graph is not None:
        out["graph_replay"] = graph
    if configs is not None:
        out["configs"] = configs
    if ceilings is not None:
        ceilings["apply_frac_of_mfma_ceiling"] = round(apply_tflops / ceilings["mfma"]["tflops"], 4)
        ceilings["ns5_frac_of_mfma_ceiling"] = round(ns5_tflops / ceilings["mfma"]["tflops"], 4)
        ceilings["rownorm_frac_of_copy_ceiling"] = round(rn_gbs / ceilings["copy"]["gbs"], 4)
        yard = ceilings["torch_matmul_bf16"]["apply_5120x5120x30720"]["tflops"]
        ceilings["apply_vs_torch_matmul_same_shape"] = round(apply_tflops / yard, 4)
        out["ceilings"] = ceilings
    if not args.no_cpu_baseline:
        say("cpu baseline: timing the float64 oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(wl, k)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
