#!/usr/bin/env python3
"""Throughput of the multi-adapter linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--w8a8]

One step is one pass of the whole hot path over one batch: device-side
segment build -> shrink -> fused linear (base GEMM with the adapter
up-projection in its epilogue), for every projection of the workload.
Batches of at most 256 rows run the segment build and the first
projection's shrink as one launch (lora_build_shrink_dev);
--separate-build times them as two.
Inputs are resident in HBM before timing; several copies of every buffer
are rotated so that a step never finds its operands in the 256 MB
Infinity Cache.  Prints one JSON line.

The default workload is the decode batch (Llama-3-8B q_proj 4096->4096,
bf16, 256 tokens, 64 slots of rank 16); --config selects another.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp32": 157.3}
# projections that read the same input and share one fused launch
# (a decoder layer's q / k / v and gate / up)
SLICE_GROUPS = {"llama_layer": [["q_proj", "k_proj", "v_proj"], ["o_proj"], ["gate_proj", "up_proj"],
                                ["down_proj"]]}
CACHE_BYTES = 256 << 20
METRIC = "multi-LoRA linear tokens/s; achieved HBM GB/s (decode) & MFMA % (prefill)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode_bgmv")
    ap.add_argument("--w8a8", action="store_true", help="fp8 base: quantise activations per token")
    ap.add_argument("--no-slices", action="store_true",
                    help="one fused call per projection (default: projections of one input share a call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-build", action="store_true",
                    help="segment build and shrink as two launches also for small batches")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "workload into profiles/ and exit")
    ap.add_argument("--counter-command", default="", help="the command lines that produced the CSVs")
    ap.add_argument("--concurrent", type=int, default=0, metavar="BASE_CUS",
                    help="one-projection workloads: time the unfused design instead, the base product on a "
                         "stream of BASE_CUS compute units and the adapter term on the others")
    ap.add_argument("--cu-layout", choices=("spread", "block"), default="spread",
                    help="base CUs: the same share of every block of 32 logical CUs, or the first BASE_CUS")
    return ap.parse_args()


# Kernel whose roofline the bench line reports, and the sources it is built from
# (a stored counter reading applies only while these are unchanged).
DOMINANT = "fused_dma_kernel"
DOMINANT_SOURCES = ["adapter_gemm_amd/csrc/fused_dma.hip", "adapter_gemm_amd/csrc/common.h"]


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in DOMINANT_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{DOMINANT}_{workload}_traffic.txt")


def summarise_counters(fetch_csv: str, write_csv: str, workload: str, copy_mb: int, command: str):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the dominant kernel,
    scaled by what the same counter reads for the calibration copy of
    copy_mb MiB (read once and written once)."""
    import csv

    def read(path, counter):
        rows = []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return rows

    copy_kib = copy_mb * 1024.0
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = read(path, counter)
        kern = [v for n, v in rows if DOMINANT in n]
        copies = [v for n, v in rows if "copy" in n.lower() and v >= 0.5 * copy_kib]
        if not kern or not copies:
            raise SystemExit(f"{path}: no {DOMINANT} or calibration-copy dispatches with {counter}")
        factor = copy_kib / (sum(copies) / len(copies))
        out[counter] = (sum(kern) / len(kern), factor, len(kern), len(copies))
    fetch_kib, ff, nk, nc = out["FETCH_SIZE"]
    write_kib, wf, _, _ = out["WRITE_SIZE"]
    traffic = (fetch_kib * ff + write_kib * wf) * 1024.0
    with open(traffic_file(workload), "w") as fh:
        fh.write(f"# HBM traffic of {DOMINANT}, workload {workload} (rocprofv3 --pmc, one counter per run)\n")
        fh.write(f"# commands: {command}\n")
        fh.write(f"source_sha256 = {sources_digest()}\n")
        fh.write(f"dispatches = {nk}\ncalibration_copy_mib = {copy_mb} ({nc} dispatches)\n")
        fh.write(f"fetch_kib_per_dispatch = {fetch_kib:.1f}\nfetch_factor = {ff:.4f}\n")
        fh.write(f"write_kib_per_dispatch = {write_kib:.1f}\nwrite_factor = {wf:.4f}\n")
        fh.write(f"traffic_bytes_per_launch = {traffic:.0f}\n")
    print(open(traffic_file(workload)).read())


def stored_traffic(workload: str):
    """Calibrated HBM bytes per launch of the dominant kernel, or None when no
    reading exists or the kernel's sources changed since it was taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != sources_digest():
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def main():
    args = parse()
    if args.counter_summary:
        summarise_counters(args.counter_summary[0], args.counter_summary[1],
                           args.config + ("_w8a8" if args.w8a8 else ""),
                           args.calibrate_copy_mb or 256, args.counter_command)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU path is a design note, not an implementation.", file=sys.stderr)
        sys.exit(2)

    import torch
    import adapter_gemm_amd as agm
    from lora_inputs import make_workload

    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = make_workload(args.config)
    T = w.T
    print(f"# workload {w.name}: {w.description}", file=sys.stderr, flush=True)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- one instance on the device ------------------------------------
    touched = w.touched_slots()
    projs = []
    inst_bytes = 0
    for p in w.projections:
        A, B = p.pool(touched)            # untouched slots stay zero: never read
        pr = {"p": p}
        pr["A"], pr["B"] = bf16(A) if p.data_dtype == "bf16" else torch.from_numpy(A).to(dev), \
            bf16(B) if p.data_dtype == "bf16" else torch.from_numpy(B).to(dev)
        del A, B
        w0 = p.w0()
        if p.base_dtype == "fp8":
            pr["W"], pr["ws"] = torch.from_numpy(w0[0]).to(dev), torch.from_numpy(w0[1]).to(dev)
        elif p.base_dtype == "bf16":
            pr["W"], pr["ws"] = bf16(w0), None
        else:
            pr["W"], pr["ws"] = torch.from_numpy(w0).to(dev), None
        del w0
        x = w.x(p)
        pr["x"] = bf16(x) if p.data_dtype == "bf16" else torch.from_numpy(x).to(dev)
        pr["rank"] = torch.from_numpy(p.slot_rank).to(dev)
        pr["scale"] = torch.from_numpy(p.slot_scale).to(dev)
        ydt = torch.bfloat16 if p.data_dtype == "bf16" else torch.float32
        pr["y"] = torch.empty(T, p.d_out, dtype=ydt, device=dev)
        pr["v"] = torch.empty(T, p.r_cap, dtype=torch.float32, device=dev)
        for k in ("A", "B", "W", "x", "y", "v"):
            inst_bytes += pr[k].numel() * pr[k].element_size()
        projs.append(pr)
    ids = torch.from_numpy(w.ids).to(dev)
    act = torch.from_numpy(w.active).to(dev)
    n_slots = w.projections[0].n_slots

    # ---- rotated copies ------------------------------------------------
    n_rot = max(1, -(-2 * CACHE_BYTES // max(inst_bytes, 1)))
    n_rot = min(n_rot, 64)
    flags = agm.FLAG_ACT_QUANT_E4M3 if args.w8a8 else 0
    names = [p.name for p in w.projections]
    if w.name in SLICE_GROUPS and not args.no_slices:
        groups = [[names.index(n) for n in g] for g in SLICE_GROUPS[w.name]]
    else:
        groups = [[j] for j in range(len(names))]
    insts = []
    for r in range(n_rot):
        inst = []
        for pr in projs:
            c = {k: (pr[k] if r == 0 else pr[k].clone()) if isinstance(pr[k], torch.Tensor) else pr[k]
                 for k in pr}
            c["pool"] = agm.pool_desc(c["A"], c["B"], c["rank"], c["scale"])
            c["base"] = agm.base_desc(c["W"], c["ws"])
            p = c["p"]
            bt = {"bf16": agm.BF16, "fp8": agm.FP8_E4M3, "fp32": agm.F32}[p.base_dtype]
            c["wsp"] = agm.fused_workspace(T, p.d_in, p.d_out, bt, flags, device=dev)
            inst.append(c)
        gws = []
        for g in groups:
            p0 = inst[g[0]]["p"]
            bt = {"bf16": agm.BF16, "fp8": agm.FP8_E4M3, "fp32": agm.F32}[p0.base_dtype]
            gws.append(agm.fused_slices_workspace(T, p0.d_in, [inst[j]["p"].d_out for j in g], bt, flags, device=dev)
                       if len(g) > 1 else None)
        seg = torch.empty(agm.segment_words(T), dtype=torch.int32, device=dev)
        insts.append((inst, seg, ids.clone(), act.clone(), gws))
    torch.cuda.synchronize()
    print(f"# {n_rot} rotated instance(s) of {inst_bytes / 1e6:.1f} MB", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    n_proj = len(projs)
    if args.concurrent:
        concurrent_line(args, w, insts, n_rot, n_slots)
        return

    n_groups = len(groups)
    # the library's one-launch rule for the segment build with the shrink
    combined = not args.separate_build and 1 <= T <= 256 and n_slots <= 1024
    j_first = groups[0][0]

    def step(i, ev=None):
        inst, seg, ids_d, act_d, gws = insts[i % n_rot]
        if ev is not None:
            ev["seg"][0].record(stream)
        if combined:
            c = inst[j_first]
            agm.build_shrink_dev(ids_d, act_d, c["pool"], seg, inst[j_first]["x"], c["v"])
        else:
            agm.build_segments_dev(ids_d, act_d, n_slots, seg)
        if ev is not None:
            ev["seg"][1].record(stream)
        for gi, g in enumerate(groups):
            x = inst[g[0]]["x"]                      # the group's one input
            for j in g:
                if combined and j == j_first:
                    continue                         # its shrink ran in the build launch
                c = inst[j]
                if ev is not None:
                    ev["shrink"][2 * j].record(stream)
                agm.shrink(c["pool"], seg, T, None, x, c["v"], launch=agm.LAUNCH_PERSISTENT)
                if ev is not None:
                    ev["shrink"][2 * j + 1].record(stream)
            if ev is not None:
                ev["fused"][2 * gi].record(stream)
            if len(g) == 1:
                c = inst[g[0]]
                agm.fused_linear(c["base"], c["pool"], seg, x, c["v"], c["y"], flags=flags, workspace=c["wsp"])
            else:
                agm.fused_linear_slices([inst[j]["base"] for j in g], [inst[j]["pool"] for j in g], seg, x,
                                        [inst[j]["v"] for j in g], [inst[j]["y"] for j in g], flags=flags,
                                        workspace=gws[gi])
            if ev is not None:
                ev["fused"][2 * gi + 1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K back-to-back steps between two events (the line's value).
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # The same K steps again with events around every launch, on the stream
    # the library launches on (torch's current stream), for each kernel's own
    # duration.  Event packets add gaps between launches, so the step time
    # above comes from the run without them.
    def mk(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    evs = [{"seg": mk(2), "shrink": mk(2 * n_proj), "fused": mk(2 * n_groups)} for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    per = {"seg": 0.0, "shrink": 0.0, "fused": 0.0}
    for ev in evs:
        per["seg"] += ev["seg"][0].elapsed_time(ev["seg"][1])
        for j in range(n_proj):
            if not (combined and j == j_first):   # one event pair per shrink launch
                per["shrink"] += ev["shrink"][2 * j].elapsed_time(ev["shrink"][2 * j + 1])
        for gi in range(n_groups):
            per["fused"] += ev["fused"][2 * gi].elapsed_time(ev["fused"][2 * gi + 1])
    per = {k: v / args.steps for k, v in per.items()}   # ms per step

    if args.calibrate_copy_mb:
        src = torch.empty(args.calibrate_copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # ---- algorithmic work --------------------------------------------------
    live = w.live()
    n_act = int(live.sum())
    alg = {"fused_bytes": 0, "fused_flops": 0, "shrink_bytes": 0, "shrink_flops": 0}
    first_of_group = {g[0] for g in groups}
    for jp, pr in enumerate(projs):
        p = pr["p"]
        el = 2 if p.data_dtype == "bf16" else 4
        wel = 1 if p.base_dtype == "fp8" else (2 if p.base_dtype == "bf16" else 4)
        used = sorted(set(int(a) for a in w.ids[live]))
        ranks = np.array([int(p.slot_rank[a]) for a in used])
        rows_r = np.array([int(p.slot_rank[a]) for a in w.ids[live]])
        adapters_A = int((ranks * p.d_in).sum()) * el
        adapters_B = int((ranks * p.d_out).sum()) * el
        v_bytes = int(rows_r.sum()) * 4
        x_once = T * p.d_in * el if jp in first_of_group else 0    # a group reads its input once
        alg["fused_bytes"] += (p.d_out * p.d_in * wel + (4 * p.d_out if p.base_dtype == "fp8" else 0)
                               + x_once + T * p.d_out * el + adapters_B + v_bytes)
        alg["fused_flops"] += 2 * T * p.d_in * p.d_out + 2 * int(rows_r.sum()) * p.d_out
        alg["shrink_bytes"] += adapters_A + n_act * p.d_in * el + v_bytes
        alg["shrink_flops"] += 2 * int(rows_r.sum()) * p.d_in
    fused_s = per["fused"] * 1e-3
    # (one launch for build and shrink: its time counts as shrink time too)
    shrink_s = (per["shrink"] + (per["seg"] if combined else 0.0)) * 1e-3
    fused_gbs = alg["fused_bytes"] / fused_s / 1e9
    fused_tfs = alg["fused_flops"] / fused_s / 1e12
    shrink_gbs = alg["shrink_bytes"] / shrink_s / 1e9
    base = w.projections[0].base_dtype
    mfma_dtype = "fp8" if (base == "fp8" and args.w8a8) else ("fp32" if base == "fp32" else "bf16")
    ridge = MFMA_PEAK_TFLOPS[mfma_dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    ai = alg["fused_flops"] / alg["fused_bytes"]
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(fused_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(fused_gbs / HBM_PEAK_GBS, 4)}
    else:
        # the fp32 path multiplies with vector FMAs (fp32 vector peak), the
        # others on MFMA at their dtype's dense peak
        pk = MFMA_PEAK_TFLOPS[mfma_dtype]
        roof = {"bound": "alu" if base == "fp32" else "mfma", "achieved": round(fused_tfs, 1), "peak": pk,
                "unit": "TFLOP/s", "frac": round(fused_tfs / pk, 4)}
    roof["kernel"] = "fused_f32_kernel" if base == "fp32" else DOMINANT
    roof["algorithmic_bytes_per_launch"] = alg["fused_bytes"] // n_groups
    roof["algorithmic_flops_per_launch"] = alg["fused_flops"] // n_groups
    # (a reading belongs to one kernel: the W8A8 option runs another one)
    roof["traffic"] = stored_traffic(w.name + ("_w8a8" if args.w8a8 else ""))

    value = T / (ms_step * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if mfma_dtype == "fp8" else ("f32" if base == "fp32" else "bf16"),
        "data": "synthetic (seeded generators; Llama-shaped; random-init adapters)",
        "config": {"workload": f"{w.name}: {w.description}",
                   "path": ("build_shrink_dev (one launch)" if combined
                            else "build_segments_dev -> shrink (persistent)") + " -> fused_linear"
                           + (" (one sliced launch per group: " + ", ".join("/".join(names[j] for j in g)
                                                                           for g in groups if len(g) > 1) + ")"
                              if any(len(g) > 1 for g in groups) else "")
                           + (" W8A8" if args.w8a8 else (" W8A16" if base == "fp8" else "")),
                   "T": T, "projections": n_proj, "fused_launches": n_groups, "live_rows": n_act,
                   "distinct_adapters": len(w.touched_slots()), "rotated_instances": n_rot},
        "roofline": roof,
        "kernels_us_per_step": {("build_shrink" if combined else "build_segments"): round(per["seg"] * 1e3, 2),
                                ("shrink_others" if combined else "shrink"): round(per["shrink"] * 1e3, 2),
                                "fused_linear": round(per["fused"] * 1e3, 2)},
        "shrink_hbm": {"achieved": round(shrink_gbs, 1), "unit": "GB/s",
                       "frac": round(shrink_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg["shrink_bytes"],
                       "includes_segment_build": combined},
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def concurrent_line(args, w, insts, n_rot: int, n_slots: int) -> None:
    """The decode step without fusion, base and adapter work side by side on
    disjoint CU sets ("From Overloaded to Guaranteed" (HALO) 4: base and LoRA
    layers on partitioned SMs): the base product alone on one CU-masked
    stream; the segment builder, the shrink and (after the base product) the
    expand on the other.  The fused step is timed in the same process for
    comparison.  One JSON line."""
    import torch
    import adapter_gemm_amd as agm
    if len(w.projections) != 1:
        sys.exit("--concurrent takes a workload of one projection (decode_bgmv, tiny_sgmv)")
    n_cus = agm.cu_count()
    k = args.concurrent
    # (the runtime refuses some masks, e.g. a single CU or 4 CUs of every 32)
    blocks = max(1, n_cus // 32)
    if not 0 < k < n_cus or (args.cu_layout == "spread" and k % blocks):
        sys.exit(f"--concurrent: 0 < BASE_CUS < {n_cus}" + (f", a multiple of {blocks}" if args.cu_layout == "spread" else ""))
    if args.cu_layout == "spread":
        base_cus = [c for c in range(n_cus) if c % 32 < k // blocks]
    else:
        base_cus = list(range(k))
    lora_cus = [c for c in range(n_cus) if c not in set(base_cus)]
    sA, sB = agm.CUMaskedStream(base_cus, n_cus), agm.CUMaskedStream(lora_cus, n_cus)
    main = torch.cuda.current_stream()
    T = w.T
    evs = [tuple(torch.cuda.Event() for _ in range(3)) for _ in range(n_rot)]

    def step_conc(i):
        inst, seg, ids_d, act_d, _ = insts[i % n_rot]
        c = inst[0]
        e0, e_base, e_lora = evs[i % n_rot]
        e0.record(main)
        sA.stream.wait_event(e0)
        sB.stream.wait_event(e0)
        agm.fused_linear(c["base"], None, None, c["x"], None, c["y"], workspace=c["wsp"], stream=sA.stream)
        e_base.record(sA.stream)
        agm.build_segments_dev(ids_d, act_d, n_slots, seg, stream=sB.stream)
        agm.shrink(c["pool"], seg, T, None, c["x"], c["v"], launch=agm.LAUNCH_PERSISTENT, stream=sB.stream)
        sB.stream.wait_event(e_base)
        agm.expand(c["pool"], seg, T, None, c["v"], c["y"], launch=agm.LAUNCH_PERSISTENT, stream=sB.stream)
        e_lora.record(sB.stream)
        main.wait_event(e_lora)

    def step_serial(i):                      # the same four calls, one stream
        inst, seg, ids_d, act_d, _ = insts[i % n_rot]
        c = inst[0]
        agm.fused_linear(c["base"], None, None, c["x"], None, c["y"], workspace=c["wsp"])
        agm.build_segments_dev(ids_d, act_d, n_slots, seg)
        agm.shrink(c["pool"], seg, T, None, c["x"], c["v"], launch=agm.LAUNCH_PERSISTENT)
        agm.expand(c["pool"], seg, T, None, c["v"], c["y"], launch=agm.LAUNCH_PERSISTENT)

    def step_fused(i):
        inst, seg, ids_d, act_d, _ = insts[i % n_rot]
        c = inst[0]
        agm.build_segments_dev(ids_d, act_d, n_slots, seg)
        agm.shrink(c["pool"], seg, T, None, c["x"], c["v"], launch=agm.LAUNCH_PERSISTENT)
        agm.fused_linear(c["base"], c["pool"], seg, c["x"], c["v"], c["y"], workspace=c["wsp"])

    # A step here costs more host time (launches, events, waits from Python)
    # than GPU time, so the main stream is held by a spin kernel while the host
    # queues every timed step; the GPU then runs them back to back and the
    # events measure GPU time only (the same for the fused step).
    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(2.4e9 * 400e-6 * args.steps))     # about 0.4 ms of spinning per step
        t0.record(main)
        h0 = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        t1.record(main)
        host_ms = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps, host_ms / args.steps

    ms_conc, host_conc = timed(step_conc)
    ms_fused, host_fused = timed(step_fused)
    ms_serial, _ = timed(step_serial)
    sA.close()
    sB.close()
    # the same two-stream step on streams without CU masks: what the
    # cross-stream waits cost by themselves
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    sA.stream, sB.stream = sA, sB
    ms_unmasked, _ = timed(step_conc)
    print(f"# host ms per step to queue: concurrent {host_conc:.3f}, fused {host_fused:.3f}", file=sys.stderr)
    out = {
        "metric": METRIC, "value": round(T / (ms_conc * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_conc, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.projections[0].base_dtype == "bf16" else "f32",
        "data": "synthetic (seeded generators; Llama-shaped; random-init adapters)",
        "config": {"workload": f"{w.name}: {w.description}",
                   "design": "concurrent CU-masked streams: base product (lora_fused_linear without a pool) on "
                             f"{len(base_cus)} CUs; build_segments_dev -> shrink -> [after the base] expand on "
                             f"{len(lora_cus)} CUs",
                   "cu_layout": args.cu_layout, "T": T, "rotated_instances": n_rot},
        "fused_ms_per_step": round(ms_fused, 5),
        "unfused_one_stream_ms_per_step": round(ms_serial, 5),
        "two_streams_without_masks_ms_per_step": round(ms_unmasked, 5),
        "concurrent_over_fused": round(ms_conc / ms_fused, 3),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, seconds: float):
    """The fp64 oracle (as it stands) on this host's cores, on a bounded
    sample of the same workload: whole batches for as long as `seconds`
    allows (at least one), or a slice of the rows for large workloads."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
    except ImportError:                       # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(cores) if threadpool_limits else None
    rows = w.T
    # large workloads: a row slice keeps the sample to ~10-30 s of CPU work
    macs = sum(p.d_in * p.d_out for p in w.projections)
    if macs * w.T > 4e10:
        rows = max(16, int(4e10 // macs))
    sel = np.arange(rows)
    ids, act = w.ids[sel], w.active[sel]
    touched = sorted(set(int(i) for i in ids[(ids >= 0) & (act != 0)]))
    data = []
    for p in w.projections:
        A, B = p.pool(touched)
        data.append((w.x(p)[sel], p.w0(), A, B, p.slot_rank, p.slot_scale))
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.build_segments(ids, act)
        for x, w0, A, B, rk, sc in data:
            oracle.linear(x, w0, ids, act, A, B, rk, sc)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = cores
    if ctx is not None:
        try:
            threads = max(i.get("num_threads", cores) for i in threadpool_info()) or cores
        except Exception:
            pass
        ctx.unregister() if hasattr(ctx, "unregister") else None
    return {"value": round(rows * n / dt, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} pass(es) of the fp64 oracle (segments + {len(w.projections)} projection(s)) "
                      f"over {rows} of {w.T} rows in {dt:.1f} s"}


if __name__ == "__main__":
    main()
