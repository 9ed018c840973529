#!/usr/bin/env python3
"""Throughput of the multi-adapter linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--configs all|none|a,b]

One step is one pass of the whole hot path over one batch: device-side
segment build -> shrink -> fused linear (base GEMM with the adapter
up-projection in its epilogue), for every projection of the workload.
Batches of at most 256 rows run the segment build and the first
projection's shrink as one launch (lora_build_shrink_dev);
--separate-build times them as two.
Inputs are resident in HBM before timing; several copies of every buffer
are rotated so that a step never finds its operands in the 256 MB
Infinity Cache.  Prints one JSON line.

The headline (`value`, `roofline`) is the prefill batch, the largest
workload by work (fused gate+up 4096->28672, bf16, 8192 tokens in 32
requests, 128 slots of ranks 8..64); --config selects another.  After it,
every workload is measured once more into `per_config` (fewer steps): the
fused path with its kernel times and roofline, for the fp8 workload both
W8A16 and W8A8, for the decode batch the unfused shrink + expand in every
launch-sizing mode against the HBM roofline, and for the Llama layer set
the launch-sizing modes of the unfused adapter term.  `cpu_baseline` is the
fp64 oracle on the host's cores (and on one thread for the two smallest
workloads), with the CPU model.
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="prefill_sgmv", choices=ALL_CONFIGS,
                    help="the headline workload (default: the prefill batch, the largest by work)")
    ap.add_argument("--configs", default="all",
                    help="workloads measured after the headline, one per_config entry each: 'all', 'none' or a "
                         "comma-separated list")
    ap.add_argument("--cpu-seconds-config", type=float, default=2.0,
                    help="oracle seconds per workload in cpu_baseline.per_config")
    ap.add_argument("--w8a8", action="store_true", help="fp8 base: quantise activations per token")
    ap.add_argument("--no-slices", action="store_true",
                    help="one fused call per projection (default: projections of one input share a call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-build", action="store_true",
                    help="segment build and shrink as two launches also for small batches")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--shrink-in-launch", action="store_true",
                    help="headline: each one-projection fused call computes its shrink in the same launch")
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


ALL_CONFIGS = ["tiny_sgmv", "decode_bgmv", "prefill_sgmv", "fp8_fused", "llama_layer"]


class Setup:
    """One workload on the device: every projection's base weight, adapter
    pool (only the slots the batch touches are filled; the others are zero
    and never read), input, output and v buffers, rotated over copies whose
    total exceeds twice the 256 MB Infinity Cache, plus the ids, the segment
    buffers and the fused workspaces of every copy."""

    def __init__(self, name: str, args, flags_list=(0,)):
        import torch
        import adapter_gemm_amd as agm
        from lora_inputs import make_workload
        dev = "cuda:0"
        self.agm = agm
        w = make_workload(name)
        self.w, self.T = w, w.T
        T = w.T

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

        touched = w.touched_slots()
        projs, inst_bytes = [], 0
        for p in w.projections:
            A, B = p.pool(touched)
            pr = {"p": p}
            mk = bf16 if p.data_dtype == "bf16" else (lambda a: torch.from_numpy(a).to(dev))
            pr["A"], pr["B"] = mk(A), mk(B)
            del A, B
            w0 = p.w0()
            if p.base_dtype == "fp8":
                pr["W"], pr["ws"] = torch.from_numpy(w0[0]).to(dev), torch.from_numpy(w0[1]).to(dev)
            else:
                pr["W"], pr["ws"] = mk(w0), None
            del w0
            pr["x"] = mk(w.x(p))
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
        self.n_slots = w.projections[0].n_slots
        self.names = [p.name for p in w.projections]
        self.inst_bytes = inst_bytes
        n_rot = min(64, max(1, -(-2 * CACHE_BYTES // max(inst_bytes, 1))))
        self.n_rot = n_rot
        self.insts = []
        bt_of = {"bf16": agm.BF16, "fp8": agm.FP8_E4M3, "fp32": agm.F32}
        for r in range(n_rot):
            inst = []
            for pr in projs:
                c = {k: (pr[k] if r == 0 else pr[k].clone()) if isinstance(pr[k], torch.Tensor) else pr[k]
                     for k in pr}
                c["pool"] = agm.pool_desc(c["A"], c["B"], c["rank"], c["scale"])
                c["base"] = agm.base_desc(c["W"], c["ws"])
                p = c["p"]
                c["wsp"] = {f: agm.fused_workspace(T, p.d_in, p.d_out, bt_of[p.base_dtype], f, device=dev)
                            for f in flags_list}
                inst.append(c)
            seg = torch.empty(agm.segment_words(T), dtype=torch.int32, device=dev)
            self.insts.append({"inst": inst, "seg": seg, "ids": ids.clone(), "act": act.clone(), "gws": {}})
        self.bt_of = bt_of
        torch.cuda.synchronize()
        print(f"# {name}: {w.description}; {n_rot} rotated instance(s) of {inst_bytes / 1e6:.1f} MB",
              file=sys.stderr, flush=True)

    def groups(self, slices: bool):
        if self.w.name in SLICE_GROUPS and slices:
            return [[self.names.index(n) for n in g] for g in SLICE_GROUPS[self.w.name]]
        return [[j] for j in range(len(self.names))]

    def group_workspaces(self, groups, flags):
        import torch
        for it in self.insts:
            key = (tuple(map(tuple, groups)), flags)
            if key in it["gws"]:
                continue
            gws = []
            for g in groups:
                p0 = it["inst"][g[0]]["p"]
                gws.append(self.agm.fused_slices_workspace(self.T, p0.d_in, [it["inst"][j]["p"].d_out for j in g],
                                                           self.bt_of[p0.base_dtype], flags, device="cuda:0")
                           if len(g) > 1 else None)
            it["gws"][key] = gws
        torch.cuda.synchronize()

    def release(self):
        import torch
        self.insts = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def ev_pair():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def algorithmic(S: Setup, groups):
    """Bytes and flops the method must move and do (each distinct live
    adapter's A and B once at its true rank, x once per input, v at fp32,
    y written once, W0 at its stored width)."""
    w, T = S.w, S.T
    live = w.live()
    n_act = int(live.sum())
    alg = {"fused_bytes": 0, "fused_flops": 0, "shrink_bytes": 0, "shrink_flops": 0, "expand_bytes": 0,
           "expand_flops": 0, "per_group_bytes": [], "per_group_flops": []}
    first_of_group = {g[0] for g in groups}
    per_proj = []
    for jp, p in enumerate(w.projections):
        el = 2 if p.data_dtype == "bf16" else 4
        wel = 1 if p.base_dtype == "fp8" else (2 if p.base_dtype == "bf16" else 4)
        used = sorted(set(int(a) for a in w.ids[live]))
        ranks = np.array([int(p.slot_rank[a]) for a in used], dtype=np.int64)
        rows_r = np.array([int(p.slot_rank[a]) for a in w.ids[live]], dtype=np.int64)
        adapters_A = int((ranks * p.d_in).sum()) * el
        adapters_B = int((ranks * p.d_out).sum()) * el
        v_bytes = int(rows_r.sum()) * 4
        x_once = T * p.d_in * el if jp in first_of_group else 0
        fb = (p.d_out * p.d_in * wel + (4 * p.d_out if p.base_dtype == "fp8" else 0) + x_once + T * p.d_out * el
              + adapters_B + v_bytes)
        ff = 2 * T * p.d_in * p.d_out + 2 * int(rows_r.sum()) * p.d_out
        per_proj.append((fb, ff))
        alg["fused_bytes"] += fb
        alg["fused_flops"] += ff
        alg["shrink_bytes"] += adapters_A + n_act * p.d_in * el + v_bytes
        alg["shrink_flops"] += 2 * int(rows_r.sum()) * p.d_in
        # the unfused expand reads B and v and reads and writes the live rows of y
        alg["expand_bytes"] += adapters_B + v_bytes + 2 * n_act * p.d_out * el
        alg["expand_flops"] += 2 * int(rows_r.sum()) * p.d_out
    for g in groups:
        alg["per_group_bytes"].append(sum(per_proj[j][0] for j in g))
        alg["per_group_flops"].append(sum(per_proj[j][1] for j in g))
    alg["n_active"] = n_act
    return alg


def roofline(bytes_, flops, seconds, base, mfma_dtype, kernel, traffic_key, launches):
    ridge = MFMA_PEAK_TFLOPS[mfma_dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    ai = flops / bytes_
    gbs = bytes_ / seconds / 1e9
    tfs = flops / seconds / 1e12
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        pk = MFMA_PEAK_TFLOPS[mfma_dtype]
        roof = {"bound": "alu" if base == "fp32" else "mfma", "achieved": round(tfs, 1), "peak": pk,
                "unit": "TFLOP/s", "frac": round(tfs / pk, 4)}
    roof["kernel"] = kernel
    roof["algorithmic_bytes_per_launch"] = bytes_ // launches
    roof["algorithmic_flops_per_launch"] = flops // launches
    tr = stored_traffic(traffic_key)
    roof["traffic"] = tr
    roof["traffic_over_algorithmic"] = None if tr is None else round(tr / (bytes_ / launches), 3)
    return roof


def fused_path(S: Setup, steps: int, warmup: int, flags: int, slices: bool, separate_build: bool,
               in_launch: bool = False):
    """The whole hot path, one step per batch: device segment build -> shrink
    -> fused linear for every projection (projections of one input share a
    sliced launch).  Returns the step time from K back-to-back steps between
    two events, and each kernel's duration from a second run of K steps with
    events around every launch (on the stream the library launches on)."""
    import torch
    agm, T = S.agm, S.T
    groups = S.groups(slices)
    S.group_workspaces(groups, flags)
    n_proj, n_groups = len(S.names), len(groups)
    # in_launch: each one-projection group's shrink runs inside its fused
    # launch ("EpiLoRA" 3.1, the decode path); the segment build is its own launch
    fl_one = flags | (agm.FLAG_SHRINK_IN_LAUNCH if in_launch else 0)
    if in_launch:
        for it in S.insts:
            for c in it["inst"]:
                if fl_one not in c["wsp"]:
                    p = c["p"]
                    c["wsp"][fl_one] = agm.fused_workspace(T, p.d_in, p.d_out, S.bt_of[p.base_dtype], fl_one,
                                                           device="cuda:0")
    combined = not separate_build and not in_launch and 1 <= T <= 256 and S.n_slots <= 1024
    j_first = groups[0][0]
    stream = torch.cuda.current_stream()
    gkey = (tuple(map(tuple, groups)), flags)

    def step(i, ev=None):
        it = S.insts[i % S.n_rot]
        inst, seg = it["inst"], it["seg"]
        if ev is not None:
            ev["seg"][0].record(stream)
        if combined:
            c = inst[j_first]
            agm.build_shrink_dev(it["ids"], it["act"], c["pool"], seg, c["x"], c["v"])
        else:
            agm.build_segments_dev(it["ids"], it["act"], S.n_slots, seg)
        if ev is not None:
            ev["seg"][1].record(stream)
        for gi, g in enumerate(groups):
            x = inst[g[0]]["x"]
            for j in g:
                if (combined and j == j_first) or (in_launch and len(g) == 1):
                    continue
                c = inst[j]
                if ev is not None:
                    ev["shrink"][j][0].record(stream)
                agm.shrink(c["pool"], seg, T, None, x, c["v"], launch=agm.LAUNCH_PERSISTENT)
                if ev is not None:
                    ev["shrink"][j][1].record(stream)
            if ev is not None:
                ev["fused"][gi][0].record(stream)
            if len(g) == 1:
                c = inst[g[0]]
                agm.fused_linear(c["base"], c["pool"], seg, x, c["v"], c["y"], flags=fl_one,
                                 workspace=c["wsp"][fl_one])
            else:
                agm.fused_linear_slices([inst[j]["base"] for j in g], [inst[j]["pool"] for j in g], seg, x,
                                        [inst[j]["v"] for j in g], [inst[j]["y"] for j in g], flags=flags,
                                        workspace=it["gws"][gkey][gi])
            if ev is not None:
                ev["fused"][gi][1].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = ev_pair()
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps

    evs = [{"seg": ev_pair(), "shrink": [ev_pair() for _ in range(n_proj)],
            "fused": [ev_pair() for _ in range(n_groups)]} for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    per = {"seg": 0.0, "shrink": 0.0, "fused": 0.0}
    fused_each = [0.0] * n_groups
    for ev in evs:
        per["seg"] += ev["seg"][0].elapsed_time(ev["seg"][1])
        for j in range(n_proj):
            if not (combined and j == j_first) and not (in_launch and any(len(g) == 1 and g[0] == j
                                                                          for g in groups)):
                per["shrink"] += ev["shrink"][j][0].elapsed_time(ev["shrink"][j][1])
        for gi in range(n_groups):
            d = ev["fused"][gi][0].elapsed_time(ev["fused"][gi][1])
            per["fused"] += d
            fused_each[gi] += d
    per = {k: v / steps for k, v in per.items()}
    fused_each = [v / steps for v in fused_each]

    alg = algorithmic(S, groups)
    base = S.w.projections[0].base_dtype
    w8a8 = bool(flags & agm.FLAG_ACT_QUANT_E4M3)
    mfma_dtype = "fp8" if (base == "fp8" and w8a8) else ("fp32" if base == "fp32" else "bf16")
    roof = roofline(alg["fused_bytes"], alg["fused_flops"], per["fused"] * 1e-3, base, mfma_dtype,
                    "fused_f32_kernel" if base == "fp32" else DOMINANT, S.w.name + ("_w8a8" if w8a8 else ""),
                    n_groups)
    shrink_s = (per["shrink"] + (per["seg"] if combined else 0.0)) * 1e-3
    # (in_launch: no shrink launch of its own; its bytes are inside the fused time)
    shrink_gbs = alg["shrink_bytes"] / shrink_s / 1e9 if shrink_s > 0 else 0.0
    names = S.names
    return {
        "ms_per_step": ms_step,
        "value": T / (ms_step * 1e-3),
        "combined": combined,
        "groups": groups,
        "path": ("build_shrink_dev (one launch)" if combined else
                 ("build_segments_dev -> fused_linear with the shrink in the same launch" if in_launch else
                  "build_segments_dev -> shrink (persistent)"))
                + ("" if in_launch else " -> fused_linear")
                + (" (one sliced launch per group: " + ", ".join("/".join(names[j] for j in g)
                                                                for g in groups if len(g) > 1) + ")"
                   if any(len(g) > 1 for g in groups) else "")
                + (" W8A8" if w8a8 else (" W8A16" if base == "fp8" else "")),
        "mfma_dtype": mfma_dtype,
        "roofline": roof,
        "kernels_us_per_step": {("build_shrink" if combined else "build_segments"): round(per["seg"] * 1e3, 2),
                                ("shrink_others" if combined else "shrink"): round(per["shrink"] * 1e3, 2),
                                "fused_linear": round(per["fused"] * 1e3, 2)},
        "fused_us_per_launch": {"/".join(names[j] for j in g): round(fused_each[gi] * 1e3, 2)
                                for gi, g in enumerate(groups)},
        "shrink_hbm": {"achieved": round(shrink_gbs, 1), "unit": "GB/s", "frac": round(shrink_gbs / HBM_PEAK_GBS, 4),
                       "algorithmic_bytes": alg["shrink_bytes"], "includes_segment_build": combined},
        "alg": alg,
    }


def quant_roofline(S: Setup, steps: int, warmup: int):
    """The W8A8 activation quantisation alone (lora_quantize_e4m3 on the
    workload's x), against the HBM roofline: T*d bf16 read, T*d codes and T
    scales written per launch; an event pair around every launch on the
    stream the library launches on."""
    import torch
    agm = S.agm
    x = S.insts[0]["inst"][0]["x"]
    T, d = int(x.shape[0]), int(x.shape[1])
    q = torch.empty(T, d, dtype=torch.uint8, device=x.device)
    s = torch.empty(T, dtype=torch.float32, device=x.device)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        agm.quantize_e4m3(x, q, s)
    torch.cuda.synchronize()
    evs = [ev_pair() for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        agm.quantize_e4m3(x, q, s)
        e1.record(stream)
    torch.cuda.synchronize()
    us = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps * 1e3
    nbytes = T * d * 2 + T * d + 4 * T
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "quant_kernel", "shape": [T, d], "us_per_launch": round(us, 2), "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes}


def unfused_adapter(S: Setup, steps: int, warmup: int, modes):
    """The adapter term without fusion: lora_shrink then lora_expand (y += s B v
    in place) for every projection, per launch-sizing mode ("LoRazor" 3.1.1-3.1.2:
    the exact tile list, the shared row bound R and the full-batch bound).  The
    segment buffer is built once per rotated copy (host planner, which also
    gives EXACT and BUCKETED their host summary); each mode's K steps run back
    to back with events around every launch.  Row tiles launched and holding
    rows are counted from the summary: exact sum_a ceil(m_a/16), bucketed
    L ceil(R/16), full batch L ceil(T/16) with L = min(T, slots)."""
    import torch
    agm, T = S.agm, S.T
    stream = torch.cuda.current_stream()
    summaries = []
    for it in S.insts:
        staging = torch.empty(agm.segment_words(T), dtype=torch.int32).pin_memory()
        summaries.append(agm.build_segments(torch.from_numpy(S.w.ids), torch.from_numpy(S.w.active), S.n_slots,
                                            it["seg"], staging))
        torch.cuda.synchronize()
    s0 = summaries[0]
    L = min(T, S.n_slots)
    tiles = {agm.LAUNCH_EXACT: s0.n_tiles_small, agm.LAUNCH_PERSISTENT: s0.n_tiles_small,
             agm.LAUNCH_BUCKETED: L * -(-s0.row_bound // 16), agm.LAUNCH_FULL_BATCH: L * -(-T // 16)}
    mode_name = {agm.LAUNCH_EXACT: "exact", agm.LAUNCH_PERSISTENT: "persistent", agm.LAUNCH_BUCKETED: "bucketed",
                 agm.LAUNCH_FULL_BATCH: "full_batch"}
    alg = algorithmic(S, [[j] for j in range(len(S.names))])
    out = {"row_tiles_with_rows": s0.n_tiles_small, "row_bound": s0.row_bound, "slots_L": L, "modes": []}
    for mode in modes:
        def step(i, ev=None):
            it = S.insts[i % S.n_rot]
            summ = summaries[i % S.n_rot]
            for c in it["inst"]:
                if ev is not None:
                    ev[0].record(stream)
                agm.shrink(c["pool"], it["seg"], T, summ, c["x"], c["v"], launch=mode)
                if ev is not None:
                    ev[1].record(stream)
                agm.expand(c["pool"], it["seg"], T, summ, c["v"], c["y"], launch=mode)
                if ev is not None:
                    ev[2].record(stream)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0, t1 = ev_pair()
        t0.record(stream)
        for i in range(steps):
            step(i)
        t1.record(stream)
        torch.cuda.synchronize()
        pair_ms = t0.elapsed_time(t1) / steps
        evs = [[tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in S.names]
               for _ in range(steps)]
        sh = ex = 0.0
        for i in range(steps):
            it_evs = evs[i]
            it = S.insts[i % S.n_rot]
            summ = summaries[i % S.n_rot]
            for c, e in zip(it["inst"], it_evs):
                e[0].record(stream)
                agm.shrink(c["pool"], it["seg"], T, summ, c["x"], c["v"], launch=mode)
                e[1].record(stream)
                agm.expand(c["pool"], it["seg"], T, summ, c["v"], c["y"], launch=mode)
                e[2].record(stream)
        torch.cuda.synchronize()
        for it_evs in evs:
            for e in it_evs:
                sh += e[0].elapsed_time(e[1])
                ex += e[1].elapsed_time(e[2])
        sh, ex = sh / steps * 1e-3, ex / steps * 1e-3           # seconds per step
        both = alg["shrink_bytes"] + alg["expand_bytes"]
        out["modes"].append({
            "mode": mode_name[mode], "row_tiles_launched": int(tiles[mode]),
            "shrink_us": round(sh * 1e6, 2), "expand_us": round(ex * 1e6, 2),
            "shrink_expand_us": round(pair_ms * 1e3, 2),
            "shrink_hbm_frac": round(alg["shrink_bytes"] / sh / 1e9 / HBM_PEAK_GBS, 4),
            "expand_hbm_frac": round(alg["expand_bytes"] / ex / 1e9 / HBM_PEAK_GBS, 4),
            "pair_hbm_frac": round(both / (pair_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    out["algorithmic_bytes"] = {"shrink": alg["shrink_bytes"], "expand": alg["expand_bytes"]}
    out["target_hbm_frac"] = 0.70
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    torch.cuda.set_device(0)
    flags = agm.FLAG_ACT_QUANT_E4M3 if args.w8a8 else 0

    if args.concurrent:
        S = Setup(args.config, args)
        concurrent_line(args, S.w, [(it["inst"], it["seg"], it["ids"], it["act"], None) for it in S.insts],
                        S.n_rot, S.n_slots)
        return

    # ---- the headline workload -------------------------------------------
    S = Setup(args.config, args, flags_list=(flags,))
    r = fused_path(S, args.steps, args.warmup, flags, not args.no_slices, args.separate_build,
                   in_launch=args.shrink_in_launch)
    if args.calibrate_copy_mb:
        src = torch.empty(args.calibrate_copy_mb << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    w = S.w
    out = {
        "metric": METRIC,
        "value": round(r["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if r["mfma_dtype"] == "fp8" else ("f32" if r["mfma_dtype"] == "fp32" else "bf16"),
        "data": "synthetic (seeded generators; Llama-shaped; random-init adapters)",
        "config": {"workload": f"{w.name}: {w.description}", "path": r["path"], "T": S.T,
                   "projections": len(S.names), "fused_launches": len(r["groups"]),
                   "live_rows": r["alg"]["n_active"], "distinct_adapters": len(w.touched_slots()),
                   "rotated_instances": S.n_rot},
        "roofline": r["roofline"],
        "kernels_us_per_step": r["kernels_us_per_step"],
        "shrink_hbm": r["shrink_hbm"],
    }
    S.release()
    del S

    # ---- every workload, one line each (the headline's numbers repeated) ---
    configs = [] if args.configs == "none" else (ALL_CONFIGS if args.configs == "all" else args.configs.split(","))
    per_cfg = {}
    steps_c, warm_c = max(5, min(args.steps, 50)), max(2, min(args.warmup, 10))
    for name in configs:
        if name == args.config and not args.w8a8:
            rr = r
            entry = _cfg_entry(rr)
            entry["same_as_headline"] = True
            per_cfg[name] = entry
            if name not in ("decode_bgmv", "llama_layer"):
                continue
        fl = (0, agm.FLAG_ACT_QUANT_E4M3) if name == "fp8_fused" else (0,)
        Sc = Setup(name, args, flags_list=fl)
        if name not in per_cfg:
            per_cfg[name] = _cfg_entry(fused_path(Sc, steps_c, warm_c, 0, not args.no_slices, args.separate_build))
        if name == "fp8_fused":
            per_cfg["fp8_fused_w8a8"] = _cfg_entry(fused_path(Sc, steps_c, warm_c, agm.FLAG_ACT_QUANT_E4M3, True,
                                                              args.separate_build))
            per_cfg["fp8_fused_w8a8"]["quant_hbm"] = quant_roofline(Sc, steps_c, warm_c)
        if name in ("decode_bgmv", "fp8_fused"):
            # the shrink inside the fused launch, against the separate launches above
            per_cfg[name + "_shrink_in_launch"] = _cfg_entry(
                fused_path(Sc, steps_c, warm_c, 0, not args.no_slices, args.separate_build, in_launch=True))
        if name == "decode_bgmv":
            per_cfg[name]["unfused_shrink_expand"] = unfused_adapter(
                Sc, steps_c, warm_c, (agm.LAUNCH_PERSISTENT, agm.LAUNCH_EXACT, agm.LAUNCH_BUCKETED,
                                      agm.LAUNCH_FULL_BATCH))
        if name == "llama_layer":
            per_cfg[name]["launch_sizing"] = unfused_adapter(
                Sc, max(5, steps_c // 2), warm_c, (agm.LAUNCH_EXACT, agm.LAUNCH_BUCKETED, agm.LAUNCH_FULL_BATCH))
        Sc.release()
        del Sc
    if per_cfg:
        out["per_config"] = per_cfg

    if not args.no_cpu_baseline:
        from lora_inputs import make_workload
        out["cpu_baseline"] = cpu_baseline(make_workload(args.config), args.cpu_seconds)
        out["cpu_baseline"]["cpu_model"] = cpu_model()
        extra = {}
        for name in configs:
            wk = make_workload(name)
            e = {"threads_all": cpu_baseline(wk, args.cpu_seconds_config)}
            if name in ("tiny_sgmv", "decode_bgmv"):
                e["threads_1"] = cpu_baseline(wk, args.cpu_seconds_config, threads=1)
            extra[name] = {k: {kk: v[kk] for kk in ("value", "unit", "cores", "sample")} for k, v in e.items()}
        if extra:
            out["cpu_baseline"]["per_config"] = extra
    print(json.dumps(out), flush=True)


def _cfg_entry(r):
    return {"ms_per_step": round(r["ms_per_step"], 5), "tokens_per_s": round(r["value"], 1),
            "path": r["path"], "kernels_us_per_step": r["kernels_us_per_step"],
            "fused_us_per_launch": r["fused_us_per_launch"], "roofline": r["roofline"],
            "shrink_hbm": r["shrink_hbm"]}


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


def cpu_baseline(w, seconds: float, threads=None):
    """The fp64 oracle (as it stands) on this host's cores, on a bounded
    sample of the same workload: whole batches for as long as `seconds`
    allows (at least one), or a slice of the rows for large workloads.
    `threads` limits the BLAS threads (default: every core this process may
    run on)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
    except ImportError:                       # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    want = cores if threads is None else threads
    ctx = threadpool_limits(want) if threadpool_limits else None
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
    used = want
    if ctx is not None:
        try:
            used = max(i.get("num_threads", want) for i in threadpool_info()) or want
        except Exception:
            pass
        ctx.unregister() if hasattr(ctx, "unregister") else None
    return {"value": round(rows * n / dt, 2), "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"{n} pass(es) of the fp64 oracle (segments + {len(w.projections)} projection(s)) "
                      f"over {rows} of {w.T} rows of {w.name} in {dt:.1f} s"}


if __name__ == "__main__":
    main()
