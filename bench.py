"""Benchmark of the SchNet CFConv energy/force MD step on one MI355X.

A step is one velocity-Verlet step of all replicas: half kick + drift,
neighbour-list rebuild (cell list, or all-pairs bit-mask tiles for replicas
of at most 512 atoms; exact fp32 predicate), one energy+force
evaluation (radial basis, filter network, CFConv, readout, analytic
backward, forces) and the second half kick.  Inputs are seeded synthetic CG
chains resident in HBM before timing starts.

The headline line is the 64 x 269-bead workload's MD rate; the same JSON line
carries, under "configs", the other workloads (evaluations and neighbour
builds with their kernel rooflines, MD under several neighbour-list
schedules) and the int16 filter weights' rate and drift.

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batched_replicas]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# peaks of one MI355X (AMD datasheet)
PEAK_HBM_GBS = 8000.0
PEAK_FP16_MFMA_TFLOPS = 2500.0
# The filter kernels compute every fp32 product as three fp16 matrix products
# (hi.hi + hi.lo + lo.hi), so the ceiling for their fp32 algorithmic FLOPs is
# a third of the dense fp16 peak.
PEAK_SPLIT_F16_TFLOPS = PEAK_FP16_MFMA_TFLOPS / 3.0

WORKLOAD_TEXT = {
    "batched_replicas": "64 replicas x 269-bead CG chain (block-diagonal CSR), rc 12 A, 3 interactions, "
                        "F=128, 50 Gaussians; velocity Verlet 2 fs, neighbour list rebuilt every step",
    "larger_cg": "16 replicas x 1000-bead compact CG chain, rc 12 A, 5 interactions, F=128, 50 Gaussians; "
                 "velocity Verlet 2 fs, rebuild every step",
    "dense_box": "15,668 particles, periodic box at 0.1/A^3, rc 6 A, 3 interactions, F=128, 32 Gaussians, "
                 "particles numbered along a Morton curve of 6 A cells; velocity Verlet 2 fs, rebuild every step",
    "dense_box_random_order": "the same periodic box with its particles in random-sequential-addition order",
    "single_protein": "1 x 269-bead CG chain, rc 12 A, 3 interactions, F=128, 50 Gaussians",
    "tiny_chain": "1 x 32-bead CG chain, rc 10 A, 2 interactions, F=32, 16 Gaussians",
}


def filter_flops_per_pair(F: int, K: int):
    """Algorithmic FLOPs of one filter evaluation (one unordered pair, shared by its two directed
    edges) in one interaction:
        forward : rbf @ A1 (2KF) + ssp(a) @ A2 (2F^2)
        backward: g_phi @ A2^T (2F^2) + g_a @ A1^T (2FK)
    Recomputed products and padding are not counted."""
    return 2 * K * F + 2 * F * F, 2 * F * F + 2 * F * K


def cfconv_algorithmic_bytes(E: int, F: int):
    """Algorithmic HBM bytes of one CFConv launch: per directed edge its filter row (4F bytes in
    fp32) and its column index (4 bytes).  The gathered input rows are served by the caches; the
    kernel itself stores each row once per pair in 24 bits and reads it from both of its edges, so
    the counters measure what it really moves."""
    return E * (4 * F + 4)


def kernel_sources() -> list:
    """The HIP sources and headers of the library (every .hip and .h under csrc/)."""
    d = os.path.join(ROOT, "schnet_cfconv_force_amd", "csrc")
    return sorted(n for n in os.listdir(d) if n.endswith((".hip", ".h")))


def source_hash() -> str:
    """sha256 of the HIP sources: hardware counters are only valid for this code."""
    import hashlib
    h = hashlib.sha256()
    for name in kernel_sources():
        with open(os.path.join(ROOT, "schnet_cfconv_force_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")


def _short_kernel(name: str) -> str:
    import re
    name = name.replace("void ", "").replace("sn::(anonymous namespace)::", "").replace("sn::", "")
    return re.sub(r"[<(].*", "", name)


def summarize_pmc(fetch_csv: str, write_csv: str, probe_mib: int, workload: str, command: str) -> str:
    """Markdown summary of two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE).

    Both counters are in KiB per dispatch.  Each is scaled by the factor that
    makes it read the known size of the probe copy (probe_mib MiB read and
    written by the copy kernel that runs first).
    """
    import collections
    import csv
    per = {}
    factor = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        agg = collections.defaultdict(list)
        probe = None
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"] and (probe is None or v > probe):
                probe = v
            agg[_short_kernel(r["Kernel_Name"])].append(v)
        factor[counter] = (probe_mib * 1024.0) / probe if probe else 1.0
        per[counter] = {k: sum(v) / len(v) for k, v in agg.items()}
    rows = []
    data = {"workload": workload, "source_hash": source_hash(), "probe_mib": probe_mib,
            "fetch_factor": round(factor["FETCH_SIZE"], 4), "write_factor": round(factor["WRITE_SIZE"], 4),
            "bytes_per_launch": {}}
    for k in sorted(per["FETCH_SIZE"], key=lambda k: -per["FETCH_SIZE"][k] - per["WRITE_SIZE"].get(k, 0)):
        if k.startswith("__amd") or k.startswith("at::"):
            continue
        f = per["FETCH_SIZE"][k]
        w = per["WRITE_SIZE"].get(k, 0.0)
        b = (f * factor["FETCH_SIZE"] + w * factor["WRITE_SIZE"]) * 1024.0
        data["bytes_per_launch"][k] = int(b)
        rows.append(f"| {k} | {f:.1f} | {w:.1f} | {b / 1e6:.1f} |")
    import json as _json
    return "\n".join([
        f"# HBM traffic per launch, {workload}",
        "",
        "Two `rocprofv3 --pmc` passes (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, mean over dispatches).",
        f"A {probe_mib} MiB device copy runs first; the counters are scaled so that it reads {probe_mib} MiB:",
        f"FETCH_SIZE x {factor['FETCH_SIZE']:.4f}, WRITE_SIZE x {factor['WRITE_SIZE']:.4f}.",
        "FETCH_SIZE counts L2 misses to the memory fabric, so reads served by the Infinity Cache count too.",
        "",
        "Commands (from the repository root):",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB / launch |",
        "|---|---|---|---|",
        *rows,
        "",
        "Machine-readable (read by bench.py; ignored once the HIP sources change):",
        "",
        "```json",
        _json.dumps(data),
        "```",
        "",
    ])


UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
                 "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS",
                 "GRBM_GUI_ACTIVE")


def summarize_util(csv_path: str, workload: str, command: str, n_simd: int = 1024, n_xcd: int = 8) -> str:
    """Markdown summary of one rocprofv3 --pmc pass over UTIL_COUNTERS, per kernel (mean per dispatch).

    MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs); LDS bank-conflict cycles per
    LDS-active cycle; VALU issue = SQ_ACTIVE_INST_VALU (quad-cycles) x 4 / (GRBM_GUI_ACTIVE x SIMDs).
    """
    import collections
    import csv
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        vals[_short_kernel(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    rows = []
    for k in ("filter_bwd_kernel", "filter_fwd_kernel", "cfconv_kernel", "chain_kernel", "tile_count_kernel",
              "tile_fill_kernel", "forces_kernel"):
        if k not in vals:
            continue
        m = {c: sum(v) / len(v) for c, v in vals[k].items()}
        # rocprofv3 sums GRBM_GUI_ACTIVE over the XCDs; the elapsed cycles are its per-XCD value
        gui = m.get("GRBM_GUI_ACTIVE", 0.0) / n_xcd
        if gui <= 0:
            continue
        mfma = 100.0 * m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * n_simd)
        valu = 100.0 * 4.0 * m.get("SQ_ACTIVE_INST_VALU", 0.0) / (gui * n_simd)
        lds_act = m.get("SQ_LDS_IDX_ACTIVE", 0.0)
        confl = m.get("SQ_LDS_BANK_CONFLICT", 0.0)
        rows.append(f"| {k} | {gui:.0f} | {mfma:.1f} % | {valu:.1f} % | {m.get('SQ_INSTS_VALU_MFMA_MOPS_F16', 0) * 512 / 1e9:.1f} "
                    f"| {confl / max(lds_act, 1.0):.4f} | {m.get('SQ_INSTS_LDS', 0):.0f} |")
    return "\n".join([
        f"# Matrix-core, VALU and LDS counters per launch, {workload}",
        "",
        "One `rocprofv3 --pmc` pass (mean per dispatch).  GUI-active cycles = GRBM_GUI_ACTIVE per XCD",
        f"(the summed counter / {n_xcd}).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI-active x {n_simd} SIMDs);",
        f"VALU active = 4 x SQ_ACTIVE_INST_VALU (quad-cycles) / (GUI-active x {n_simd});",
        "F16 MFMA GFLOP = 512 x SQ_INSTS_VALU_MFMA_MOPS_F16 / 1e9;",
        "LDS conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles per active cycle).",
        "",
        "Command (repository root):",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | GUI-active cycles | MFMA busy | VALU active | F16 MFMA GFLOP | LDS conflict cycles / active | LDS instructions |",
        "|---|---|---|---|---|---|---|",
        *rows,
        "",
    ])


CACHE_COUNTERS = ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCP_TOTAL_CACHE_ACCESSES_sum",
                  "TCP_TCC_READ_REQ_sum", "TCP_TCC_READ_REQ_LATENCY_sum")


def summarize_cache(csv_path: str, workload: str, command: str) -> str:
    """Markdown summary of one rocprofv3 --pmc pass over CACHE_COUNTERS, per kernel (mean per
    dispatch): L2 hit rate, L2 read requests to DRAM, vector L1 accesses, L1-to-L2 read requests and
    their mean latency."""
    import collections
    import csv
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        vals[_short_kernel(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    rows = []
    for k in ("filter_bwd_kernel", "filter_fwd_kernel", "cfconv_kernel", "chain_kernel", "tile_count_kernel",
              "tile_fill_kernel", "forces_kernel"):
        if k not in vals:
            continue
        m = {c: sum(v) / len(v) for c, v in vals[k].items()}
        hit, miss = m.get("TCC_HIT_sum", 0.0), m.get("TCC_MISS_sum", 0.0)
        req = m.get("TCP_TCC_READ_REQ_sum", 0.0)
        lat = m.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / req if req > 0 else 0.0
        rows.append(f"| {k} | {100.0 * hit / max(hit + miss, 1.0):.1f} % | {hit + miss:.3g} | "
                    f"{m.get('TCC_EA0_RDREQ_DRAM_sum', 0.0):.3g} | {m.get('TCP_TOTAL_CACHE_ACCESSES_sum', 0.0):.3g} | "
                    f"{req:.3g} | {lat:.0f} |")
    return "\n".join([
        f"# L1 and L2 counters per launch, {workload}",
        "",
        "One `rocprofv3 --pmc` pass (mean per dispatch).  L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS);",
        "DRAM read requests = TCC_EA0_RDREQ_DRAM (L2 misses sent to memory); L1 accesses =",
        "TCP_TOTAL_CACHE_ACCESSES; L1-to-L2 reads = TCP_TCC_READ_REQ and their mean latency in cycles =",
        "TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ.",
        "",
        "Command (repository root):",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | L2 hit rate | L2 requests | DRAM read requests | L1 accesses | L1-to-L2 reads | mean L1-to-L2 read latency (cycles) |",
        "|---|---|---|---|---|---|---|",
        *rows,
        "",
    ])


def summarize_stats(csv_path: str, workload: str, command: str) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run (its kernel_stats.csv), one row per
    kernel: calls, average / min / max duration in microseconds and share of GPU time."""
    import csv
    rows = []
    for r in csv.DictReader(open(csv_path)):
        name = r.get("Name") or r.get("KernelName") or ""
        calls = int(float(r.get("Calls", 0)))
        avg = float(r.get("AverageNs", 0.0)) / 1e3
        mn = float(r.get("MinNs", 0.0)) / 1e3
        mx = float(r.get("MaxNs", 0.0)) / 1e3
        pct = float(r.get("Percentage", 0.0))
        if name.startswith("Cijk_"):
            label = "vendor fp16 GEMM (the device-rate probe)"
        elif "copyBuffer" in name:
            label = "runtime copy kernel (probes and host transfers)"
        else:
            label = _short_kernel(name) + (name[name.find("<"):name.find(">") + 1] if "<" in name else "")
        rows.append((pct, f"| {label} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.2f} % |"))
    rows.sort(key=lambda t: -t[0])
    return "\n".join([
        f"# rocprofv3 kernel statistics, {workload}",
        "",
        "Command (repository root, MI355X):",
        "",
        "```",
        command,
        "```",
        "",
        "The run covers the device-rate probes, the initial neighbour build and evaluation, the warm-up,",
        "uninstrumented and event-timed MD steps, and the fixed-list evaluations and neighbour builds that",
        "bench.py times after them; every library kernel runs on one stream, so each duration is that",
        "kernel alone.  Durations in microseconds, from the kernel_stats.csv that the command writes.",
        "",
        "| kernel | calls | average us | min us | max us | share of GPU time |",
        "|---|---|---|---|---|---|",
        *[r for _, r in rows],
        "",
    ])


def load_traffic(workload: str):
    import json as _json
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        data = _json.loads(blob)
    except (IndexError, ValueError):
        return None
    if data.get("source_hash") != source_hash():
        return None
    return data["bytes_per_launch"]


def event_times(fn, n: int):
    """Per-call milliseconds of fn() from HIP events on the current stream."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def measured_peaks(torch):
    """Device rates to set the datasheet peaks beside: a 1 GiB device-to-device
    copy (read + write bytes / time) and a large fp16 GEMM in the vendor
    library (divided by three for the split-fp16 product rate)."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    ms = event_times(lambda: b.copy_(a), 10)
    copy = 2 * 4 * n / (min(ms) * 1e-3) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, dtype=torch.float16, device="cuda")
    y = torch.randn(m, m, dtype=torch.float16, device="cuda")
    torch.matmul(x, y)
    ms = event_times(lambda: torch.matmul(x, y), 10)
    gemm = 2 * m ** 3 / (min(ms) * 1e-3) / 1e12
    return {"hbm_copy_GBs": round(copy, 1), "f16_gemm_TFLOPs": round(gemm, 1),
            "split_f16_mfma_TFLOPs_via_gemm": round(gemm / 3, 1),
            "how": "1 GiB float32 device copy (2 x 4 B per element); 8192^3 fp16 torch.matmul; best of 10"}


def cpu_baseline(cfg, seconds: float):
    """Time the CPU oracle (as it is) on a bounded sample of the same workload."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    rp = cfg["replica_ptr"]
    B = len(rp) - 1
    n_sample = min(B, 4)
    idx = [int(b) for b in np.linspace(0, B - 1, n_sample).round()]
    t0 = time.perf_counter()
    done = 0
    while True:
        for b in idx:
            s, e = rp[b], rp[b + 1]
            sub = np.array([0, e - s], np.int32)
            csr = O.neighbors_bruteforce(cfg["pos"][s:e], sub, cfg["hyper"]["cutoff"], cfg["box"])
            O.energy_forces(cfg["params"], cfg["hyper"], cfg["types"][s:e], cfg["pos"][s:e], sub, csr, cfg["box"])
            done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    per_replica = dt / done
    evals_per_s = 1.0 / (per_replica * B)
    return {"value": evals_per_s, "unit": "evals/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} single-replica oracle evaluations (brute-force neighbour list + fp64 energy "
                      f"and forces) of replicas {idx}, {dt:.1f} s, scaled to all {B} replicas",
            "seconds": round(dt, 2), "host_cpu_count": os.cpu_count(), "blas_threads": int(threads),
            "threads_note": "NumPy fp64; its BLAS calls (the matrix products) use blas_threads threads, "
                            "the rest of the oracle one"}


# ---------------------------------------------------------------------------
# measured runs


class Workload:
    """One seeded workload on the device: model, system, positions, velocities, initial forces."""

    def __init__(self, sn, torch, name: str, fmt: int = 0, math: int = 0):
        import numpy as np
        import synth
        self.sn, self.torch, self.name = sn, torch, name
        cfg = synth.make_config(name)
        self.cfg = cfg
        h = cfg["hyper"]
        self.N, self.B = len(cfg["pos"]), len(cfg["replica_ptr"]) - 1
        self.F, self.K, self.I = h["n_features"], h["n_rbf"], h["n_interactions"]
        self.cutoff = h["cutoff"]
        if "vel" not in cfg:
            cfg["vel"] = synth.maxwell_boltzmann(self.N, cfg["replica_ptr"], 110.0, 300.0, 2)
            cfg["inv_mass"] = np.full(self.N, 1.0 / 110.0, np.float32)
        self.model = sn.Model(cfg["params"], h, filter_format=fmt, filter_math=math)
        self.system = sn.System(cfg["replica_ptr"], cfg["types"], cfg["box"])
        self.capacity = self.N * 200
        self.ws = sn.workspace(self.model, self.system, self.capacity)
        self.row_ptr = torch.empty(self.N + 1, dtype=torch.int32, device="cuda")
        self.col = torch.empty(self.capacity, dtype=torch.int32, device="cuda")
        self.rev = torch.empty(self.capacity, dtype=torch.int32, device="cuda")
        self.reset()

    def reset(self):
        torch, sn, cfg = self.torch, self.sn, self.cfg
        self.pos = torch.from_numpy(cfg["pos"]).cuda()
        self.vel = torch.from_numpy(cfg["vel"]).cuda()
        self.inv_mass = torch.from_numpy(cfg["inv_mass"]).cuda()
        rp, col, rev, E = sn.build_csr_neighbors(self.system, self.pos, self.cutoff, self.capacity, self.ws)
        self.E = E
        self.row_ptr.copy_(rp)
        self.col[:E].copy_(col)
        self.rev[:E].copy_(rev)
        _, self.forces = sn.energy_forces(self.model, self.system, self.pos, self.row_ptr, self.col, self.rev, E,
                                          self.ws)
        torch.cuda.synchronize()

    def md(self, n, skin=0.0, rebuild_every=1, graph=False, epot=None, ekin=None):
        """n MD steps in one call; returns each step's edge count."""
        import synth
        if n <= 0:
            return []
        elog = self.torch.zeros(n, dtype=self.torch.int32, device="cuda")
        self.sn.verlet_step(self.model, self.system, self.pos, self.vel, self.forces, self.inv_mass, 2.0,
                            synth.FORCE_TO_ACCEL, n, self.cutoff + skin, self.capacity, self.ws, epot, ekin,
                            csr=(self.row_ptr, self.col, self.rev), edge_log=elog, rebuild_every=rebuild_every,
                            graph=graph)
        return [int(e) for e in elog.cpu().tolist()]

    def eval(self):
        self.sn.energy_forces(self.model, self.system, self.pos, self.row_ptr, self.col, self.rev, self.E, self.ws,
                              forces=self.forces)

    def build(self):
        return self.sn.build_csr_neighbors(self.system, self.pos, self.cutoff, self.capacity, self.ws)

    def time_md(self, steps, warmup, **kw):
        """Wall-clock seconds per MD step (one call of `steps` steps, no timing events inside)."""
        self.reset()
        self.md(warmup, **kw)
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        edges = self.md(steps, **kw)
        self.torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps, edges

    def profile(self, fn, n):
        """Per kernel class: (total ms, launches) from HIP events around every launch of n calls."""
        sn = self.sn
        sn.profile_enable(True)
        sn.profile_collect()
        for _ in range(n):
            fn()
        self.torch.cuda.synchronize()
        prof = sn.profile_collect()
        sn.profile_enable(False)
        return prof


def kernel_rooflines(prof, P, E, F, K, traffic=None, flops_pairs=None):
    """Roofline entries of the filter kernels (matrix cores, fp16 peak) and the CFConv (HBM).

    prof: per class (total ms, launches) over launches that each processed P pairs / E directed
    edges (flops_pairs overrides the pair count summed over all launches of a class).
    traffic: counter bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled), or None."""
    fwd_pp, bwd_pp = filter_flops_per_pair(F, K)
    out = {}
    for name, per_pair, kern in (("filter_bwd", bwd_pp, "filter_bwd_kernel"), ("filter_fwd", fwd_pp,
                                                                                "filter_fwd_kernel")):
        if name not in prof:
            continue
        ms, n = prof[name]
        pairs = flops_pairs[name] if flops_pairs else P * n
        flops = per_pair * pairs
        achieved = flops / (ms * 1e-3) / 1e12
        out[name] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_MFMA_TFLOPS, 4),
                     "traffic": traffic.get(kern) if traffic else None,
                     "avg_launch_us": round(1e3 * ms / n, 2), "flops_per_launch": int(flops / n),
                     "flops_basis": "fp32 algorithmic FLOPs of one filter evaluation per unordered pair "
                                    f"({per_pair} per pair; recompute and padding not counted)",
                     "mfma_dtype": "f16 (each fp32 product as three fp16 products)",
                     "frac_of_split_peak": round(achieved / PEAK_SPLIT_F16_TFLOPS, 4),
                     "split_peak_TFLOPs": round(PEAK_SPLIT_F16_TFLOPS, 1)}
    if "cfconv" in prof:
        ms, n = prof["cfconv"]
        us = 1e3 * ms / n
        alg = cfconv_algorithmic_bytes(E, F)
        r = {"bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s", "avg_launch_us": round(us, 2),
             "algorithmic_bytes_per_launch": int(alg),
             "algorithmic_GBs": round(alg / (us * 1e-6) / 1e9, 1),
             "algorithmic_basis": "4F + 4 bytes per directed edge (an fp32 filter row and a column index)"}
        t = traffic.get("cfconv_kernel") if traffic else None
        if t:
            achieved = t / (us * 1e-6) / 1e9
            r.update({"achieved": round(achieved, 1), "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": t,
                      "achieved_basis": "hardware counters (FETCH_SIZE + WRITE_SIZE, scaled) / launch time"})
        else:
            r.update({"achieved": None, "frac": None, "traffic": None,
                      "achieved_basis": "no counter profile for the current kernels"})
        out["cfconv"] = r
    return out


def kernels_table(prof, steps):
    return {k: {"ms_per_step": v[0] / steps, "launches_per_step": v[1] / steps, "avg_us": 1e3 * v[0] / max(v[1], 1)}
            for k, v in prof.items()}


def measure_eval_config(sn, torch, name, n_rep=20):
    """Fixed-CSR evaluations, the neighbour build, one evaluation with its rebuild, and the kernel
    rooflines of one workload."""
    import numpy as np
    W = Workload(sn, torch, name)
    for _ in range(3):
        W.eval()
    torch.cuda.synchronize()
    assert sn.read_status(W.ws) == sn.SN_OK
    ev = event_times(W.eval, n_rep)
    nb = event_times(W.build, n_rep)
    both = event_times(lambda: (W.build(), W.eval()), n_rep)
    prof = W.profile(W.eval, 5)
    med = float(np.median(ev))
    res = {"workload": WORKLOAD_TEXT[name], "n_atoms": W.N, "n_replicas": W.B, "n_edges": W.E,
           "eval_ms": {"median": round(med, 4), "min": round(float(np.min(ev)), 4), "n": n_rep},
           "evals_per_s": round(1e3 / med, 2), "edges_per_s": round(W.E * 1e3 / med, 1),
           "neighbour_build_ms": {"median": round(float(np.median(nb)), 4), "min": round(float(np.min(nb)), 4)},
           "rebuild_plus_eval_ms": round(float(np.median(both)), 4),
           "roofline_kernels": kernel_rooflines(prof, W.E // 2, W.E, W.F, W.K, load_traffic(name)),
           "kernels": kernels_table(prof, 5)}
    return W, res


def md_variants(W, steps, warmup, variants):
    """MD steps/s and aggregate ns/day of a workload under several neighbour-list schedules."""
    out = {}
    for label, kw in variants:
        sec, edges = W.time_md(steps, warmup, **kw)
        out[label] = {"steps_per_s": round(1.0 / sec, 2), "ms_per_step": round(sec * 1e3, 4),
                      "ns_per_day": round(W.B / sec * 2.0 * 1e-6 * 86400.0, 1), "edges_mean": round(
                          sum(edges) / len(edges), 1), "schedule": kw}
    return out


def mode_drift(sn, torch, mode: str, steps=100):
    """Drift of an alternative filter mode from the default (fp32 weights, fp32-accurate products) on
    the 64 x 269 workload: mode "int16" (per-output-channel int16 filter weights) or "fp16_math" (one
    fp16 product per filter-network product).  One evaluation at the same neighbour list (relative
    energy change, RMS force change over RMS force), the difference of the total-energy traces over
    `steps` MD steps (fp64 logs), and both MD rates (timed alternately, best of two)."""
    import numpy as np
    kw = {"int16": {"fmt": 1}, "fp16_math": {"math": 1}}[mode]
    runs, work = {}, {}
    for alt in (0, 1):
        W = Workload(sn, torch, "batched_replicas", **(kw if alt else {}))
        e, f = sn.energy_forces(W.model, W.system, W.pos, W.row_ptr, W.col, W.rev, W.E, W.ws)
        e = e.cpu().numpy().astype(np.float64)
        f = f.cpu().numpy().astype(np.float64)
        ep = torch.zeros((steps, W.B), dtype=torch.float64, device="cuda")
        ek = torch.zeros((steps, W.B), dtype=torch.float64, device="cuda")
        W.md(steps, epot=ep, ekin=ek)
        tot = (ep + ek).cpu().numpy()
        runs[alt] = (e, f, tot, ek.cpu().numpy())
        work[alt] = W
    sec = {0: float("inf"), 1: float("inf")}
    for _ in range(2):
        for alt in (0, 1):
            sec[alt] = min(sec[alt], work[alt].time_md(20, 3)[0])
    e0, f0, t0, k0 = runs[0]
    e1, f1, t1, _ = runs[1]
    W1 = work[1]
    prof = W1.profile(lambda: W1.md(1), 10)

    def slope_per_ns(tot):
        # least-squares slope of each replica's total energy over time (2 fs steps)
        t_ns = np.arange(tot.shape[0]) * 2.0e-6
        tc = t_ns - t_ns.mean()
        return (tc[:, None] * (tot - tot.mean(axis=0))).sum(axis=0) / max((tc ** 2).sum(), 1e-30)
    s0, s1 = slope_per_ns(t0), slope_per_ns(t1)
    return {"kernels": {k: v for k, v in kernels_table(prof, 10).items() if k.startswith("filter")},
            "rel_dE_max": float(np.abs(e1 - e0).max() / np.abs(e0).max()),
            "rms_dF_over_rms_F": float(np.sqrt(((f1 - f0) ** 2).mean() / (f0 ** 2).mean())),
            "etot_trace_max_abs_diff_kcal_mol": float(np.abs(t1 - t0).max()),
            "etot_trace_diff_over_mean_ekin": float(np.abs(t1 - t0).max() / k0.mean()),
            "etot_drift_fp32_kcal_mol": float(np.abs(t0 - t0[0]).max()),
            f"etot_drift_{mode}_kcal_mol": float(np.abs(t1 - t1[0]).max()),
            "etot_slope_fp32_kcal_mol_per_ns": {"mean": float(s0.mean()), "max_abs": float(np.abs(s0).max())},
            f"etot_slope_{mode}_kcal_mol_per_ns": {"mean": float(s1.mean()), "max_abs": float(np.abs(s1).max())},
            "md_steps": steps,
            "md_steps_per_s_fp32": round(1.0 / sec[0], 2), f"md_steps_per_s_{mode}": round(1.0 / sec[1], 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batched_replicas", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--filter-format", type=int, default=0, choices=[0, 1])
    ap.add_argument("--graph", action="store_true", help="replay the MD steps as a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="only the headline workload")
    ap.add_argument("--drift-steps", type=int, default=0,
                    help="only the long-run drift of the int16 weights and of the fp16-product filter against "
                         "the default on the 64 x 269 workload, over this many MD steps; one JSON line")
    ap.add_argument("--no-measure-peaks", dest="measure_peaks", action="store_false",
                    help="skip the device-copy and fp16-GEMM rate measurements (fractions of measured rates)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first copy a buffer of this many MiB (calibrates hardware byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary of two rocprofv3 --pmc runs to profiles/ and exit")
    ap.add_argument("--pmc-command", default="", help="command line recorded in the traffic summary")
    ap.add_argument("--summarize-util", metavar="CSV",
                    help="write the MFMA/VALU/LDS counter summary of one rocprofv3 --pmc run to profiles/ and exit")
    ap.add_argument("--summarize-cache", metavar="CSV",
                    help="write the L1/L2 counter summary of one rocprofv3 --pmc run to profiles/ and exit")
    ap.add_argument("--summarize-stats", metavar="CSV",
                    help="write the summary of a rocprofv3 --kernel-trace --stats run to profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_stats:
        md = summarize_stats(args.summarize_stats, args.workload, args.pmc_command)
        with open(os.path.join(ROOT, "profiles", f"kernel_stats_{args.workload}.md"), "w") as f:
            f.write(md)
        print(md)
        return
    if args.summarize_cache:
        md = summarize_cache(args.summarize_cache, args.workload, args.pmc_command)
        with open(os.path.join(ROOT, "profiles", f"cache_{args.workload}.md"), "w") as f:
            f.write(md)
        print(md)
        return
    if args.summarize_util:
        md = summarize_util(args.summarize_util, args.workload, args.pmc_command)
        with open(os.path.join(ROOT, "profiles", f"mfma_lds_{args.workload}.md"), "w") as f:
            f.write(md)
        print(md)
        return
    if args.summarize_pmc:
        md = summarize_pmc(*args.summarize_pmc, args.copy_probe_mb, args.workload, args.pmc_command)
        with open(traffic_file(args.workload), "w") as f:
            f.write(md)
        print(md)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.drift_steps > 0 and args.gpus == 1 and world == 1:
        import torch
        import schnet_cfconv_force_amd as sn
        out = {"drift_steps": args.drift_steps, "workload": WORKLOAD_TEXT["batched_replicas"]}
        for mode in ("int16", "fp16_math"):
            print(f"[bench] {args.drift_steps}-step drift, {mode}", file=sys.stderr, flush=True)
            out[mode] = mode_drift(sn, torch, mode, steps=args.drift_steps)
        print(json.dumps(out))
        return
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not part of "
              f"this build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import schnet_cfconv_force_amd as sn

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.copy_probe_mb > 0:
        src = torch.ones(args.copy_probe_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # device rates first (untimed for the headline; they also bring the GPU out of idle)
    peaks = measured_peaks(torch) if args.measure_peaks else None

    # ---------------------------------------------------------------- headline
    log(f"headline: {args.workload} MD, {args.steps} steps")
    W = Workload(sn, torch, args.workload, fmt=args.filter_format)
    N, B, F, K, I = W.N, W.B, W.F, W.K, W.I
    W.md(args.warmup, graph=args.graph)
    torch.cuda.synchronize()
    # uninstrumented pass (no timing events in the stream)
    t0 = time.perf_counter()
    edges = W.md(args.steps, graph=args.graph)
    torch.cuda.synchronize()
    sec_plain = (time.perf_counter() - t0) / args.steps
    # instrumented pass: HIP events around every kernel on the launch stream (the graph is not used
    # here: launches recorded into a graph are not timed individually)
    sn.profile_enable(True)
    sn.profile_collect()
    t0 = time.perf_counter()
    edges_p = W.md(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = sn.profile_collect()
    sn.profile_enable(False)
    assert sn.read_status(W.ws) == sn.SN_OK
    sec_events = (t1 - t0) / args.steps
    evals_per_s = 1.0 / sec_plain
    E_mean = float(np.mean(edges))
    P_total = sum(e // 2 for e in edges_p)
    ns_per_day = B * evals_per_s * 2.0 * 1e-6 * 86400.0

    # fixed-CSR energy+force evaluations (the same kernels without rebuild / integration)
    # the last step (of the instrumented pass) rebuilt the list at the final positions, into W's
    # list buffers
    E_last = edges_p[-1]
    W.E = E_last
    for _ in range(3):
        W.eval()
    torch.cuda.synchronize()
    n_fixed = max(20, args.steps)
    t2 = time.perf_counter()
    for _ in range(n_fixed):
        W.eval()
    torch.cuda.synchronize()
    fixed_evals_per_s = n_fixed / (time.perf_counter() - t2)
    eval_ms = event_times(W.eval, n_fixed)
    assert sn.read_status(W.ws) == sn.SN_OK
    nb_ms = event_times(W.build, n_fixed)

    traffic = load_traffic(args.workload)
    pairs_per_class = {k: P_total * I for k in ("filter_fwd", "filter_bwd")}
    rl = kernel_rooflines(prof, None, int(E_mean), F, K, traffic, flops_pairs=pairs_per_class)
    dominant = max(prof.items(), key=lambda kv: kv[1][0])[0]
    main_rl = rl.get(dominant) or rl.get("filter_bwd")

    out = {
        "metric": "energy+force evals/sec and edges/sec at 1 GPU; aggregate ns/day (2 fs step)",
        "value": round(evals_per_s, 2),
        "unit": "evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec_plain * 1e3, 4),
        "ms_per_step_with_kernel_events": round(sec_events * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 (fp32-accurate split-fp16 MFMA products, filter rows stored in 24 bits)"
                 + (", int16 filter weights" if args.filter_format else ""),
        "data": "synthetic (seeded CG chains / particle box, random-init weights)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload, "n_atoms": N,
                   "n_replicas": B, "n_edges_mean": round(E_mean, 1), "n_interactions": I, "n_features": F,
                   "n_rbf": K, "dt_fs": 2.0, "graph_replay": bool(args.graph), "parallelism": "single GPU"},
        "edges_per_s": round(E_mean * evals_per_s, 1),
        "ns_per_day": round(ns_per_day, 1),
        "evals_per_s_fixed_csr": round(fixed_evals_per_s, 2),
        "edges_per_s_fixed_csr": round(E_last * fixed_evals_per_s, 1),
        "eval_ms_fixed_csr": {"median": round(float(np.median(eval_ms)), 4), "min": round(float(np.min(eval_ms)), 4),
                              "n": len(eval_ms)},
        "neighbour_build_ms": {"median": round(float(np.median(nb_ms)), 4), "min": round(float(np.min(nb_ms)), 4),
                               "n": len(nb_ms)},
        "peak_device_memory_bytes": int(torch.cuda.max_memory_allocated()),
        "workspace_bytes": int(W.ws.numel()),
        "roofline": main_rl,
        "roofline_kernels": rl,
        "dominant_kernel": dominant,
        "kernels": kernels_table(prof, args.steps),
        "context": {"pages_ns_per_day": 1000, "pages_hardware": "1x NVIDIA RTX PRO 6000, 64 x 269-bead 1ENH"},
    }
    if peaks:
        out["measured_peaks"] = peaks
        for r in rl.values():
            if r.get("achieved") is None:
                continue
            ref = peaks["hbm_copy_GBs"] if r["unit"] == "GB/s" else peaks["f16_gemm_TFLOPs"]
            r["frac_vs_measured"] = round(r["achieved"] / ref, 4)
    del W
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- the other workloads
    if not args.no_configs:
        configs = {}
        md_kw = [("rebuild_every_step", {}), ("rebuild_every_step_graph", {"graph": True}),
                 ("skin_0.5A_graph", {"skin": 0.5, "rebuild_every": 0, "graph": True}),
                 ("skin_1A_graph", {"skin": 1.0, "rebuild_every": 0, "graph": True})]
        for name in ("tiny_chain", "single_protein", "larger_cg", "dense_box", "dense_box_random_order"):
            log(f"config {name}")
            Wc, res = measure_eval_config(sn, torch, name)
            if name in ("tiny_chain", "single_protein"):
                res["md"] = md_variants(Wc, 200, 20, md_kw)
            elif name != "dense_box_random_order":
                res["md"] = md_variants(Wc, 10, 3, md_kw[:2])
            configs[name] = res
            del Wc
            torch.cuda.empty_cache()
        log("config batched_replicas neighbour-list schedules")
        Wb = Workload(sn, torch, "batched_replicas")
        configs["batched_replicas"] = {"workload": WORKLOAD_TEXT["batched_replicas"],
                                       "md": md_variants(Wb, 20, 3, md_kw)}
        del Wb
        torch.cuda.empty_cache()
        log("config batched_replicas with int16 filter weights")
        configs["batched_replicas_int16"] = {
            "workload": WORKLOAD_TEXT["batched_replicas"] + "; per-output-channel int16 filter weights",
            **mode_drift(sn, torch, "int16")}
        log("config batched_replicas with one fp16 product per filter product")
        configs["batched_replicas_fp16_filter_math"] = {
            "workload": WORKLOAD_TEXT["batched_replicas"] + "; filter network with one fp16 product per fp32 "
                        "product (reduced precision, not the headline arithmetic)",
            **mode_drift(sn, torch, "fp16_math")}
        out["configs"] = configs
    if not args.no_cpu_baseline:
        log("cpu baseline")
        cfg = __import__("synth").make_config(args.workload)
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
