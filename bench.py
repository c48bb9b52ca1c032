"""Benchmark of the MI355X LSH-attention forward (hash, sort, chunk attention, combine).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload paper_64k]

One step = the four calls over one batch of synthetic input already resident in
HBM.  Prints one JSON line.  The K timed steps are bracketed by two HIP events
and nothing else; per-call times come from a second pass of K steps with an
event pair around every call (event records cost host time, which a small step,
bound by the host time of its calls, would otherwise include).  `roofline` describes the call with the
largest time: achieved = algorithmic bytes (or FLOPs) per launch / its average
duration.  `traffic` is the HBM traffic per launch of that kernel measured with
rocprofv3 counters (profiles/pmc_traffic.json), or null when those counters were
taken on a different kernel source.  Every call also carries its MFMA and HBM
fractions and, for the four steps, the target fraction it is held to.
`cpu_baseline` is the CPU oracle timed on this host's cores (a process pool,
one BLAS thread per worker) on the same workload (a prefix of each sequence
above 64K positions), run before the first GPU call; `hash_check` counts the
near-ties and mismatches of the GPU's buckets against the oracle's on the
positions it hashed.

Other modes:
    --layer D_MODEL      time the attention layer instead: the shared-QK and value
                         projections of x [B, L, D_MODEL], the four calls and the
                         output projection (a second workload; no CPU baseline)
    --block D_MODEL      time one Reformer block forward and its input recompute
                         (the reversible inverse) at this model width, feed-forward
                         width --d-ff (default 4 x D_MODEL), --chunk-rows rows per
                         feed-forward chunk (no CPU baseline)
    --graph              also time the step captured into one HIP graph and replayed
                         (launch overhead removed; `value` is then the replay rate)
    --backward           time forward + backward (lsh_attn_backward with a synthetic
                         loss gradient at the output; no CPU baseline)
    --copy-calibration   run only a plain 1 GiB device copy (for scaling the
                         FETCH_SIZE / WRITE_SIZE counters)
    --pmc-summary F W CF CW   turn four rocprofv3 --pmc output folders (FETCH_SIZE
                         and WRITE_SIZE on the benchmark, then on the copy) into
                         profiles/pmc_traffic.json (no GPU needed)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
METRIC = "LSH-attn fwd tokens/s at L=64K, 8 heads, 8 rounds; % MFMA/HBM peak"
# Sources whose text decides each call's kernels (device helpers included): the
# committed counter figures are only used while these files are unchanged.
KERNEL_SOURCES = {
    "lsh_hash": ["lsh_hash.hip", "lsh_device.h"],
    "lsh_sort": ["lsh_sort.hip"],
    "lsh_chunk_attn": ["lsh_chunk_attn.h", "lsh_chunk_attn.hip", "lsh_chunk_attn_bf16_d64.hip",
                       "lsh_chunk_attn_bf16_d128.hip", "lsh_chunk_attn_f32_d64.hip",
                       "lsh_chunk_attn_f32_d128.hip", "lsh_device.h"],
    "lsh_combine_rounds": ["lsh_combine.hip", "lsh_device.h"],
    "lsh_attn_backward": ["lsh_attn_bwd.hip", "lsh_chunk_attn.h", "lsh_device.h"],
    "lsh_project_in": ["lsh_linear.hip", "lsh_device.h"],
    "lsh_project_out": ["lsh_linear.hip", "lsh_device.h"],
    "lsh_project_out_add": ["lsh_linear.hip", "lsh_device.h"],
    "lsh_ffn": ["lsh_linear.hip", "lsh_device.h"],
}
KERNEL_SYMBOLS = {"lsh_hash": "k_hash", "lsh_sort": "k_sort_*", "lsh_chunk_attn": "k_chunk_attn",
                  "lsh_combine_rounds": "k_combine", "lsh_attn_backward": "k_attn_bwd",
                  "lsh_project_in": "k_linear", "lsh_project_out_add": "k_linear",
                  "lsh_ffn": "k_linear",
                  "lsh_project_out": "k_linear"}
LAYER_METRIC = "LSH-attention layer fwd tokens/s (projections + the four calls)"
BACKWARD_METRIC = "LSH-attention fwd+bwd tokens/s (the four calls + lsh_attn_backward)"
BLOCK_METRIC = "Reformer block fwd + input recompute tokens/s (reversible halves, chunked FFN)"
PMC_TRAFFIC = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def algorithmic_work(w, d_model=None, d_ff=None):
    """Algorithmic FLOPs and HBM bytes per launch of each call.

    TR = token-head-rounds, T = token-heads, e = bytes per element.
      hash     2*d*(nb/2) FLOP per TR; reads qk once (T*d*e) and R, writes 4 B per TR
      sort     reads the bucket (4 B), writes perm (4 B) and cid (2 B): 10 B per TR
      attn     8*c*d FLOP per TR (QK^T and PV over a 2c-key window); gathers the qk
               and v rows once and writes the o_rounds row (3*d*e), reads perm (4),
               writes lse (4), reads the cid row (2*n_r) per TR
      combine  reads n_r rows and lse values, writes one row: n_r*(d*e+4) + d*e per T
      project_in   2*(2*H*d)*d_model FLOP per token; reads x and both weights once,
                   writes qk and v
      project_out  2*d_model*H*d FLOP per token; reads o and w_o, writes y
                   (project_out_add also reads the residual)
      ffn      2*2*d_model*d_ff FLOP per token; reads x, the residual and the
               weights, writes y (the hidden chunk stays out of the count)
      backward  20*c*d FLOP per TR (scores, dP, dQ, dK, dV over the 2c-key window);
                per TR gathers qk, v, d_o rows and writes three bf16 partial rows
                (6*d*e), reads perm, cid, LSE and Delta (12 + 2*n_r); per T the
                prep reads o, d_o and n_r lse values and writes LSE, Delta, and the
                reduce reads 3*n_r partial rows and writes two float32 rows
    """
    e = 2 if w.dtype == "bf16" else 4
    T = w.batch * w.heads * w.seq_len
    TR = T * w.n_rounds
    d, nb = w.d_head, w.n_buckets
    work = {
        "lsh_hash": {"flops": 2.0 * d * (nb // 2) * TR,
                     "bytes": T * d * e + w.n_rounds * d * (nb // 2) * e + 4.0 * TR},
        "lsh_sort": {"flops": 0.0, "bytes": 10.0 * TR},
        "lsh_chunk_attn": {"flops": 8.0 * w.chunk * d * TR,
                           "bytes": TR * (3.0 * d * e + 8 + 2 * w.n_rounds)},
        "lsh_combine_rounds": {"flops": 0.0,
                               "bytes": T * (w.n_rounds * (d * e + 4.0) + d * e)},
    }
    work["lsh_attn_backward"] = {
        "flops": 20.0 * w.chunk * d * TR,
        "bytes": TR * (6.0 * d * e + 12 + 2 * w.n_rounds)
        + T * (2.0 * d * e + 4 * w.n_rounds + 8)
        + T * (3.0 * w.n_rounds * d * e + 2 * d * 4)}
    if d_model:
        M, hd = w.batch * w.seq_len, w.heads * d
        work["lsh_project_in"] = {"flops": 2.0 * M * 2 * hd * d_model,
                                  "bytes": e * (M * d_model + 2.0 * hd * d_model + 2.0 * M * hd)}
        work["lsh_project_out"] = {"flops": 2.0 * M * d_model * hd,
                                   "bytes": e * (M * hd + d_model * hd + 1.0 * M * d_model)}
        work["lsh_project_out_add"] = {"flops": 2.0 * M * d_model * hd,
                                       "bytes": e * (M * hd + d_model * hd + 2.0 * M * d_model)}
    if d_model and d_ff:
        M = w.batch * w.seq_len
        work["lsh_ffn"] = {"flops": 4.0 * M * d_model * d_ff,
                           "bytes": e * (3.0 * M * d_model + 2.0 * d_model * d_ff + d_ff + d_model)}
    return work


def bound_of(name, w):
    """Binding roofline of each call at the benchmark sizes: the hash and the
    projections are dense contractions (hundreds to thousands of FLOP per byte),
    the others stream memory (the backward does about 65 FLOP per byte at
    the 64K-token workload, far below the MFMA/HBM balance)."""
    return "mfma" if name in ("lsh_hash", "lsh_project_in", "lsh_project_out", "lsh_project_out_add",
                             "lsh_ffn") else "hbm"


# Targets per call: at least this fraction of the MI355X peak, of the named
# resource (chunk attention: bf16 MFMA; hash, sort and combine: HBM).
TARGET_FRACTION = {"lsh_chunk_attn": ("mfma", 0.5), "lsh_hash": ("hbm", 0.6),
                   "lsh_sort": ("hbm", 0.6), "lsh_combine_rounds": ("hbm", 0.6)}


def both_fractions(name, w, ms, d_model=None, d_ff=None):
    """(MFMA fraction, HBM fraction) of a call's algorithmic FLOPs and bytes at
    the published peaks, whichever binds it."""
    work = algorithmic_work(w, d_model, d_ff)[name]
    sec = ms * 1e-3
    mfma = work["flops"] / sec / (PEAK_MFMA_TFLOPS[w.dtype] * 1e12)
    hbm = work["bytes"] / sec / (PEAK_HBM_GBS * 1e9)
    return round(mfma, 4), round(hbm, 4)


def roofline_entry(name, w, ms, d_model=None, d_ff=None):
    work = algorithmic_work(w, d_model, d_ff)[name]
    if bound_of(name, w) == "mfma":
        ach = work["flops"] / (ms * 1e-3) / 1e12
        peak = PEAK_MFMA_TFLOPS[w.dtype]
        unit = "TFLOP/s"
    else:
        ach = work["bytes"] / (ms * 1e-3) / 1e9
        peak = PEAK_HBM_GBS
        unit = "GB/s"
    return {"bound": bound_of(name, w), "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4)}


def source_sha(name):
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "lsh_attention_02_amd", "csrc", fn), "rb") as f:
            h.update(fn.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_for(name, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    if not os.path.exists(PMC_TRAFFIC):
        return None
    with open(PMC_TRAFFIC) as f:
        rec = json.load(f)
    ent = rec.get("workloads", {}).get(workload, {}).get("kernels", {}).get(name)
    if not ent or ent.get("source_sha256") != source_sha(name):
        return None
    return ent.get("hbm_bytes_per_launch")


# The oracle's per-token work does not depend on the sequence length at a fixed
# bucket count, chunk and round count (the hash costs d * nb/2 per token-round,
# a query attends to 2 * chunk keys, the sort is linear), so a prefix of every
# (batch row, head) measures the same tokens/s as the whole sequence.  Longer
# sequences are timed on a prefix of this many positions.
CPU_BASELINE_MAX_POSITIONS = 65536


def cpu_baseline(w, x, flags=0):
    """The oracle timed on this host's cores: a process pool (oracle/pool.py),
    one BLAS thread per worker, over the (batch row, head) slices and rounds of
    the workload (a prefix of each slice when L is above
    CPU_BASELINE_MAX_POSITIONS).  Must run before the first GPU call: its
    workers are spawned processes.  Returns (the JSON entry, the oracle's
    buckets and margins of the positions it hashed)."""
    import numpy as np
    from oracle.pool import MAX_WORKERS, OraclePool, host_cores

    Lp = min(w.seq_len, CPU_BASELINE_MAX_POSITIONS)
    qk = np.ascontiguousarray(x["qk"][:, :, :Lp])
    v = np.ascontiguousarray(x["v"][:, :, :Lp])
    # Each hash job holds a few [16384, n_buckets] float64 arrays; keep the
    # workers' peak within half the memory available.
    per_job = 3 * 16384 * w.n_buckets * 8 + 64 * (2 << 20)
    avail = _mem_available()
    cores = min(host_cores(), MAX_WORKERS)
    workers = max(1, min(cores, int(0.5 * avail / per_job))) if avail else cores
    with OraclePool(workers) as pool:
        out = pool.forward(qk, v, x["R"], w.n_buckets, w.chunk, w.causal,
                           dup_correct=not (flags & 1), wrap=bool(flags & 2),
                           same_bucket=bool(flags & 4), keep=("buckets", "margins", "o"))
    assert np.isfinite(out["o"]).all()
    sec = out["seconds"]
    tokens = w.batch * Lp
    sample = (f"the whole workload: {w.batch * w.heads} (batch row, head) slices x {w.n_rounds} rounds x "
              f"{w.seq_len} positions" if Lp == w.seq_len else
              f"the first {Lp} of the {w.seq_len} positions of all {w.batch * w.heads} (batch row, head) "
              f"slices, {w.n_rounds} rounds (same buckets, chunk and rounds: the same work per token)")
    entry = {"value": round(tokens / sec["total"], 1), "unit": "tokens/s", "cores": workers,
             "kind": "oracle",
             "sample": f"{sample}; hash+sort {sec['hash_sort']:.1f} s, attention {sec['attention']:.1f} s, "
                       f"combine {sec['combine']:.1f} s wall-clock on {workers} worker processes "
                       f"(one BLAS thread each) of {host_cores()} host cores"}
    return entry, out["buckets"], out["margins"], Lp


def _mem_available():
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return 0


def hash_check(gpu_buckets, ref_buckets, margins, Lp, L):
    """Near-ties and mismatches of the GPU's buckets against the oracle's on
    the positions the CPU baseline hashed."""
    import numpy as np
    near = margins <= 1.0e-4
    mism = gpu_buckets[..., :Lp] != ref_buckets
    return {"hashes": int(mism.size), "near_ties": int(near.sum()), "mismatches": int(mism.sum()),
            "mismatches_beyond_near_ties": int((mism & ~near).sum()),
            "sample": "every hash" if Lp == L else f"the hashes of the first {Lp} positions"}


def pmc_summary(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands):
    """HBM bytes per launch of each call from rocprofv3 counter CSVs.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, each from a run of its own)
    are scaled by what the same counter reads for the 1 GiB device copy of
    --copy-calibration (rocclr's copyBuffer kernel), so that the factor turns
    the counter into bytes the way a copy of known size defines them."""
    import csv
    import collections

    def per_kernel(d, counter):
        sums = collections.defaultdict(list)
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    sums[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return sums

    def copy_factor(d, counter, nbytes):
        vals = [v for k, vs in per_kernel(d, counter).items() if "copyBuffer" in k for v in vs]
        if not vals:
            raise SystemExit(f"no copyBuffer dispatch with {counter} in {d}")
        return nbytes / (1024.0 * sum(vals) / len(vals))

    gib = float(1 << 30)
    ff = copy_factor(copy_fetch_dir, "FETCH_SIZE", gib)
    wf = copy_factor(copy_write_dir, "WRITE_SIZE", gib)
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    from synthetic_inputs import WORKLOADS
    work = algorithmic_work(WORKLOADS[workload])
    kernels = {}
    for name, sym in KERNEL_SYMBOLS.items():
        prefix = sym.rstrip("*")

        def per_launch(table):
            # Launch count = dispatches of the call's first kernel; the sort's
            # kernels add up to one call.
            hits = {k: v for k, v in table.items()
                    if re.search(r"::" + re.escape(prefix) + r"\w*[<(]", k)}
            if not hits:
                return None
            launches = max(len(v) for v in hits.values())
            return sum(sum(v) for v in hits.values()) / launches
        f_kib, w_kib = per_launch(fetch), per_launch(write)
        if f_kib is None or w_kib is None or name not in work:
            continue
        hbm = 1024.0 * (f_kib * ff + w_kib * wf)
        kernels[name] = {
            "source_sha256": source_sha(name),
            "fetch_kib_per_launch": round(f_kib, 1), "write_kib_per_launch": round(w_kib, 1),
            "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": work[name]["bytes"],
            "traffic_over_algorithmic": round(hbm / work[name]["bytes"], 3),
        }
    rec = {}
    if os.path.exists(PMC_TRAFFIC):
        with open(PMC_TRAFFIC) as f:
            rec = json.load(f)
        if "workloads" not in rec:          # an older single-workload record
            rec = {}
    rec.update({"fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                "calibration": "1 GiB device copy (bench.py --copy-calibration), counter read "
                               "per copyBuffer dispatch"})
    rec.setdefault("workloads", {})[workload] = {"commands": commands, "kernels": kernels}
    with open(PMC_TRAFFIC, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec["workloads"][workload], indent=1))


def trace_summary(workload, stats_csv, bench_log, command, out_md, title="forward pass"):
    """A rocprofv3 --kernel-trace --stats summary (the library's kernels) next to
    the per-call event times the same bench run printed, as a short Markdown file."""
    import csv
    from synthetic_inputs import WORKLOADS
    rows = [r for r in csv.DictReader(open(stats_csv)) if "lshk::" in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    w = WORKLOADS[workload]
    line = [l for l in open(bench_log) if l.startswith("{")][-1]
    res = json.loads(line)
    out = [f"# Kernel trace summary: {title}, {workload} workload", "",
           f"Workload {workload}: {w.description} (synthetic, seed {w.seed}).", "",
           "Command (repository root, MI355X):", "",
           "    cd /root/repo && export TMPDIR=/tmp", f"    {command}", "",
           "Library kernels only (torch kernels of the input upload omitted); averages over every "
           "launch of the run, warm-up included.", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share of library GPU time |",
           "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("(anonymous namespace)::", "").replace("lshk::", "")
        name = re.sub(r"\(.*", "", name).replace("void ", "").replace("attn::", "")
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")
    out += ["", "Per-call averages the same run printed (HIP events on the launch stream, from a "
                "pass of as many steps after the timed ones), with each call's fraction of the "
                "MFMA and HBM peaks:", "",
            "| call | ms | MFMA fraction | HBM fraction |", "|---|---|---|---|"]
    for n, e in res["kernels"].items():
        out.append(f"| {n} | {e['ms']:.4f} | {e['mfma_frac']:.3f} | {e['hbm_frac']:.3f} |")
    out += ["", f"bench.py ms_per_step in this run: {res['ms_per_step']} "
                f"({res['value'] / 1e6:.1f} M tokens/s)", ""]
    with open(out_md, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


# Counters of the two --pmc passes that --counter-summary reads (each pass within
# the per-pass limits of the SQ and GRBM blocks); MfmaUtil, VALUBusy, LdsUtil,
# LDSBankConflict and OccupancyPercent are rocprofv3's derived metrics.
COUNTER_PASSES = [
    "MfmaUtil VALUBusy SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_WAVES",
    "LdsUtil LDSBankConflict OccupancyPercent SQ_WAIT_INST_ANY SQ_WAVE_CYCLES",
]


def counter_summary(workload, dirs, out_md, title="forward pass", extra=""):
    """Per-kernel means over every dispatch of rocprofv3 --pmc counter runs (one
    folder per pass), as a short Markdown table."""
    import csv
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if "lshk::" not in name:
                    continue
                name = name.replace("(anonymous namespace)::", "").replace("lshk::", "")
                name = re.sub(r"\(.*", "", name).replace("void ", "").replace("attn::", "")
                vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    cols = [("MfmaUtil", "MFMA busy %", 1), ("VALUBusy", "VALU busy %", 1), ("LdsUtil", "LDS busy %", 1),
            ("LDSBankConflict", "LDS bank-conflict %", 1), ("OccupancyPercent", "occupancy %", 1),
            ("SQ_WAIT_INST_ANY", "wait-any / wave-cycles %", None),
            ("SQ_INSTS_VALU", "VALU instr per wave", "w"), ("SQ_INSTS_MFMA", "MFMA instr per wave", "w"),
            ("SQ_INSTS_LDS", "LDS instr per wave", "w")]
    from synthetic_inputs import WORKLOADS
    w = WORKLOADS[workload]
    cmd = ("rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python bench.py --steps 2 "
           "--warmup 1 --no-cpu-baseline --workload " + workload + extra)
    out = [f"# Hardware counters: {title}, {workload} workload", "",
           f"Workload {workload}: {w.description} (synthetic, seed {w.seed}).", "",
           "Commands (repository root, MI355X), one counter pass each:", "",
           "    cd /root/repo && export TMPDIR=/tmp"]
    out += [f"    {cmd.format(c=c, d=d)}" for c, d in zip(COUNTER_PASSES, dirs)]
    out += ["", "Means over every dispatch of each kernel (warm-up included).  MfmaUtil, VALUBusy, "
                "LdsUtil, LDSBankConflict and OccupancyPercent are rocprofv3's derived metrics "
                "(percent of the kernel's GPU-active cycles, per SIMD or CU); per-wave counts are the "
                "instruction counters divided by SQ_WAVES; wait-any is SQ_WAIT_INST_ANY over "
                "SQ_WAVE_CYCLES.", "",
            "| kernel | " + " | ".join(c[1] for c in cols) + " |",
            "|---|" + "---|" * len(cols)]
    mean = lambda xs: sum(xs) / len(xs)
    for name in sorted(vals, key=lambda n: -mean(vals[n].get("SQ_WAVE_CYCLES", [0]))):
        v = vals[name]
        cells = []
        for key, _, kind in cols:
            if key not in v:
                cells.append("–")
            elif kind == "w":
                cells.append(f"{mean(v[key]) / max(1.0, mean(v.get('SQ_WAVES', [1]))):.0f}")
            elif kind is None:
                cyc = mean(v.get("SQ_WAVE_CYCLES", [0]))
                cells.append(f"{100 * mean(v[key]) / cyc:.0f}" if cyc else "–")
            else:
                cells.append(f"{mean(v[key]):.1f}")
        out.append(f"| `{name}` | " + " | ".join(cells) + " |")
    out.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def copy_calibration():
    """A plain 1 GiB device-to-device copy: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters, and the practical HBM copy bandwidth."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    reps = 5
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        b.copy_(a)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                      "launches": reps + 1, "ms_per_copy": round(ms, 4),
                      "read_plus_write_GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="paper_64k")
    ap.add_argument("--flags", type=int, default=0,
                    help="LSH_FLAG_* bits for the attention variants (0: the method as described)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as one captured HIP graph (replayed); per-call times stay eager")
    ap.add_argument("--block", type=int, default=0, metavar="D_MODEL",
                    help="time a Reformer block forward + its input recompute at this model width")
    ap.add_argument("--d-ff", type=int, default=0, help="feed-forward width (default 4 x D_MODEL)")
    ap.add_argument("--chunk-rows", type=int, default=16384, help="positions per feed-forward chunk")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (gradients of qk and v)")
    ap.add_argument("--layer", type=int, default=0, metavar="D_MODEL",
                    help="time the attention layer (projections included) at this model width")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="write profiles/forward_<workload>_kernel_stats.md from a rocprofv3 "
                         "--kernel-trace --stats run of this benchmark (no GPU needed)")
    ap.add_argument("--counter-summary", nargs=2, metavar=("PASS1_DIR", "PASS2_DIR"),
                    help="write profiles/counters_<workload>.md from the two rocprofv3 --pmc passes "
                         "of COUNTER_PASSES (no GPU needed)")
    ap.add_argument("--pmc-summary", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/pmc_traffic.json from rocprofv3 --pmc output folders")
    args = ap.parse_args()
    if args.trace_summary:
        stats, blog = args.trace_summary
        wl = args.workload
        mode, extra, title, tag = "forward", "", "forward pass", ""
        if args.backward:
            mode, extra, title = "backward", " --backward", "forward + backward (lsh_attn_backward)"
        elif args.layer:
            mode, extra, tag = "layer", f" --layer {args.layer}", f"_d{args.layer}"
            title = f"attention layer (projections around the four steps) at d_model {args.layer}"
        elif args.block:
            mode, extra, tag = "block", f" --block {args.block}", f"_d{args.block}"
            title = f"Reformer block forward and input recompute at d_model {args.block}"
        trace = "trace" if mode == "forward" else f"trace_{mode}"
        cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/{trace}_{wl} "
               f"-o run -- python bench.py --no-cpu-baseline --workload {wl}{extra}")
        trace_summary(wl, stats, blog, cmd,
                      os.path.join(ROOT, "profiles", f"{mode}_{wl}{tag}_kernel_stats.md"), title)
        return
    if args.counter_summary:
        mode, extra, title, tag = "", "", "forward pass", ""
        if args.backward:
            mode, extra, title = "backward_", " --backward", "forward + backward (lsh_attn_backward)"
        elif args.layer:
            mode, extra, tag = "layer_", f" --layer {args.layer}", f"_d{args.layer}"
            title = f"attention layer (projections around the four steps) at d_model {args.layer}"
        elif args.block:
            mode, extra, tag = "block_", f" --block {args.block}", f"_d{args.block}"
            title = f"Reformer block forward and input recompute at d_model {args.block}"
        counter_summary(args.workload, args.counter_summary,
                        os.path.join(ROOT, "profiles", f"counters_{mode}{args.workload}{tag}.md"), title, extra)
        return
    if args.pmc_summary:
        fd, wd, cfd, cwd = args.pmc_summary
        cmd = ("rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python bench.py "
               "--steps 2 --warmup 1 --no-cpu-baseline --workload " + args.workload)
        ccmd = "rocprofv3 --pmc {c} --output-format csv -d {d} -o run -- python bench.py --copy-calibration"
        pmc_summary(args.workload, fd, wd, cfd, cwd,
                    [cmd.format(c="FETCH_SIZE", d=fd), cmd.format(c="WRITE_SIZE", d=wd),
                     ccmd.format(c="FETCH_SIZE", d=cfd), ccmd.format(c="WRITE_SIZE", d=cwd)])
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the forward pass shards over batch rows and heads "
              "with no exchange, so a multi-GPU figure is not produced (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import lsh_attention_02_amd as lsh
    from synthetic_inputs import (WORKLOADS, make_block_inputs, make_grad, make_inputs,
                                  make_layer_inputs)

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    blk = args.block
    bwd_mode = args.backward
    if blk and (args.layer or args.backward):
        raise SystemExit("--block, --layer and --backward are separate modes")
    dm = args.layer or blk
    dff = (args.d_ff or 4 * blk) if blk else None
    x = (make_block_inputs(w, dm, dff) if blk else make_layer_inputs(w, dm)) if dm else make_inputs(w)
    # The CPU baseline spawns worker processes, so it runs before the first GPU call.
    base = None
    if not args.no_cpu_baseline and not dm and not bwd_mode:
        base = cpu_baseline(w, x, flags=args.flags)
    cfg = lsh.LSHConfig(w.batch, w.heads, w.seq_len, w.d_head, w.n_buckets, w.n_rounds, w.chunk,
                        w.causal, dtype=w.dtype, flags=args.flags)
    tdt = cfg.torch_dtype
    B, H, L, d, nr = w.batch, w.heads, w.seq_len, w.d_head, w.n_rounds
    if blk:
        bt = {k: torch.from_numpy(a).to(dev).to(tdt) for k, a in x.items()}
        xin = bt["x2"]
        wts = [bt["w_qk"], bt["w_v"], bt["w_o"]]
        qk = torch.empty((B, H, L, d), dtype=tdt, device=dev)
        v = torch.empty((B, H, L, d), dtype=tdt, device=dev)
        y1, y2, r1, r2 = (torch.empty((B, L, dm), dtype=tdt, device=dev) for _ in range(4))
        hidden = torch.empty(lsh.lsh_ffn_workspace_bytes(B * L, dff, args.chunk_rows), dtype=torch.uint8,
                             device=dev)
        y = r1
    elif dm:
        xin = torch.from_numpy(x["x"]).to(dev).to(tdt)
        wts = [torch.from_numpy(x[k]).to(dev).to(tdt) for k in ("w_qk", "w_v", "w_o")]
        qk = torch.empty((B, H, L, d), dtype=tdt, device=dev)
        v = torch.empty((B, H, L, d), dtype=tdt, device=dev)
        y = torch.empty((B, L, dm), dtype=tdt, device=dev)
    else:
        qk = torch.from_numpy(x["qk"]).to(dev).to(tdt)
        v = torch.from_numpy(x["v"]).to(dev).to(tdt)
    R = torch.from_numpy(x["R"]).to(dev).to(tdt)
    buckets = torch.empty((B, H, nr, L), dtype=torch.int32, device=dev)
    perm = torch.empty((B, H, nr, L), dtype=torch.int32, device=dev)
    cid = torch.empty((B, H, L, nr), dtype=torch.int16, device=dev)
    o_r = torch.empty((B, H, nr, L, d), dtype=tdt, device=dev)
    lse = torch.empty((B, H, nr, L), dtype=torch.float32, device=dev)
    o = torch.empty((B, H, L, d), dtype=tdt, device=dev)
    ws = lsh.sort_workspace(cfg, dev)
    stream = torch.cuda.Stream(device=dev)
    names = ["lsh_hash", "lsh_sort", "lsh_chunk_attn", "lsh_combine_rounds"]
    calls = [
        lambda: lsh.lsh_hash(cfg, qk, R, buckets, stream=stream),
        lambda: lsh.lsh_sort(cfg, buckets, perm, cid, ws, stream=stream),
        lambda: lsh.lsh_chunk_attn(cfg, qk, v, perm, cid, o_r, lse, stream=stream),
        lambda: lsh.lsh_combine_rounds(cfg, o_r, lse, o, stream=stream),
    ]
    bwd = args.backward
    if bwd:
        if dm:
            raise SystemExit("--backward and --layer are separate modes")
        d_o = torch.from_numpy(make_grad(w)).to(dev).to(tdt)
        d_qk = torch.empty((B, H, L, d), dtype=torch.float32, device=dev)
        d_v = torch.empty((B, H, L, d), dtype=torch.float32, device=dev)
        bws = lsh.backward_workspace(cfg, dev)
        names = names + ["lsh_attn_backward"]
        calls = calls + [lambda: lsh.lsh_attn_backward(cfg, qk, v, perm, cid, lse, o, d_o, d_qk, d_v,
                                                       workspace=bws, stream=stream)]
    if blk:
        # forward: y1 = x1 + Attention(x2), y2 = x2 + FFN(y1); then the recompute
        # x2 = y2 - FFN(y1), x1 = y1 - Attention(x2) (into r2, r1)
        core_names, core_calls = names, calls
        ffn = lambda xx, res, sign, out: lsh.lsh_ffn(xx, bt["w1"], bt["b1"], bt["w2"], bt["b2"], res, sign,
                                                     args.chunk_rows, y=out, hidden=hidden, stream=stream)
        names = (["fwd:lsh_project_in"] + ["fwd:" + n for n in core_names]
                 + ["fwd:lsh_project_out_add", "fwd:lsh_ffn", "inv:lsh_ffn", "inv:lsh_project_in"]
                 + ["inv:" + n for n in core_names] + ["inv:lsh_project_out_add"])
        calls = ([lambda: lsh.lsh_project_in(cfg, dm, bt["x2"], wts[0], wts[1], qk, v, stream=stream)]
                 + core_calls
                 + [lambda: lsh.lsh_project_out_add(cfg, dm, o, wts[2], bt["x1"], 1.0, y1, stream=stream),
                    lambda: ffn(y1, bt["x2"], 1.0, y2),
                    lambda: ffn(y1, y2, -1.0, r2),
                    lambda: lsh.lsh_project_in(cfg, dm, r2, wts[0], wts[1], qk, v, stream=stream)]
                 + core_calls
                 + [lambda: lsh.lsh_project_out_add(cfg, dm, o, wts[2], y1, -1.0, r1, stream=stream)])
    elif dm:
        names = ["lsh_project_in"] + names + ["lsh_project_out"]
        calls = ([lambda: lsh.lsh_project_in(cfg, dm, xin, wts[0], wts[1], qk, v, stream=stream)]
                 + calls + [lambda: lsh.lsh_project_out(cfg, dm, o, wts[2], y, stream=stream)])

    def step(evs=None):
        for i, c in enumerate(calls):
            if evs is not None:
                evs[i][0].record(stream)
            c()
            if evs is not None:
                evs[i][1].record(stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(args.steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        # per-call times: the same number of steps again, an event pair around each call
        ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in calls]
              for _ in range(args.steps)]
        for k in range(args.steps):
            step(ev[k])
        torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    eager_ms_per_step = ms_per_step
    if args.graph:
        # the same step captured into one HIP graph; every call is asynchronous
        # on `stream` and allocates nothing, so the capture records the kernels
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        gs = torch.cuda.Event(enable_timing=True)
        ge = torch.cuda.Event(enable_timing=True)
        gs.record(stream)
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                graph.replay()
        ge.record(stream)
        torch.cuda.synchronize()
        ms_per_step = gs.elapsed_time(ge) / args.steps
    per_call = {n: float(np.mean([ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)]))
                for i, n in enumerate(names)}
    assert torch.isfinite((y if dm else o).float()).all().item(), "non-finite output"
    if bwd:
        assert torch.isfinite(d_qk).all().item() and torch.isfinite(d_v).all().item(), "non-finite gradient"

    tokens = B * L
    value = tokens / (ms_per_step * 1e-3)
    kind = lambda n: n.split(":")[-1]         # block mode: "fwd:" / "inv:" prefixes
    dominant = max(per_call, key=per_call.get)
    roof = roofline_entry(kind(dominant), w, per_call[dominant], dm, dff)
    work = algorithmic_work(w, dm, dff)[kind(dominant)]
    # the committed counters were taken on the method without variant flags
    roof["traffic"] = traffic_for(dominant, w.name) if args.flags == 0 and not dm and not bwd else None
    roof["kernel"] = KERNEL_SYMBOLS[kind(dominant)]
    if blk:
        roof["call"] = dominant
    roof["algorithmic_per_launch"] = work["flops"] if roof["bound"] == "mfma" else work["bytes"]
    roof["mfma_frac"], roof["hbm_frac"] = both_fractions(kind(dominant), w, per_call[dominant], dm, dff)
    kernels = {}
    for n in names:
        e = roofline_entry(kind(n), w, per_call[n], dm, dff)
        e["ms"] = round(per_call[n], 4)
        e["mfma_frac"], e["hbm_frac"] = both_fractions(kind(n), w, per_call[n], dm, dff)
        tgt = TARGET_FRACTION.get(kind(n))
        if tgt and not dm and not bwd and not blk:
            got = e[tgt[0] + "_frac"]
            e["target"] = {"of": tgt[0], "frac": tgt[1], "met": got >= tgt[1]}
        kernels[n] = e

    result = {
        "metric": (BLOCK_METRIC if blk else LAYER_METRIC if dm else BACKWARD_METRIC if bwd else METRIC),
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "seq_len": L, "d_head": d,
                   "n_buckets": w.n_buckets, "n_rounds": nr, "chunk": w.chunk,
                   "causal": w.causal, "flags": args.flags, **({"d_model": dm} if dm else {}),
                   **({"d_ff": dff, "chunk_rows": args.chunk_rows} if blk else {}),
                   **({"graph": True, "eager_ms_per_step": round(eager_ms_per_step, 4)}
                      if args.graph else {}),
                   **({"backward": True} if bwd else {})},
        "roofline": roof, "kernels": kernels,
    }
    if base is not None:
        entry, ref_b, ref_m, Lp = base
        result["cpu_baseline"] = entry
        result["hash_check"] = hash_check(buckets.cpu().numpy(), ref_b, ref_m, Lp, L)
    result["env"] = {"torch": torch.__version__, "hip": torch.version.hip,
                     "device": torch.cuda.get_device_name(0),
                     "host_cores": len(os.sched_getaffinity(0))}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
