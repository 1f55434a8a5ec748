"""Benchmark of the MSA forward path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for prefill, the block selection (the fused proxy + top-k pass when topk <= 17,
else proxy block max scores and top-k over every row chunk),
then the block-sparse attention; for decode, one sparse decode call.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ...]

Prints one JSON line.  The headline workload is the 32K causal sparse prefill
(32 query heads, 8 KV heads, top-k 16); the 128K varlen prefill and the
32 x 131072 fp8 paged decode (with the workload's fixed selections, and as a
whole step with its own indexer pass) are reported under "extra".  Throughput is
measured with inputs resident in HBM, between a synchronize on both sides of
exactly K timed steps.  The roofline entry times the dominant kernel with HIP
events recorded by the library on the stream it launches on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill tok/s + MFMA util @32K/128K; paged fp8 decode tok/s @131K"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0
# matrix-core peak of each proxy pair: fp4 x fp8 products run at the fp8 rate
PROXY_PEAK = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS, "mxfp4": PEAK_FP8_TFLOPS, "mxfp4_qk": PEAK_FP4_TFLOPS}
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {
    "bwd_dq": "sparse_prefill.hip", "bwd_dkv": "sparse_prefill.hip", "bwd_dq_sum": "sparse_prefill.hip",
    "bwd_dq_sum_bfp": "sparse_prefill.hip",
    "proxy_maxscore": "proxy_maxscore.hip", "topk_select": "topk_select.hip", "proxy_topk": "proxy_maxscore.hip",
    "csr": "sparse_prefill.hip",
    "partial_attn": "sparse_prefill.hip", "local_merge": "sparse_prefill.hip", "decode": "sparse_decode.hip",
    "decode_merge": "sparse_decode.hip", "proxy_onerow": "proxy_maxscore.hip",
    "proxy_onerow_mxfp4": "proxy_maxscore.hip", "topk_wave": "topk_select.hip",
    "topk_wave_exact": "topk_select.hip", "topk_refine": "proxy_maxscore.hip",
    "kl_dq_sum": "sparse_prefill.hip", "kl_dense_dq": "proxy_kl.hip", "kl_dense_dk": "proxy_kl.hip",
    "dense_fwd": "dense_attn.hip", "dense_dq": "dense_attn.hip", "dense_dkv": "sparse_prefill.hip",
}


def source_hash(kernel: str) -> str:
    p = os.path.join(ROOT, "block_sparse_top_amd", "csrc", KERNEL_SOURCES[kernel])
    h = hashlib.sha256()
    for f in (p, os.path.join(ROOT, "block_sparse_top_amd", "csrc", "device_common.hpp")):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch, if a committed summary for the
    current kernel source exists (null otherwise).  The summary's last line
    is a JSON object."""
    p = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__traffic.txt")
    if not os.path.exists(p):
        return None
    last = [ln for ln in open(p).read().splitlines() if ln.startswith("{")][-1]
    d = json.loads(last)
    if d.get("source_hash") != source_hash(kernel):
        return None
    return d.get("bytes_per_launch")


# ----------------------------------------------------------------------------
# rocprofv3 summaries (run on the host from the CSV files rocprofv3 wrote)
# ----------------------------------------------------------------------------
COPY_BYTES = 1 << 30           # calibration copy: bytes read and bytes written per launch
PMC_ARGS = ("--steps 2 --warmup 1 --no-cpu-baseline --no-peaks --profile-run --extra "
            "prefill_32k_backward,decode_131k,decode_step_131k,decode_step_mxfp4_131k --copy-calibration")
# counters are collected on the library's kernels and the calibration copy only
PMC_FILTER = '--kernel-include-regex "msa|bitwise_not"'
PMC_CMDS = {
    "FETCH_SIZE": f"rocprofv3 --pmc FETCH_SIZE {PMC_FILTER} -f csv -d gpurun_out/pmc_fetch -o f -- python bench.py "
                  f"{PMC_ARGS}",
    "WRITE_SIZE": f"rocprofv3 --pmc WRITE_SIZE {PMC_FILTER} -f csv -d gpurun_out/pmc_write -o w -- python bench.py "
                  f"{PMC_ARGS}",
}
TRACE_CMD = "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/kt -o kt -- python bench.py"
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE")
MFMA_PMC_ARGS = ("--steps 2 --warmup 1 --no-cpu-baseline --no-peaks --profile-run --extra "
                 "prefill_128k,prefill_32k_mxfp4,prefill_32k_backward,warmup_32k,decode_131k,decode_step_131k")
MFMA_CMD = (f"rocprofv3 --pmc {MFMA_COUNTERS} {PMC_FILTER} -f csv -d gpurun_out/pmc_mfma -o m -- python bench.py "
            f"{MFMA_PMC_ARGS}")
STALL_COUNTERS = {
    "a": "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
         "SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_ANY",
    "b": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_INSTS_SALU "
         "SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU_TRANS_F32"}
STALL_PMC_ARGS = "--steps 2 --warmup 1 --no-cpu-baseline --no-peaks --profile-run --extra prefill_32k_backward"
STALL_CMDS = {k: f"rocprofv3 --pmc {v} --kernel-include-regex \"msa\" -f csv -d gpurun_out/stall_{k} -o s -- python "
                 f"bench.py {STALL_PMC_ARGS}" for k, v in STALL_COUNTERS.items()}
NUM_CU, SIMD_PER_CU, NUM_XCD = 256, 4, 8
SECTION_OF_KERNEL = {"decode": "decode_fp8_b32_131k", "decode_merge": "decode_fp8_b32_131k",
                     "proxy_onerow": "decode_step_b32_131k", "topk_wave": "decode_step_b32_131k",
                     "topk_wave_exact": "decode_step_b32_131k",
                     "proxy_onerow_mxfp4": "decode_step_mxfp4_b32_131k"}


def _short_kernel(name: str):
    import re
    if "bitwise_not" in name:
        return "copy"
    m = re.search(r"msa::\(anonymous namespace\)::(\w+?)(_kernel)?[<(]", name)
    return m.group(1) if m else None


def summarize_counters(fetch_csv: str, write_csv: str):
    """Per-launch HBM bytes of every library kernel from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by the factor that makes
    the same counter read the known size of the calibration copy."""
    import collections
    import csv

    def per_kernel(path, counter):
        acc = collections.defaultdict(dict)          # kernel -> dispatch -> KiB
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k = _short_kernel(r["Kernel_Name"])
            if k is not None:
                acc[k][int(r["Dispatch_Id"])] = acc[k].get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
        return {k: (sum(v.values()) / len(v), len(v)) for k, v in acc.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    f_fac = COPY_BYTES / (fetch["copy"][0] * 1024.0)
    w_fac = COPY_BYTES / (write["copy"][0] * 1024.0)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    written = []
    for k in sorted(set(fetch) & set(write)):
        if k == "copy" or k not in KERNEL_SOURCES:
            continue
        wl = SECTION_OF_KERNEL.get(k, "prefill_32k_gqa4")
        fb = fetch[k][0] * 1024.0 * f_fac
        wb = write[k][0] * 1024.0 * w_fac
        d = {"kernel": k, "workload": wl, "bytes_per_launch": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
             "fetch_kib_raw": fetch[k][0], "write_kib_raw": write[k][0], "dispatches": fetch[k][1],
             "fetch_factor": f_fac, "write_factor": w_fac, "source_hash": source_hash(k)}
        txt = (f"# HBM traffic of {k} on {wl} (rocprofv3 counters, per dispatch)\n"
               f"# fetch: {PMC_CMDS['FETCH_SIZE']}\n# write: {PMC_CMDS['WRITE_SIZE']}\n"
               f"# summary: python bench.py --summarize-counters gpurun_out/pmc_fetch/f_counter_collection.csv "
               f"gpurun_out/pmc_write/w_counter_collection.csv\n"
               f"# calibration: a streaming int32 copy reading and writing {COPY_BYTES} B per launch reads "
               f"FETCH_SIZE {fetch['copy'][0]:.0f} KiB and WRITE_SIZE {write['copy'][0]:.0f} KiB, "
               f"factors {f_fac:.4f} and {w_fac:.4f}\n"
               f"# {k}: {fetch[k][1]} dispatches, FETCH_SIZE {fetch[k][0]:.0f} KiB, WRITE_SIZE {write[k][0]:.0f} KiB "
               f"-> {fb / 1e9:.3f} GB read + {wb / 1e9:.3f} GB written = {(fb + wb) / 1e9:.3f} GB per launch\n"
               + json.dumps(d) + "\n")
        path = os.path.join(ROOT, "profiles", f"{k}__{wl}__traffic.txt")
        open(path, "w").write(txt)
        written.append(path)
    return written


def summarize_mfma(mfma_csv: str, bench_err: str, out_name: str):
    """Matrix-core and LDS counters per library kernel and workload from one
    rocprofv3 --pmc run (MFMA_CMD): MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE x 1024 SIMDs); counted matrix FLOPs = MOPS x 512 (the
    counters count 512-FLOP units); LDS active = SQ_LDS_IDX_ACTIVE /
    (GRBM_GUI_ACTIVE x 256 CUs); bank conflicts per LDS-active cycle.  A
    dispatch belongs to the workload bench.py marked last before it."""
    import collections
    import csv
    disp = collections.defaultdict(lambda: collections.defaultdict(float))
    kname, grbm, start_ts, dur_ns = {}, collections.defaultdict(float), {}, {}
    for r in csv.DictReader(open(mfma_csv)):
        k = _short_kernel(r["Kernel_Name"])
        if k is None:
            continue
        d = int(r["Dispatch_Id"])
        kname[d] = k
        start_ts[d] = int(r.get("Start_Timestamp") or 0)
        c, v = r["Counter_Name"], float(r["Counter_Value"])
        if c == "GRBM_GUI_ACTIVE":
            # reported summed over the 8 XCDs: per-XCD busy cycles
            grbm[d] = max(grbm[d], v / NUM_XCD)
        else:
            disp[d][c] += v
        dur_ns[d] = int(r.get("End_Timestamp") or 0) - int(r.get("Start_Timestamp") or 0)
    # workload of each dispatch: the last "[bench-mark] <entry> <ns>" line (the
    # host's monotonic clock, the trace's time origin) before its start
    import bisect
    names = {"main": "prefill_32k_gqa4", "prefill_128k": "prefill_varlen_128k_gqa8",
             "prefill_32k_mxfp4": "prefill_32k_gqa4_mxfp4", "prefill_32k_backward": "prefill_32k_gqa4_backward",
             "warmup_32k": "prefill_32k_gqa4_warmup", "decode_131k": "decode_fp8_b32_131k",
             "decode_step_131k": "decode_step_b32_131k", "decode_step_mxfp4_131k": "decode_step_mxfp4_b32_131k",
             "prefill_1m_fp8proxy": "prefill_1m_fp8proxy"}
    marks = sorted((int(ln.split()[2]), names.get(ln.split()[1], ln.split()[1]))
                   for ln in open(bench_err).read().splitlines() if ln.startswith("[bench-mark] "))
    mark_t = [t for t, _ in marks]
    sec = {}
    for d, t0 in start_ts.items():
        if kname.get(d) in (None, "copy"):
            continue
        i = bisect.bisect_right(mark_t, t0) - 1
        sec[d] = marks[i][1] if i >= 0 else "?"
    g = collections.OrderedDict()
    for d in sorted(sec):
        g.setdefault((sec[d], kname[d]), []).append(d)
    out = ["# Matrix-core and LDS counters per kernel (rocprofv3 --pmc, per dispatch, averaged)",
           f"# command: {MFMA_CMD}",
           f"# summary: python bench.py --summarize-mfma gpurun_out/pmc_mfma/m_counter_collection.csv <bench stderr> "
           f"{out_name}",
           "# MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs); counted matrix FLOPs = "
           "(MOPS_BF16 + MOPS_F8 + MOPS_F6F4) x 512; LDS active = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE x 256 CUs); "
           "conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
           "# GRBM_GUI_ACTIVE is reported summed over the 8 XCDs; per-XCD cycles / dispatch duration gives the "
           "clock column",
           "", "| workload | kernel | dispatches | avg us | clock GHz | MFMA busy | bf16 GFLOP | fp8 GFLOP | "
               "fp4/fp6 GFLOP | counted TFLOP/s | LDS active | LDS conflicts |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    rows = []
    for (wl, k), ds in g.items():
        cyc = np.mean([grbm[d] for d in ds])
        busy = np.mean([disp[d]["SQ_VALU_MFMA_BUSY_CYCLES"] / max(1.0, grbm[d] * NUM_CU * SIMD_PER_CU) for d in ds])
        fb = np.mean([disp[d]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 for d in ds]) / 1e9
        f8 = np.mean([disp[d]["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512 for d in ds]) / 1e9
        f4 = np.mean([disp[d]["SQ_INSTS_VALU_MFMA_MOPS_F6F4"] * 512 for d in ds]) / 1e9
        lds = np.mean([disp[d]["SQ_LDS_IDX_ACTIVE"] / max(1.0, grbm[d] * NUM_CU) for d in ds])
        bc = np.mean([disp[d]["SQ_LDS_BANK_CONFLICT"] / max(1.0, disp[d]["SQ_LDS_IDX_ACTIVE"]) for d in ds])
        us = np.mean([dur_ns[d] for d in ds]) / 1e3
        ghz = cyc / max(1e-9, us * 1e3)
        tfs = (fb + f8 + f4) * 1e9 / max(1e-12, us * 1e-6) / 1e12
        out.append(f"| {wl} | {k} | {len(ds)} | {us:.1f} | {ghz:.2f} | {100 * busy:.1f}% | {fb:.1f} | {f8:.1f} | "
                   f"{f4:.1f} | {tfs:.0f} | {100 * lds:.1f}% | {100 * bc:.2f}% |")
        rows.append({"workload": wl, "kernel": k, "dispatches": len(ds), "avg_us": us, "clock_ghz": ghz,
                     "mfma_busy": busy, "bf16_gflop": fb, "fp8_gflop": f8, "fp6f4_gflop": f4,
                     "counted_tflops": tfs, "lds_active": lds, "lds_conflict": bc})
    out += ["", json.dumps({"rows": rows}), ""]
    path = os.path.join(ROOT, "profiles", out_name)
    open(path, "w").write("\n".join(out))
    return path


def summarize_stalls(a_csv: str, b_csv: str, out_name: str):
    """Where the waves of each library kernel spend their cycles (two
    rocprofv3 --pmc passes over the 32K prefill and backward, STALL_CMDS),
    as fractions of SQ_WAVE_CYCLES: waiting at s_waitcnt (memory or LDS),
    waiting for an issue slot or a dependency, and issuing VALU, LDS, VMEM or
    any instruction; plus instruction counts per MFMA."""
    import collections
    import csv

    def load(path):
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        kn = {}
        for r in csv.DictReader(open(path)):
            k = _short_kernel(r["Kernel_Name"])
            if k is None or k == "copy":
                continue
            d = int(r["Dispatch_Id"])
            kn[d] = k
            per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        agg = collections.defaultdict(lambda: collections.defaultdict(float))
        n = collections.Counter()
        for d, c in per.items():
            n[kn[d]] += 1
            for name, v in c.items():
                agg[kn[d]][name] += v
        return agg, n

    a, na = load(a_csv)
    b, _ = load(b_csv)
    out = ["# Wave cycles and instruction mix per kernel (rocprofv3 --pmc, 32K prefill and backward, summed over "
           "dispatches)",
           f"# pass a: {STALL_CMDS['a']}", f"# pass b: {STALL_CMDS['b']}",
           f"# summary: python bench.py --summarize-stalls <pass a csv> <pass b csv> {out_name}",
           "# fractions of SQ_WAVE_CYCLES (cycles summed over resident waves): wait = at s_waitcnt, dep = waiting "
           "for an issue slot or an operand, valu / lds / vmem / any = issuing that kind",
           "", "| kernel | dispatches | wait | dep | valu | lds | vmem | any issue | VALU / MFMA | LDS / MFMA | "
           "transcendental / MFMA | MFMA-VALU co-issue / wave cycle |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    rows = []
    for k in sorted(a, key=lambda x: -a[x]["SQ_WAVE_CYCLES"]):
        x, y = a[k], b.get(k, {})
        wc = x["SQ_WAVE_CYCLES"] or 1.0
        mf = y.get("SQ_INSTS_MFMA", 0.0)
        per = (lambda c: f"{y.get(c, 0.0) / mf:.1f}" if mf else "")
        row = {"kernel": k, "dispatches": na[k]}
        row.update({c: x[c] / wc for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
                                           "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_ANY")})
        row.update({c: y.get(c, 0.0) for c in STALL_COUNTERS["b"].split()})
        rows.append(row)
        out.append(f"| {k} | {na[k]} | {row['SQ_WAIT_ANY']:.2f} | {row['SQ_WAIT_INST_ANY']:.2f} | "
                   f"{row['SQ_ACTIVE_INST_VALU']:.2f} | {row['SQ_ACTIVE_INST_LDS']:.2f} | "
                   f"{row['SQ_ACTIVE_INST_VMEM']:.2f} | {row['SQ_ACTIVE_INST_ANY']:.2f} | {per('SQ_INSTS_VALU')} | "
                   f"{per('SQ_INSTS_LDS')} | {per('SQ_INSTS_VALU_TRANS_F32')} | "
                   f"{y.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0.0) / wc:.3f} |")
    out.append("")
    out.append(json.dumps({"rows": rows}))
    path = os.path.join(ROOT, "profiles", out_name)
    open(path, "w").write("\n".join(out) + "\n")
    return path


def summarize_trace(trace_csv: str, bench_json: str, bench_err: str, out_name: str):
    """Kernel durations from a rocprofv3 kernel trace, per workload, next to
    the per-launch averages that bench.py measured with HIP events in the same
    run.  bench.py stamps the host's monotonic clock on stderr before each
    workload ("[bench-mark] <entry> <ns>"); the trace's dispatch timestamps
    count from the same origin, so a dispatch belongs to the last workload
    marked before it started."""
    import bisect
    import collections
    import csv
    line = [ln for ln in open(bench_json).read().splitlines() if ln.startswith("{")][-1]
    b = json.loads(line)
    ev = [(b["config"]["workload"], b["roofline"])]
    name_of = {"main": b["config"]["workload"]}
    for key, r in (b.get("extra") or {}).items():
        ev.append((r["workload"], r["roofline"]))
        name_of[key] = r["workload"]
    marks = []
    for ln in open(bench_err).read().splitlines():
        if ln.startswith("[bench-mark] "):
            _, key, ns = ln.split()
            marks.append((int(ns), name_of.get(key, key)))
    marks.sort()
    mark_t = [t for t, _ in marks]
    rows = []
    for r in sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"])):
        k = _short_kernel(r["Kernel_Name"])
        if k is None or k == "copy":
            continue
        grid = "x".join(r[f"Grid_Size_{a}"] for a in "XYZ")
        t0 = int(r["Start_Timestamp"])
        i = bisect.bisect_right(mark_t, t0) - 1
        sec = marks[i][1] if i >= 0 else "before the first mark"
        rows.append((k, grid, (int(r["End_Timestamp"]) - t0) * 1e-6, sec))
    section = [sec for (_, _, _, sec) in rows]
    rows = [(k, grid, ms) for (k, grid, ms, _) in rows]
    g = collections.OrderedDict()
    for (k, grid, ms), sec in zip(rows, section):
        g.setdefault((sec, k, grid), []).append(ms)
    out = [f"# Kernel durations, rocprofv3 kernel trace of the default benchmark run",
           f"# command: {TRACE_CMD}",
           f"# summary: python bench.py --summarize-trace gpurun_out/kt/kt_kernel_trace.csv <bench stdout> "
           f"<bench stderr> {out_name}",
           "", "| workload | kernel | grid | calls | avg ms | min ms | max ms | total ms |",
           "|---|---|---|---|---|---|---|---|"]
    for (sec, k, grid), v in sorted(g.items(), key=lambda kv: str(kv[0][0])):
        out.append(f"| {sec} | {k} | {grid} | {len(v)} | {np.mean(v):.4f} | {min(v):.4f} | {max(v):.4f} | "
                   f"{sum(v):.3f} |")
    out += ["", "HIP-event averages that bench.py reported for the dominant kernel of each workload in this run:", ""]
    # profiling names that share a kernel symbol with another entry
    symbol_of = {"dense_dkv": "bwd_dkv", "kl_dq_sum": "bwd_dq_sum", "proxy_topk": "proxy_maxscore",
                 "topk_select": "topk"}
    for wl, r in ev:
        kk = symbol_of.get(r["kernel"], r["kernel"])
        tr = np.mean(g.get((wl, kk, next((gr for (s2, k2, gr) in g if s2 == wl and k2 == kk), "")), [float("nan")]))
        out.append(f"- {wl}: {r['kernel']} {r['avg_launch_ms']:.4f} ms per launch by HIP events, {tr:.4f} ms in the "
                   f"trace ({r['launches_per_step']} launches per step); {r['achieved']:.1f} {r['unit']} "
                   f"= {100 * r['frac']:.1f}% of {r['peak']:.0f}")
    out += ["", "bench.py line of this run:", "", "```", line, "```", ""]
    path = os.path.join(ROOT, "profiles", out_name)
    open(path, "w").write("\n".join(out))
    return path


def copy_calibration(reps=3):
    """A plain streaming copy of known size (int32 bitwise not: COPY_BYTES read
    and COPY_BYTES written per launch), profiled beside the library kernels to
    scale the HBM byte counters."""
    import torch
    src = torch.arange(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


# ----------------------------------------------------------------------------
# peaks measured on this device, reported beside the published ones
# ----------------------------------------------------------------------------
MEASURED = {}
PROFILE_RUN = [False]   # set by --profile-run: legs take fixed small step counts


def measure_peaks(msa):
    """A plain streaming copy (int32 bitwise not over 2 GiB read + 2 GiB
    written, HIP events) for HBM, and the library's matrix-core loop
    (msa_diag_mfma_rate: register operands, two waves per SIMD) for bf16, fp8
    and FP4."""
    import torch
    n = (2 << 30) // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    e1.record()
    e1.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    MEASURED.update({
        "hbm_gbs": 2.0 * n * 4 / (copy_ms * 1e-3) / 1e9,
        "bf16_tflops": msa.msa_diag_mfma_rate("bf16", 20000),
        "fp8_tflops": msa.msa_diag_mfma_rate("fp8", 20000),
        "fp4_tflops": msa.msa_diag_mfma_rate("mxfp4_qk", 20000),
        "method": "HBM: int32 streaming copy of 2 GiB read + 2 GiB written (HIP events, 10 launches); matrix "
                  "cores: msa_diag_mfma_rate, 2 waves per SIMD, 4 independent 32x32 MFMA chains on register "
                  "operands, 20000 rounds",
    })
    return dict(MEASURED)


MEASURED_KEY = {"GB/s": "hbm_gbs"}
PEAK_KEY = {PEAK_BF16_TFLOPS: "bf16_tflops", PEAK_FP8_TFLOPS: "fp8_tflops", PEAK_FP4_TFLOPS: "fp4_tflops",
            PEAK_HBM_GBS: "hbm_gbs"}


def with_measured(roof: dict) -> dict:
    """Add the fraction of the peak measured on this device to a roofline entry."""
    key = PEAK_KEY.get(roof.get("peak"))
    mp = MEASURED.get(key) if key else None
    if mp and roof.get("achieved") is not None:
        roof["measured_peak"] = mp
        roof["frac_measured"] = roof["achieved"] / mp
    return roof


def time_by_duration(step, warm_ms=50.0, rep_ms=200.0):
    """At least warm_ms of warm-up steps, then one timed block of steps sized
    from the warm-up rate to last at least rep_ms, between a synchronize on
    both sides.  Returns (ms per step, steps timed)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= warm_ms:
                break
    per = (time.perf_counter() - t0) * 1e3 / n
    reps = max(16, int(math.ceil(rep_ms / per)))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / reps, reps


def stream_event_ms(step, warm_ms=50.0, rep_ms=200.0):
    """Per-step time from one pair of HIP events recorded on the launch stream
    around a block of back-to-back steps (no per-dispatch events): for a
    step that is a single kernel launch, that kernel's average duration
    including the gaps between launches."""
    import torch
    per, _ = time_by_duration(step, warm_ms, 20.0)   # warm-up, and the step time the block is sized from
    n = max(16, int(math.ceil(rep_ms / per)))
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(n):
        step()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / n, n


def host_cost_us(step, n=200):
    """Host time to enqueue one step (binding, argument checks, launches),
    measured without waiting for the device."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        step()
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    return (t1 - t0) * 1e6 / n


def graph_time(step, sets, warm_ms=50.0, rep_ms=200.0):
    """The same steps captured once in a HIP graph (`sets` consecutive steps,
    so the rotated input sets all appear) and replayed: device time per step
    without the host's launch cost."""
    import torch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):       # metadata uploaded on the capture stream before capture
        for _ in range(2 * sets):
            step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(sets):
            step()
    ms, reps = time_by_duration(g.replay, warm_ms, rep_ms)
    del g
    return ms / sets, reps * sets


# ----------------------------------------------------------------------------
# algorithmic work
# ----------------------------------------------------------------------------
def visible_keys_per_row(sel, qo_lens, kv_lens, device):
    """Selected causally visible keys per (row, group) from a selection tensor."""
    import torch
    T, Hkv, k = sel.shape
    pos = torch.cat([torch.arange(kv - qo, kv, device=device) for qo, kv in zip(qo_lens, kv_lens)])
    b = sel.long()
    valid = (b >= 0) & (b <= (pos // 128)[:, None, None])
    n = torch.clamp(pos[:, None, None] - 128 * b + 1, max=128)
    return torch.where(valid, n, torch.zeros_like(n)).sum(dim=2)   # [T, Hkv]


FWD_RECORD_BYTES = 152   # one forward partial record: 144 B of 9-bit values + {lse, step}
KV_PAGE_PAIR_BYTES = {"bf16": 2 * 128 * 128 * 2, "fp8": 2 * 128 * 128, "mxfp4": 2 * 8704}


def partial_attn_bytes(sel, qo_lens, kv_lens, G, kv_dtype, device):
    """HBM bytes the partial attention moves in its formulation: per (row,
    group) slot other than the row's own block, the G heads' gathered q rows
    (G x 256 B read) and their partial records (G x 152 B written), plus each
    selected (group, block) K/V page pair once."""
    import torch
    T, Hkv, k = sel.shape
    pos = torch.cat([torch.arange(kv - qo, kv, device=device) for qo, kv in zip(qo_lens, kv_lens)])
    base, acc = [], 0
    for qo, kv in zip(qo_lens, kv_lens):   # first global block of each row's sequence
        base.append(torch.full((qo,), acc, dtype=torch.long, device=device))
        acc += (kv + 127) // 128
    base = torch.cat(base)
    b = sel.long()
    ent = (b >= 0) & (b < (pos // 128)[:, None, None])
    n_e = int(ent.sum().item())
    g = torch.arange(Hkv, device=device)[None, :, None].expand_as(b)
    keys = (g * acc + base[:, None, None] + b)[ent]
    n_pages = int(torch.unique(keys).numel())
    return n_e * G * (256 + FWD_RECORD_BYTES) + n_pages * KV_PAGE_PAIR_BYTES[kv_dtype]


def proxy_flops(qo_lens, kv_lens, P, d=128):
    pairs = sum(sum(range(kv - qo + 1, kv + 1)) for qo, kv in zip(qo_lens, kv_lens))
    return 2.0 * d * pairs * P


# ----------------------------------------------------------------------------
# runners
# ----------------------------------------------------------------------------
def time_steps(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def kernel_profile(msa, plan, step, names, reps=3):
    """Per-kernel total ms per step, averaged over `reps` steps.  Two
    unprofiled steps are queued first so that the profiled ones start on a
    busy GPU (after an idle gap the first kernel of a step runs slower)."""
    import torch
    out = {}
    for n in names:
        step()
        step()
        msa.msa_profile_kernel(plan, n)
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        ms, cnt = msa.msa_profile_read(plan)
        msa.msa_profile_kernel(plan, None)
        if cnt:
            out[n] = (ms / reps, cnt // reps)
    return out


def timed_with_kernel(msa, plan, step, steps, warmup, kernel):
    """Time K steps; the library brackets every launch of `kernel` with events."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    msa.msa_profile_kernel(plan, kernel)
    msa.msa_profile_read(plan)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    kms, launches = msa.msa_profile_read(plan)
    msa.msa_profile_kernel(plan, None)
    return ms_step, kms / max(1, launches), launches


def prefill_bench(msa, n_cfg, steps, warmup, max_rows=0, attn_window=0, profile_reps=3):
    import torch
    from synthetic.gen import workload, seed_of
    from synthetic.device_gen import make_inputs_device
    w = workload(n_cfg)
    inp = make_inputs_device(w, seed_of(n_cfg))
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, kv_dtype=w.kv_dtype, proxy_dtype=w.proxy_dtype,
                        max_rows_per_call=max_rows, attn_window_rows=attn_window)
    T = w.total_rows
    sel = torch.empty((T, w.num_kv_heads, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((T, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    ms_buf = msa.max_score_buffer(plan)

    def step():
        msa.run_prefill(plan, inp.proxy_q, inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale, inp.q,
                        inp.k_pages, inp.v_pages, inp.kv_indices, sel, out, None, ms_buf, k_scale=inp.k_scale,
                        v_scale=inp.v_scale)

    step()
    torch.cuda.synchronize()
    lowp = w.proxy_dtype != "bf16"
    stages = ((["proxy_topk"] + (["topk_refine"] if lowp else [])) if w.topk <= 17
              else ["proxy_maxscore", "topk_select"]) + ["csr", "partial_attn", "merge"]
    per_kernel = kernel_profile(msa, plan, step, stages, reps=profile_reps)
    dominant = max(per_kernel, key=lambda n: per_kernel[n][0])
    ms_step, k_ms, launches = timed_with_kernel(msa, plan, step, steps, warmup, dominant)
    launches_per_step = launches // steps
    nvis = visible_keys_per_row(sel, w.qo_lens, w.kv_lens, "cuda")
    G = w.num_qo_heads // w.num_kv_heads
    f_main = 4.0 * 128 * float(nvis.sum().item()) * G
    f_proxy = proxy_flops(w.qo_lens, w.kv_lens, w.num_proxy_heads)
    proxy_peak = PROXY_PEAK[w.proxy_dtype]
    # work per launch of the dominant kernel (launches cover equal shares of a step)
    if dominant in ("proxy_maxscore", "proxy_topk"):
        work, peak, unit, bound = f_proxy / launches_per_step, proxy_peak, "TFLOP/s", "mfma"
    elif dominant == "partial_attn":
        work, peak, unit, bound = f_main / launches_per_step, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:  # bandwidth-bound helper kernels: count their compulsory bytes
        work, peak, unit, bound = None, PEAK_HBM_GBS, "GB/s", "hbm"
    achieved = (work / (k_ms * 1e-3) / 1e12) if (work is not None) else None
    roof = with_measured({"kernel": dominant, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                          "frac": (achieved / peak) if achieved is not None else None,
                          "traffic": traffic_from_profiles(dominant, w.name), "avg_launch_ms": k_ms,
                          "launches_per_step": launches_per_step,
                          "work_per_launch": work, "work_unit": "FLOP" if unit == "TFLOP/s" else "B"})
    if dominant == "partial_attn":
        # the same launch against the HBM roof: the bytes this formulation
        # moves (gathered q, records, K/V pages), counted from the selection
        fb = partial_attn_bytes(sel, w.qo_lens, w.kv_lens, G, w.kv_dtype, "cuda") / launches_per_step
        gbs = fb / (k_ms * 1e-3) / 1e9
        mh = MEASURED.get("hbm_gbs")
        roof["hbm_view"] = {"bytes_per_launch": fb, "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": gbs / PEAK_HBM_GBS, "frac_measured": (gbs / mh) if mh else None,
                            "basis": "gathered q (G x 256 B) + partial records (G x 152 B) per non-local "
                                     "(row, group) slot, + each selected K/V page pair once"}
    stage_ms = {n: v[0] for n, v in per_kernel.items()}
    pstage = "proxy_topk" if "proxy_topk" in stage_ms else "proxy_maxscore"
    p_ach = f_proxy / (stage_ms[pstage] * 1e-3) / 1e12
    proxy_roof = with_measured({"kernel": pstage, "proxy_dtype": w.proxy_dtype, "achieved": p_ach, "peak": proxy_peak,
                                "unit": "TFLOP/s", "frac": p_ach / proxy_peak})
    tflops = (f_main + f_proxy) / (ms_step * 1e-3) / 1e12
    # matrix-core utilisation of the step: the time the step's FLOPs need at
    # each dtype's peak (bf16 attention, proxy at its own dtype) over the step time
    util = (f_main / PEAK_BF16_TFLOPS + f_proxy / proxy_peak) / 1e12 / (ms_step * 1e-3)
    mb, mpx = MEASURED.get("bf16_tflops"), MEASURED.get(PEAK_KEY[proxy_peak])
    util_m = (f_main / mb + f_proxy / mpx) / 1e12 / (ms_step * 1e-3) if (mb and mpx) else None
    res = {
        "workload": w.name, "tok_per_s": T / (ms_step * 1e-3), "ms_per_step": ms_step,
        "tflops": tflops, "mfma_util": util, "mfma_util_measured": util_m,
        "flops": {"proxy": f_proxy, "main": f_main}, "stage_ms": stage_ms, "roofline": roof,
        "proxy_roofline": proxy_roof,
        "config": {"workload": w.name, "qo_lens": w.qo_lens if len(w.qo_lens) <= 8 else None, "total_rows": T,
                   "num_qo_heads": w.num_qo_heads, "num_kv_heads": w.num_kv_heads,
                   "num_proxy_heads": w.num_proxy_heads, "topk": w.topk, "page_size": 128, "head_dim": 128,
                   "proxy_dtype": w.proxy_dtype, "kv_dtype": w.kv_dtype, "max_rows_per_call": plan.max_rows_per_call},
    }
    return res, (w, inp, sel)


WINDOWS = (0, 8192, 4096, 2048)   # 0: the whole call (the default window)


def window_sweep(msa, n_cfg, steps, warmup, mark):
    """The sparse prefill at attention windows of 32K (the default), 8K, 4K
    and 2K rows, each without and with XCD pinning of the work items
    (MSA_XCD_PIN, read when a plan is made).  One JSON line per setting."""
    import torch
    from synthetic.gen import workload
    T = workload(n_cfg).total_rows
    for W in WINDOWS:
        for pin in ("0", "1"):
            os.environ["MSA_XCD_PIN"] = pin
            mark(f"sweep_{n_cfg}_{W or T}_{pin}")
            r, _ = prefill_bench(msa, n_cfg, steps, warmup, attn_window=W, profile_reps=1)
            print(json.dumps({"window_sweep": r["config"]["workload"], "window": W or T, "xcd_pin": pin == "1",
                              "launches_per_step": (T + (W or T) - 1) // (W or T),
                              "ms_per_step": r["ms_per_step"], "stage_ms": r["stage_ms"]}), flush=True)
            torch.cuda.empty_cache()
    os.environ.pop("MSA_XCD_PIN", None)


SWEEP_CMDS = {c: f"rocprofv3 --pmc {c} {PMC_FILTER} -f csv -d gpurun_out/sweep_{c.lower()} -o s -- python bench.py "
                 f"--window-sweep 2 --profile-run --copy-calibration"
              for c in ("FETCH_SIZE", "WRITE_SIZE")}


def summarize_window_sweep(fetch_csv: str, fetch_err: str, write_csv: str, write_err: str, sweep_stdout: str,
                           out_name: str):
    """partial_attn HBM bytes per step and stage times of each window-sweep
    setting: a counter run's dispatches belong to the setting that run marked
    last before them; bytes scaled by the calibration copy in the same run."""
    import bisect
    import collections
    import csv

    def per_setting(path, counter, err):
        marks = sorted((int(ln.split()[2]), ln.split()[1]) for ln in open(err).read().splitlines()
                       if ln.startswith("[bench-mark] sweep_"))
        mark_t = [t for t, _ in marks]
        disp, start, kn = collections.defaultdict(float), {}, {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k = _short_kernel(r["Kernel_Name"])
            if k not in ("copy", "partial_attn"):
                continue
            d = int(r["Dispatch_Id"])
            disp[d] += float(r["Counter_Value"])
            start[d] = int(r.get("Start_Timestamp") or 0)
            kn[d] = k
        copy = [disp[d] for d in disp if kn[d] == "copy"]
        fac = COPY_BYTES / (sum(copy) / len(copy) * 1024.0)
        acc = collections.defaultdict(list)
        for d in disp:
            if kn[d] != "partial_attn":
                continue
            i = bisect.bisect_right(mark_t, start[d]) - 1
            if i >= 0:
                acc[marks[i][1]].append(disp[d] * 1024.0 * fac)
        return {k: sum(v) / len(v) for k, v in acc.items()}, fac

    fetch, ff = per_setting(fetch_csv, "FETCH_SIZE", fetch_err)
    write, wf = per_setting(write_csv, "WRITE_SIZE", write_err)
    timing = [json.loads(ln) for ln in open(sweep_stdout).read().splitlines() if ln.startswith('{"window_sweep"')]
    out = ["# Sparse prefill (prefill_32k_gqa4): attention window x XCD pinning of the work items",
           f"# timing: python bench.py --window-sweep 2",
           f"# fetch: {SWEEP_CMDS['FETCH_SIZE']}",
           f"# write: {SWEEP_CMDS['WRITE_SIZE']}",
           f"# summary: python bench.py --summarize-window-sweep <fetch csv> <fetch run stderr> <write csv> "
           f"<write run stderr> <timing stdout> {out_name}",
           f"# counters per partial_attn dispatch x launches per step; calibration factors {ff:.4f} (fetch), "
           f"{wf:.4f} (write)",
           "",
           "| window (rows) | XCD pinning | launches / step | step ms | partial_attn ms / step | merge ms | "
           "partial_attn read GB / step | written GB / step |",
           "|---|---|---|---|---|---|---|---|"]
    for t in timing:
        key = f"sweep_2_{t['window']}_{'1' if t['xcd_pin'] else '0'}"
        n = t["launches_per_step"]
        fb = fetch.get(key)
        wb = write.get(key)
        out.append(f"| {t['window']} | {'yes' if t['xcd_pin'] else 'no'} | {n} | {t['ms_per_step']:.3f} | "
                   f"{t['stage_ms']['partial_attn']:.3f} | {t['stage_ms']['merge']:.3f} | "
                   f"{'' if fb is None else f'{fb * n / 1e9:.3f}'} | {'' if wb is None else f'{wb * n / 1e9:.3f}'} |")
    path = os.path.join(ROOT, "profiles", out_name)
    open(path, "w").write("\n".join(out) + "\n")
    return path


def backward_bench(msa, n_cfg, steps, warmup, kl=False):
    """The training backward of the sparse prefill attention on one workload:
    the forward runs once (selection, output, lse), then each step is
    msa_sparse_attn_prefill_backward with a fixed upstream gradient (with `kl`,
    msa_sparse_attn_prefill_backward_kl: the same plus the gradient of the
    proxy's distillation loss)."""
    import torch
    from synthetic.gen import workload, seed_of
    from synthetic.device_gen import make_inputs_device
    w = workload(n_cfg)
    inp = make_inputs_device(w, seed_of(n_cfg))
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, proxy_dtype=w.proxy_dtype)
    T, Hq, Hkv = w.total_rows, w.num_qo_heads, w.num_kv_heads
    sel = torch.empty((T, Hkv, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    msa.run_prefill(plan, inp.proxy_q, inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale, inp.q, inp.k_pages,
                    inp.v_pages, inp.kv_indices, sel, out, lse)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed_of(n_cfg) + 77)
    dout = torch.randn((T, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    dq = torch.empty((T, Hq, 128), dtype=torch.float32, device="cuda")
    dk = torch.empty((inp.k_pages.shape[0], Hkv, 128, 128), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    if kl:
        dpq = torch.empty((T, Hkv, 128), dtype=torch.float32, device="cuda")
        dpk = torch.empty_like(dk)
        plse = torch.empty((T, Hkv), dtype=torch.float32, device="cuda")

    def step():
        if kl:
            msa.msa_sparse_attn_prefill_backward_kl(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, out,
                                                    lse, dout, inp.proxy_q, inp.proxy_k_pages, 1.0, dq, dk, dv, dpq,
                                                    dpk, plse)
        else:
            msa.msa_sparse_attn_prefill_backward(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, sel, out,
                                                 lse, dout, dq, dk, dv)

    step()
    torch.cuda.synchronize()
    stages = ["csr", "bwd_dq", "bwd_dq_sum", "bwd_dkv"]
    if kl:
        stages += ["kl_dq_sum", "kl_dense_dq", "kl_dense_dk"]
    per_kernel = kernel_profile(msa, plan, step, stages)
    heavy = ("bwd_dq", "bwd_dkv", "kl_dense_dq", "kl_dense_dk") if kl else ("bwd_dq", "bwd_dkv")
    dominant = max(heavy, key=lambda n: per_kernel[n][0])
    ms_step, k_ms, launches = timed_with_kernel(msa, plan, step, steps, warmup, dominant)
    nvis = visible_keys_per_row(sel, w.qo_lens, w.kv_lens, "cuda")
    G = Hq // Hkv
    pairs = float(nvis.sum().item()) * G          # (selected visible key, query head) pairs
    dense = 0.0                                   # (visible key, proxy head) pairs of the dense proxy
    for qo, kv in zip(w.qo_lens, w.kv_lens):
        first = kv - qo
        dense += (qo * (first + 1) + qo * (qo - 1) / 2) * Hkv
    # algorithmic products, 2*128 FLOP per pair each: S, dP, dQ in bwd_dq; dV, dK in
    # bwd_dkv (its recomputation of S and dP is not counted); with the proxy term
    # one more sparse product in each, and S, dQ, dK over the dense proxy pairs
    # (kl_dense_dq's first sweep, which only finds the log-sum-exp, is not counted)
    per_kernel_products = {"bwd_dq": (3 + kl) * pairs, "bwd_dkv": (2 + kl) * pairs,
                           "kl_dense_dq": 2 * dense, "kl_dense_dk": dense}
    f_total = (5 + 2 * kl) * 2 * 128 * pairs + (3 * 2 * 128 * dense if kl else 0.0)
    work = 2 * 128 * per_kernel_products[dominant] / (launches // steps)
    achieved = work / (k_ms * 1e-3) / 1e12
    roof = {"kernel": dominant, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic_from_profiles(dominant, w.name),
            "avg_launch_ms": k_ms, "launches_per_step": launches // steps, "work_per_launch": work, "work_unit": "FLOP"}
    roof = with_measured(roof)
    name = w.name + ("_backward_kl" if kl else "_backward")
    grads = "dq, dk, dv, dproxy_q, dproxy_k (fp32)" if kl else "dq, dk, dv (fp32)"
    return {
        "workload": name, "tok_per_s": T / (ms_step * 1e-3), "ms_per_step": ms_step,
        "tflops": f_total / (ms_step * 1e-3) / 1e12, "stage_ms": {n: v[0] for n, v in per_kernel.items()},
        "roofline": roof,
        "config": {"workload": name, "total_rows": T, "num_qo_heads": Hq, "num_kv_heads": Hkv,
                   "num_proxy_heads": w.num_proxy_heads, "topk": w.topk, "head_dim": 128, "kv_dtype": "bf16",
                   "grads": grads},
    }


def warmup_bench(msa, n_cfg, steps, warmup):
    """The warm-up mode on one workload: one step = the dense causal forward
    (msa_dense_attn_prefill) and its backward with the proxy distillation
    gradient against the dense main distribution
    (msa_dense_attn_prefill_backward)."""
    import torch
    from synthetic.gen import workload, seed_of
    from synthetic.device_gen import make_inputs_device
    w = workload(n_cfg)
    inp = make_inputs_device(w, seed_of(n_cfg))
    plan = msa.msa_plan(w.qo_lens, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads,
                        w.num_proxy_kv_heads, topk=w.topk, proxy_dtype=w.proxy_dtype)
    T, Hq, Hkv = w.total_rows, w.num_qo_heads, w.num_kv_heads
    N = inp.k_pages.shape[0]
    out = torch.empty((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed_of(n_cfg) + 78)
    dout = torch.randn((T, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    dq = torch.empty((T, Hq, 128), dtype=torch.float32, device="cuda")
    dk = torch.empty((N, Hkv, 128, 128), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    dpq = torch.empty((T, Hkv, 128), dtype=torch.float32, device="cuda")
    dpk = torch.empty_like(dk)
    plse = torch.empty((T, Hkv), dtype=torch.float32, device="cuda")

    def step():
        msa.msa_dense_attn_prefill(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, out, lse)
        msa.msa_dense_attn_prefill_backward(plan, inp.q, inp.k_pages, inp.v_pages, inp.kv_indices, out, lse, dout,
                                            dq, dk, dv, inp.proxy_q, inp.proxy_k_pages, 1.0, dpq, dpk, plse)

    step()
    torch.cuda.synchronize()
    stages = ["dense_fwd", "dense_dq", "dense_dkv", "kl_dense_dq", "kl_dense_dk"]
    per_kernel = kernel_profile(msa, plan, step, stages)
    dominant = max(stages, key=lambda n: per_kernel[n][0])
    ms_step, k_ms, launches = timed_with_kernel(msa, plan, step, steps, warmup, dominant)
    dense = 0.0                                   # causally visible (row, key) pairs per KV head
    for qo, kv in zip(w.qo_lens, w.kv_lens):
        dense += qo * (kv - qo + 1) + qo * (qo - 1) / 2
    G = Hq // Hkv
    main_pairs = dense * Hq                       # (row, query head, key)
    proxy_pairs = dense * Hkv                     # (row, proxy head, key)
    # products of 2*128 FLOP per pair: forward S, PV; backward S, dP, dQ (dense_dq), dV, dK (dense_dkv;
    # its S, dP recomputation not counted); the proxy term's pk^T P and P^T pq over the main pairs;
    # the dense proxy S, dQ (kl_dense_dq) and dK (kl_dense_dk) over the proxy pairs
    products = {"dense_fwd": 2 * main_pairs, "dense_dq": 4 * main_pairs, "dense_dkv": 3 * main_pairs,
                "kl_dense_dq": 2 * proxy_pairs, "kl_dense_dk": proxy_pairs}
    f_total = 256 * sum(products.values())
    work = 256 * products[dominant] / (launches // steps)
    achieved = work / (k_ms * 1e-3) / 1e12
    roof = {"kernel": dominant, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic_from_profiles(dominant, w.name),
            "avg_launch_ms": k_ms, "launches_per_step": launches // steps, "work_per_launch": work, "work_unit": "FLOP"}
    roof = with_measured(roof)
    name = w.name + "_warmup"
    return {
        "workload": name, "tok_per_s": T / (ms_step * 1e-3), "ms_per_step": ms_step,
        "tflops": f_total / (ms_step * 1e-3) / 1e12, "stage_ms": {n: v[0] for n, v in per_kernel.items()},
        "roofline": roof,
        "config": {"workload": name, "total_rows": T, "num_qo_heads": Hq, "num_kv_heads": Hkv,
                   "num_proxy_heads": w.num_proxy_heads, "head_dim": 128, "kv_dtype": "bf16",
                   "step": "dense forward + backward (dq, dk, dv, dproxy_q, dproxy_k)", "G": G},
    }


def decode_bench(msa, steps, warmup, sets=4):
    import torch
    from synthetic.gen import workload, seed_of, decode_picks
    from synthetic.device_gen import make_inputs_device
    w = workload(4)
    inp = make_inputs_device(w, seed_of(4))
    # independent (q, picks) sets rotated per step so that the selected working
    # set (sets x 143 MB) exceeds the 256 MB Infinity Cache
    qs, sels = [inp.q], [inp.kv_block_indexes]
    for j in range(1, sets):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed_of(4) * 100 + j)
        qs.append(torch.randn(inp.q.shape, generator=g, device="cuda").to(torch.bfloat16))
        sels.append(torch.from_numpy(decode_picks(w, seed_of(4) * 100 + j)).cuda())
    plan = msa.msa_plan(None, w.kv_lens, w.num_qo_heads, w.num_kv_heads, topk=w.topk, kv_dtype="fp8", mode="decode")
    out = torch.empty((w.num_seqs, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    it = [0]

    def step():
        j = it[0] % sets
        it[0] += 1
        msa.msa_sparse_attn_decode(plan, qs[j], inp.k_pages, inp.v_pages, inp.k_scale, inp.v_scale, inp.kv_indices,
                                   sels[j], out)

    step()
    torch.cuda.synchronize()
    per_kernel = kernel_profile(msa, plan, step, ["decode", "decode_merge"])
    # the kernel by its own HIP events (a separate pass); the step by duration,
    # eagerly and replayed from a HIP graph, with no profiling events attached
    _, k_ms, launches = timed_with_kernel(msa, plan, step, steps, warmup, "decode")
    launches_per_step = max(1, launches // steps)
    k_timing = "per-dispatch HIP events"
    if "decode_merge" not in per_kernel and launches_per_step == 1 and not PROFILE_RUN[0]:
        # the step is this one kernel: a pair of events around a block of
        # back-to-back launches on the launch stream times it without the
        # per-dispatch events' own cost (a few microseconds a launch)
        k_ms, _ = stream_event_ms(step)
        k_timing = "HIP events on the launch stream around a block of back-to-back launches (one launch per step)"
    if PROFILE_RUN[0]:
        ms_step, timed = time_steps(step, steps, warmup), steps
        host_us, g_ms, g_steps = None, float("nan"), 0
    else:
        ms_step, timed = time_by_duration(step)
        host_us = host_cost_us(step)
        g_ms, g_steps = graph_time(step, sets)
    # compulsory bytes of one decode launch: selected K and V pages (fp8) + q + scales + indices + partials out
    nsel = sum(int((s >= 0).sum().item()) for s in sels) / sets
    kv_bytes = nsel * 2 * 128 * 128
    q_bytes = w.num_seqs * w.num_qo_heads * 128 * 2
    work = kv_bytes + q_bytes
    achieved = work / (k_ms * 1e-3) / 1e9
    step_bytes = work + w.num_seqs * w.num_qo_heads * 128 * 2
    roof = with_measured({"kernel": "decode", "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                          "traffic": traffic_from_profiles("decode", w.name), "avg_launch_ms": k_ms,
                          "launch_timing": k_timing,
                          "launches_per_step": launches_per_step, "work_per_launch": work, "work_unit": "B"})
    return {
        "workload": w.name, "tok_per_s": w.num_seqs / (ms_step * 1e-3), "ms_per_step": ms_step,
        "timing": f"by duration: >= 50 ms warm-up, then {timed} steps (>= 200 ms) between synchronizes, no "
                  f"profiling events",
        "step_gbs": step_bytes / (ms_step * 1e-3) / 1e9, "hbm_frac_step": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "host_us_per_step": host_us,
        "graph": {"ms_per_step": g_ms, "tok_per_s": w.num_seqs / (g_ms * 1e-3), "steps": g_steps,
                  "hbm_frac_step": step_bytes / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "stage_ms": {n: v[0] for n, v in per_kernel.items()}, "roofline": roof,
        "config": {"workload": w.name, "batch": w.num_seqs, "kv_len": w.kv_lens[0], "num_qo_heads": w.num_qo_heads,
                   "num_kv_heads": w.num_kv_heads, "slots": w.topk, "kv_dtype": "fp8", "rotated_sets": sets},
    }


def decode_step_bench(msa, steps, warmup, sets=4, wn=6):
    """A whole decode step at 32 x 131072: the indexer pass (fused proxy +
    top-k on a one-query-row plan; 8 fp8 proxy heads sharing one fp8 (workload
    6) or MXFP4 (workload 7) proxy-K head) and the fp8 sparse decode on its
    selection.  Four independent (proxy q, q) sets are rotated per step."""
    import torch
    from synthetic.gen import workload, seed_of
    from synthetic.device_gen import make_inputs_device
    w = workload(wn)
    S = w.num_seqs
    inp = make_inputs_device(w, seed_of(wn))
    pqs, qs = [inp.proxy_q], [inp.q]
    for j in range(1, sets):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed_of(wn) * 100 + j)
        pq = torch.randn(inp.proxy_q.shape, generator=g, device="cuda") / inp.proxy_q_scale[None, :, None]
        pqs.append(pq.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8))
        qs.append(torch.randn(inp.q.shape, generator=g, device="cuda").to(torch.bfloat16))
    ip = msa.msa_plan([1] * S, w.kv_lens, w.num_qo_heads, w.num_kv_heads, w.num_proxy_heads, w.num_proxy_kv_heads,
                      topk=w.topk, proxy_dtype=w.proxy_dtype)
    dp = msa.msa_plan(None, w.kv_lens, w.num_qo_heads, w.num_kv_heads, topk=w.topk, kv_dtype="fp8", mode="decode")
    sel = torch.empty((S, w.num_kv_heads, w.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((S, w.num_qo_heads, 128), dtype=torch.bfloat16, device="cuda")
    it = [0]

    def step():
        j = it[0] % sets
        it[0] += 1
        msa.msa_proxy_topk_select(ip, pqs[j], inp.proxy_k_pages, inp.proxy_q_scale, inp.proxy_k_scale, inp.kv_indices,
                                  0, S, sel)
        msa.msa_sparse_attn_decode(dp, qs[j], inp.k_pages, inp.v_pages, inp.k_scale, inp.v_scale, inp.kv_indices, sel,
                                   out)

    step()
    torch.cuda.synchronize()
    stage = {}
    for plan, names in ((ip, ["proxy_topk", "topk_select"]), (dp, ["decode"])):
        for n, v in kernel_profile(msa, plan, step, names).items():
            stage[n] = v[0]
    _, k_ms, launches = timed_with_kernel(msa, ip, step, steps, warmup, "proxy_topk")
    if PROFILE_RUN[0]:
        ms_step, timed = time_steps(step, steps, warmup), steps
        host_us, g_ms, g_steps = None, float("nan"), 0
    else:
        ms_step, timed = time_by_duration(step)
        host_us = host_cost_us(step)
        g_ms, g_steps = graph_time(step, sets)
    # compulsory bytes of one indexer launch: every visible proxy-K block
    # (fp8: 128 x 128 B; MXFP4: 128 x (64 + 4) B) + the fp8 proxy q
    nb = sum(-(-L // 128) for L in w.kv_lens)
    kblock = 128 * 128 if w.proxy_dtype == "fp8" else 128 * (64 + 4)
    work = nb * w.num_proxy_kv_heads * kblock + S * w.num_proxy_heads * 128
    achieved = work / (k_ms * 1e-3) / 1e9
    kname = "proxy_onerow" if w.proxy_dtype == "fp8" else "proxy_onerow_mxfp4"
    roof = with_measured({"kernel": kname, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                          "traffic": traffic_from_profiles(kname, w.name), "avg_launch_ms": k_ms,
                          "launches_per_step": max(1, launches // steps), "work_per_launch": work, "work_unit": "B"})
    return {
        "workload": w.name, "tok_per_s": S / (ms_step * 1e-3), "ms_per_step": ms_step, "stage_ms": stage,
        "timing": f"by duration: >= 50 ms warm-up, then {timed} steps (>= 200 ms) between synchronizes, no "
                  f"profiling events",
        "host_us_per_step": host_us,
        "graph": {"ms_per_step": g_ms, "tok_per_s": S / (g_ms * 1e-3), "steps": g_steps},
        "roofline": roof,
        "config": {"workload": w.name, "batch": S, "kv_len": w.kv_lens[0], "num_qo_heads": w.num_qo_heads,
                   "num_kv_heads": w.num_kv_heads, "num_proxy_heads": w.num_proxy_heads,
                   "num_proxy_kv_heads": w.num_proxy_kv_heads, "proxy_dtype": w.proxy_dtype, "kv_dtype": "fp8",
                   "slots": w.topk, "rotated_sets": sets},
    }


def cpu_baseline(w, inp, sel, rows=256):
    """The fp64 oracle as it stands, on a bounded sample of rows of the same
    workload: proxy scores, selection and attention for `rows` rows spread
    over the sequence.  Returns tok/s of the sample."""
    import oracle as O
    from synthetic.device_gen import to_host
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    T = w.total_rows
    sample = np.unique(np.linspace(0, T - 1, rows).astype(np.int64))
    h = {k: to_host(getattr(inp, k)) for k in ("q", "k_pages", "v_pages", "kv_indices", "proxy_q", "proxy_k_pages",
                                                "proxy_q_scale", "proxy_k_scale")}
    t0 = time.perf_counter()
    ms = O.proxy_block_maxscore(h["proxy_q"], h["proxy_k_pages"], h["kv_indices"], w.qo_lens, w.kv_lens, 128,
                                w.proxy_sm_scale, w.proxy_dtype, h["proxy_q_scale"], h["proxy_k_scale"], rows=sample)
    osel = O.topk_select(ms, w.qo_lens, w.kv_lens, 128, w.topk, rows=sample)
    full_sel = np.zeros((T, w.num_kv_heads, w.topk), np.int32)
    full_sel[sample] = osel
    O.sparse_attention(h["q"], h["k_pages"], h["v_pages"], h["kv_indices"], full_sel, w.qo_lens, w.kv_lens, 128,
                       w.sm_scale, rows=sample)
    dt = time.perf_counter() - t0
    model, physical = cpu_info()
    return {"value": len(sample) / dt, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "physical_cores": physical, "logical_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{len(sample)} rows evenly spaced over the {T}-row {w.name} workload "
                      f"(proxy scores, top-k and attention for each), {dt:.1f} s wall"}


def cpu_info():
    """(model name, physical cores among the CPUs this process may run on)."""
    model, cores = None, set()
    allowed = os.sched_getaffinity(0)
    try:
        cpu = phys = None
        for ln in open("/proc/cpuinfo"):
            k, _, v = ln.partition(":")
            k, v = k.strip(), v.strip()
            if k == "processor":
                cpu, phys = int(v), None
            elif k == "model name" and model is None:
                model = v
            elif k == "physical id":
                phys = v
            elif k == "core id" and cpu in allowed:
                cores.add((phys, v))
    except OSError:
        pass
    return model, (len(cores) or None)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="skip the 128K prefill and decode entries")
    ap.add_argument("--extra", default="prefill_128k,prefill_1m_fp8proxy,prefill_32k_mxfp4,prefill_32k_backward,"
                                       "prefill_32k_backward_kl,warmup_32k,decode_131k,decode_step_131k,"
                                       "decode_step_mxfp4_131k",
                    help="comma-separated extra entries: prefill_128k, prefill_1m_fp8proxy, prefill_32k_mxfp4, "
                         "prefill_32k_backward, prefill_32k_backward_kl, prefill_128k_backward (not by default), "
                         "warmup_32k, decode_131k, decode_step_131k, decode_step_mxfp4_131k (or none)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--profile-run", action="store_true",
                    help="under a profiler: fixed small step counts, no duration-timed, host-cost or graph legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a streaming copy of known size (for scaling HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: write profiles/<kernel>__<workload>__traffic.txt from two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_CSV", "BENCH_STDOUT", "BENCH_STDERR", "OUT_NAME"),
                    help="host only: write a kernel-duration summary under profiles/ from a rocprofv3 kernel trace")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("MFMA_CSV", "BENCH_STDERR", "OUT_NAME"),
                    help="host only: write a matrix-core / LDS counter summary under profiles/")
    ap.add_argument("--summarize-stalls", nargs=3, metavar=("PASS_A_CSV", "PASS_B_CSV", "OUT_NAME"),
                    help="host only: write the wave-cycle / instruction-mix summary under profiles/")
    ap.add_argument("--window-sweep", type=int, metavar="CFG",
                    help="only the sparse prefill of workload CFG at attention windows 32K/8K/4K/2K, without and with "
                         "XCD pinning (one JSON line each)")
    ap.add_argument("--summarize-window-sweep", nargs=6,
                    metavar=("FETCH_CSV", "FETCH_STDERR", "WRITE_CSV", "WRITE_STDERR", "SWEEP_STDOUT", "OUT_NAME"),
                    help="host only: write the window-sweep summary under profiles/")
    args = ap.parse_args()
    if args.summarize_counters:
        for p in summarize_counters(*args.summarize_counters):
            print(p)
        return
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace))
        return
    if args.summarize_mfma:
        print(summarize_mfma(*args.summarize_mfma))
        return
    if args.summarize_stalls:
        print(summarize_stalls(*args.summarize_stalls))
        return
    if args.summarize_window_sweep:
        print(summarize_window_sweep(*args.summarize_window_sweep))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (see the design notes on "
              "sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from block_sparse_top_amd import msa
    torch.cuda.set_device(0)
    PROFILE_RUN[0] = args.profile_run
    extras = [] if args.no_extra or args.extra == "none" else [e for e in args.extra.split(",") if e]
    for e in extras:
        if e not in ("prefill_128k", "prefill_1m_fp8proxy", "prefill_32k_mxfp4", "prefill_32k_backward",
                     "prefill_32k_backward_kl",
                     "prefill_128k_backward", "warmup_32k", "decode_131k", "decode_step_131k",
                     "decode_step_mxfp4_131k"):
            ap.error(f"unknown extra entry {e}")
    if args.copy_calibration:
        print("[bench] calibration copy", file=sys.stderr, flush=True)
        copy_calibration()
    def mark(key):   # host monotonic clock before a workload's first launch (trace summaries split on it)
        torch.cuda.synchronize()
        print(f"[bench-mark] {key} {time.monotonic_ns()}", file=sys.stderr, flush=True)
    if args.window_sweep:
        steps, warm = (2, 1) if args.profile_run else (args.steps, args.warmup)
        window_sweep(msa, args.window_sweep, steps, warm, mark)
        return

    peaks = None
    if not args.no_peaks:
        print("[bench] measured peaks (streaming copy, matrix-core loops)", file=sys.stderr, flush=True)
        peaks = measure_peaks(msa)
    print("[bench] prefill 32k", file=sys.stderr, flush=True)
    mark("main")
    main_res, (w, inp, sel) = prefill_bench(msa, 2, args.steps, args.warmup)
    extra = {}
    if "prefill_128k" in extras:
        print("[bench] prefill 128k varlen", file=sys.stderr, flush=True)
        mark("prefill_128k")
        r3, _ = prefill_bench(msa, 3, max(2, args.steps // 2), 1)
        extra["prefill_128k"] = r3
    if "prefill_1m_fp8proxy" in extras:
        print("[bench] prefill 1M tokens, fp8 proxy", file=sys.stderr, flush=True)
        mark("prefill_1m_fp8proxy")
        r5, _ = prefill_bench(msa, 5, 2, 1, profile_reps=1)
        extra["prefill_1m_fp8proxy"] = r5
        import torch as _t
        _t.cuda.empty_cache()
    if "prefill_32k_mxfp4" in extras:
        print("[bench] prefill 32k, MXFP4 proxy q and K, MXFP4 K/V", file=sys.stderr, flush=True)
        mark("prefill_32k_mxfp4")
        r8, _ = prefill_bench(msa, 8, args.steps, args.warmup)
        extra["prefill_32k_mxfp4"] = r8
    if "prefill_32k_backward" in extras:
        print("[bench] prefill 32k backward", file=sys.stderr, flush=True)
        mark("prefill_32k_backward")
        extra["prefill_32k_backward"] = backward_bench(msa, 2, args.steps, args.warmup)
    if "prefill_32k_backward_kl" in extras:
        print("[bench] prefill 32k backward with the proxy distillation gradient", file=sys.stderr, flush=True)
        mark("prefill_32k_backward_kl")
        extra["prefill_32k_backward_kl"] = backward_bench(msa, 2, args.steps, args.warmup, kl=True)
    if "prefill_128k_backward" in extras:
        print("[bench] prefill 128k varlen backward", file=sys.stderr, flush=True)
        mark("prefill_128k_backward")
        extra["prefill_128k_backward"] = backward_bench(msa, 3, max(2, args.steps // 2), 1)
    if "warmup_32k" in extras:
        print("[bench] warm-up mode 32k: dense forward and backward with the proxy gradient", file=sys.stderr,
              flush=True)
        mark("warmup_32k")
        extra["warmup_32k"] = warmup_bench(msa, 2, max(2, args.steps // 2), 1)
    if "decode_131k" in extras:
        print("[bench] decode 131k fp8", file=sys.stderr, flush=True)
        mark("decode_131k")
        extra["decode_131k"] = decode_bench(msa, args.steps if args.profile_run else max(50, args.steps * 10),
                                            1 if args.profile_run else 10)
    if "decode_step_131k" in extras:
        print("[bench] decode step (indexer + decode) 131k fp8", file=sys.stderr, flush=True)
        mark("decode_step_131k")
        extra["decode_step_131k"] = decode_step_bench(msa, args.steps if args.profile_run else max(50, args.steps * 10),
                                                      1 if args.profile_run else 10)
    if "decode_step_mxfp4_131k" in extras:
        print("[bench] decode step (indexer + decode) 131k, MXFP4 proxy K", file=sys.stderr, flush=True)
        mark("decode_step_mxfp4_131k")
        extra["decode_step_mxfp4_131k"] = decode_step_bench(
            msa, args.steps if args.profile_run else max(50, args.steps * 10), 1 if args.profile_run else 10, wn=7)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp, sel, args.cpu_rows)
    line = {
        "metric": METRIC, "value": main_res["tok_per_s"], "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1), device generator)",
        "config": main_res["config"], "roofline": main_res["roofline"], "cpu_baseline": cpu,
        "mfma_util": main_res["mfma_util"], "tflops": main_res["tflops"], "stage_ms": main_res["stage_ms"],
        "flops": main_res["flops"], "proxy_roofline": main_res["proxy_roofline"],
        "mfma_util_measured": main_res["mfma_util_measured"], "measured_peaks": peaks, "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
