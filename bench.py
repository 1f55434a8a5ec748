"""Benchmark of the MSA forward path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
for prefill, proxy block max scores and top-k selection over every row chunk,
then the block-sparse attention; for decode, one sparse decode call.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ...]

Prints one JSON line.  The headline workload is the 32K causal sparse prefill
(32 query heads, 8 KV heads, top-k 16); the 128K varlen prefill and the
32 x 131072 fp8 paged decode are reported under "extra".  Throughput is
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
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {
    "proxy_maxscore": "proxy_maxscore.hip", "topk_select": "topk_select.hip", "csr": "sparse_prefill.hip",
    "partial_attn": "sparse_prefill.hip", "merge": "sparse_prefill.hip", "decode": "sparse_decode.hip",
    "decode_merge": "sparse_decode.hip",
}


def source_hash(kernel: str) -> str:
    p = os.path.join(ROOT, "block_sparse_top_amd", "csrc", KERNEL_SOURCES[kernel])
    h = hashlib.sha256()
    for f in (p, os.path.join(ROOT, "block_sparse_top_amd", "csrc", "device_common.hpp")):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """Counter-measured HBM bytes per launch, if a committed summary for the
    current kernel source exists (null otherwise)."""
    p = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_hash") != source_hash(kernel):
        return None
    return d.get("bytes_per_launch")


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


def kernel_profile(msa, plan, step, names):
    """Per-kernel total ms over one step (each kernel in its own step)."""
    import torch
    out = {}
    for n in names:
        msa.msa_profile_kernel(plan, n)
        step()
        torch.cuda.synchronize()
        ms, cnt = msa.msa_profile_read(plan)
        msa.msa_profile_kernel(plan, None)
        if cnt:
            out[n] = (ms, cnt)
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


def prefill_bench(msa, n_cfg, steps, warmup, max_rows=0, attn_window=0):
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
                        inp.k_pages, inp.v_pages, inp.kv_indices, sel, out, None, ms_buf)

    step()
    torch.cuda.synchronize()
    per_kernel = kernel_profile(msa, plan, step, ["proxy_maxscore", "topk_select", "csr", "partial_attn", "merge"])
    dominant = max(per_kernel, key=lambda n: per_kernel[n][0])
    ms_step, k_ms, launches = timed_with_kernel(msa, plan, step, steps, warmup, dominant)
    launches_per_step = launches // steps
    nvis = visible_keys_per_row(sel, w.qo_lens, w.kv_lens, "cuda")
    G = w.num_qo_heads // w.num_kv_heads
    f_main = 4.0 * 128 * float(nvis.sum().item()) * G
    f_proxy = proxy_flops(w.qo_lens, w.kv_lens, w.num_proxy_heads)
    proxy_peak = PEAK_FP8_TFLOPS if w.proxy_dtype == "fp8" else PEAK_BF16_TFLOPS
    # work per launch of the dominant kernel (launches cover equal shares of a step)
    if dominant == "proxy_maxscore":
        work, peak, unit, bound = f_proxy / launches_per_step, proxy_peak, "TFLOP/s", "mfma"
    elif dominant == "partial_attn":
        work, peak, unit, bound = f_main / launches_per_step, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:  # bandwidth-bound helper kernels: count their compulsory bytes
        work, peak, unit, bound = None, PEAK_HBM_GBS, "GB/s", "hbm"
    achieved = (work / (k_ms * 1e-3) / 1e12) if (work is not None) else None
    roof = {"kernel": dominant, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": (achieved / peak) if achieved is not None else None,
            "traffic": traffic_from_profiles(dominant, w.name), "avg_launch_ms": k_ms,
            "launches_per_step": launches_per_step,
            "work_per_launch": work, "work_unit": "FLOP" if unit == "TFLOP/s" else "B"}
    stage_ms = {n: v[0] for n, v in per_kernel.items()}
    tflops = (f_main + f_proxy) / (ms_step * 1e-3) / 1e12
    res = {
        "workload": w.name, "tok_per_s": T / (ms_step * 1e-3), "ms_per_step": ms_step,
        "tflops": tflops, "mfma_util": tflops / PEAK_BF16_TFLOPS,
        "flops": {"proxy": f_proxy, "main": f_main}, "stage_ms": stage_ms, "roofline": roof,
        "config": {"workload": w.name, "qo_lens": w.qo_lens if len(w.qo_lens) <= 8 else None, "total_rows": T,
                   "num_qo_heads": w.num_qo_heads, "num_kv_heads": w.num_kv_heads,
                   "num_proxy_heads": w.num_proxy_heads, "topk": w.topk, "page_size": 128, "head_dim": 128,
                   "proxy_dtype": w.proxy_dtype, "max_rows_per_call": plan.max_rows_per_call},
    }
    return res, (w, inp, sel)


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
    ms_step, k_ms, launches = timed_with_kernel(msa, plan, step, steps, warmup, "decode")
    # compulsory bytes of one decode launch: selected K and V pages (fp8) + q + scales + indices + partials out
    nsel = sum(int((s >= 0).sum().item()) for s in sels) / sets
    kv_bytes = nsel * 2 * 128 * 128
    q_bytes = w.num_seqs * w.num_qo_heads * 128 * 2
    work = kv_bytes + q_bytes
    achieved = work / (k_ms * 1e-3) / 1e9
    step_bytes = work + w.num_seqs * w.num_qo_heads * 128 * 2
    roof = {"kernel": "decode", "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profiles("decode", w.name),
            "avg_launch_ms": k_ms, "launches_per_step": launches // steps, "work_per_launch": work, "work_unit": "B"}
    return {
        "workload": w.name, "tok_per_s": w.num_seqs / (ms_step * 1e-3), "ms_per_step": ms_step,
        "step_gbs": step_bytes / (ms_step * 1e-3) / 1e9, "hbm_frac_step": step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "stage_ms": {n: v[0] for n, v in per_kernel.items()}, "roofline": roof,
        "config": {"workload": w.name, "batch": w.num_seqs, "kv_len": w.kv_lens[0], "num_qo_heads": w.num_qo_heads,
                   "num_kv_heads": w.num_kv_heads, "slots": w.topk, "kv_dtype": "fp8", "rotated_sets": sets},
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
    return {"value": len(sample) / dt, "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(sample)} rows evenly spaced over the {T}-row {w.name} workload "
                      f"(proxy scores, top-k and attention for each), {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="skip the 128K prefill and decode entries")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path (see the design notes on "
              "sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from block_sparse_top_amd import msa
    torch.cuda.set_device(0)
    print("[bench] prefill 32k", file=sys.stderr, flush=True)
    main_res, (w, inp, sel) = prefill_bench(msa, 2, args.steps, args.warmup)
    extra = {}
    if not args.no_extra:
        print("[bench] prefill 128k varlen", file=sys.stderr, flush=True)
        r3, _ = prefill_bench(msa, 3, max(2, args.steps // 2), 1)
        extra["prefill_128k"] = r3
        print("[bench] decode 131k fp8", file=sys.stderr, flush=True)
        extra["decode_131k"] = decode_bench(msa, max(50, args.steps * 10), 10)
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
        "flops": main_res["flops"], "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
