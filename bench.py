#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X: KV-cache GB/s per decode step.

A step is one decode step of each of the three workloads the metric names,
back to back on one stream:
  * GQA g=4, 8B-shaped layer:  B=32, h_q=32, h_kv=8, D=128, T=4096, bf16
  * GQA g=8, 70B-shaped layer: B=16, h_q=64, h_kv=8, D=128, ragged
    seq_lens ~ U[1024, 32768] (seed 0), T_max=32768, bf16
  * absorbed MLA, DeepSeek-V2-shaped layer: B=64, H=128, d_c=512, d_r=64,
    T=4096, bf16 (when the MLA kernel is built)
Each call is split into its two kernels (split-KV partial, log-sum-exp merge).
A first pass of K steps records HIP events around every kernel on the launch
stream (``config.breakdown``); the timed pass of K steps records events only
around the dominant partial kernel (``roofline``), because every event record
adds a few microseconds to a step. ``value`` = KV-cache bytes of the step
(valid positions only) divided by the wall time of a step in the timed pass.
The MHA (Llama-2-7B layer) and MQA (7B-shaped, one KV head) workloads are
timed separately, and the tiny fp32 workload as the latency of one call; they
are reported in ``config.breakdown`` only. Per-call and per-step figures come
with their median and 10th/90th percentiles over the K steps.

Inputs are seeded synthetic tensors (``workloads``), resident in HBM before
the timed region. The working set (> 1.6 GB per step) is far larger than the
256 MB last-level cache, so every step streams the caches from HBM.

The ``cpu_baseline`` leg times the fp64 oracle on a bounded sample of the
same workloads on the host cores (rank 0, N=1 only).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(xs, q):
    """q-th percentile (0..100) of a list, linear interpolation between order statistics."""
    ys = sorted(xs)
    if not ys:
        return float("nan")
    k = (len(ys) - 1) * q / 100.0
    lo = int(math.floor(k))
    hi = min(lo + 1, len(ys) - 1)
    return ys[lo] + (ys[hi] - ys[lo]) * (k - lo)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------- algorithmic work

def gqa_work(w, lens):
    """Bytes and FLOPs the method must move/do for one GQA decode step (valid positions only)."""
    e = 2 if "bfloat16" in str(w.dtype) else 4
    sum_n = int(sum(min(max(int(x), 0), w.T_max) for x in lens))
    kv = 2 * w.h_kv * w.D * e * sum_n
    q_out = 2 * w.B * w.h_q * w.D * e
    flops = 4 * w.h_q * w.D * sum_n
    return kv, q_out + 4 * w.B, flops


def mla_work(w, lens):
    sum_n = int(sum(min(max(int(x), 0), w.T_max) for x in lens))
    kv = sum_n * (w.d_c + w.d_r) * 2
    q_out = w.B * w.H * (w.d_c + w.d_r + w.d_c) * 2
    flops = 2 * w.H * sum_n * ((w.d_c + w.d_r) + w.d_c)
    return kv, q_out + 4 * w.B, flops


# ----------------------------------------------------------------------------- traffic record

def traffic_for(kernel_src: str, kernel_name: str):
    """HBM bytes per launch measured with rocprofv3 counters, if still valid for this source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    ent = rec.get("kernels", {}).get(kernel_name)
    if not ent or ent.get("source_sha256") != sha:
        return None
    return ent.get("hbm_bytes_per_launch")


COPY_CAL_BYTES = 1 << 30   # size of the plain device-to-device copy used to calibrate counters
COPY_CAL_REPS = 4


def copy_calibration(dev):
    """Plain device-to-device copies of a known size (read COPY_CAL_BYTES, write COPY_CAL_BYTES).

    Run after the timed region when --copy-calibration is given, so that a
    rocprofv3 counter run over the same command can scale FETCH_SIZE and
    WRITE_SIZE to bytes."""
    import torch
    a = torch.ones(COPY_CAL_BYTES // 2, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(COPY_CAL_REPS):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def _norm_kernel_name(full: str) -> str:
    s = full.replace("attn::(anonymous namespace)::", "")
    if s.startswith("void "):
        s = s[5:]
    return s.split("(")[0].strip()


def _read_counter(path: str, counter: str):
    """[(dispatch_id, kernel_name, value)] for one counter from a rocprofv3 counter_collection CSV."""
    import csv
    out = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            out.append((int(row["Dispatch_Id"]), _norm_kernel_name(row["Kernel_Name"]),
                        float(row["Counter_Value"])))
    return out


def write_traffic(fetch_csv: str, write_csv: str, command: str):
    """Turn two rocprofv3 --pmc runs of ``bench.py --copy-calibration`` (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) into profiles/traffic.json.

    The calibration copies are the copy-kernel dispatches issued after the last
    attention kernel; each moves COPY_CAL_BYTES in and out, so
    factor = COPY_CAL_BYTES / (counter KiB * 1024) converts a counter reading to bytes."""
    srcs = {"gqa_partial": os.path.join(ROOT, "mla_kv_cache_amd", "csrc", "gqa_decode.hip"),
            "gqa_matrix": os.path.join(ROOT, "mla_kv_cache_amd", "csrc", "gqa_matrix.hip"),
            "gqa_mma16": os.path.join(ROOT, "mla_kv_cache_amd", "csrc", "gqa_mma16.hip"),
            "mla_partial": os.path.join(ROOT, "mla_kv_cache_amd", "csrc", "mla_decode.hip"),
            "lse_merge": os.path.join(ROOT, "mla_kv_cache_amd", "csrc", "lse_merge.hip"),
            "split_merge": os.path.join(ROOT, "mla_kv_cache_amd", "csrc", "lse_merge.hip")}
    res = {"command": command, "copy_bytes": COPY_CAL_BYTES, "kernels": {}}
    per = {}
    for cname, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _read_counter(path, cname)
        attn = [r for r in rows if any(r[1].startswith(k) for k in srcs)]
        last = max(r[0] for r in attn)
        cal = [r[2] for r in rows if r[0] > last and "copyBuffer" in r[1]]
        if not cal:
            raise SystemExit(f"{path}: no calibration copy dispatches after the attention kernels")
        kib = sum(cal) / len(cal)
        factor = COPY_CAL_BYTES / (kib * 1024.0)
        res[cname] = {"copy_kib_per_dispatch": kib, "factor": factor, "copy_dispatches": len(cal)}
        for _, name, v in attn:
            per.setdefault(name, {}).setdefault(cname, []).append(v * 1024.0 * factor)
    for name, d in sorted(per.items()):
        src = next(p for k, p in srcs.items() if name.startswith(k))
        fb = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"])
        wb = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"])
        res["kernels"][name] = {
            "source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
            "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
            "hbm_bytes_per_launch": round(fb + wb), "launches": len(d["FETCH_SIZE"])}
    out = os.path.join(ROOT, "profiles", "traffic.json")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


def summarize_counters(csvs, trace_csv=None):
    """Markdown table of per-dispatch hardware counters averaged per kernel, from
    rocprofv3 --pmc counter_collection CSVs (one or more passes).

    Derived columns (MI355X: 32 shader engines, 256 CUs, 1,024 SIMDs):
      cycles = SQ_BUSY_CYCLES / 32 (cycles with waves present, summed over the
        32 shader engines: the kernel's duration in cycles when it fills the chip);
      MHz = cycles / the kernel-trace duration (the clock the kernel ran at);
      MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1,024 SIMDs x cycles);
      VALU issue = 4 x SQ_ACTIVE_INST_VALU / (1,024 x cycles) (quad-cycles waves spend
        issuing VALU instructions, summed over waves, per SIMD-cycle);
      LDS bank conflicts = SQ_LDS_BANK_CONFLICT / (256 CUs x cycles) (stalled cycles per CU-cycle);
      L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS)."""
    import csv
    per = {}
    for path in csvs:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                name = _norm_kernel_name(row["Kernel_Name"])
                if name.startswith("__amd"):
                    continue
                d = per.setdefault(name, {})
                d.setdefault(row["Counter_Name"], {}).setdefault(row["Dispatch_Id"], 0.0)
                d[row["Counter_Name"]][row["Dispatch_Id"]] += float(row["Counter_Value"])
    dur = {}
    if trace_csv:
        with open(trace_csv, newline="") as f:
            for row in csv.DictReader(f):
                name = _norm_kernel_name(row["Kernel_Name"])
                dur.setdefault(name, []).append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)

    def avg(d, c):
        v = d.get(c)
        return sum(v.values()) / len(v) if v else None

    lines = ["| Kernel | dispatches | us (trace) | cycles / dispatch | MHz | MFMA busy | VALU issue | "
             "LDS bank conflicts | L2 hit rate |",
             "|---|---|---|---|---|---|---|---|---|"]
    for name, d in sorted(per.items()):
        busy = avg(d, "SQ_BUSY_CYCLES")
        cyc = busy / 32 if busy else None
        us = sum(dur[name]) / len(dur[name]) if name in dur else None
        mfma, valu = avg(d, "SQ_VALU_MFMA_BUSY_CYCLES"), avg(d, "SQ_ACTIVE_INST_VALU")
        bank, lds = avg(d, "SQ_LDS_BANK_CONFLICT"), avg(d, "SQ_ACTIVE_INST_LDS")
        hit = avg(d, "TCC_HIT") if "TCC_HIT" in d else avg(d, "TCC_HIT_sum")
        miss = avg(d, "TCC_MISS") if "TCC_MISS" in d else avg(d, "TCC_MISS_sum")
        ndisp = max(len(v) for v in d.values())
        f = lambda x, fmt: (fmt.format(x) if x is not None else "-")
        lines.append("| `{}` | {} | {} | {} | {} | {} | {} | {} | {} |".format(
            name, ndisp, f(us, "{:.1f}"), f(cyc, "{:,.0f}"),
            f(cyc / us if cyc and us else None, "{:,.0f}"),
            f(mfma / (1024 * cyc) if mfma is not None and cyc else None, "{:.1%}"),
            f(4 * valu / (1024 * cyc) if valu is not None and cyc else None, "{:.1%}"),
            f(bank / (256 * cyc) if bank is not None and cyc else None, "{:.2%}"),
            f(hit / (hit + miss) if hit is not None and miss is not None and hit + miss > 0 else None, "{:.1%}")))
    raw = ["", "Raw averages per dispatch:", "",
           "| Kernel | " + " | ".join(sorted({c for d in per.values() for c in d})) + " |",
           "|---|" + "---|" * len({c for d in per.values() for c in d})]
    cols = sorted({c for d in per.values() for c in d})
    for name, d in sorted(per.items()):
        raw.append("| `{}` | ".format(name) + " | ".join(
            "{:,.0f}".format(avg(d, c)) if avg(d, c) is not None else "-" for c in cols) + " |")
    return "\n".join(lines + raw)


# ----------------------------------------------------------------------------- widened rows

def _time_calls(fn, stream, warmup, iters):
    """Average HIP-event time (us) of one library call (all its kernels) on the launch stream."""
    import torch
    for _ in range(max(1, warmup)):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters


def time_next_rows(m, W, dev, stream, items, warmup, iters):
    """Time the rows built beside the decode path, on the bench's own inputs (not in `value`):
    the decode step that appends the new row (GQA g=8, MLA), sliding-window decode, the
    paged cache (the same caches in 64-position pages at permuted physical slots) and the
    MLA absorption products around the decode."""
    import torch
    res = {}
    by = {it["name"]: it for it in items}
    if "gqa8" in by:
        it = by["gqa8"]
        w = it["w"]
        q, k, v, lens = it["gpu"]
        before = (lens - 1).to(torch.int32)
        idx = (torch.arange(w.B, device=dev), slice(None), (lens - 1).long())
        kn, vn = k[idx].clone(), v[idx].clone()         # re-append the last row: the cache stays as it was
        ws = torch.empty(m.attn_decode_gqa_workspace_bytes(w.B, w.h_q, w.h_kv, w.D, w.T_max, w.dtype),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        us = _time_calls(lambda: m.attn_decode_gqa_step(q, kn, vn, k, v, before, w.scale, out, ws),
                         stream, warmup, iters)
        res["gqa8_step"] = {"workload": w.name + ", append + attend", "us": round(us, 2),
                            "kv_GBps": round(it["kv"] / (us * 1e-6) / 1e9, 1)}
        for window in (4096,):
            span = int(sum(min(int(x), window) for x in lens.tolist()))
            kvb = 2 * w.h_kv * w.D * 2 * span
            wsw = torch.empty(m.attn_decode_gqa_workspace_bytes(w.B, w.h_q, w.h_kv, w.D, window, w.dtype),
                              dtype=torch.uint8, device=dev)
            us = _time_calls(lambda: m.attn_decode_gqa_window(q, k, v, lens, window, w.scale, out, wsw),
                             stream, warmup, iters)
            res[f"gqa8_window{window}"] = {"workload": w.name + f", sliding window {window}",
                                           "us": round(us, 2), "kv_bytes": kvb,
                                           "kv_GBps": round(kvb / (us * 1e-6) / 1e9, 1)}
        # paged: the same cache cut into 64-position pages at randomly permuted physical slots
        ps = 64
        npg = w.T_max // ps
        perm = torch.randperm(w.B * npg, generator=torch.Generator().manual_seed(0)).to(dev)
        def paginate(x):
            pages = torch.empty((w.B * npg, w.h_kv, ps, w.D), dtype=x.dtype, device=dev)
            pages[perm] = x.view(w.B, w.h_kv, npg, ps, w.D).transpose(1, 2).reshape(w.B * npg, w.h_kv, ps, w.D)
            return pages
        kp, vp = paginate(k), paginate(v)
        table = perm.view(w.B, npg).to(torch.int32)
        us = _time_calls(lambda: m.attn_decode_gqa_paged(q, kp, vp, table, lens, w.scale, out, ws),
                         stream, warmup, iters)
        res["gqa8_paged64"] = {"workload": w.name + ", 64-position pages, permuted", "us": round(us, 2),
                               "kv_GBps": round(it["kv"] / (us * 1e-6) / 1e9, 1)}
        del kp, vp
    if "mla" in by:
        it = by["mla"]
        w = it["w"]
        qn, qr, lat, lens = it["gpu"]
        before = (lens - 1).to(torch.int32)
        new = lat[torch.arange(w.B, device=dev), (lens - 1).long()].clone()
        ws = torch.empty(m.attn_decode_mla_workspace_bytes(w.B, w.H, w.d_c, w.d_r, w.T_max),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((w.B, w.H, w.d_c), dtype=torch.bfloat16, device=dev)
        us = _time_calls(lambda: m.attn_decode_mla_step(qn, qr, new, lat, before, w.scale, out, ws),
                         stream, warmup, iters)
        res["mla_step"] = {"workload": w.name + ", append + attend", "us": round(us, 2),
                           "kv_GBps": round(it["kv"] / (us * 1e-6) / 1e9, 1)}
        ps = 64
        npg = w.T_max // ps
        perm = torch.randperm(w.B * npg, generator=torch.Generator().manual_seed(1)).to(dev)
        lp = torch.empty((w.B * npg, ps, w.d_c + w.d_r), dtype=lat.dtype, device=dev)
        lp[perm] = lat.view(w.B * npg, ps, w.d_c + w.d_r)
        table = perm.view(w.B, npg).to(torch.int32)
        us = _time_calls(lambda: m.attn_decode_mla_paged(qn, qr, lp, table, lens, w.scale, out, ws),
                         stream, warmup, iters)
        res["mla_paged64"] = {"workload": w.name + ", 64-position pages, permuted", "us": round(us, 2),
                              "kv_GBps": round(it["kv"] / (us * 1e-6) / 1e9, 1)}
        del lp
        # the absorption products around the decode: W_UK and W_UV of [H, d_c, 128], page init scale
        d_h = d_v = 128
        g = torch.Generator().manual_seed(2)
        qh = torch.randn((w.B, w.H, d_h), generator=g).to(torch.bfloat16).to(dev)
        w_uk = (torch.randn((w.H, w.d_c, d_h), generator=g) / w.d_c ** 0.5).to(torch.bfloat16).to(dev)
        w_uv = (torch.randn((w.H, w.d_c, d_v), generator=g) / w.d_c ** 0.5).to(torch.bfloat16).to(dev)
        q_lat = torch.empty((w.B, w.H, w.d_c), dtype=torch.bfloat16, device=dev)
        o = torch.empty((w.B, w.H, d_v), dtype=torch.bfloat16, device=dev)
        for name, fn, nbytes in (
                ("mla_absorb_q", lambda: m.attn_mla_absorb_q(qh, w_uk, q_lat),
                 2 * (w.B * w.H * d_h + w.H * w.d_c * d_h + w.B * w.H * w.d_c)),
                ("mla_up_v", lambda: m.attn_mla_up_v(out, w_uv, o),
                 2 * (w.B * w.H * w.d_c + w.H * w.d_c * d_v + w.B * w.H * d_v))):
            us = _time_calls(fn, stream, warmup, iters)
            flops = 2 * w.B * w.H * d_h * w.d_c
            res[name] = {"workload": f"B={w.B}, H={w.H}, d_c={w.d_c}, d_head=128, bf16 weights [H, d_c, 128]",
                         "us": round(us, 2), "bytes": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                         "TFLOPs": round(flops / (us * 1e-6) / 1e12, 2)}
    return res


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(items, budget_s=15.0):
    """Time the fp64 oracle on whole sequences of each workload until the budget is spent.

    Reported: KV GB/s of the oracle (sampled bytes / time), the host's CPU model
    and thread count, and the oracle's decode steps/s, estimated as one over the
    sum, across workloads, of the sampled time scaled up to the whole workload
    (by its share of the workload's KV bytes)."""
    import numpy as np  # noqa: F401
    import torch
    import oracle
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    done_bytes, t_used, parts = 0, 0.0, []
    step_est = 0.0
    per = budget_s / max(1, len(items))
    for name, kind, w, cpu in items:
        t0 = time.perf_counter()
        nseq = 0
        wl_bytes = 0
        total = gqa_work(w, cpu[3].tolist())[0] if kind == "gqa" else mla_work(w, cpu[3].tolist())[0]
        for b in range(w.B):
            if kind == "gqa":
                q, k, v, lens = cpu
                oracle.decode_gqa(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b:b + 1], w.scale)
                wl_bytes += gqa_work(w, lens[b:b + 1])[0]
            else:
                qn, qr, lat, lens = cpu
                oracle.decode_mla(qn[b:b + 1], qr[b:b + 1], lat[b:b + 1], lens[b:b + 1], w.scale, w.d_c)
                wl_bytes += mla_work(w, lens[b:b + 1])[0]
            nseq += 1
            if time.perf_counter() - t0 >= per:
                break
        dt = time.perf_counter() - t0
        t_used += dt
        done_bytes += wl_bytes
        step_est += dt * total / max(1, wl_bytes)
        parts.append(f"{name}: {nseq}/{w.B} sequences in {dt:.1f}s")
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "decode_steps_per_s": round(1.0 / step_est, 4) if step_est > 0 else None,
            "sample": "; ".join(parts) +
            " (fp64 oracle, whole sequences, KV bytes of the sampled sequences / time; "
            "steps/s scales each workload's sampled time to all its sequences)"}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--skip-mha", action="store_true", help="do not time the MHA and MQA breakdown workloads")
    ap.add_argument("--skip-next", action="store_true",
                    help="do not time the decode-step and sliding-window variants")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 counter CSVs and exit")
    ap.add_argument("--traffic-command", default="", help="command recorded with --traffic-from")
    ap.add_argument("--counters-from", nargs="+", metavar="CSV",
                    help="print a per-kernel table of rocprofv3 counter CSVs (and exit)")
    ap.add_argument("--trace", metavar="KERNEL_TRACE_CSV", help="kernel trace for --counters-from durations")
    args = ap.parse_args()

    if args.counters_from:
        print(summarize_counters(args.counters_from, args.trace))
        return

    if args.traffic_from:
        write_traffic(args.traffic_from[0], args.traffic_from[1], args.traffic_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs on a single MI355X and has no "
              "multi-GPU path. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import mla_kv_cache_amd as m

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    m.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    mla_ok = True
    try:
        m.attn_decode_mla_plan(W.MLA_V2.B, W.MLA_V2.H, W.MLA_V2.d_c, W.MLA_V2.d_r, W.MLA_V2.T_max)
    except m.AttnError:
        mla_ok = False

    # ---- inputs (seeded, drawn on the host, copied once into HBM)
    specs = [("gqa4", "gqa", W.GQA4_8B, True), ("gqa8", "gqa", W.GQA8_70B, True)]
    if mla_ok:
        specs.append(("mla", "mla", W.MLA_V2, True))
    if not args.skip_mha:
        specs.append(("mha7b", "gqa", W.MHA_7B, False))
        specs.append(("mqa", "gqa", W.MQA_7B, False))
    items, cpu_items = [], []
    for name, kind, w, in_step in specs:
        t0 = time.perf_counter()
        cpu = W.gqa_inputs(w) if kind == "gqa" else W.mla_inputs(w)
        gpu = tuple(x.to(dev) for x in cpu)
        log(f"[bench] inputs {name}: {time.perf_counter() - t0:.1f}s")
        lens = cpu[3].tolist()
        if kind == "gqa":
            q, k, v, gl = gpu
            P, NP, ws = m.attn_decode_gqa_plan(w.B, w.h_q, w.h_kv, w.D, w.T_max, w.dtype)
            out = torch.empty_like(q)
            kv, other, flops = gqa_work(w, lens)
            # attn_decode_gqa's work-balanced split (bf16), one stage per call
            wsb = torch.empty(ws, dtype=torch.uint8, device=dev)
            P, NP = "work-balanced split, 128-position units", None

            def partial(q=q, k=k, v=v, gl=gl, wsb=wsb, out=out, w=w):
                m.attn_decode_gqa_split(q, k, v, gl, wsb, scale=w.scale, out=out)

            def merge(q=q, k=k, v=v, gl=gl, wsb=wsb, out=out, w=w):
                m.attn_decode_gqa_split_merge(q, k, v, gl, wsb, scale=w.scale, out=out)
            if w.group <= 4:
                kname, srcf = f"gqa_partial_po_kernel<{w.D}, {w.group}, true>", "gqa_decode.hip"
            elif w.group <= 64:
                kname, srcf = f"gqa_mma16_kernel<{w.D}, {w.group}, true>", "gqa_mma16.hip"
            else:
                kname, srcf = f"gqa_matrix_kernel<{w.D}, {w.group}, true>", "gqa_matrix.hip"
            src = os.path.join(ROOT, "mla_kv_cache_amd", "csrc", srcf)
        else:
            qn, qr, lat, gl = gpu
            P, NP, ws = m.attn_decode_mla_plan(w.B, w.H, w.d_c, w.d_r, w.T_max)
            po = torch.empty((w.B, w.H, NP, w.d_c), dtype=torch.float32, device=dev)
            pl = torch.empty((w.B, w.H, NP), dtype=torch.float32, device=dev)
            out = torch.empty((w.B, w.H, w.d_c), dtype=torch.bfloat16, device=dev)
            kv, other, flops = mla_work(w, lens)

            def partial(qn=qn, qr=qr, lat=lat, gl=gl, P=P, po=po, pl=pl, w=w):
                m.attn_decode_mla_partial(qn, qr, lat, gl, w.scale, P, part_out=po, part_lse=pl)

            def merge(po=po, pl=pl, gl=gl, P=P, out=out, w=w):
                m.attn_decode_merge(po, pl, gl, w.T_max, P, out=out)
            kname = f"mla_partial_kernel<{4 if w.H >= 128 else w.H // 32}, false>"
            src = os.path.join(ROOT, "mla_kv_cache_amd", "csrc", "mla_decode.hip")
        items.append(dict(name=name, kind=kind, w=w, partial=partial, merge=merge, kv=kv,
                          other=other, flops=flops, P=P, NP=NP, kname=kname, src=src,
                          in_step=in_step, gpu=gpu))
        if in_step:
            cpu_items.append((name, kind, w, cpu))
        else:
            del cpu
    torch.cuda.synchronize()

    step_items = [it for it in items if it["in_step"]]

    def run_step(record=None, only=None, only_evs=None, step_evs=None):
        # record: events around every kernel; only: the name of the one
        # workload whose partial kernel alone is bracketed by only_evs;
        # step_evs: one event at the start of the step.
        if step_evs is not None:
            step_evs.record(stream)
        for it in step_items:
            if record is not None:
                record[it["name"]][0].record(stream)
            elif only == it["name"]:
                only_evs[0].record(stream)
            it["partial"]()
            if record is not None:
                record[it["name"]][1].record(stream)
            elif only == it["name"]:
                only_evs[1].record(stream)
            it["merge"]()
            if record is not None:
                record[it["name"]][2].record(stream)

    def summary_us(ms_list):
        us = [x * 1e3 for x in ms_list]
        return {"median": round(pct(us, 50), 2), "p10": round(pct(us, 10), 2),
                "p90": round(pct(us, 90), 2), "mean": round(sum(us) / len(us), 2)}

    def breakdown_entry(it, pt, mt, ct, note=None):
        call_ms, part_ms, merge_ms = pct(ct, 50), pct(pt, 50), pct(mt, 50)
        it["partial_ms"] = part_ms
        e = {"workload": it["w"].name, "partition_size": it["P"], "partitions": it["NP"],
             "call_us": summary_us(ct), "partial_us": round(part_ms * 1e3, 2),
             "merge_us": round(merge_ms * 1e3, 2), "kv_bytes": it["kv"],
             "kv_GBps": round(it["kv"] / (call_ms * 1e-3) / 1e9, 1),
             "kv_frac_hbm_peak": round(it["kv"] / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "partial_kernel_GBps": round((it["kv"] + it["other"]) / (part_ms * 1e-3) / 1e9, 1),
             "partial_frac_hbm_peak": round((it["kv"] + it["other"]) / (part_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if it["kind"] == "mla":
            tf = it["flops"] / (call_ms * 1e-3) / 1e12
            e["call_TFLOPs"] = round(tf, 1)
            e["mfma_frac_bf16_peak"] = round(tf / BF16_MFMA_PEAK_TFLOPS, 4)
        if note:
            e["note"] = note
        return e

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # Per-kernel breakdown: a pass of its own with events around every
    # kernel (each event record adds a few microseconds to the step, so this
    # pass is not the one whose wall time is reported). Medians and p10/p90
    # are over the K steps; kv_frac_hbm_peak is the whole call's (partial
    # kernel + merge) median.
    evs = [{it["name"]: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for it in step_items}
           for _ in range(args.steps)]
    for s_ in range(args.steps):
        run_step(evs[s_])
    torch.cuda.synchronize()

    # Whole calls: a pass with events only around each call (partial kernel +
    # merge, as one library call issues them), no event between the two.
    cevs = [{it["name"]: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for it in step_items}
            for _ in range(args.steps)]
    for s_ in range(args.steps):
        for it in step_items:
            cevs[s_][it["name"]][0].record(stream)
            it["partial"]()
            it["merge"]()
            cevs[s_][it["name"]][1].record(stream)
    torch.cuda.synchronize()

    breakdown = {}
    for it in step_items:
        pt = [evs[s_][it["name"]][0].elapsed_time(evs[s_][it["name"]][1]) for s_ in range(args.steps)]
        mt = [evs[s_][it["name"]][1].elapsed_time(evs[s_][it["name"]][2]) for s_ in range(args.steps)]
        ct = [cevs[s_][it["name"]][0].elapsed_time(cevs[s_][it["name"]][1]) for s_ in range(args.steps)]
        breakdown[it["name"]] = breakdown_entry(it, pt, mt, ct)

    # Step-time distribution: one event at each step boundary.
    sevs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for s_ in range(args.steps):
        run_step(step_evs=sevs[s_])
    sevs[-1].record(stream)
    torch.cuda.synchronize()
    step_ms = [sevs[i].elapsed_time(sevs[i + 1]) for i in range(args.steps)]

    # The timed region: K steps with events only around the dominant partial
    # kernel (the roofline's launch duration comes from these).
    dom = max(step_items, key=lambda it: it["partial_ms"])
    dom_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        run_step(only=dom["name"], only_evs=dom_evs[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    dom_ms = sum(e[0].elapsed_time(e[1]) for e in dom_evs) / args.steps

    # Workloads timed on their own, not part of the step (MHA 7B, MQA): calls
    # back to back on the stream, one pass with events around each kernel and
    # one with events around each whole call.
    for it in items:
        if it["in_step"]:
            continue
        for _ in range(args.warmup):
            it["partial"]()
            it["merge"]()
        e3 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        e2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for s_ in range(args.steps):
            e3[s_][0].record(stream)
            it["partial"]()
            e3[s_][1].record(stream)
            it["merge"]()
            e3[s_][2].record(stream)
        for s_ in range(args.steps):
            e2[s_][0].record(stream)
            it["partial"]()
            it["merge"]()
            e2[s_][1].record(stream)
        torch.cuda.synchronize()
        pts = [e[0].elapsed_time(e[1]) for e in e3]
        mts = [e[1].elapsed_time(e[2]) for e in e3]
        cts = [e[0].elapsed_time(e[1]) for e in e2]
        breakdown[it["name"]] = breakdown_entry(it, pts, mts, cts, note="timed alone, not part of the step")

    # The tiny fp32 workload: latency of one library call (latency-bound, microseconds only).
    tw = W.TINY_GQA
    tq, tk, tv, tl = (x.to(dev) for x in W.gqa_inputs(tw))
    tws = torch.empty(m.attn_decode_gqa_workspace_bytes(tw.B, tw.h_q, tw.h_kv, tw.D, tw.T_max, tw.dtype),
                      dtype=torch.uint8, device=dev)
    tout = torch.empty_like(tq)
    for _ in range(max(1, args.warmup)):
        m.attn_decode_gqa(tq, tk, tv, tl, scale=tw.scale, out=tout, workspace=tws)
    te = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s_ in range(args.steps):
        te[s_][0].record(stream)
        m.attn_decode_gqa(tq, tk, tv, tl, scale=tw.scale, out=tout, workspace=tws)
        te[s_][1].record(stream)
    torch.cuda.synchronize()
    tts = [e[0].elapsed_time(e[1]) for e in te]
    breakdown["tiny"] = {"workload": tw.name, "call_us": summary_us(tts),
                         "note": "latency-bound (262 KB of KV): microseconds only, no roofline fraction; "
                                 "calls back to back on the stream"}

    if not args.skip_next:
        breakdown["next_rows"] = time_next_rows(m, W, dev, stream, items, args.warmup, args.steps)

    step_kv = sum(it["kv"] for it in step_items)
    value = step_kv / (ms_per_step * 1e-3) / 1e9

    achieved = (dom["kv"] + dom["other"]) / (dom_ms * 1e-3) / 1e9
    traffic = traffic_for(dom["src"], dom["kname"])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom["kname"], "workload": dom["w"].name,
                "avg_launch_us": round(dom_ms * 1e3, 2),
                "algorithmic_bytes_per_launch": dom["kv"] + dom["other"],
                "whole_call_frac": {it["name"]: breakdown[it["name"]]["kv_frac_hbm_peak"]
                                    for it in items}}

    res = {
        "metric": "KV-cache GB/s per decode step (GQA g=4, GQA g=8, MLA)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": " + ".join(it["w"].name for it in step_items),
                   "step_kv_bytes": step_kv,
                   "kv_frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                   "decode_steps_per_s": round(1e3 / ms_per_step, 2),
                   "step_us": summary_us(step_ms),
                   "breakdown": breakdown},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cpu_items, args.cpu_budget)
    if args.copy_calibration:
        copy_calibration(dev)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
