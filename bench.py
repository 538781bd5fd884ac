"""Benchmark of the MSA hot path on one MI355X.

One step = one pass of every hot-path row at 128K and 1M context, on seeded
synthetic inputs resident in HBM (64 query / 4 KV heads, d_h 128, d_idx 64,
B_k 128, k 16, bf16):
  prefill128k    131072-token causal prefill with planted retrieval blocks
                 (contiguous cache): msa_index_topk + msa_sparse_prefill
  prefill1m      the last 8192 queries of a 1,048,576-token paged cache:
                 msa_index_topk + msa_sparse_prefill
  decode64x128k  one decode step of 64 sequences x 131072 tokens (paged,
                 4 rotating query sets): msa_index_topk + msa_sparse_decode
After the timed steps, 256 decode steps of the 1M sequence (batch 1) give
the decode latency p50 / p99, eager and from a HIP graph.
``value`` is prefill tokens/s over the step's four prefill calls; the decode
legs are reported in microseconds per step.  Each ABI call is timed with HIP
events on the stream it is launched on; ``roofline`` covers the dominant
kernel (kp_kernel, the KV-outer pass) and ``roofline.call`` the whole
msa_sparse_prefill call; ``rooflines`` lists every call.  The dense GQA
kernel is timed at the 128K shape for comparison, outside the step.  The
float64 oracle is timed on a bounded sample on the host (cpu_baseline).

Other workloads print their own JSON line: step32k (the 32K prefill with the
64 x 128K decode), prefill128k (planted, with the retrieval check), long1m,
decode_fp8 (e4m3 and MXFP8 caches), backward32k (the training path's gradient
call at the 32K prefill shape), project (index projections + RoPE), copy
(bandwidth calibration) and peak (achievable MFMA rate and copy bandwidth).

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5]
                       [--workload step|step32k|prefill128k|long1m|decode_fp8|backward32k|project|copy|peak]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synth import MODEL_SHAPE, gen_decode_paged, gen_long_context, gen_planted_prefill, gen_prefill  # noqa: E402
from synth.inputs import MXFP8  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
BLOCK = 128


# ----------------------------------------------------------- work accounting

def prefill_counts(n_q, q_start, shape=MODEL_SHAPE):
    """Algorithmic work of one prefill call, exact causal counts.

    index: 2 * d_idx FLOPs per (query, group, key) score over the strictly
      past blocks (the diagonal block is kept without scoring);
    main: 4 * d_h FLOPs per (query head, visible selected key): k-1 full past
      blocks (fewer early on) plus the visible part of the diagonal block."""
    p = q_start + np.arange(n_q, dtype=np.int64)
    diag = p // BLOCK
    past_keys = (BLOCK * diag).sum()
    idx_flops = 2.0 * shape.d_idx * shape.h_kv * float(past_keys)
    visible = BLOCK * np.minimum(shape.top_k - 1, diag) + (p % BLOCK) + 1
    main_flops = 4.0 * shape.h_q * shape.d_h * float(visible.sum())
    dense_flops = 4.0 * shape.h_q * shape.d_h * float((p + 1).sum())
    return idx_flops, main_flops, dense_flops


def decode_bytes(seq_lens, shape=MODEL_SHAPE, esz=2, cache_esz=None, mx=False):
    """Algorithmic HBM bytes of one decode step: the index keys of every past
    page (index scan) and the visible keys/values of the k selected pages.
    ``cache_esz``: bytes per cached element (default ``esz``; 1 for e4m3);
    ``mx``: MXFP8 caches, one more scale byte per 32 cached elements."""
    cesz = (esz if cache_esz is None else cache_esz) + (1.0 / 32 if mx else 0.0)
    L = np.asarray(seq_lens, dtype=np.int64)
    diag = (L - 1) // BLOCK
    idx_bytes = float((BLOCK * diag * shape.d_idx * cesz).sum())
    vis = BLOCK * np.minimum(shape.top_k - 1, diag) + (L - 1) % BLOCK + 1
    main_bytes = float((vis * shape.h_kv * shape.d_h * cesz * 2).sum())
    main_bytes += float(len(L) * shape.h_q * shape.d_h * esz * 2)  # q in, o out
    dense_bytes = float((L * shape.h_kv * shape.d_h * esz * 2).sum())
    return idx_bytes, main_bytes, dense_bytes


# ----------------------------------------------------------------- timing

class CallTimer:
    """HIP events around ABI calls on the current (launch) stream."""

    def __init__(self, names):
        self.names = names
        self.records = {n: [] for n in names}

    def step(self, fns):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
        evs[0].record()
        for i, fn in enumerate(fns):
            fn()
            evs[i + 1].record()
        return evs

    def collect(self, ev_lists):
        torch.cuda.synchronize()
        for evs in ev_lists:
            for i, n in enumerate(self.names):
                self.records[n].append(evs[i].elapsed_time(evs[i + 1]))

    def mean_ms(self, n):
        return float(np.mean(self.records[n]))

    def pct(self, n, q):
        return float(np.percentile(self.records[n], q))


def roofline(bound, work, ms, unit, call=None, workload="step"):
    peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
    if unit == "TFLOP/s":
        achieved = work / (ms * 1e-3) / 1e12
    else:
        achieved = work / (ms * 1e-3) / 1e9
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_bytes(workload, call)}


# ------------------------------------------------------------- HBM traffic
#
# Measured HBM bytes per ABI call come from two rocprofv3 counter runs of this
# script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what
# the same counter reads for a plain device-to-device copy of known size
# (``--workload copy``).  ``--summarize-traffic`` turns the four CSV files into
# profiles/traffic.json, stamped with a hash of the kernel sources; the bench
# reports null once the sources have changed since.

TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30
# kernels of each ABI call (substring of the kernel name)
CALL_KERNELS = {
    "index_prefill": ["ki_prefill_kernel", "ki_merge_kernel"],
    # name prefixes: the schedule counts and scatters in LDS (ks_*_lds_kernel) or
    # with global atomics (ks_zero + ks_count/ks_scatter) depending on the size
    "sparse_prefill": ["ks_zero", "ks_count", "ks_scan_a", "ks_scan_b", "ks_scan_c", "ks_scatter", "ks_items",
                       "kp_kernel", "km_kernel"],
    "index_decode": ["ki_decode_scan_kernel", "ki_decode_select_kernel"],
    "sparse_decode": ["kd_kernel", "kd_merge_kernel"],
}
CALL_FIRST = {"index_prefill": "ki_prefill_kernel", "sparse_prefill": "ks_count",
              "index_decode": "ki_decode_scan_kernel", "sparse_decode": "kd_kernel"}
# Legs of the default run, in launch order: two prefill legs (each starts with
# an index prefill launch), then the 64 x 128K decode step (its index scan is the
# first after the 1M prefill); the 1M decode steps of the latency probe follow
# the last step, so every later index scan belongs to them.
STEP_PREFILL_LEGS = ("prefill128k", "prefill1m")
TRAFFIC_KERNELS = ("ki_prefill_kernel", "kp_kernel", "km_kernel", "ki_decode_scan_kernel", "kd_kernel")


def source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_attention_branch_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    with open(os.path.join(ROOT, "include", "msa.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic():
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as fh:
        t = json.load(fh)
    return t if t.get("source_hash") == source_hash() else None


def traffic_bytes(workload, call):
    """Measured HBM bytes per call of `call` in `workload` (a workload or a leg
    of the default step), or None when not measured for the current sources."""
    t = _traffic()
    if call is None or t is None:
        return None
    rec = t.get("workloads", {}).get(workload, {}).get(call)
    return None if rec is None else rec["bytes"]


def kernel_traffic(workload, kernel):
    """Measured HBM bytes per launch of `kernel`, or None (see traffic_bytes)."""
    t = _traffic()
    if t is None:
        return None
    rec = t.get("kernels", {}).get(workload, {}).get(kernel)
    return None if rec is None else rec["bytes_per_launch"]


def _pmc_rows(path, counter):
    import csv
    out = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return out


def step_legs(names):
    """Leg of each dispatch of a default-step run, from the launch order:
    an index-prefill launch opens the next prefill leg (128K, 1M, 128K, ...);
    an index-scan launch opens a decode leg, the first after the 1M prefill
    being the 64 x 128K step and the rest the 1M steps.  Kernels that belong to
    no call (cache appends, the dense comparison, copies) get None."""
    legs = []
    leg, n_pre, n_dec = None, 0, 0
    mine = [k for ks in CALL_KERNELS.values() for k in ks]
    for n in names:
        if "ki_prefill_kernel" in n:
            leg = STEP_PREFILL_LEGS[n_pre % 2]
            n_pre += 1
            n_dec = 0
        elif "ki_decode_scan_kernel" in n:
            leg = "decode64x128k" if n_dec == 0 else "decode1m"
            n_dec += 1
        legs.append(leg if any(k in n for k in mine) else None)
    return legs


def summarize_traffic(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Per-call HBM bytes from rocprofv3 counter CSVs; writes profiles/traffic.json.

    FETCH_SIZE and WRITE_SIZE are read per dispatch (KiB; several rows of one
    dispatch add up) and scaled by the ratio of a plain copy's known bytes to
    what the same counter read for it.  For the default step ("step") each
    dispatch is attributed to its leg (step_legs) and a call's bytes are
    averaged over that leg's occurrences; other workloads are one leg."""
    def per_dispatch(path, counter):
        d = {}
        for name, did, v in _pmc_rows(path, counter):
            d[did] = (name, d.get(did, (name, 0.0))[1] + v)
        return [d[k] for k in sorted(d)]

    def copy_factor(path, counter):
        vals = [v for n, v in per_dispatch(path, counter) if "copy" in n.lower()]
        if not vals:
            raise SystemExit(f"no copy kernel in {path}")
        kib = float(np.median(vals))
        return (COPY_BYTES / 1024.0) / kib, kib

    ff, fk = copy_factor(copy_fetch_csv, "FETCH_SIZE")
    wf, wk = copy_factor(copy_write_csv, "WRITE_SIZE")
    runs = {"fetch": (per_dispatch(fetch_csv, "FETCH_SIZE"), ff), "write": (per_dispatch(write_csv, "WRITE_SIZE"), wf)}
    t = _traffic() or {"workloads": {}, "kernels": {}}
    t["source_hash"] = source_hash()
    t["copy_calibration"] = {"bytes": COPY_BYTES, "fetch_kib_read": fk, "write_kib_read": wk,
                             "fetch_factor": ff, "write_factor": wf}
    leg_names = ([workload] if workload != "step" else list(STEP_PREFILL_LEGS) + ["decode64x128k", "decode1m"])
    for leg_name in leg_names:
        res = {}
        for call, kernels in CALL_KERNELS.items():
            tot = {}
            for key, (rows, fac) in runs.items():
                legs = step_legs([n for n, _ in rows]) if workload == "step" else [workload] * len(rows)
                sel = [(n, v) for (n, v), lg in zip(rows, legs) if lg == leg_name]
                n_calls = sum(1 for n, _ in sel if CALL_FIRST[call] in n)
                if n_calls == 0:
                    break
                kib = sum(v for n, v in sel if any(k in n for k in kernels))
                tot[key] = kib * 1024.0 * fac / n_calls
            if len(tot) == 2:
                res[call] = {"fetch_bytes": round(tot["fetch"]), "write_bytes": round(tot["write"]),
                             "bytes": round(tot["fetch"] + tot["write"])}
        t["workloads"][leg_name] = res
    kres = {}
    for kname in TRAFFIC_KERNELS:
        rec = {}
        for key, (rows, fac) in runs.items():
            vals = [v for n, v in rows if kname in n and "merge" not in n]
            if vals:
                rec[key] = float(np.mean(vals)) * 1024.0 * fac
        if len(rec) == 2:
            kres[kname] = {"fetch_bytes_per_launch": round(rec["fetch"]), "write_bytes_per_launch": round(rec["write"]),
                           "bytes_per_launch": round(rec["fetch"] + rec["write"])}
    t.setdefault("kernels", {})[workload] = kres
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(t, fh, indent=1)
    print(json.dumps(t))


def _short(name, width=66):
    return name if len(name) <= width else name[:width - 3] + "..."


def summarize_stats(stats_csv):
    """Print the kernel-statistics table of a rocprofv3 --stats run (its
    kernel_stats.csv), and the launch-weighted mean of the KV-outer kernel's
    instances (the per-launch figure of the step's roofline)."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    print(f"{'kernel':66s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'total_ms':>10s} {'pct':>6s}")
    for r in rows:
        if float(r["Percentage"]) < 0.005:
            continue
        print(f"{_short(r['Name']):66s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
              f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
              f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}")
    kp = [(int(r["Calls"]), float(r["AverageNs"]) / 1e3) for r in rows if "kp_kernel" in r["Name"]]
    if kp:
        n = sum(c for c, _ in kp)
        terms = " + ".join(f"{c} x {a:.2f}" for c, a in kp)
        print(f"\nkp_kernel, launch-weighted mean over its instances: ({terms}) / {n} = "
              f"{sum(c * a for c, a in kp) / n:.1f} us")


def summarize_counters(sq_csv, tcc_csv):
    """Print per-kernel averages of the SQ and TCC counter runs (rocprofv3
    --pmc counter_collection.csv files): matrix-core busy share, VALU
    instructions per MFMA instruction and L2 hit rate."""
    import csv
    import collections
    import re

    def load(path):
        d = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            did = int(r["Dispatch_Id"])
            d[did][r["Counter_Name"]] += float(r["Counter_Value"])
            names[did] = r["Kernel_Name"]
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for did, c in d.items():
            m = re.search(r"(k[a-z_]+_kernel)", names[did])
            for cn, v in c.items():
                agg[m.group(1) if m else names[did]][cn].append(v)
        return agg

    sq, tcc = load(sq_csv), load(tcc_csv)
    mean = lambda xs: sum(xs) / len(xs) if xs else 0.0  # noqa: E731
    print(f"{'kernel':26s} {'launches':>8s} {'mfma_busy':>9s} {'valu/mfma':>9s} {'valu_insts':>11s} {'mfma_insts':>11s} "
          f"{'lds_insts':>10s} {'waves':>7s} {'gui_cycles':>11s} {'l2_hit':>7s}")
    order = ["ki_prefill_kernel", "ki_merge_kernel", "ks_count_lds_kernel", "ks_scatter_lds_kernel", "ks_items_kernel",
             "kp_kernel", "km_kernel", "ki_decode_scan_kernel", "ki_decode_select_kernel", "kd_kernel",
             "kd_merge_kernel"]
    for k in order:
        a = sq.get(k)
        if not a:
            continue
        gui = mean(a["GRBM_GUI_ACTIVE"])
        busy = mean(a["SQ_VALU_MFMA_BUSY_CYCLES"]) / (gui / 8 * 1024) if gui else 0.0  # 8 XCDs, 1024 SIMDs
        valu, mfma = mean(a["SQ_INSTS_VALU"]), mean(a["SQ_INSTS_MFMA"])
        ratio = f"{valu / mfma:9.2f}" if mfma else f"{'-':>9s}"
        h, m = mean(tcc[k]["TCC_HIT_sum"]), mean(tcc[k]["TCC_MISS_sum"])
        print(f"{k:26s} {len(a['GRBM_GUI_ACTIVE']):8d} {busy:9.3f} {ratio} {valu:11.4g} {mfma:11.4g} "
              f"{mean(a['SQ_INSTS_LDS']):10.4g} {mean(a['SQ_WAVES']):7.0f} {gui:11.4g} {h / (h + m) if h + m else 0:7.3f}")


def traffic_table():
    """Print the per-call and per-kernel tables of profiles/traffic.json."""
    with open(TRAFFIC_JSON) as fh:
        t = json.load(fh)
    print(f"{'leg':16s} {'call':16s} {'fetch_GB':>10s} {'write_GB':>10s} {'total_GB':>10s}")
    for leg, calls in t["workloads"].items():
        for c, r in calls.items():
            print(f"{leg:16s} {c:16s} {r['fetch_bytes'] / 1e9:10.3f} {r['write_bytes'] / 1e9:10.3f} {r['bytes'] / 1e9:10.3f}")
    for w, ks in t.get("kernels", {}).items():
        print(f"\n{'kernel (' + w + ')':26s} {'fetch_MB':>10s} {'write_MB':>10s} {'total_MB':>10s}")
        for k, r in ks.items():
            print(f"{k:26s} {r['fetch_bytes_per_launch'] / 1e6:10.1f} {r['write_bytes_per_launch'] / 1e6:10.1f} "
                  f"{r['bytes_per_launch'] / 1e6:10.1f}")


def bench_copy(args):
    """A plain device-to-device copy of COPY_BYTES (counter calibration)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(max(1, args.steps)):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(1, args.steps)
    # a read-only stream of 4 GiB (torch's sum), for the achievable read rate
    big = torch.ones(4 * COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    big.sum()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(max(1, args.steps)):
        big.sum(dtype=torch.float32)
    e1.record()
    torch.cuda.synchronize()
    rms = e0.elapsed_time(e1) / max(1, args.steps)
    print(json.dumps({"workload": "copy", "bytes": COPY_BYTES, "ms": round(ms, 4),
                      "read_plus_write_GBs": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1),
                      "read_only_bytes": 4 * COPY_BYTES, "read_only_ms": round(rms, 4),
                      "read_only_GBs": round(4 * COPY_BYTES / (rms * 1e-3) / 1e9, 1)}))


def bench_peak(msa, args):
    """Achievable peaks next to the published ones: a dense bf16 MFMA loop
    (msa_probe_mfma on 4 workgroups of 4 waves per CU) and the copy above."""
    n_wg, iters = 4 * 256, 4000
    out = torch.empty(n_wg, dtype=torch.float32, device="cuda")
    msa.probe_mfma(n_wg, 100, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(max(3, args.steps)):
        e0.record()
        msa.probe_mfma(n_wg, iters, out)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts)[len(ts) // 2]
    fl = n_wg * 4.0 * iters * 8 * 32768
    tf = fl / (ms * 1e-3) / 1e12
    print(json.dumps({"workload": "peak", "mfma_bf16_tflops": round(tf, 1), "mfma_spec_tflops": PEAK_BF16_TFLOPS,
                      "mfma_frac_of_spec": round(tf / PEAK_BF16_TFLOPS, 4), "mfma_ms": round(ms, 4)}))
    bench_copy(args)


def kernel_roofline(kern, main_flops, call_rl, workload="step"):
    """Roofline of the dominant kernel, kp_kernel (the KV-outer pass of
    msa_sparse_prefill, which does all of the main branch's MFMA work):
    achieved = the main branch's algorithmic FLOPs per step / launches per step
    (FLOPs per launch) / the kernel's mean launch time, both from HIP events
    recorded around each launch on its stream.  ``call`` repeats the figure for
    the whole msa_sparse_prefill call (schedule, KV-outer pass and merge)."""
    k = kern.get("kp_kernel")
    if not k:
        return dict(call_rl, name="msa_sparse_prefill")
    per_launch = main_flops / k["launches_per_step"]
    achieved = per_launch / (k["avg_launch_ms"] * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": kernel_traffic(workload, "kp_kernel"),
            "name": "kp_kernel", "avg_launch_ms": k["avg_launch_ms"], "launches_per_step": k["launches_per_step"],
            "flops_per_launch": per_launch,
            "call": {"name": "msa_sparse_prefill", "achieved": call_rl["achieved"], "frac": call_rl["frac"]}}


# ------------------------------------------------------------ CPU baseline

def host_info():
    """CPU model, logical CPUs and the BLAS threads the oracle runs with."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas_threads": int(threads)}


def _time_rows(fn, rows, budget_s):
    """Run fn(row) over rows until budget_s has passed (at least 4 rows); returns (rows done, seconds)."""
    t0 = time.perf_counter()
    done = 0
    for i in rows:
        fn(int(i))
        done += 1
        if time.perf_counter() - t0 > budget_s and done >= 4:
            break
    return done, time.perf_counter() - t0


def cpu_baseline_prefill(inp, shape, budget_s=12.0, seed=0):
    """Time the float64 oracle on sampled query rows of one contiguous prefill input."""
    from oracle import msa_oracle as orc
    q_idx = inp["q_idx"].double().cpu().numpy()
    k_idx = inp["k_idx"].double().cpu().numpy()
    k = inp["k"].double().cpu().numpy()
    v = inp["v"].double().cpu().numpy()
    q = inp["q"]
    n = q.shape[0]

    def row(i):
        ids, _, _ = orc.index_topk(q_idx[i:i + 1], k_idx, i, shape.top_k)
        orc.sparse_attention(q[i:i + 1].double().cpu().numpy(), k, v, ids, i)

    done, dt = _time_rows(row, np.random.default_rng(seed).permutation(n), budget_s)
    return done, dt


def cpu_baseline_chunk_1m(lc, shape, budget_s=8.0, seed=0):
    """Time the float64 oracle on sampled query rows of the 1M-context chunk.
    The oracle's index branch reads the whole contiguous index-key sequence
    (gathered from the pages once, outside the timing).  Its main branch reads
    only the selected blocks, so each row is handed the selected blocks of its
    four groups packed in ascending order (block ids renumbered to that packed
    sequence, which keeps them ascending and the diagonal block last)."""
    from oracle import msa_oracle as orc
    n_ctx, q_start = lc["n_ctx"], lc["q_start"]
    pt = lc["page_table"][0]
    nb = -(-n_ctx // BLOCK)
    k_idx = lc["k_idx_pages"][pt[:nb].long()].reshape(nb * BLOCK, -1)[:n_ctx].double().cpu().numpy()
    q_idx = lc["chunk_q_idx"].double().cpu().numpy()
    nq = q_idx.shape[0]

    def row(i):
        ids, _, _ = orc.index_topk(q_idx, k_idx, q_start, shape.top_k, rows=[i])
        p = q_start + i
        blocks = sorted(set(int(b) for b in ids[0].ravel() if b >= 0))
        pages = pt[torch.tensor(blocks, device=pt.device)].long()
        kk = lc["k_pages"][pages].transpose(1, 2).reshape(len(blocks) * BLOCK, shape.h_kv, shape.d_h)
        vv = lc["v_pages"][pages].transpose(1, 2).reshape(len(blocks) * BLOCK, shape.h_kv, shape.d_h)
        pos = {b: j for j, b in enumerate(blocks)}
        ids_c = np.where(ids >= 0, np.vectorize(lambda b: pos.get(int(b), -1))(ids), -1)
        p_c = pos[p // BLOCK] * BLOCK + p % BLOCK
        orc.sparse_attention(lc["chunk_q"][i:i + 1].double().cpu().numpy(), kk.double().cpu().numpy(),
                             vv.double().cpu().numpy(), ids_c, p_c)

    return _time_rows(row, np.random.default_rng(seed).permutation(nq), budget_s)


def cpu_baseline_decode(dec, shape, n_seqs=2):
    from oracle import msa_oracle as orc
    t_total = 0.0
    pt = dec["page_table"]
    for s in range(n_seqs):
        L = int(dec["seq_lens"][s])
        nb = -(-L // BLOCK)
        pages = pt[s, :nb].long()
        kp = dec["k_pages"][pages].double().cpu().numpy()
        vp = dec["v_pages"][pages].double().cpu().numpy()
        ip = dec["k_idx_pages"][pages].double().cpu().numpy()
        local_pt = np.arange(nb)[None, :]
        qi = dec["q_idx"][0, s:s + 1].double().cpu().numpy()
        q = dec["q"][0, s:s + 1].double().cpu().numpy()
        t0 = time.perf_counter()
        ids, _, _ = orc.index_topk_decode(qi, ip, local_pt, [L], shape.top_k)
        orc.sparse_decode(q, kp, vp, local_pt, [L], ids)
        t_total += time.perf_counter() - t0
    per_seq = t_total / n_seqs
    return {"us_per_step_extrapolated": round(per_seq * dec["q"].shape[1] * 1e6, 1),
            "sample": f"{n_seqs} of {dec['q'].shape[1]} sequences, {t_total:.1f} s, extrapolated per sequence"}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="step", choices=["step", "step32k", "prefill128k", "long1m", "decode_fp8",
                                                             "backward32k", "project", "copy", "peak"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the per-kernel event timing pass (ABI-call events only)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                             "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json for --workload from rocprofv3 counter CSVs (no GPU)")
    ap.add_argument("--traffic-table", action="store_true", help="print the tables of profiles/traffic.json (no GPU)")
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV",
                    help="print the kernel table of a rocprofv3 --stats run (no GPU)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("SQ_CSV", "TCC_CSV"),
                    help="print per-kernel averages of the SQ and TCC counter runs (no GPU)")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(args.workload, *args.summarize_traffic)
        return
    if args.traffic_table:
        traffic_table()
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the library has no "
              "multi-GPU path (it would shard by KV group, decode batch or KV-block range).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from block_sparse_attention_branch_amd import msa
    msa.lib()
    if args.workload == "copy":
        bench_copy(args)
    elif args.workload == "peak":
        bench_peak(msa, args)
    elif args.workload == "step":
        bench_step(msa, args)
    elif args.workload == "step32k":
        bench_step32k(msa, args)
    elif args.workload == "decode_fp8":
        bench_decode_fp8(msa, args)
    elif args.workload == "prefill128k":
        bench_prefill_only(msa, args, planted=True)
    elif args.workload == "backward32k":
        bench_backward(msa, args)
    elif args.workload == "project":
        bench_project(msa, args)
    else:
        bench_long(msa, args)


def bench_step(msa, args):
    """The default step: every hot-path call at 128K and 1M context.

    Legs of a timed step, in launch order:
      prefill128k    planted 131072-token causal prefill (contiguous cache):
                     msa_index_topk + msa_sparse_prefill over all queries;
      prefill1m      chunked prefill of the last 8192 queries of a 1,048,576-token
                     paged cache: msa_index_topk + msa_sparse_prefill;
      decode64x128k  one decode step of 64 sequences x 131072 tokens, paged,
                     4 rotating query sets: msa_index_topk + msa_sparse_decode.
    After the timed steps, a latency probe:
      decode1m       256 decode steps of the 1M sequence (batch 1) per timed
                     step, each after appending its token to the caches; every
                     step is launched on an idle GPU and timed on its own
                     (p50 / p99), then 256 replays of the step from a HIP graph.
    The probe runs outside the timed steps because its idle gaps let the GPU
    clock down, which would slow the prefill launched after it.
    ``value`` = prefill tokens of the step / the GPU time of the four prefill
    calls (HIP events on the launch stream)."""
    dev = "cuda"
    shape = MODEL_SHAPE
    B, L_dec = 64, 131072
    t_gen = time.perf_counter()
    big = gen_planted_prefill(131072, shape, device=dev)
    lc = gen_long_context(device=dev)
    dec = gen_decode_paged(B, L_dec, shape, seed=3, device=dev, n_query_sets=4)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    s_idx = msa.make_shape(shape.h_q, shape.h_kv, shape.d_h, shape.d_idx, shape.top_k, msa.MSA_BF16)

    def wsz(op, **kw):
        return torch.empty(max(1, msa.workspace_size(op, s_idx, **kw)), dtype=torch.uint8, device=dev)

    # leg prefill128k
    n_a = big["q"].shape[0]
    bidx_a = torch.empty((n_a, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev)
    o_a = torch.empty_like(big["q"])
    ws_ia, ws_pa = wsz(msa.OP_INDEX, n_q=n_a, n_kv=n_a), wsz(msa.OP_PREFILL, n_q=n_a, n_kv=n_a)
    # leg prefill1m
    n_ctx, q_start = lc["n_ctx"], lc["q_start"]
    n_b = lc["chunk_q"].shape[0]
    pt_l = lc["page_table"]
    bidx_b = torch.empty((n_b, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev)
    o_b = torch.empty_like(lc["chunk_q"])
    ws_ib = wsz(msa.OP_INDEX, n_q=n_b, q_start=q_start, n_kv=n_ctx)
    ws_pb = wsz(msa.OP_PREFILL, n_q=n_b, q_start=q_start, n_kv=n_ctx)
    # leg decode64x128k
    mp_c = dec["page_table"].shape[1]
    bidx_c = [torch.empty((B, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev) for _ in range(4)]
    o_c = torch.empty((B, shape.h_q, shape.d_h), dtype=torch.bfloat16, device=dev)
    ws_ic, ws_dc = wsz(msa.OP_INDEX_DECODE, batch=B, n_q=1, max_pages=mp_c), wsz(msa.OP_DECODE, batch=B, n_q=1)
    qsets = [dec["q"][i].contiguous() for i in range(4)]
    qisets = [dec["q_idx"][i].contiguous() for i in range(4)]
    # leg decode1m
    n_dec = lc["step_q"].shape[0]
    sl_d = torch.tensor([n_ctx], dtype=torch.int32, device=dev)
    bidx_d = torch.empty((1, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev)
    o_d = torch.empty((1, shape.h_q, shape.d_h), dtype=torch.bfloat16, device=dev)
    ws_id = wsz(msa.OP_INDEX_DECODE, batch=1, n_q=1, max_pages=pt_l.shape[1])
    ws_dd = wsz(msa.OP_DECODE, batch=1, n_q=1)
    app_page = [int(pt_l[0, (n_ctx + t) // BLOCK]) for t in range(n_dec)]

    prefill_calls = [
        lambda: msa.index_topk(big["q_idx"], big["k_idx"], top_k=16, out=bidx_a, workspace=ws_ia),
        lambda: msa.sparse_prefill(big["q"], big["k"], big["v"], bidx_a, out=o_a, workspace=ws_pa),
        lambda: msa.index_topk(lc["chunk_q_idx"], lc["k_idx_pages"], top_k=16, q_start=q_start, page_table=pt_l[0],
                               n_kv=n_ctx, out=bidx_b, workspace=ws_ib),
        lambda: msa.sparse_prefill(lc["chunk_q"], lc["k_pages"], lc["v_pages"], bidx_b, q_start=q_start,
                                   page_table=pt_l[0], n_kv=n_ctx, out=o_b, workspace=ws_pb),
    ]

    def decode_c(j):
        return [lambda: msa.index_topk(qisets[j], dec["k_idx_pages"], top_k=16, page_table=dec["page_table"],
                                       seq_lens=dec["seq_lens"], out=bidx_c[j], workspace=ws_ic),
                lambda: msa.sparse_decode(qsets[j], dec["k_pages"], dec["v_pages"], dec["page_table"],
                                          dec["seq_lens"], bidx_c[j], out=o_c, workspace=ws_dc)]

    def append(t):
        # the new token's K, V and index key go into the cache before its step
        pg, row = app_page[t], (n_ctx + t) % BLOCK
        lc["k_pages"][pg, :, row] = lc["step_k"][t]
        lc["v_pages"][pg, :, row] = lc["step_v"][t]
        lc["k_idx_pages"][pg, row] = lc["step_k_idx"][t]
        sl_d.fill_(n_ctx + t + 1)

    def decode_1m(t):
        return [lambda: msa.index_topk(lc["step_q_idx"][t], lc["k_idx_pages"], top_k=16, page_table=pt_l,
                                       seq_lens=sl_d, out=bidx_d, workspace=ws_id),
                lambda: msa.sparse_decode(lc["step_q"][t], lc["k_pages"], lc["v_pages"], pt_l, sl_d, bidx_d,
                                          out=o_d, workspace=ws_dd)]

    names = ["prefill128k_index", "prefill128k_sparse", "prefill1m_index", "prefill1m_sparse",
             "decode64x128k_index", "decode64x128k_sparse"]
    timer = CallTimer(names)
    d1m = CallTimer(["decode1m_index", "decode1m_sparse"])

    def run_step(s, timed):
        calls = prefill_calls + decode_c(s % 4)
        return timer.step(calls) if timed else [f() for f in calls]

    for w in range(args.warmup):
        run_step(w, False)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for s in range(args.steps):
        evs.append(run_step(s, True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect(evs)
    print(f"[bench] {args.steps} steps in {wall:.3f}s", file=sys.stderr, flush=True)
    # Kernel timing: steps again with every launch of the hot kernels bracketed
    # by HIP events on its stream (after the timed region: the extra events add
    # gaps between launches that would inflate the call times).
    kern = {}
    if not args.no_kernel_timing:
        reps = min(args.steps, 5)
        for k in TRAFFIC_KERNELS:
            msa.profile_read(k)
        msa.profile_enable(True)
        for s in range(reps):
            run_step(s, False)
        torch.cuda.synchronize()
        msa.profile_enable(False)
        for k in TRAFFIC_KERNELS:
            tot, cnt = msa.profile_read(k)
            if cnt:
                kern[k] = {"launches_per_step": cnt / reps, "avg_launch_ms": round(tot / cnt, 5),
                           "ms_per_step": round(tot / reps, 4)}
    # latency probe: the 1M decode steps, each launched on an idle GPU
    for t in range(16):
        append(t)
        for f in decode_1m(t):
            f()
    evds = []
    for s in range(args.steps):
        for t in range(n_dec):
            append(t)
            torch.cuda.synchronize()
            evds.append(d1m.step(decode_1m(t)))
    d1m.collect(evds)
    print(f"[bench] {len(evds)} decode steps at 1M timed", file=sys.stderr, flush=True)
    # the same steps replayed from a captured HIP graph (new queries and the
    # sequence length written into the captured buffers before each replay)
    qb, qib = lc["step_q"][0].clone(), lc["step_q_idx"][0].clone()

    def dstep():
        msa.index_topk(qib, lc["k_idx_pages"], top_k=16, page_table=pt_l, seq_lens=sl_d, out=bidx_d, workspace=ws_id)
        msa.sparse_decode(qb, lc["k_pages"], lc["v_pages"], pt_l, sl_d, bidx_d, out=o_d, workspace=ws_dd)

    sl_d.fill_(n_ctx + 1)
    dstep()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dstep()
    torch.cuda.synchronize()
    graph_ms = []
    for t in range(n_dec):
        qb.copy_(lc["step_q"][t])
        qib.copy_(lc["step_q_idx"][t])
        sl_d.fill_(n_ctx + t + 1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms.append(e0.elapsed_time(e1))
    graph_us = np.array(graph_ms) * 1e3
    del graph

    t = {n: timer.mean_ms(n) for n in names}
    dstep_us = (np.array(d1m.records["decode1m_index"]) + np.array(d1m.records["decode1m_sparse"])) * 1e3
    t1m_i, t1m_s = d1m.mean_ms("decode1m_index"), d1m.mean_ms("decode1m_sparse")
    prefill_ms = t["prefill128k_index"] + t["prefill128k_sparse"] + t["prefill1m_index"] + t["prefill1m_sparse"]
    fa = prefill_counts(n_a, 0, shape)
    fb = prefill_counts(n_b, q_start, shape)
    dc = decode_bytes([L_dec] * B, shape)
    dd = decode_bytes([n_ctx + n_dec // 2], shape)  # mid-run length of the 1M decode steps
    kd = {"prefill128k": ("ki_prefill_kernel+ki_merge_kernel", "ks_* schedule + kp_kernel + km_kernel"),
          "prefill1m": ("ki_prefill_kernel+ki_merge_kernel", "ks_* schedule + kp_kernel + km_kernel"),
          "decode64x128k": ("ki_decode_scan_kernel+ki_decode_select_kernel", "kd_kernel(+kd_merge_kernel)"),
          "decode1m": ("ki_decode_scan_kernel+ki_decode_select_kernel", "kd_kernel+kd_merge_kernel")}
    rl = {}
    for leg, (bound, unit, wi, ws, ti, ts, recs) in {
            "prefill128k": ("mfma", "TFLOP/s", fa[0], fa[1], "prefill128k_index", "prefill128k_sparse", timer),
            "prefill1m": ("mfma", "TFLOP/s", fb[0], fb[1], "prefill1m_index", "prefill1m_sparse", timer),
            "decode64x128k": ("hbm", "GB/s", dc[0], dc[1], "decode64x128k_index", "decode64x128k_sparse", timer),
            "decode1m": ("hbm", "GB/s", dd[0], dd[1], "decode1m_index", "decode1m_sparse", d1m)}.items():
        for call, work, nm, kn in (("index", wi, ti, kd[leg][0]), ("sparse", ws, ts, kd[leg][1])):
            ms_ = recs.mean_ms(nm)
            abi = ("index_prefill" if leg.startswith("prefill") else "index_decode") if call == "index" else \
                ("sparse_prefill" if leg.startswith("prefill") else "sparse_decode")
            rl[f"{leg}_{call}"] = dict(roofline(bound, work, ms_, unit, abi, leg), kernel=kn, ms=round(ms_, 4),
                                       p10_ms=round(recs.pct(nm, 10), 4), p90_ms=round(recs.pct(nm, 90), 4))
    legs = {
        "prefill128k": {"tokens": n_a, "ms": round(t["prefill128k_index"] + t["prefill128k_sparse"], 4),
                        "tokens_per_s": round(n_a / ((t["prefill128k_index"] + t["prefill128k_sparse"]) * 1e-3), 1)},
        "prefill1m": {"tokens": n_b, "ctx": n_ctx, "ms": round(t["prefill1m_index"] + t["prefill1m_sparse"], 4),
                      "tokens_per_s": round(n_b / ((t["prefill1m_index"] + t["prefill1m_sparse"]) * 1e-3), 1)},
        "decode64x128k": {"us_per_step": round((t["decode64x128k_index"] + t["decode64x128k_sparse"]) * 1e3, 2)},
        "decode1m": {"us_p50": round(float(np.percentile(dstep_us, 50)), 1),
                     "us_p99": round(float(np.percentile(dstep_us, 99)), 1),
                     "us_mean": round(float(dstep_us.mean()), 1), "steps_timed": int(dstep_us.size),
                     "graph_us_p50": round(float(np.percentile(graph_us, 50)), 1),
                     "graph_us_p99": round(float(np.percentile(graph_us, 99)), 1)},
    }
    # retrieval check of the planted workload (a property of the output, not timed)
    got = bidx_a.cpu()
    des = big["designated"]
    legs["prefill128k"]["planted_blocks_retrieved"] = bool(all(
        set(big["planted_blocks"][r].tolist()) <= set(got[int(i), r].tolist())
        for i in des[:256] for r in range(shape.h_kv)))

    dense = None
    if not args.no_dense:
        od = torch.empty_like(big["q"])
        msa.dense_prefill(big["q"], big["k"], big["v"], out=od)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        msa.dense_prefill(big["q"], big["k"], big["v"], out=od)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1)
        ta = t["prefill128k_index"] + t["prefill128k_sparse"]
        dense = {"workload": "prefill 1x131072", "ms": round(dms, 3), "tflops": round(fa[2] / (dms * 1e-3) / 1e12, 1),
                 "speedup_msa_prefill_vs_dense": round(dms / ta, 2), "kernel": "kg_kernel (Q-outer, Eq. (1))"}
        del od

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host ...", file=sys.stderr, flush=True)
        na_done, na_s = cpu_baseline_prefill(big, shape, budget_s=10.0)
        nb_done, nb_s = cpu_baseline_chunk_1m(lc, shape, budget_s=8.0)
        sec_a, sec_b = na_s / na_done, nb_s / nb_done
        hi = host_info()
        cpu = {"value": round((n_a + n_b) / (n_a * sec_a + n_b * sec_b), 3), "unit": "tokens/s",
               "cores": hi["blas_threads"], "kind": "oracle",
               "sample": f"{na_done} random query rows of the 131072-token planted prefill ({na_s:.1f} s) and "
                         f"{nb_done} random rows of the 8192-query chunk at 1M context ({nb_s:.1f} s), each row "
                         f"the index top-k and sparse attention of all 4 groups / 64 heads; per-row times scaled to "
                         f"the step's {n_a} + {n_b} prefill tokens",
               "host": hi, "decode": cpu_baseline_decode(dec, shape)}

    main_fl = fa[1] + fb[1]
    line = {
        "metric": "MSA prefill tok/s + decode us/step at 128K/1M ctx; % MFMA / HBM roofline",
        "value": round((n_a + n_b) / (prefill_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic, seeded (planted-needle index keys at 128K, N(0,1) elsewhere); no weights",
        "config": {"workload": "step = prefill 1x131072 planted (whole causal prefill) + prefill chunk of the "
                               "last 8192 queries at 1048576 ctx (paged) + decode step 64x131072 paged; after the "
                               "timed steps, 256 decode steps (batch 1) at 1048576 ctx per step, each launched on "
                               "an idle GPU; 64 q / 4 kv heads, d_h 128, d_idx 64, B_k 128, k 16, diagonal block "
                               "kept",
                   "prefill_tokens_per_step": n_a + n_b, "seq_len": n_a, "long_ctx": n_ctx, "decode_batch": B,
                   "decode_ctx": L_dec, "long_decode_steps": n_dec, "parallelism": "single GPU"},
        "prefill_ms": round(prefill_ms, 4),
        "decode_us_per_step": legs["decode64x128k"]["us_per_step"],
        "decode_1m_us_p50": legs["decode1m"]["us_p50"],
        "decode_1m_us_p99": legs["decode1m"]["us_p99"],
        "legs": legs,
        "roofline": kernel_roofline(kern, main_fl, roofline("mfma", main_fl, t["prefill128k_sparse"]
                                                             + t["prefill1m_sparse"], "TFLOP/s"), "step"),
        "rooflines": rl,
        "kernels": kern,
        "dense_gqa": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def bench_step32k(msa, args):
    """The 32K prefill + 64 x 128K decode step (the smaller prefill configuration)."""
    dev = "cuda"
    shape = MODEL_SHAPE
    n = 32768
    t_gen = time.perf_counter()
    pre = gen_prefill(n, shape, dtype=torch.bfloat16, seed=1, device=dev)
    dec = gen_decode_paged(64, 131072, shape, seed=3, device=dev, n_query_sets=4)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    # outputs and workspaces allocated once, outside the timed region
    bidx = torch.empty((n, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev)
    o = torch.empty_like(pre["q"])
    s_idx = msa.make_shape(shape.h_q, shape.h_kv, shape.d_h, shape.d_idx, shape.top_k, msa.MSA_BF16)
    ws_idx = torch.empty(max(1, msa.workspace_size(msa.OP_INDEX, s_idx, n_q=n, n_kv=n)), dtype=torch.uint8, device=dev)
    ws_pre = torch.empty(max(1, msa.workspace_size(msa.OP_PREFILL, s_idx, n_q=n, n_kv=n)), dtype=torch.uint8, device=dev)
    B = 64
    mp = dec["page_table"].shape[1]
    dbidx = [torch.empty((B, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev) for _ in range(4)]
    do = torch.empty((B, shape.h_q, shape.d_h), dtype=torch.bfloat16, device=dev)
    ws_di = torch.empty(max(1, msa.workspace_size(msa.OP_INDEX_DECODE, s_idx, batch=B, n_q=1, max_pages=mp)),
                        dtype=torch.uint8, device=dev)
    ws_dd = torch.empty(max(1, msa.workspace_size(msa.OP_DECODE, s_idx, batch=B, n_q=1)), dtype=torch.uint8, device=dev)
    qsets = [dec["q"][i].contiguous() for i in range(4)]
    qisets = [dec["q_idx"][i].contiguous() for i in range(4)]

    def calls(step):
        j = step % 4
        return [
            lambda: msa.index_topk(pre["q_idx"], pre["k_idx"], top_k=16, out=bidx, workspace=ws_idx),
            lambda: msa.sparse_prefill(pre["q"], pre["k"], pre["v"], bidx, out=o, workspace=ws_pre),
            lambda: msa.index_topk(qisets[j], dec["k_idx_pages"], top_k=16, page_table=dec["page_table"],
                                   seq_lens=dec["seq_lens"], out=dbidx[j], workspace=ws_di),
            lambda: msa.sparse_decode(qsets[j], dec["k_pages"], dec["v_pages"], dec["page_table"],
                                      dec["seq_lens"], dbidx[j], out=do, workspace=ws_dd),
        ]

    names = ["index_prefill", "sparse_prefill", "index_decode", "sparse_decode"]
    timer = CallTimer(names)
    for w in range(args.warmup):
        for fn in calls(w):
            fn()
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for s in range(args.steps):
        evs.append(timer.step(calls(s)))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect(evs)
    print(f"[bench] {args.steps} steps in {wall:.3f}s", file=sys.stderr, flush=True)
    # Kernel timing: the same steps again, with every launch of the hot kernels
    # bracketed by HIP events on its stream.  Run after the timed region above
    # because the extra events add gaps between launches (they would inflate
    # the call times that `value` is computed from).
    kern = {}
    if not args.no_kernel_timing:
        kern_names = ("ki_prefill_kernel", "kp_kernel", "km_kernel", "ki_decode_scan_kernel", "kd_kernel")
        for k in kern_names:
            msa.profile_read(k)
        msa.profile_enable(True)
        for s in range(args.steps):
            for fn in calls(s):
                fn()
        torch.cuda.synchronize()
        msa.profile_enable(False)
        for k in kern_names:
            tot, cnt = msa.profile_read(k)
            if cnt:
                kern[k] = {"launches_per_step": cnt / args.steps, "avg_launch_ms": round(tot / cnt, 5),
                           "ms_per_step": round(tot / args.steps, 4)}

    ms_step = wall * 1e3 / args.steps
    t_ip, t_sp = timer.mean_ms("index_prefill"), timer.mean_ms("sparse_prefill")
    t_id, t_sd = timer.mean_ms("index_decode"), timer.mean_ms("sparse_decode")
    prefill_ms = t_ip + t_sp
    idx_fl, main_fl, dense_fl = prefill_counts(n, 0, shape)
    didx_b, dmain_b, ddense_b = decode_bytes([131072] * B, shape)
    rl = {
        "index_prefill": dict(roofline("mfma", idx_fl, t_ip, "TFLOP/s", "index_prefill", "step32k"),
                              kernel="ki_prefill_kernel+ki_merge_kernel"),
        "sparse_prefill": dict(roofline("mfma", main_fl, t_sp, "TFLOP/s", "sparse_prefill", "step32k"),
                               kernel="ks_* schedule + kp_kernel + km_kernel (per window)"),
        "index_decode": dict(roofline("hbm", didx_b, t_id, "GB/s", "index_decode", "step32k"),
                             kernel="ki_decode_scan_kernel+ki_decode_select_kernel"),
        "sparse_decode": dict(roofline("hbm", dmain_b, t_sd, "GB/s", "sparse_decode", "step32k"),
                              kernel="kd_kernel+kd_merge_kernel"),
    }
    for k_, ms_ in (("index_prefill", t_ip), ("sparse_prefill", t_sp), ("index_decode", t_id), ("sparse_decode", t_sd)):
        rl[k_]["ms"] = round(ms_, 4)
        rl[k_]["p10_ms"] = round(timer.pct(k_, 10), 4)
        rl[k_]["p90_ms"] = round(timer.pct(k_, 90), 4)

    dense = None
    if not args.no_dense:
        od = torch.empty_like(pre["q"])
        msa.dense_prefill(pre["q"], pre["k"], pre["v"], out=od)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        reps = 3
        for _ in range(reps):
            msa.dense_prefill(pre["q"], pre["k"], pre["v"], out=od)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / reps
        dense = {"ms": round(dms, 3), "tflops": round(dense_fl / (dms * 1e-3) / 1e12, 1),
                 "speedup_msa_prefill_vs_dense": round(dms / prefill_ms, 2),
                 "kernel": "kg_kernel (Q-outer, Eq. (1))"}
        del od

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host ...", file=sys.stderr, flush=True)
        done, dt = cpu_baseline_prefill(pre, shape)
        hi = host_info()
        cpu = {"value": round(done / dt, 3), "unit": "tokens/s", "cores": hi["blas_threads"], "kind": "oracle",
               "sample": f"{done} random query rows of the 32768-token prefill (index top-k + sparse attention, "
                         f"all 4 groups / 64 heads), {dt:.1f} s", "host": hi,
               "decode": cpu_baseline_decode(dec, shape)}

    line = {
        "metric": "MSA prefill tok/s + decode us/step (32K prefill variant); % MFMA / HBM roofline",
        "value": round(n / (prefill_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic, seeded (N(0,1)/sqrt(d) prefill, N(0,1) decode); no weights",
        "config": {"workload": "prefill 1x32768 + decode step 64x131072 paged; 64 q / 4 kv heads, d_h 128, "
                               "d_idx 64, B_k 128, k 16, causal, diagonal block kept",
                   "global_batch": 1, "seq_len": n, "decode_batch": B, "decode_ctx": 131072,
                   "parallelism": "single GPU"},
        "prefill_ms": round(prefill_ms, 4),
        "decode_us_per_step": round((t_id + t_sd) * 1e3, 2),
        "roofline": kernel_roofline(kern, main_fl, rl["sparse_prefill"], "step32k"),
        "rooflines": rl,
        "kernels": kern,
        "dense_gqa": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def bench_decode_fp8(msa, args):
    """The 64 x 131072 paged decode step with 8-bit K, V and K_idx caches
    (bf16 queries and outputs), 4 rotating query sets: e4m3 codes used as
    stored, then MXFP8 (the same codes with one E8M0 scale per 32 elements)."""
    res = _decode_8bit(msa, args, mx=False)
    res["mxfp8"] = _decode_8bit(msa, args, mx=True)
    res["mxfp8"].pop("workload")
    print(json.dumps(res))


def _decode_8bit(msa, args, mx):
    dev = "cuda"
    shape = MODEL_SHAPE
    B, L = 64, 131072
    dec = gen_decode_paged(B, L, shape, seed=3, device=dev, n_query_sets=4,
                           cache_dtype=MXFP8 if mx else torch.float8_e4m3fn)
    ks, vs, kis = dec.get("k_pages_scale"), dec.get("v_pages_scale"), dec.get("k_idx_pages_scale")
    s_idx = msa.make_shape(shape.h_q, shape.h_kv, shape.d_h, shape.d_idx, shape.top_k, msa.MSA_BF16,
                           cache_dtype=msa.MSA_MXFP8_E4M3 if mx else msa.MSA_FP8_E4M3)
    mp = dec["page_table"].shape[1]
    dbidx = [torch.empty((B, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev) for _ in range(4)]
    do = torch.empty((B, shape.h_q, shape.d_h), dtype=torch.bfloat16, device=dev)
    ws_di = torch.empty(max(1, msa.workspace_size(msa.OP_INDEX_DECODE, s_idx, batch=B, n_q=1, max_pages=mp)),
                        dtype=torch.uint8, device=dev)
    ws_dd = torch.empty(max(1, msa.workspace_size(msa.OP_DECODE, s_idx, batch=B, n_q=1)), dtype=torch.uint8,
                        device=dev)
    qsets = [dec["q"][i].contiguous() for i in range(4)]
    qisets = [dec["q_idx"][i].contiguous() for i in range(4)]

    def calls(j):
        return [lambda: msa.index_topk(qisets[j], dec["k_idx_pages"], top_k=16, page_table=dec["page_table"],
                                       seq_lens=dec["seq_lens"], out=dbidx[j], workspace=ws_di, k_idx_scale=kis),
                lambda: msa.sparse_decode(qsets[j], dec["k_pages"], dec["v_pages"], dec["page_table"],
                                          dec["seq_lens"], dbidx[j], out=do, workspace=ws_dd, k_scale=ks, v_scale=vs)]
    timer = CallTimer(["index_decode", "sparse_decode"])
    for w in range(args.warmup):
        for f in calls(w % 4):
            f()
    torch.cuda.synchronize()
    evs = [timer.step(calls(i % 4)) for i in range(args.steps)]
    timer.collect(evs)
    t_id, t_sd = timer.mean_ms("index_decode"), timer.mean_ms("sparse_decode")
    didx_b, dmain_b, _ = decode_bytes([L] * B, shape, cache_esz=1, mx=mx)
    del dec
    torch.cuda.empty_cache()
    return {"workload": "decode 64 x 131072 paged, e4m3 K/V/K_idx caches, bf16 queries",
            "decode_us_per_step": round((t_id + t_sd) * 1e3, 2),
            "index_us": round(t_id * 1e3, 2), "sparse_us": round(t_sd * 1e3, 2),
            "index_roofline": roofline("hbm", didx_b, t_id, "GB/s"),
            "sparse_roofline": roofline("hbm", dmain_b, t_sd, "GB/s")}


def bench_prefill_only(msa, args, planted=True):
    """Planted 131072-token prefill (index + sparse prefill)."""
    dev = "cuda"
    shape = MODEL_SHAPE
    n = 131072
    inp = gen_planted_prefill(n, shape, device=dev) if planted else gen_prefill(n, shape, device=dev)
    bidx = torch.empty((n, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev)
    o = torch.empty_like(inp["q"])
    s_idx = msa.make_shape(shape.h_q, shape.h_kv, shape.d_h, shape.d_idx, shape.top_k, msa.MSA_BF16)
    ws_idx = torch.empty(max(1, msa.workspace_size(msa.OP_INDEX, s_idx, n_q=n, n_kv=n)), dtype=torch.uint8, device=dev)
    ws_pre = torch.empty(max(1, msa.workspace_size(msa.OP_PREFILL, s_idx, n_q=n, n_kv=n)), dtype=torch.uint8, device=dev)
    fns = [lambda: msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=16, out=bidx, workspace=ws_idx),
           lambda: msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, out=o, workspace=ws_pre)]
    timer = CallTimer(["index_prefill", "sparse_prefill"])
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    evs = [timer.step(fns) for _ in range(args.steps)]
    timer.collect(evs)
    t_ip, t_sp = timer.mean_ms("index_prefill"), timer.mean_ms("sparse_prefill")
    idx_fl, main_fl, dense_fl = prefill_counts(n, 0, shape)
    dense = None
    if not args.no_dense:
        # the dense comparison kernel at the same shape, for the speedup at 128K
        od = torch.empty_like(inp["q"])
        msa.dense_prefill(inp["q"], inp["k"], inp["v"], out=od)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        msa.dense_prefill(inp["q"], inp["k"], inp["v"], out=od)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1)
        dense = {"ms": round(dms, 2), "tflops": round(dense_fl / (dms * 1e-3) / 1e12, 1),
                 "speedup_msa_prefill_vs_dense": round(dms / (t_ip + t_sp), 2)}
        del od
    got = bidx.cpu()
    des = inp["designated"]
    hit = all(set(inp["planted_blocks"][r].tolist()) <= set(got[int(i), r].tolist())
              for i in des[:256] for r in range(shape.h_kv))
    print(json.dumps({"workload": "prefill 1x131072 planted", "index_ms": round(t_ip, 3),
                      "sparse_ms": round(t_sp, 3), "tokens_per_s": round(n / ((t_ip + t_sp) * 1e-3), 1),
                      "index_roofline": roofline("mfma", idx_fl, t_ip, "TFLOP/s"),
                      "sparse_roofline": roofline("mfma", main_fl, t_sp, "TFLOP/s"),
                      "planted_blocks_retrieved": bool(hit), "dense_gqa": dense}))


def bench_backward(msa, args):
    """msa_sparse_prefill_backward at the 32K prefill shape, without and with
    the KL-alignment term.  Algorithmic work of the attention gradients: five
    d_h-wide products per (query head, visible selected key) -- S, dP, dV, dK,
    dQ -- i.e. 10 * d_h FLOPs, 2.5x the forward's main branch."""
    dev = "cuda"
    shape = MODEL_SHAPE
    n = 32768
    inp = gen_prefill(n, shape, dtype=torch.bfloat16, seed=1, device=dev)
    bidx = msa.index_topk(inp["q_idx"], inp["k_idx"], top_k=shape.top_k)
    o, lse = msa.sparse_prefill(inp["q"], inp["k"], inp["v"], bidx, with_lse=True)
    d_o = torch.randn(inp["q"].shape, generator=torch.Generator(device=dev).manual_seed(2), device=dev,
                      dtype=torch.float32).to(torch.bfloat16)
    s = msa.make_shape(shape.h_q, shape.h_kv, shape.d_h, shape.d_idx, shape.top_k, msa.MSA_BF16)
    ws = torch.empty(max(1, msa.workspace_size(msa.OP_PREFILL_BACKWARD_KL, s, n_q=n, n_kv=n)), dtype=torch.uint8,
                     device=dev)
    outs = (torch.empty_like(inp["q"]), torch.empty_like(inp["k"]), torch.empty_like(inp["v"]))
    fns = [lambda: msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], bidx, o, lse, d_o, out=outs,
                                               workspace=ws),
           lambda: msa.sparse_prefill_backward(inp["q"], inp["k"], inp["v"], bidx, o, lse, d_o, out=outs,
                                               workspace=ws, q_idx=inp["q_idx"], k_idx=inp["k_idx"],
                                               kl_scale=1.0 / (n * shape.h_kv))]
    timer = CallTimer(["backward", "backward_kl"])
    for _ in range(args.warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    evs = [timer.step(fns) for _ in range(args.steps)]
    timer.collect(evs)
    t, t_kl = timer.mean_ms("backward"), timer.mean_ms("backward_kl")
    kern = {}
    if not args.no_kernel_timing:
        reps = min(args.steps, 5)
        msa.profile_enable(True)
        for _ in range(reps):
            fns[0]()
        torch.cuda.synchronize()
        msa.profile_enable(False)
        for k_ in ("kbq_kernel", "kbkv_kernel"):
            tot, cnt = msa.profile_read(k_)
            if cnt:
                kern[k_] = {"launches_per_call": cnt / reps, "avg_launch_ms": round(tot / cnt, 5),
                            "ms_per_call": round(tot / reps, 4)}
    _, main_fl, _ = prefill_counts(n, 0, shape)
    bwd_fl = 2.5 * main_fl
    print(json.dumps({"workload": "backward 1x32768 (dq, dk, dv of the sparse prefill), 64 q / 4 kv heads, "
                                  "d_h 128, d_idx 64, k 16, bf16", "ms": round(t, 3),
                      "p10_ms": round(timer.pct("backward", 10), 3), "p90_ms": round(timer.pct("backward", 90), 3),
                      "ms_with_kl_alignment": round(t_kl, 3),
                      "tokens_per_s": round(n / (t * 1e-3), 1), "flops": bwd_fl,
                      "roofline": roofline("mfma", bwd_fl, t, "TFLOP/s"), "kernels": kern}))


def bench_project(msa, args):
    """msa_index_project (index projections + RoPE + index-key append) for a
    64-sequence decode step and a 32768-token prefill, at d_model 6144 (the
    pages give no hidden size; 6144 is an assumed width), 4 groups, d_idx 64,
    RoPE on 64 dims.  Work: 2 * d_model * (h_kv + 1) * d_idx FLOPs per token;
    bytes: the weights once plus x, q_idx and the appended keys."""
    dev = "cuda"
    dm, h_kv, di = 6144, 4, 64
    g = torch.Generator(device=dev).manual_seed(5)
    wq = (torch.randn(h_kv, di, dm, generator=g, device=dev) / dm ** 0.5).to(torch.bfloat16)
    wk = (torch.randn(di, dm, generator=g, device=dev) / dm ** 0.5).to(torch.bfloat16)
    res = {}
    for name, n in (("decode64", 64), ("prefill32k", 32768)):
        x = torch.randn(n, dm, generator=g, device=dev).to(torch.bfloat16)
        if name == "decode64":
            pos = torch.full((n,), 131071, dtype=torch.int32, device=dev)
            cache = torch.zeros(65536, 128, di, dtype=torch.bfloat16, device=dev)
            pt = torch.randperm(65536, device=dev).to(torch.int32).view(64, 1024)
            seq = torch.arange(n, dtype=torch.int32, device=dev)
            fn = [lambda: msa.index_project(x, wq, wk, pos, cache, page_table=pt, seq=seq, out=qo, workspace=ws)]
        else:
            pos = torch.arange(n, dtype=torch.int32, device=dev)
            cache = torch.zeros(n, di, dtype=torch.bfloat16, device=dev)
            fn = [lambda: msa.index_project(x, wq, wk, pos, cache, out=qo, workspace=ws)]
        qo = torch.empty(n, h_kv, di, dtype=torch.bfloat16, device=dev)
        shp = msa.make_shape(h_kv, h_kv, 128, di, 16, msa.MSA_BF16)
        ws = torch.empty(max(1, msa.workspace_size(msa.OP_INDEX_PROJECT, shp, n_q=n, n_kv=dm)), dtype=torch.uint8,
                         device=dev)
        timer = CallTimer([name])
        for _ in range(args.warmup):
            fn[0]()
        torch.cuda.synchronize()
        evs = [timer.step(fn) for _ in range(args.steps)]
        timer.collect(evs)
        t = timer.mean_ms(name)
        fl = 2.0 * n * dm * (h_kv + 1) * di
        byts = (h_kv + 1) * di * dm * 2 + n * dm * 2 + n * (h_kv + 1) * di * 2
        res[name] = {"tokens": n, "us": round(t * 1e3, 2), "tflops": round(fl / (t * 1e-3) / 1e12, 2),
                     "mfma_frac": round(fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "gbs": round(byts / (t * 1e-3) / 1e9, 1), "hbm_frac": round(byts / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    print(json.dumps({"workload": "index projections + RoPE + k_idx append, d_model 6144 (assumed), 4 groups, d_idx 64, "
                                  "RoPE 64", "results": res}))


def bench_long(msa, args):
    """1M-token paged cache: chunked prefill of the last 8192 queries, then
    256 decode steps (each appends its token first), batch 1, launched call by
    call and then replayed from a captured HIP graph."""
    dev = "cuda"
    shape = MODEL_SHAPE
    lc = gen_long_context(device=dev)
    n_ctx, q_start = lc["n_ctx"], lc["q_start"]
    nq = lc["chunk_q"].shape[0]
    pt = lc["page_table"]
    bidx = torch.empty((nq, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev)
    o = torch.empty_like(lc["chunk_q"])
    s_idx = msa.make_shape(shape.h_q, shape.h_kv, shape.d_h, shape.d_idx, shape.top_k, msa.MSA_BF16)
    ws_idx = torch.empty(max(1, msa.workspace_size(msa.OP_INDEX, s_idx, n_q=nq, q_start=q_start, n_kv=n_ctx)),
                         dtype=torch.uint8, device=dev)
    ws_pre = torch.empty(max(1, msa.workspace_size(msa.OP_PREFILL, s_idx, n_q=nq, q_start=q_start, n_kv=n_ctx)),
                         dtype=torch.uint8, device=dev)
    fns = [lambda: msa.index_topk(lc["chunk_q_idx"], lc["k_idx_pages"], top_k=16, q_start=q_start,
                                  page_table=pt[0], n_kv=n_ctx, out=bidx, workspace=ws_idx),
           lambda: msa.sparse_prefill(lc["chunk_q"], lc["k_pages"], lc["v_pages"], bidx, q_start=q_start,
                                      page_table=pt[0], n_kv=n_ctx, out=o, workspace=ws_pre)]
    timer = CallTimer(["index_prefill", "sparse_prefill"])
    for _ in range(max(1, args.warmup // 2)):
        for f in fns:
            f()
    torch.cuda.synchronize()
    evs = [timer.step(fns) for _ in range(max(3, args.steps // 2))]
    timer.collect(evs)
    t_ip, t_sp = timer.mean_ms("index_prefill"), timer.mean_ms("sparse_prefill")
    idx_fl, main_fl, _ = prefill_counts(nq, q_start, shape)
    # decode steps
    seq_lens = torch.tensor([n_ctx], dtype=torch.int32, device=dev)
    dbidx = torch.empty((1, shape.h_kv, shape.top_k), dtype=torch.int32, device=dev)
    do = torch.empty((1, shape.h_q, shape.d_h), dtype=torch.bfloat16, device=dev)
    mp = pt.shape[1]
    ws_di = torch.empty(max(1, msa.workspace_size(msa.OP_INDEX_DECODE, s_idx, batch=1, n_q=1, max_pages=mp)),
                        dtype=torch.uint8, device=dev)
    ws_dd = torch.empty(max(1, msa.workspace_size(msa.OP_DECODE, s_idx, batch=1, n_q=1)), dtype=torch.uint8, device=dev)
    n_dec = lc["step_q"].shape[0]
    step_ms = []
    for t in range(n_dec):
        pos = n_ctx + t
        page = pt[0, pos // BLOCK].long()
        row = pos % BLOCK
        lc["k_pages"][page, :, row] = lc["step_k"][t]
        lc["v_pages"][page, :, row] = lc["step_v"][t]
        lc["k_idx_pages"][page, row] = lc["step_k_idx"][t]
        seq_lens.fill_(pos + 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        msa.index_topk(lc["step_q_idx"][t], lc["k_idx_pages"], top_k=16, page_table=pt, seq_lens=seq_lens,
                       out=dbidx, workspace=ws_di)
        msa.sparse_decode(lc["step_q"][t], lc["k_pages"], lc["v_pages"], pt, seq_lens, dbidx, out=do,
                          workspace=ws_dd)
        e1.record()
        torch.cuda.synchronize()
        step_ms.append(e0.elapsed_time(e1))
    step_us = np.array(step_ms[8:]) * 1e3
    # The same steps again, the two calls captured once in a HIP graph and
    # replayed: new query rows and the sequence length are written into the
    # captured buffers before each replay, as a serving loop would do.
    qb = lc["step_q"][0].clone()
    qib = lc["step_q_idx"][0].clone()

    def dstep():
        msa.index_topk(qib, lc["k_idx_pages"], top_k=16, page_table=pt, seq_lens=seq_lens, out=dbidx,
                       workspace=ws_di)
        msa.sparse_decode(qb, lc["k_pages"], lc["v_pages"], pt, seq_lens, dbidx, out=do, workspace=ws_dd)

    seq_lens.fill_(n_ctx + 1)
    dstep()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dstep()
    torch.cuda.synchronize()
    graph_ms = []
    for t in range(n_dec):
        qb.copy_(lc["step_q"][t])
        qib.copy_(lc["step_q_idx"][t])
        seq_lens.fill_(n_ctx + t + 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms.append(e0.elapsed_time(e1))
    graph_us = np.array(graph_ms[8:]) * 1e3
    print(json.dumps({"workload": "1M context: chunked prefill 8192 @ q_start 1040384 + 256 decode steps",
                      "chunk_index_ms": round(t_ip, 3), "chunk_sparse_ms": round(t_sp, 3),
                      "chunk_tokens_per_s": round(nq / ((t_ip + t_sp) * 1e-3), 1),
                      "chunk_index_roofline": roofline("mfma", idx_fl, t_ip, "TFLOP/s"),
                      "chunk_sparse_roofline": roofline("mfma", main_fl, t_sp, "TFLOP/s"),
                      "decode_us_p50": round(float(np.percentile(step_us, 50)), 1),
                      "decode_us_p99": round(float(np.percentile(step_us, 99)), 1),
                      "decode_graph_us_p50": round(float(np.percentile(graph_us, 50)), 1),
                      "decode_graph_us_p99": round(float(np.percentile(graph_us, 99)), 1)}))


if __name__ == "__main__":
    main()
