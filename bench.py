"""Benchmark of the packed varlen causal attention hot path on one MI355X.

One step = plan the pack on the host (SH-Tiles, eq. 8 pair counts, Algorithm 2
placement onto the CUs), upload the plan, run the persistent forward kernel and
the backward (row dot D, dK/dV kernel, dQ kernel), with per-CU busy records.
The host builds each step's plan one step ahead, on a worker thread, while the
GPU runs the previous step.  Inputs (q, k, v, dout) are resident in HBM before
timing starts.  Throughput counts only unmasked causal pairs:
FLOPs_fwd = 4 d h_q sum_j l_j (l_j + 1) / 2, FLOPs_bwd = 2.5 FLOPs_fwd.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
After the train_256k step the same line reports the forward of the 1M-token head share
(L = 1048576, 8 Q / 1 KV heads, one 600000-token sample plus filler) as "fwd_share_1m".
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6       # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "packed varlen causal attn TFLOP/s (fwd, fwd+bwd), % bf16 MFMA peak, CU max/mean"
# what the device code is compiled from (package-relative), flags included
DEVICE_SOURCES = ["csrc/attn_fwd.hip", "csrc/attn_bwd.hip", "csrc/attn_bwd_dq.hip", "csrc/bwd_common.h",
                  "csrc/device_common.h", "csrc/plan_layout.h", "build.py"]
# Algorithmic FLOPs per unmasked (query, key, head) pair for each kernel:
#   forward: QK^T and PV (2 x 2d); dK/dV pass: S recompute, dP, dV, dK (4 x 2d);
#   dQ pass: dQ (2d) -- its S and dP recomputations are not algorithmic work.
KERNEL_FLOPS_PER_PAIR = {"fwd": 4, "bwd_dkdv": 8, "bwd_dq": 2}
KERNEL_SYMBOL = {"fwd": "attn_fwd_kernel", "bwd_dkdv": "attn_bwd_dkdv_kernel",
                 "bwd_dq": "attn_bwd_dq_kernel"}
PLACEMENT_NAMES = {0: "algorithm2", 1: "round_robin", 2: "algorithm2_l2"}


def source_hash() -> str:
    """Hash of the device sources with comments and blank lines removed (code changes only)."""
    import re
    h = hashlib.sha256()
    for name in DEVICE_SOURCES:
        with open(os.path.join(ROOT, "packed_varlen_attention_cu_amd", name)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        for line in text.splitlines():
            line = re.sub(r"//.*", "", line).strip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def causal_pairs(cu) -> int:
    lens = np.diff(np.asarray(cu, dtype=np.int64))
    return int((lens * (lens + 1) // 2).sum())


def cu_busy_ratio(rec_bytes, num_cus):
    import packed_varlen_attention_cu_amd as lib
    r = rec_bytes.view(lib.RECORD_DTYPE)[:num_cus]
    busy = (r["t_end"] - r["t_start"]).astype(np.float64)
    ran = r["n_items"] > 0
    if not ran.any():
        return None, None
    # key of the physical CU: XCC id, SE id, SH id, CU id
    hw = r["hw_id"].astype(np.int64)
    key = (r["xcc_id"].astype(np.int64) & 0xF) << 16 | ((hw >> 13) & 0x7) << 8 | ((hw >> 12) & 1) << 4 | ((hw >> 8) & 0xF)
    per_cu = {}
    for k_, b, ok in zip(key, busy, ran):
        if ok:
            per_cu[int(k_)] = per_cu.get(int(k_), 0.0) + b
    vals = np.array(list(per_cu.values()))
    return float(vals.max() / vals.mean()), len(per_cu)


def cpu_baseline(w, cu, tensors, scale, with_bwd=True, budget_s=15.0):
    """The fp64 oracle's forward (+ backward) on a bounded sample of the same pack."""
    from concurrent.futures import ThreadPoolExecutor, FIRST_COMPLETED, wait
    import oracle.attention as A
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:          # pragma: no cover
        threadpool_limits = None
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    g = w.h_q // w.h_kv
    lens = np.diff(np.asarray(cu, dtype=np.int64))
    # Units of work, heaviest first: the last 64 query rows of every (sample,
    # KV head) pair, then the last 256, 1024, ... rows (each unit recomputes
    # its own rows from scratch), until the time budget is spent.
    units = []
    order = np.argsort(-lens, kind="stable")
    tail = 64
    while tail < 4 * int(lens.max()):
        for j in order:
            n = int(lens[j])
            if n > tail // 4 or tail == 64:
                for kv in range(w.h_kv):
                    if n > 0:
                        units.append((int(j), kv, max(0, n - tail)))
        tail *= 4
    def run(unit):
        j, kv, first = unit
        s, e = int(cu[j]), int(cu[j + 1])
        q = A.widen_bf16(tensors["q"][s:e])
        k = A.widen_bf16(tensors["k"][s:e])
        v = A.widen_bf16(tensors["v"][s:e])
        do = A.widen_bf16(tensors["dout"][s:e]) if with_bwd else None
        for h in range(kv * g, (kv + 1) * g):
            A.head_rows(q, k, v, 0, e - s, h, kv, first, e - s, scale)
        if with_bwd:
            A.backward_tail(q, k, v, do, 0, e - s, kv, first, scale)
        n = e - s
        return g * ((n * (n + 1) - first * (first + 1)) // 2)

    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    pairs = 0
    done = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        pending = set()
        it = iter(units)
        for _ in range(cores):
            u = next(it, None)
            if u is not None:
                pending.add(ex.submit(run, u))
        while pending:
            fin, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in fin:
                pairs += f.result()
                done += 1
            if time.perf_counter() - t0 < budget_s:
                u = next(it, None)
                if u is not None:
                    pending.add(ex.submit(run, u))
    elapsed = time.perf_counter() - t0
    if ctx is not None:
        ctx.restore_original_limits()
    flops = (3.5 if with_bwd else 1.0) * 4 * w.head_dim * pairs
    full = (3.5 if with_bwd else 1.0) * 4 * w.head_dim * w.h_q * int((lens * (lens + 1) // 2).sum())
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "extrapolated_full_config_s": round(full / (flops / elapsed), 1),
            "sample": f"fp64 numpy oracle {'fwd+bwd' if with_bwd else 'fwd'} on {done} (sample, KV head) units of the same pack "
                      f"(the last 64, then 256, 1024, ... query rows of each sample, heaviest first, until "
                      f"{budget_s:.0f} s were spent; {pairs} causal pair-heads) in {elapsed:.1f} s"}


def cpu_oracle_full(workloads=("tiny_2k", "gqa_32k", "skew_128k_b")):
    """The complete fp64 forward oracle (every sample, every head) on whole packs, timed on the
    host cores (one worker thread per core, one BLAS thread each, one (sample, head) per task);
    prints a markdown table."""
    import synth
    import oracle.attention as A
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:          # pragma: no cover
        threadpool_limits = None
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    print(f"| workload | L | h_q/h_kv | d | samples | fwd FLOPs | oracle s | oracle TFLOP/s | cores |")
    print("|---|---|---|---|---|---|---|---|---|", flush=True)
    for name in workloads:
        w = synth.WORKLOADS[name]
        lens = synth.make_lengths(w, 0)
        cu = synth.cu_seqlens(lens)
        t = synth.make_tensors(w, 0)
        q, k, v = (A.widen_bf16(t[n]) for n in ("q", "k", "v"))
        scale = 1.0 / math.sqrt(w.head_dim)
        g = w.h_q // w.h_kv
        units = [(int(cu[j]), int(cu[j + 1]), h) for j in range(len(lens)) if lens[j] > 0 for h in range(w.h_q)]
        units.sort(key=lambda u: -(u[1] - u[0]))

        def run(u):
            s_, e_, h = u
            return A.head_rows(q, k, v, s_, e_, h, h // g, 0, e_ - s_, scale)

        ctx = threadpool_limits(limits=1) if threadpool_limits else None
        t0 = time.perf_counter()
        with ThreadPoolExecutor(cores) as ex:
            for _ in ex.map(run, units):
                pass
        el = time.perf_counter() - t0
        if ctx is not None:
            ctx.restore_original_limits()
        flops = 4.0 * w.head_dim * w.h_q * int((lens.astype(np.int64) * (lens + 1) // 2).sum())
        print(f"| {name} | {w.total_tokens} | {w.h_q}/{w.h_kv} | {w.head_dim} | {len(lens)} | {flops:.3g} | "
              f"{el:.1f} | {flops / el / 1e12:.3f} | {cores} |", flush=True)


def traffic_for(kernel, workload, launches_bytes_fn):
    """HBM bytes per launch of `kernel` from the committed counter summary, if current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return launches_bytes_fn(t)


def summarize_pmc(fetch_dir, write_dir, workload, copy_bytes):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into profiles/traffic_*.json.

    Each counter is scaled by what it reads for the calibration copy of
    ``copy_bytes`` (a plain device-to-device copy run by --calibrate-copy)."""
    import sqlite3

    def read(d, counter):
        rows = []
        for p in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            con = sqlite3.connect(p)
            rows += list(con.execute("select kernel_name, value from counters_collection where counter_name = ?",
                                     (counter,)))
        return rows

    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")

    def per_kernel(rows, sym):
        v = [x for name, x in rows if sym + "<" in name]
        return float(np.mean(v)) if v else None

    def copy_value(rows):
        v = [x for name, x in rows if "copyBuffer" in name]
        return max(v) if v else None

    fc, wc = copy_value(fetch), copy_value(write)
    out = []
    for kernel, sym in KERNEL_SYMBOL.items():
        f_kib, w_kib = per_kernel(fetch, sym), per_kernel(write, sym)
        if f_kib is None or w_kib is None or not fc or not wc:
            continue
        rec = {"kernel": kernel, "symbol": sym, "workload": workload, "source_hash": source_hash(),
               "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
               "copy_bytes": copy_bytes, "copy_fetch_kib": fc, "copy_write_kib": wc,
               "fetch_bytes_per_kib": copy_bytes / fc, "write_bytes_per_kib": copy_bytes / wc}
        rec["hbm_bytes_per_launch"] = f_kib * rec["fetch_bytes_per_kib"] + w_kib * rec["write_bytes_per_kib"]
        path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        out.append(path)
    print(json.dumps({"written": out}))


def _dbs(d):
    return sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))


def _short(name):
    """Kernel name without namespaces and argument lists: attn_fwd_kernel<128, 1, 8>."""
    base = name.replace("(anonymous namespace)::", "").split("(")[0].replace("libra::", "")
    return base.replace("void ", "").strip()


def summarize_trace(d):
    """Markdown table of every kernel in a rocprofv3 --kernel-trace database."""
    import sqlite3
    rows = {}
    for p in _dbs(d):
        con = sqlite3.connect(p)
        q = "select name, duration, lds_size, grid_x, workgroup_x from kernels"
        for name, dur, lds, gx, wx in con.execute(q):
            r = rows.setdefault(name, {"d": [], "meta": (lds, gx, wx)})
            r["d"].append(dur)
    total = sum(sum(r["d"]) for r in rows.values())
    print("| kernel | calls | total ms | avg ms | min ms | max ms | % | LDS bytes | grid (threads) | workgroup |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for name, r in sorted(rows.items(), key=lambda kv: -sum(kv[1]["d"])):
        d_ = np.array(r["d"], dtype=np.float64) / 1e6
        lds, gx, wx = r["meta"]
        print(f"| `{_short(name)}` | {len(d_)} | {d_.sum():.3f} | {d_.mean():.3f} | {d_.min():.3f} | "
              f"{d_.max():.3f} | {100 * d_.sum() * 1e6 / total:.2f} | {lds} | {gx} | {wx} |")


def summarize_counters(dirs, clock_ghz=2.4, num_cus=256):
    """Markdown table of rocprofv3 --pmc counters per kernel (mean over its dispatches), with
    MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x CUs x 4 SIMDs), kernel cycles
    = its duration in the same run x the shader clock, and the LDS bank-conflict share
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    import sqlite3
    vals, durs = {}, {}
    for d in dirs:
        for p in _dbs(d):
            con = sqlite3.connect(p)
            for k, c, v in con.execute("select kernel_name, counter_name, value from counters_collection"):
                if "libra::" in k:
                    vals.setdefault(_short(k), {}).setdefault(c, []).append(v)
            for name, dur in con.execute("select name, duration from kernels"):
                if "libra::" in name:
                    durs.setdefault(_short(name), []).append(dur)
    counters = sorted({c for v in vals.values() for c in v})
    kernels = sorted(vals)
    print("| counter | " + " | ".join(f"`{k}`" for k in kernels) + " |")
    print("|---|" + "---|" * len(kernels))
    mean = {k: {c: float(np.mean(v)) for c, v in vals[k].items()} for k in kernels}
    for c in counters:
        print(f"| {c} | " + " | ".join(f"{mean[k][c]:.4g}" if c in mean[k] else "" for k in kernels) + " |")

    def derived(k):
        m, out = mean[k], {}
        dur = float(np.median(durs[k])) * 1e-9 if k in durs else None
        if dur and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            out["MFMA util"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (dur * clock_ghz * 1e9 * num_cus * 4)
        if "SQ_LDS_BANK_CONFLICT" in m and m.get("SQ_LDS_IDX_ACTIVE"):
            out["LDS bank-conflict share"] = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_LDS_IDX_ACTIVE"]
        if m.get("SQ_INSTS_MFMA"):
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VALU_TRANS_F32"):
                if c in m:
                    out[c.replace("SQ_INSTS_", "") + " per MFMA"] = m[c] / m["SQ_INSTS_MFMA"]
        if m.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
            out["VALU co-issued share of MFMA-busy cycles"] = m["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"]
        if dur and "GRBM_GUI_ACTIVE" in m:
            # GRBM_GUI_ACTIVE sums the eight XCDs' busy clocks: their mean clock over the kernel
            out["GPU clock GHz (GRBM_GUI_ACTIVE / 8 / duration)"] = m["GRBM_GUI_ACTIVE"] / 8 / dur / 1e9
        if dur:
            out["kernel ms (this run)"] = dur * 1e3
        return out
    der = {k: derived(k) for k in kernels}
    names = sorted({n for v in der.values() for n in v})
    if names:
        print()
        print("| derived | " + " | ".join(f"`{k}`" for k in kernels) + " |")
        print("|---|" + "---|" * len(kernels))
        for n in names:
            print(f"| {n} | " + " | ".join(f"{der[k][n]:.3f}" if n in der[k] else "" for k in kernels) + " |")


def sweep():
    """Forward on every workload at seed 0; the skewed and the uniform 128K packs alone and pooled
    into one launch; then the per-CU balance of the skewed and uniform packs at seeds 0-2 under
    Algorithm 2 and under round-robin placement."""
    import torch
    import synth
    print("| workload | L | h_q/h_kv | d | samples | max sample | fwd ms | TFLOP/s | % bf16 peak | "
          "CU busy max/mean | planned load max/mean | plan ms |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|", flush=True)
    for wl in ("tiny_2k", "gqa_32k", "skew_128k_a", "skew_128k_b", "share_1m", "train_256k"):
        o = measure(wl, 0, 0, True, 5, 2, False, quiet=True)
        c = o["config"]
        print(f"| {wl} | {c['total_tokens']} | {c['h_q']}/{c['h_kv']} | {c['head_dim']} | {c['samples']} | "
              f"{c['max_sample']} | {o['kernel_ms']['fwd']:.3f} | {o['fwd_tflops']:.1f} | "
              f"{100 * o['fwd_frac_peak']:.1f} | {o['cu_busy_max_over_mean']['fwd']:.3f} | "
              f"{o['plan_load_max_over_mean']:.4f} | {o['plan_ms']:.2f} |", flush=True)
        torch.cuda.empty_cache()
    print()
    print("| launch | fwd ms | TFLOP/s | CU busy max/mean |")
    print("|---|---|---|---|", flush=True)
    total = 0.0
    for wl in ("skew_128k_a", "skew_128k_b", "skew_128k_a+skew_128k_b"):
        o = measure(wl, 0, 0, True, 5, 2, False, quiet=True)
        if "+" not in wl:
            total += o["kernel_ms"]["fwd"]
        label = f"pool of two packs ({wl}), one launch" if "+" in wl else f"{wl} alone"
        print(f"| {label} | {o['kernel_ms']['fwd']:.3f} | {o['fwd_tflops']:.1f} | "
              f"{o['cu_busy_max_over_mean']['fwd']:.3f} |", flush=True)
        torch.cuda.empty_cache()
    print(f"| the two packs in two launches (sum) | {total:.3f} | | |", flush=True)
    print()
    print("| workload | seed | sum of squared lengths | placement | fwd ms | TFLOP/s | CU busy max/mean | "
          "planned load max/mean |")
    print("|---|---|---|---|---|---|---|---|", flush=True)
    for wl in ("skew_128k_a", "skew_128k_b", "share_1m"):
        for seed in (0, 1, 2):
            sq = int((synth.make_lengths(synth.WORKLOADS[wl], seed).astype(np.int64) ** 2).sum())
            for assign in (0, 1):
                o = measure(wl, seed, assign, True, 3, 1, False, quiet=True)
                print(f"| {wl} | {seed} | {sq:.4g} | {'Algorithm 2' if assign == 0 else 'round-robin'} | "
                      f"{o['kernel_ms']['fwd']:.3f} | {o['fwd_tflops']:.1f} | "
                      f"{o['cu_busy_max_over_mean']['fwd']:.3f} | {o['plan_load_max_over_mean']:.4f} |", flush=True)
                torch.cuda.empty_cache()


def ab_table(workloads, rounds=2):
    """Plan variants side by side: Algorithm 2 with executed-work item costs (the default), with
    eq. 8 pair costs, and with the L2 residency term; rounds interleave the variants so that
    drifting clocks hit them alike."""
    import torch
    variants = [("algorithm2, executed cost", 0, 0), ("algorithm2, pair cost", 0, 1),
                ("algorithm2 + L2 term, executed cost", 2, 0)]
    print("| workload | plan | round | fwd ms | fwd TFLOP/s | dK/dV ms | dQ ms | step TFLOP/s | "
          "CU busy max/mean fwd / dK/dV / dQ |")
    print("|---|---|---|---|---|---|---|---|---|", flush=True)
    for wl in workloads:
        fwd_only = wl != "train_256k"
        for rnd in range(rounds):
            for label, assign, cost in variants:
                o = measure(wl, 0, assign, fwd_only, 5, 2, False, quiet=True, cost=cost)
                km, busy = o["kernel_ms"], o["cu_busy_max_over_mean"]
                print(f"| {wl} | {label} | {rnd} | {km['fwd']:.3f} | {o['fwd_tflops']:.1f} | "
                      f"{km.get('bwd_dkdv', float('nan')):.3f} | {km.get('bwd_dq', float('nan')):.3f} | "
                      f"{o['value'] if not fwd_only else float('nan'):.1f} | "
                      + " / ".join(f"{busy[k]:.3f}" for k in ("fwd", "bwd_dkdv", "bwd_dq") if k in busy) + " |",
                      flush=True)
                torch.cuda.empty_cache()


def granularity():
    """Forward of train_256k at seed 0 for SH-Tiles of B tokens x W heads: the planner cuts
    work items inside tiles, so B and W set where items are cut and how many query heads
    share one K/V block copy (W < 4 leaves W heads per item)."""
    import torch
    print("| tile tokens B | tile heads W | tiles | forward items | heads per item | fwd ms | TFLOP/s | "
          "CU busy max/mean | planned load max/mean | plan ms |")
    print("|---|---|---|---|---|---|---|---|---|---|", flush=True)
    for b_ in (512, 2048, 8192, 32768):
        for w_ in (1, 2, 4, 8):
            o = measure("train_256k", 0, 0, True, 5, 2, False, quiet=True, tiling=(b_, w_))
            ps = o["plan_sizes"]
            print(f"| {b_} | {w_} | {ps['tiles']} | {ps['fwd_items']} | {min(w_, 4)} | "
                  f"{o['kernel_ms']['fwd']:.3f} | {o['fwd_tflops']:.1f} | "
                  f"{o['cu_busy_max_over_mean']['fwd']:.3f} | {o['plan_load_max_over_mean']:.4f} | "
                  f"{o['plan_ms']:.2f} |", flush=True)
            torch.cuda.empty_cache()


def simulate(packs=3, seed=0):
    """Configuration simulator (host only; the single-GPU counterpart of the pages' replay of
    VRSP and the placer over windows for candidate configurations).  For packs of train_256k's
    shape and each SH-Tile shape (B tokens x W heads): the planner's intra-GPU imbalance per
    queue (largest over mean planned load) and the bytes the kernels stream into LDS (each item
    copies its K/V blocks, or its Q/dO blocks for dK/dV, once), which is what smaller tiles cost
    on one GPU in place of the pages' exchange volume.  Inter-pool imbalance is VRSP's
    (--vrsp); it does not depend on B or W."""
    import synth
    import packed_varlen_attention_cu_amd as lib
    w0 = synth.WORKLOADS["train_256k"]
    d, blk = w0.head_dim, 64
    print("| tile tokens B | tile heads W | tiles | fwd items | fwd planned max/mean | dQ planned max/mean | "
          "dK/dV planned max/mean | streamed K/V + Q/dO bytes (GB) | plan ms |")
    print("|---|---|---|---|---|---|---|---|---|", flush=True)
    lens = [synth.make_lengths(w0, seed + i) for i in range(packs)]
    for b_ in (512, 2048, 8192, 32768):
        for w_ in (1, 2, 4, 8):
            agg = {"tiles": 0, "items": 0, "f": [], "q": [], "k": [], "bytes": 0.0, "ms": []}
            for ln in lens:
                cu = synth.cu_seqlens(ln)
                t0 = time.perf_counter()
                p_ = lib.Plan(cu, total_tokens=w0.total_tokens, h_q=w0.h_q, h_kv=w0.h_kv, head_dim=d,
                              tile_tokens=b_, tile_heads=w_)
                agg["ms"].append((time.perf_counter() - t0) * 1e3)
                i_ = p_.info
                n = i_.num_cus
                agg["tiles"] += i_.n_tiles
                agg["items"] += i_.n_items
                agg["f"].append(i_.load_max / (i_.load_sum / n))
                agg["q"].append(i_.dq_load_max / (i_.dq_load_sum / n))
                agg["k"].append(i_.kv_load_max / (i_.kv_load_sum / n))
                starts = cu[np.searchsorted(cu, np.arange(w0.total_tokens), side="right") - 1]
                for its in (p_.items, p_.dq_items):       # K and V blocks per item
                    r0 = its["row0"].astype(np.int64)
                    ks = starts[r0] & ~(blk - 1)
                    nb = (r0 + its["nrows"] - ks + blk - 1) // blk
                    agg["bytes"] += float(nb.sum()) * 2 * blk * d * 2
                kv = p_.kv_items                          # Q and dO blocks of every head per step
                r0 = kv["row0"].astype(np.int64)
                ends = np.searchsorted(cu, r0 + kv["nrows"] - 1, side="right")
                qb = (cu[ends] - (r0 & ~(blk - 1)) + blk - 1) // blk
                agg["bytes"] += float((qb * kv["nheads"]).sum()) * 2 * blk * d * 2
            print(f"| {b_} | {w_} | {agg['tiles'] // packs} | {agg['items'] // packs} | "
                  f"{np.mean(agg['f']):.4f} | {np.mean(agg['q']):.4f} | {np.mean(agg['k']):.4f} | "
                  f"{agg['bytes'] / packs / 1e9:.1f} | {np.median(agg['ms']):.1f} |", flush=True)


def vrsp_report(windows=20, seed=0):
    """Variance-reduced sequence placement (host only): time per window, and the residual
    inter-pool imbalance R - 1 (max / mean pool workload - 1) under the sampler's index order,
    a seeded random grouping and VRSP, over windows of 128 synthetic packed sequences."""
    import synth
    import packed_varlen_attention_cu_amd as lib
    import oracle.vrsp as V

    def window(L, w_seed, D):
        w = synth.WORKLOADS["train_256k"].with_tokens(L, first_lengths=())
        return np.array([int((synth.make_lengths(w, w_seed * 1000 + i).astype(np.int64) ** 2).sum())
                         for i in range(D)], dtype=np.int64)

    print("| window D | pool size P | library, µs per window (median of 2000 calls, 1 thread) | "
          "oracle (Python), µs per window | pages |")
    print("|---|---|---|---|---|", flush=True)
    for D, ref in ((128, "48 µs"), (256, "106 µs")):
        F = window(262144, seed, D)
        ts = []
        for _ in range(2000):
            t0 = time.perf_counter_ns()
            lib.libra_vrsp(F, 8)
            ts.append(time.perf_counter_ns() - t0)
        to = []
        Fl = F.tolist()
        for _ in range(50):
            t0 = time.perf_counter_ns()
            V.vrsp(Fl, 8)
            to.append(time.perf_counter_ns() - t0)
        print(f"| {D} | 8 | {np.median(ts) / 1e3:.1f} | {np.median(to) / 1e3:.0f} | {ref} |", flush=True)
    t_call = []
    cu = np.array([0, 1], dtype=np.int32)
    for _ in range(2000):
        t0 = time.perf_counter_ns()
        lib.libra_pack_workload(cu)
        t_call.append(time.perf_counter_ns() - t0)
    print(f"\nA trivial library call through the same binding takes {np.median(t_call) / 1e3:.1f} µs "
          "(included above).\n")

    print("| packs of | P | pools K | R - 1, index order | R - 1, random grouping | R - 1, VRSP | "
          "lower bound (largest pack / mean pool - 1) |")
    print("|---|---|---|---|---|---|---|", flush=True)
    rng = np.random.default_rng(seed)
    for L, label in ((262144, "256K tokens"), (1048576, "1M tokens")):
        wins = [window(L, seed + 1 + r, 128) for r in range(windows)]
        for P in (2, 4, 8, 16, 32, 64):
            idx, rnd, vr, lb = [], [], [], []
            for F in wins:
                K = len(F) // P
                lb.append(max(0.0, float(F.max()) / (float(F.sum()) / K) - 1.0))
                idx.append(V.imbalance([int(F[k * P:(k + 1) * P].sum()) for k in range(K)]))
                perm = rng.permutation(len(F))
                rnd.append(V.imbalance([int(F[perm[k * P:(k + 1) * P]].sum()) for k in range(K)]))
                vr.append(V.imbalance(lib.libra_vrsp(F, P)[2].tolist()))
            print(f"| {label} | {P} | {len(wins[0]) // P} | {np.mean(idx):.4f} | {np.mean(rnd):.4f} | "
                  f"{np.mean(vr):.5f} | {np.mean(lb):.5f} |", flush=True)


_INPUTS = {}


def pooled_inputs(workload, seed, names):
    """Workload, sample lengths and bf16 tensors of one pack, or of a pool "a+b+...": the packs
    concatenated into one (the block-diagonal mask keeps them apart), planned and launched once.
    Kept for the next call with the same arguments (the A/B tables time several plans of one
    pack)."""
    key = (workload, seed, tuple(names))
    if key not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[key] = _make_inputs(workload, seed, names)
    return _INPUTS[key]


def _make_inputs(workload, seed, names):
    import synth
    parts = [synth.WORKLOADS[n] for n in workload.split("+")]
    w0 = parts[0]
    for p_ in parts[1:]:
        if (p_.h_q, p_.h_kv, p_.head_dim, p_.tile_tokens, p_.tile_heads) != \
                (w0.h_q, w0.h_kv, w0.head_dim, w0.tile_tokens, w0.tile_heads):
            raise ValueError(f"pool members must share heads, head_dim and tiling: {workload}")
    lengths = [synth.make_lengths(p_, seed) for p_ in parts]
    tensors = [synth.make_tensors(p_, seed, names=names) for p_ in parts]
    if len(parts) == 1:
        return w0, lengths[0], tensors[0]
    w = w0.with_tokens(sum(p_.total_tokens for p_ in parts), name=workload)
    return (w, np.concatenate(lengths),
            {n: np.concatenate([t[n] for t in tensors]) for n in names})


def measure(workload="train_256k", seed=0, assign=0, fwd_only=False, steps=10, warmup=2, cpu=True,
            calibrate_copy=0, quiet=False, tiling=None, dump_records=None, speed_calibration=True,
            cost=0, item_overhead=0, tau=0.03, num_cus=0):
    """Time `steps` steps of the hot path on cuda:0; returns the JSON record.  `tiling`
    = (tile_tokens, tile_heads) replaces the workload's SH-Tile shape."""
    import torch
    import synth
    import packed_varlen_attention_cu_amd as lib

    do_bwd = not fwd_only
    names = ("q", "k", "v", "dout") if do_bwd else ("q", "k", "v")
    w, lengths, host = pooled_inputs(workload, seed, names)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cu = synth.cu_seqlens(lengths)

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = up(host["q"]), up(host["k"]), up(host["v"])
    dout = up(host["dout"]) if do_bwd else None
    L, d = w.total_tokens, w.head_dim
    scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((w.h_q, L), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if do_bwd else (None,) * 3

    tile_tokens, tile_heads = tiling if tiling else (w.tile_tokens, w.tile_heads)
    plan_kw = dict(total_tokens=L, h_q=w.h_q, h_kv=w.h_kv, head_dim=d, tile_tokens=tile_tokens,
                   tile_heads=tile_heads, assign=assign, cost=cost, item_overhead=item_overhead, tau=tau,
                   num_cus=num_cus)
    plan0 = lib.Plan(cu, **plan_kw)
    ncu = plan0.info.num_cus
    ws_b = torch.empty(max(1, lib.libra_attn_bwd_workspace(plan0.host)), dtype=torch.uint8, device=dev)
    rec = torch.zeros(3 * ncu * lib.RECORD_DTYPE.itemsize, dtype=torch.uint8, device=dev)   # warm-up steps
    cu_dev = torch.from_numpy(cu.copy()).to(dev)
    plan_dev = torch.empty(plan0.host.nbytes, dtype=torch.uint8, device=dev)

    if calibrate_copy:
        n = calibrate_copy << 20
        a_ = torch.empty(n, dtype=torch.uint8, device=dev)
        b_ = torch.empty(n, dtype=torch.uint8, device=dev)
        b_.copy_(a_)
        torch.cuda.synchronize()
        del a_, b_

    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    names_ = ("fwd", "bwd_prepare", "bwd_dkdv", "bwd_dq")
    ev = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names_}
          for _ in range(steps)]
    recs = [torch.zeros(3 * ncu * lib.RECORD_DTYPE.itemsize, dtype=torch.uint8, device=dev) for _ in range(steps)]
    times = {n: [] for n in names_}
    plan_ms = []

    # The host planner runs one step ahead on a worker thread (the planner call
    # releases the GIL): the plan of step i + 1 is built while the GPU runs
    # step i, so planning stays off the GPU's critical path, as the method
    # intends.  Every step still builds its own plan inside the timed region.
    def make_plan():
        t0 = time.perf_counter()
        plan = lib.Plan(cu, **plan_kw)                                  # host planner (a1-a3)
        plan_ms.append((time.perf_counter() - t0) * 1e3)
        return plan

    planner = ThreadPoolExecutor(1)

    def step(plan, i, record):
        # plan upload; the copy waits for the previous step's kernels, which read plan_dev
        plan_dev.copy_(torch.from_numpy(plan.host))
        wsb = ws_b.numel()
        r = recs[i] if record else rec
        r_f, r_kv, r_q = r[:ncu * 32], r[ncu * 32:2 * ncu * 32], r[2 * ncu * 32:]

        def timed(name, fn):
            if record:
                ev[i][name][0].record(stream)
            fn()
            if record:
                ev[i][name][1].record(stream)

        timed("fwd", lambda: lib.libra_attn_fwd(plan.host, plan_dev, q, k, v, cu_dev, o, lse, scale, r_f, sh))
        if do_bwd:
            timed("bwd_prepare", lambda: lib.libra_attn_bwd_prepare(plan.host, o, dout, lse, ws_b, wsb, sh))
            timed("bwd_dkdv", lambda: lib.libra_attn_bwd_dkdv(plan.host, plan_dev, q, k, v, dout, lse, cu_dev,
                                                              dk, dv, scale, ws_b, wsb, r_kv, sh))
            timed("bwd_dq", lambda: lib.libra_attn_bwd_dq(plan.host, plan_dev, q, k, v, dout, lse, cu_dev, dq,
                                                          scale, ws_b, wsb, r_q, sh))

    nxt = planner.submit(make_plan)
    plan = None
    for _ in range(warmup):
        plan = nxt.result()
        nxt = planner.submit(make_plan)
        step(plan, 0, False)
    torch.cuda.synchronize()
    speed = None
    if plan is not None and speed_calibration and assign in (0, 2):
        # The eight XCDs sustain different clocks; the last warm-up launch's per-CU records give
        # each one's rate, and the timed steps' plans place work by finish time on it.
        r = rec.cpu().numpy()
        parts = [(lib.QUEUE_FWD, r[:ncu * 32])]
        if do_bwd:
            parts += [(lib.QUEUE_KV, r[ncu * 32:2 * ncu * 32]), (lib.QUEUE_DQ, r[2 * ncu * 32:])]
        num = np.zeros(8)
        den = 0.0
        for q_, rr in parts:
            rec_ = rr.view(lib.RECORD_DTYPE)[:ncu]
            b_ = float((rec_["t_end"] - rec_["t_start"]).astype(np.float64).sum())
            num += b_ * lib.libra_worker_speed(plan.host, q_, rec_).astype(np.float64)
            den += b_
        speed = [int(round(x)) for x in num / den] if den > 0 else None
        if speed:
            plan_kw["worker_speed"] = speed
            nxt.result()
            nxt = planner.submit(make_plan)                             # re-plan with the speeds
    plan_ms.clear()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        plan = nxt.result()
        nxt = planner.submit(make_plan)                                 # the next step's plan
        step(plan, i, True)
        if not quiet:
            print(f"step {i + 1}/{steps} enqueued", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nxt.result()
    planner.shutdown()

    if dump_records:
        # per-workgroup busy time (constant-rate clock ticks) next to the planner's load of the
        # same queue, for the last timed step
        import packed_varlen_attention_cu_amd as lib_
        r = recs[steps - 1].cpu().numpy()
        out_ = {}
        for n, rr, its, off in (("fwd", r[:ncu * 32], plan.items, plan.cu_off),
                                ("bwd_dkdv", r[ncu * 32:2 * ncu * 32], plan.kv_items, plan.kv_cu_off),
                                ("bwd_dq", r[2 * ncu * 32:], plan.dq_items, plan.dq_cu_off)):
            if n.startswith("bwd") and not do_bwd:
                continue
            rec_ = rr.view(lib_.RECORD_DTYPE)[:ncu]
            item_cost = its["cost"].astype(np.int64)
            out_[n] = [{"w": w_, "xcc": int(rec_["xcc_id"][w_]), "hw": int(rec_["hw_id"][w_]),
                        "busy": int(rec_["t_end"][w_] - rec_["t_start"][w_]), "n_items": int(rec_["n_items"][w_]),
                        "planned": int(item_cost[off[w_]:off[w_ + 1]].sum()),
                        "items": [int(x) for x in its["id"][off[w_]:off[w_ + 1]]]}
                       for w_ in range(ncu)]
        with open(dump_records, "w") as f:
            json.dump(out_, f)

    busy = {"fwd": [], "bwd_dkdv": [], "bwd_dq": []}
    for i in range(steps):
        for n, (a_, b_) in ev[i].items():
            if n.startswith("bwd") and not do_bwd:
                continue
            times[n].append(a_.elapsed_time(b_))
        r = recs[i]
        for n, rr in (("fwd", r[:ncu * 32]), ("bwd_dkdv", r[ncu * 32:2 * ncu * 32]), ("bwd_dq", r[2 * ncu * 32:])):
            if n.startswith("bwd") and not do_bwd:
                continue
            raw = rr.cpu().numpy()
            flags = raw.view(lib.RECORD_DTYPE)[:ncu]["flags"]
            if (flags != 0).any():
                raise RuntimeError(f"{n}: per-CU records flag {sorted(set(int(x) for x in flags if x))} "
                                   "(plan mismatch or an expired wait): the step's results are not valid")
            ratio, _ = cu_busy_ratio(raw, ncu)
            busy[n].append(ratio)
    ms_step = wall / steps * 1e3
    pairs = causal_pairs(cu) * w.h_q
    assert pairs == plan0.info.total_pairs, "planner pair count disagrees with the closed form"
    fwd_flops = 4.0 * d * pairs
    total_flops = fwd_flops * (3.5 if do_bwd else 1.0)
    avg = {n: float(np.mean(t)) for n, t in times.items() if t}
    fwd_ms = avg["fwd"]
    kernels = {n: avg[n] for n in KERNEL_FLOPS_PER_PAIR if n in avg}
    dom = max(kernels, key=kernels.get)
    achieved = KERNEL_FLOPS_PER_PAIR[dom] * d * pairs / (kernels[dom] * 1e-3) / 1e12
    traffic = traffic_for(dom, workload, lambda t: t["hbm_bytes_per_launch"])

    out = {
        "metric": METRIC,
        "value": round(total_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "total_tokens": L, "h_q": w.h_q, "h_kv": w.h_kv,
                   "head_dim": d, "sh_tile": [tile_tokens, tile_heads], "samples": int(len(lengths)),
                   "max_sample": int(lengths.max()), "seed": seed, "pass": "fwd+bwd" if do_bwd else "fwd",
                   "placement": PLACEMENT_NAMES[assign], "item_cost": ("executed", "pairs")[cost],
                   "num_cus": ncu},
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "fwd_frac_peak": round(fwd_flops / (avg["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {n: round(t, 4) for n, t in avg.items()},
        "plan_ms": round(float(np.mean(plan_ms)), 3),
        "cu_busy_max_over_mean": {n: round(float(np.mean(b)), 4) for n, b in busy.items() if b},
        "plan_load_max_over_mean": round(plan0.info.load_max / (plan0.info.load_sum / ncu), 5),
        "worker_speed": speed,
        "plan_sizes": {"tiles": plan0.info.n_tiles, "fwd_items": plan0.info.n_items,
                       "dq_items": plan0.info.n_dq_items, "kv_items": plan0.info.n_kv_items},
        "flops_fwd": fwd_flops,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if do_bwd:
        bwd_ms = avg["bwd_prepare"] + avg["bwd_dkdv"] + avg["bwd_dq"]
        out["bwd_tflops"] = round(2.5 * fwd_flops / (bwd_ms * 1e-3) / 1e12, 2)
        out["fwd_bwd_kernels_tflops"] = round(3.5 * fwd_flops / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2)
    if cpu:
        out["cpu_baseline"] = cpu_baseline(w, cu, host, scale, with_bwd=do_bwd)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="train_256k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--assign", type=int, default=0,
                    help="0: Algorithm 2 placement, 1: round-robin, 2: Algorithm 2 with the L2 residency term")
    ap.add_argument("--cost", choices=("executed", "pairs"), default="executed",
                    help="forward / dQ item cost: executed query-key slots or eq. 8 pairs")
    ap.add_argument("--item-overhead", type=int, default=0, help="cost added to every work item")
    ap.add_argument("--tau", type=float, default=0.03, help="soft-target slack of Algorithm 2")
    ap.add_argument("--num-cus", type=int, default=0,
                    help="workers (persistent workgroups) the plan places on; 0: one per CU (256)")
    ap.add_argument("--no-share-1m", action="store_true",
                    help="skip the forward of the 1M-token head share that follows the train_256k step")
    ap.add_argument("--cpu-oracle-full", action="store_true",
                    help="time the complete fp64 forward oracle on the 2K, 32K and uniform 128K packs (host only)")
    ap.add_argument("--ab", nargs="+", metavar="WORKLOAD",
                    help="plan variants side by side (executed vs pair cost, L2 term) on these workloads")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="run one plain device copy of this size first (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="DIR", help="markdown table of a rocprofv3 --kernel-trace run")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR", help="markdown table of rocprofv3 --pmc runs")
    ap.add_argument("--simulate", action="store_true",
                    help="host-only configuration simulator: planner imbalance and streamed bytes per SH-Tile shape")
    ap.add_argument("--vrsp", action="store_true",
                    help="host-only: variance-reduced sequence placement timing and pool balance")
    ap.add_argument("--no-speed-calibration", action="store_true",
                    help="plan with equal worker speeds instead of the per-XCD rates of the warm-up")
    ap.add_argument("--dump-records", metavar="PATH",
                    help="write each workgroup's busy time and planned load (last timed step) as JSON")
    ap.add_argument("--granularity", action="store_true",
                    help="forward of train_256k against the SH-Tile shape (tile tokens x tile heads)")
    ap.add_argument("--sweep", action="store_true",
                    help="forward on every workload (and seeds 0-2 and both placements on the skewed and "
                         "uniform packs); prints a markdown table")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      args.calibrate_copy * (1 << 20))
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.vrsp:
        vrsp_report()
        return
    if args.cpu_oracle_full:
        cpu_oracle_full()
        return
    if args.simulate:
        simulate()
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); sharding this path over "
              "several GPUs is a design note and is not run here.", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep()
        return
    if args.granularity:
        granularity()
        return
    if args.ab:
        ab_table(args.ab)
        return
    out = measure(args.workload, args.seed, args.assign, args.fwd_only, args.steps, args.warmup,
                  not args.no_cpu_baseline, args.calibrate_copy, dump_records=args.dump_records,
                  speed_calibration=not args.no_speed_calibration, cost=("executed", "pairs").index(args.cost),
                  item_overhead=args.item_overhead, tau=args.tau, num_cus=args.num_cus)
    if args.workload == "train_256k" and not args.fwd_only and not args.no_share_1m:
        # The other configuration the forward target names: the 1M-token head share, forward only.
        s1 = measure("share_1m", args.seed, args.assign, True, 5, 2, False, quiet=True,
                     cost=("executed", "pairs").index(args.cost), item_overhead=args.item_overhead, tau=args.tau)
        c = s1["config"]
        out["fwd_share_1m"] = {"tflops": s1["fwd_tflops"], "frac_peak": s1["fwd_frac_peak"],
                               "fwd_ms": round(s1["kernel_ms"]["fwd"], 3), "steps": 5,
                               "cu_busy_max_over_mean": s1["cu_busy_max_over_mean"]["fwd"],
                               "config": {k: c[k] for k in ("total_tokens", "h_q", "h_kv", "head_dim", "sh_tile",
                                                             "samples", "max_sample")}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
