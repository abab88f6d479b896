#!/usr/bin/env python3
"""Benchmark of the MILO hot path on one MI355X.

One step = one pass of the whole path over the workload's KV cache: compress
every K block and every V block of every layer (Gram -> eigensolve ->
singular-value refinement -> rank allocation -> factors), then one decode step
of every layer over the compressed blocks.  Inputs (planted-spectrum blocks and
queries, seeded) are generated on the GPU and resident in HBM before timing.

Prints ONE JSON line.  `value` is context tokens (sum over sequences of the
tokens attended in the decode step) per second of step time, the K and V
compression calls on two streams (--compress-streams); the breakdown reports
compression blocks/s and decode context-tokens/s on their own, and a roofline
entry for every kernel from per-kernel HIP-event timings taken in a second pass
of the same steps with every call on one stream.

  python bench.py [--steps K] [--warmup W] [--config 4] [--no-cpu-baseline]
  python bench.py --calibrate-copy     # plain copy kernel for HBM counter calibration
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

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_VEC_TFLOPS = 157.3   # fp32 vector (packed)
# fp32 vector without packed instructions (the build disables them):
# 256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA) x 2.4 GHz
PEAK_FP32_VEC_NONPACKED_TFLOPS = 78.6
METRIC = ("compressed-KV decode context-tokens/s (+HBM %peak); blocks/s compressed (+MFMA %)")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--factor-dtype", default=None, help="bf16 | i8 | i4 | i2 (default: the config's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the host-offloaded cache measurement (compressed vs full KV over PCIe)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--decode-only-steps", type=int, default=20,
                    help="extra decode-only passes after the timed steps (reported separately)")
    ap.add_argument("--ingest-stats", metavar="CSV",
                    help="rocprofv3 kernel_stats.csv -> profiles/kernel_stats_<workload>.txt (no GPU)")
    ap.add_argument("--ingest-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 counter_collection.csv of the bench (FETCH_SIZE, WRITE_SIZE) and of "
                         "--calibrate-copy -> profiles/<kernel>_traffic.json (no GPU)")
    ap.add_argument("--ingest-mfma", metavar="CSV",
                    help="rocprofv3 counter_collection.csv of the bench with SQ_INSTS_VALU_MFMA_MOPS_BF16, "
                         "SQ_INSTS_VALU_MFMA_MOPS_F32, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE -> "
                         "profiles/<kernel>_mfma.json (no GPU)")
    ap.add_argument("--compress-streams", type=int, default=2,
                    help="streams the compression calls of a step alternate between (1 or 2; with 2 the K "
                         "and V calls overlap, so one's QR chain runs beside the other's Gram)")
    ap.add_argument("--compress-chunks", type=int, default=1,
                    help="compression calls per kind (runs of whole layers)")
    ap.add_argument("--filter-csv", nargs=2, metavar=("IN", "OUT"),
                    help="copy the rows of a rocprofv3 CSV that belong to libmilo's kernels (no GPU)")
    ap.add_argument("--extra", default="2,1,4:i4,4:i2",
                    help="other workloads measured after the main one (config indices, or 'none'): "
                         "multi-layer ones as whole steps, one-layer ones warm and cold; "
                         "'c:fmt' runs config c with factor format fmt (with its offload step)")
    ap.add_argument("--command", action="append", default=[],
                    help="with --ingest-*: the command(s) that produced the CSV files")
    return ap.parse_args()


# kernel -> the sources that define it (the traffic records are tied to their hash)
KERNEL_SOURCES = {"gram": ["gram.hip", "common.hpp"], "jacobi": ["jacobi.hip"], "tridiag": ["eigh.hip"], "qr_chain": ["eigh.hip"],
                  "qr_apply": ["eigh.hip"],
                  "refine": ["refine.hip", "common.hpp"], "alloc": ["alloc.hip"],
                  "project": ["project.hip", "common.hpp"], "reconstruct": ["reconstruct.hip", "common.hpp"],
                  "decode": ["decode.hip", "common.hpp"], "decode_tail": ["decode.hip", "common.hpp"],
                  "decode_combine": ["decode.hip", "common.hpp"],
                  "decode_tables": ["decode.hip"]}


def kernel_key(name):
    """libmilo kernel name (as rocprofv3 prints it) -> bench kernel key."""
    for frag, key in (("gram_kernel", "gram"), ("gram_bf16_kernel", "gram"), ("jacobi_kernel", "jacobi"), ("tridiag_kernel", "tridiag"), ("qr_chain_kernel", "qr_chain"),
                      ("qr_apply_kernel", "qr_apply"),
                      ("refine_kernel", "refine"), ("alloc_kernel", "alloc"), ("project_kernel", "project"),
                      ("project_bf16_kernel", "project"), ("reconstruct_kernel", "reconstruct"),
                      ("reconstruct_bf16_kernel", "reconstruct"), ("decode_tables_kernel", "decode_tables"),
                      ("decode_combine_kernel", "decode_combine")):
        if frag in name:
            return key
    if "decode_kernel<" in name:  # <factor type, tail type>: -1 = no tail
        return "decode" if ", -1>" in name else "decode_tail"
    return None


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def workload_slug(cfg):
    return (f"{cfg.layers}L_b{cfg.batch}_kv{cfg.n_kv_heads}_q{cfg.n_q_heads}_"
            f"{cfg.attended_blocks}x{cfg.block_len}")


def ingest_stats(args):
    from synthetic import CONFIGS
    cfg = CONFIGS[args.config]
    rows = _read_csv(args.ingest_stats)
    lines = [f"# rocprofv3 kernel statistics: {cfg.workload}", ""]
    for c in args.command:
        lines.append(f"command: {c}")
    lines += ["", f"{'kernel':16s} {'calls':>7s} {'avg_us':>12s} {'total_ms':>11s} {'share':>7s}  name"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        key = kernel_key(r["Name"]) or "-"
        lines.append(f"{key:16s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:12.2f} "
                     f"{float(r['TotalDurationNs']) / 1e6:11.2f} {float(r['Percentage']):6.2f}%  {r['Name'][:110]}")
    out = os.path.join(ROOT, "profiles", f"kernel_stats_{workload_slug(cfg)}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel name, value)} for one counter (summed over its instances)."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = r["Dispatch_Id"]
        name, v = acc.get(d, (r["Kernel_Name"], 0.0))
        acc[d] = (name, v + float(r["Counter_Value"]))
    return acc


def ingest_traffic(args):
    from synthetic import CONFIGS
    cfg = CONFIGS[args.config]
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.ingest_traffic
    copy_bytes = 1 << 30

    def copy_factor(path, counter):
        d = _per_dispatch(_read_csv(path), counter)
        vals = [v * 1024 for n, v in d.values() if "bitwise_not" in n.lower()]
        if not vals:
            vals = [v * 1024 for n, v in list(d.values())[-3:]]
        vals.sort()
        return vals[len(vals) // 2] / copy_bytes

    f_fetch = copy_factor(cfetch_csv, "FETCH_SIZE")
    f_write = copy_factor(cwrite_csv, "WRITE_SIZE")
    per = {}
    for path, counter, fac, slot in ((fetch_csv, "FETCH_SIZE", f_fetch, 0), (write_csv, "WRITE_SIZE", f_write, 1)):
        for name, v in _per_dispatch(_read_csv(path), counter).values():
            key = kernel_key(name)
            if key is None:
                continue
            rec = per.setdefault(key, [[], []])
            rec[slot].append(v * 1024 / fac)
    lines = [f"# HBM traffic per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE): {cfg.workload}", "",
             f"calibration: a plain {copy_bytes} B device copy reads {f_fetch:.4f} x and writes "
             f"{f_write:.4f} x its size by these counters; values below are divided by that factor", ""]
    for c in args.command:
        lines.append(f"command: {c}")
    lines += ["", f"{'kernel':16s} {'dispatches':>10s} {'fetch_MB':>12s} {'write_MB':>12s} {'total_MB':>12s}"]
    for key, (fv, wv) in sorted(per.items()):
        if not fv or not wv:
            continue
        fb, wb = sum(fv) / len(fv), sum(wv) / len(wv)
        h = hashlib.sha256()
        for n in KERNEL_SOURCES[key]:
            with open(os.path.join(ROOT, "block_wise_rank_amd", "csrc", n), "rb") as f:
                h.update(f.read())
        rec = {"kernel": key, "workload": cfg.workload, "source_hash": h.hexdigest()[:16],
               "bytes_per_launch": fb + wb, "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
               "dispatches": len(fv), "copy_calibration": {"fetch": f_fetch, "write": f_write},
               "commands": args.command}
        with open(os.path.join(ROOT, "profiles", f"{key}_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
        lines.append(f"{key:16s} {len(fv):10d} {fb / 1e6:12.2f} {wb / 1e6:12.2f} {(fb + wb) / 1e6:12.2f}")
    out = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_slug(cfg)}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def _per_dispatch_reduce(rows, counter, how):
    """{dispatch id: (kernel name, value)} for one counter, its instances reduced
    by `how` (sum or max)."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = r["Dispatch_Id"]
        name, v = acc.get(d, (r["Kernel_Name"], None))
        x = float(r["Counter_Value"])
        acc[d] = (name, x if v is None else (v + x if how == "sum" else max(v, x)))
    return acc


SIMD_NUM = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
CLOCK_HZ = 2.4e9   # MI355X peak engine clock


def ingest_mfma(args):
    """MFMA counters of the bench run -> per kernel: MFMA flops per launch
    (SQ_INSTS_VALU_MFMA_MOPS_* x 512, the unit rocprofv3's MfmaFlops uses) and the
    MFMA busy share (SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs / (GRBM_GUI_ACTIVE x
    SIMDs), rocprofv3's MfmaUtil)."""
    from synthetic import CONFIGS
    cfg = CONFIGS[args.config]
    rows = _read_csv(args.ingest_mfma)
    bf16 = _per_dispatch_reduce(rows, "SQ_INSTS_VALU_MFMA_MOPS_BF16", "sum")
    f32 = _per_dispatch_reduce(rows, "SQ_INSTS_VALU_MFMA_MOPS_F32", "sum")
    busy = _per_dispatch_reduce(rows, "SQ_VALU_MFMA_BUSY_CYCLES", "sum")
    active = _per_dispatch_reduce(rows, "GRBM_GUI_ACTIVE", "max")
    dur = {}
    for r in rows:  # dispatch duration (ns) from the record's own timestamps
        dur[r["Dispatch_Id"]] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    per = {}
    for dsp, (name, v) in bf16.items():
        key = kernel_key(name)
        if key is None:
            continue
        flops = 512.0 * (v + f32.get(dsp, (name, 0.0))[1])
        util = busy_dur = None
        if dsp in busy and dsp in active and active[dsp][1] > 0:
            util = 100.0 * busy[dsp][1] / (active[dsp][1] * SIMD_NUM)
        if dsp in busy and dur.get(dsp, 0) > 0:
            busy_dur = 100.0 * busy[dsp][1] / (dur[dsp] * 1e-9 * CLOCK_HZ * SIMD_NUM)
        per.setdefault(key, []).append((flops, util, busy_dur, dur.get(dsp)))
    lines = [f"# MFMA counters per launch (rocprofv3 --pmc): {cfg.workload}", "",
             "flops = 512 x (SQ_INSTS_VALU_MFMA_MOPS_BF16 + SQ_INSTS_VALU_MFMA_MOPS_F32) (rocprofv3's MfmaFlops);",
             f"busy_dur = SQ_VALU_MFMA_BUSY_CYCLES / (dispatch duration x {CLOCK_HZ / 1e9:g} GHz x {SIMD_NUM} SIMDs);",
             f"util_rocprof = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x {SIMD_NUM}) (rocprofv3's MfmaUtil; its",
             "GRBM_GUI_ACTIVE reads several times the dispatch's cycles here, so it understates the busy share)", ""]
    for c in args.command:
        lines.append(f"command: {c}")
    lines += ["", f"{'kernel':16s} {'dispatches':>10s} {'mfma_GFLOP':>12s} {'dur_ms':>9s} {'TFLOP/s':>9s} "
                  f"{'busy_dur_%':>10s} {'util_rocprof_%':>14s}"]

    def mean(xs):
        xs = [x for x in xs if x is not None]
        return sum(xs) / len(xs) if xs else None
    for key, vals in sorted(per.items()):
        fl = mean([v[0] for v in vals])
        util, bd, dms = mean([v[1] for v in vals]), mean([v[2] for v in vals]), mean([v[3] for v in vals])
        rec = {"kernel": key, "workload": cfg.workload, "source_hash": source_hash(*KERNEL_SOURCES[key]),
               "mfma_flops_per_launch": fl, "mfma_busy_pct": None if bd is None else round(bd, 3),
               "mfma_util_rocprof_pct": None if util is None else round(util, 3),
               "profiled_duration_ms": None if dms is None else round(dms / 1e6, 4),
               "dispatches": len(vals), "commands": args.command}
        if fl > 0:
            with open(os.path.join(ROOT, "profiles", f"{key}_mfma.json"), "w") as f:
                json.dump(rec, f, indent=1)
        tf = fl / (dms * 1e-9) / 1e12 if dms else 0.0
        lines.append(f"{key:16s} {len(vals):10d} {fl / 1e9:12.2f} {(dms or 0) / 1e6:9.3f} {tf:9.1f} "
                     f"{'-' if bd is None else f'{bd:.2f}':>10s} {'-' if util is None else f'{util:.2f}':>14s}")
    out = os.path.join(ROOT, "profiles", f"mfma_{workload_slug(cfg)}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def calibrate_copy():
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters (run it under rocprofv3 --pmc)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        # an elementwise kernel that reads and writes n bytes (a plain copy_ may
        # go to a DMA engine, which the counters do not see)
        torch.bitwise_not(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}))


def hbm_reference(torch, gib=8, reps=5):
    """What this board's HBM delivers to plain torch kernels, after the timed
    regions: a streaming read (an fp32 tensor of `gib` GiB summed row-wise as
    [65536, -1], the fastest torch read found) and a copy (read + write).  The
    HBM-bound kernels are also reported as a fraction of the read rate."""
    n = gib << 30
    x = torch.zeros(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    xf = x.view(torch.float32).view(65536, -1)

    def med(fn):
        ts = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]
    read_ms = med(lambda: xf.sum(dim=1))
    copy_ms = med(lambda: y.copy_(x))
    del x, y, xf
    torch.cuda.empty_cache()
    return {"read_GBs": round(n / read_ms / 1e6, 1), "copy_GBs": round(2 * n / copy_ms / 1e6, 1),
            "bytes": n, "how": f"torch: {gib} GiB as fp32 [65536, -1].sum(dim=1) (read); copy_ (read + write); "
                                  f"median of {reps}"}


def annotate_reference(res, ref):
    """frac_of_read_reference beside frac for every GB/s entry of a workload's result."""
    for r in (res.get("rooflines") or {}).values():
        if r.get("unit") == "GB/s":
            r["frac_of_read_reference"] = round(r["achieved"] / ref["read_GBs"], 4)
    for r in (res.get("decode_only_rooflines") or {}).values():
        if "achieved_GBs" in r:
            r["frac_of_read_reference"] = round(r["achieved_GBs"] / ref["read_GBs"], 4)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_wise_rank_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, src_hash):
    """HBM traffic per launch measured by rocprofv3 --pmc (profiles/<kernel>_traffic.json),
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load_mfma(kernel, src_hash):
    """MFMA counters per launch (profiles/<kernel>_mfma.json), or None when absent
    or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec if rec.get("source_hash") == src_hash else None


# bf16 MFMA products each kernel issues per product of the method (term splits):
# refine: V^T in 2 bf16 terms for bf16 X, both operands in 3 terms (6 products of
# term order <= 2) for fp32 X; project: (x dtype, factor dtype) -> products.
REFINE_TERMS = {2: 2, 4: 6}
PROJECT_TERMS = {("bf16", "bf16"): 1, ("bf16", "i8"): 1, ("bf16", "f32"): 3, ("bf16", "i4"): 3,
                 ("bf16", "i2"): 3, ("f32", "bf16"): 3, ("f32", "i8"): 3, ("f32", "f32"): 6,
                 ("f32", "i4"): 6, ("f32", "i2"): 6}
GRAM_TERMS = {2: 1, 4: 6}


def tridiag_executed_flops(d=128):
    """Flops the tridiagonalisation kernel issues per matrix.  Step k (of d - 2)
    runs on the waves that hold a row > k; each of their threads (one per row)
    takes the dot product of its row with v over the groups of eight columns not
    wholly <= k (2 flops a column) and updates its row over the groups of four
    columns not wholly <= k (two FMAs an entry)."""
    total = 0
    for k in range(d - 2):
        threads = sum(64 for w in range(d // 64) if 64 * w + 63 > k)
        dot = d - 8 * ((k + 1) // 8)
        upd = d - 4 * ((k + 1) // 4)
        total += threads * (2 * dot + 4 * upd)
    return total


def qr_apply_executed_flops(rotations, d=128):
    """Flops the rotation kernel issues per matrix: the rows of Q (d - 2
    reflectors, a dot product and an update per row over the entries the
    reflector touches, in groups of eight: about d^3 / 2 FMAs in all) and every
    rotation applied to every row (two products and two FMAs: 6 flops; the
    identity rotations that fill a step's first and last groups of eight are not
    counted)."""
    touched = sum(d - (k + 1) // 8 * 8 for k in range(d - 2))
    return 2 * d * touched * 2 + 6.0 * d * rotations


def run_workload(cfg, fdt, steps, warmup, *, decode_only_steps=20, want_rebuild=True, want_offload=True,
                 want_cpu=True, counters=True, compress_streams=1, compress_chunks=1):
    """Generate the workload's inputs in HBM, time `steps` whole steps (compress
    every K and V block of every layer, then one decode step of every layer) and
    price every kernel against its roofline.  Returns the result dict."""
    import numpy as np
    import torch

    import block_wise_rank_amd as milo
    from synthetic import pool_layout
    from synthetic.planted import layer_inputs, queries, selection, tail_inputs

    dev = torch.device("cuda")
    T, d, L, H, Hq = cfg.block_len, cfg.head_dim, cfg.layers, cfg.n_kv_heads, cfg.n_q_heads
    nb_layer = cfg.blocks_per_layer
    n_all = nb_layer * L

    # ---------------- inputs (resident in HBM) ----------------
    t0 = time.time()
    xdt = torch.float32 if cfg.storage == "f32" else torch.bfloat16
    X = {k: torch.empty((n_all, T, d), dtype=xdt, device=dev) for k in ("k", "v")}
    for layer in range(L):
        for kind in ("k", "v"):
            X[kind][layer * nb_layer:(layer + 1) * nb_layer] = layer_inputs(
                cfg, layer, kind, device=dev, sub_batch=512)
        if layer % 6 == 0:
            log(f"[cfg{cfg.idx}] generated layer {layer + 1}/{L} ({time.time() - t0:.1f}s)")
    Q = [queries(cfg, layer, device=dev) for layer in range(L)]
    q_pos = torch.full((cfg.batch,), cfg.context_len + cfg.tail_len, dtype=torch.int64, device=dev)
    sel = selection(cfg)
    sel_kw = {}
    if sel is not None:
        sel_kw = dict(sel_ptr=torch.tensor(np.cumsum([0] + [len(s) for s in sel]), dtype=torch.int32, device=dev),
                      sel_blk=torch.tensor(sum(sel, []), dtype=torch.int32, device=dev),
                      sel_max=cfg.sel_blocks)
    tails = []
    tl = tp = None
    if cfg.tail_len:
        for layer in range(L):
            tails.append((tail_inputs(cfg, layer, "k", device=dev), tail_inputs(cfg, layer, "v", device=dev)))
        tl = torch.full((cfg.batch,), cfg.tail_len, dtype=torch.int32, device=dev)
        tp = torch.full((cfg.batch,), cfg.context_len, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    log(f"[cfg{cfg.idx}] inputs ready: {2 * n_all} blocks, "
        f"{2 * X['k'].numel() * X['k'].element_size() / 1e9:.1f} GB in {gen_s:.1f}s")

    # ---------------- outputs and workspaces ----------------
    pp1, bud1 = pool_layout(cfg)
    n_pools = len(bud1) * L
    pp = [p * cfg.blocks_per_seq for p in range(n_pools + 1)]
    bud = bud1 * L
    arena_bytes = milo.milo_arena_bytes(fdt, T, d, pp, bud)
    F = {k: milo.Factors.alloc(fdt, n_all, T, d, arena_bytes, device=dev) for k in ("k", "v")}
    sigma = {k: torch.empty((n_all, d), dtype=torch.float32, device=dev) for k in ("k", "v")}
    sweeps = {k: torch.empty(n_all, dtype=torch.int32, device=dev) for k in ("k", "v")}
    # Compression calls: one per kind over every layer, or `compress_chunks` calls
    # per kind over runs of whole layers; with two streams, consecutive calls
    # alternate between them (each stream its own workspace), so that one call's
    # HBM-bound passes can share the chip with another's eigensolve.  A chunk's
    # factors sit in its own slice of the arena (offsets relative to the slice).
    chunks = max(1, min(compress_chunks, L))
    bounds = [round(i * L / chunks) for i in range(chunks + 1)]
    layer_bytes = arena_bytes // L  # pools are identical per layer
    CF = {k: [] for k in ("k", "v")}
    for k in ("k", "v"):
        for c in range(chunks):
            l0, l1 = bounds[c], bounds[c + 1]
            f = F[k].view(l0 * nb_layer, (l1 - l0) * nb_layer)
            f.arena = F[k].arena[l0 * layer_bytes:l1 * layer_bytes] if chunks > 1 else F[k].arena
            CF[k].append((l0, l1, f))
    calls = [(k, c) for c in range(chunks) for k in ("k", "v")]
    side = torch.cuda.Stream() if compress_streams > 1 else None
    ws_blocks = max((l1 - l0) for l0, l1, _ in CF["k"]) * nb_layer
    ws_bytes = milo.milo_compress_workspace_bytes(ws_blocks, T, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws2 = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if side is not None else None
    outs = [torch.empty((cfg.batch, Hq, d), dtype=xdt, device=dev) for _ in range(L)]

    def layer_factors(kind, layer):
        for l0, l1, f in CF[kind]:
            if l0 <= layer < l1:
                return f.view((layer - l0) * nb_layer, nb_layer)
        raise IndexError(layer)

    def decode_kw(layer):
        kw = dict(sel_kw)
        if cfg.tail_len:
            kw.update(tail_k=tails[layer][0], tail_v=tails[layer][1], tail_len=tl, tail_pos0=tp)
        return kw

    def decode_layer(layer, dws):
        milo.milo_decode_attention(Q[layer], q_pos, layer_factors("k", layer), layer_factors("v", layer),
                                   cfg.blocks_per_seq, H, outs[layer], workspace=dws, **decode_kw(layer))

    dws_bytes = milo.decode_workspace_bytes(Q[0], layer_factors("k", 0), layer_factors("v", 0),
                                            cfg.blocks_per_seq, H, outs[0], q_pos=q_pos, **decode_kw(0))
    dws = torch.empty(dws_bytes, dtype=torch.uint8, device=dev)
    main_stream = torch.cuda.current_stream()

    def compress_all(one_stream=False):
        two = side is not None and not one_stream
        if two:
            side.wait_stream(main_stream)
        for i, (kind, c) in enumerate(calls):
            l0, l1, f = CF[kind][c]
            lo, n = l0 * nb_layer, (l1 - l0) * nb_layer
            p0 = l0 * len(bud1)
            npl = (l1 - l0) * len(bud1)
            ppc = [pp[p0 + j] - pp[p0] for j in range(npl + 1)]
            st = main_stream if (not two or i % 2 == 0) else side
            milo.milo_compress_blocks(X[kind][lo:lo + n], ppc, bud[p0:p0 + npl], cfg.eps2,
                                      sigma[kind][lo:lo + n], f, sweeps_out=sweeps[kind][lo:lo + n],
                                      workspace=ws if st is main_stream else ws2, stream=st)
        if two:
            main_stream.wait_stream(side)

    def step(record=None, one_stream=False):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        compress_all(one_stream)
        ev[1].record()
        for layer in range(L):
            decode_layer(layer, dws)
        ev[2].record()
        if record is not None:
            record.append(ev)

    # ---------------- warmup + timed steps ----------------
    log(f"[cfg{cfg.idx}] warmup {warmup} step(s)")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    rec = []
    t_start = time.perf_counter()
    for i in range(steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    comp_ms = sum(e[0].elapsed_time(e[1]) for e in rec) / steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in rec) / steps
    step_ms = wall * 1e3 / steps
    log(f"[cfg{cfg.idx}] timed {steps} step(s): {step_ms:.1f} ms/step "
        f"(compress {comp_ms:.1f}, decode {dec_ms:.2f})")
    # per-kernel times for the rooflines: the same steps again with every call on
    # one stream, so that no kernel's duration includes another's
    milo.milo_profile_read()
    milo.milo_profile_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(None, one_stream=True)
    torch.cuda.synchronize()
    one_ms = (time.perf_counter() - t1) * 1e3 / steps
    prof = milo.milo_profile_read()
    milo.milo_profile_enable(False)
    if side is not None:
        log(f"[cfg{cfg.idx}] one stream: {one_ms:.1f} ms/step")
    n_bad = int((sweeps["k"] < 0).sum() + (sweeps["v"] < 0).sum())

    # decode-only passes over the same compressed cache (the per-token regime)
    dec_only_ms, prof_dec = None, {}
    if decode_only_steps > 0:
        milo.milo_profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(decode_only_steps):
            for layer in range(L):
                decode_layer(layer, dws)
        e1.record()
        torch.cuda.synchronize()
        dec_only_ms = e0.elapsed_time(e1) / decode_only_steps
        prof_dec = milo.milo_profile_read()
        milo.milo_profile_enable(False)

    # the same decode-only pass recorded once into a graph and replayed (launch
    # gaps between the 3 L kernels of a step removed); each replay's outputs are
    # checked against the eager pass's
    dec_graph = None
    if decode_only_steps > 0:
        try:
            ref = [o.clone() for o in outs]
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for layer in range(L):
                    decode_layer(layer, dws)
            graph.replay()
            torch.cuda.synchronize()
            same = all(torch.equal(o, r) for o, r in zip(outs, ref))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(decode_only_steps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            same = same and all(torch.equal(o, r) for o, r in zip(outs, ref))
            g_ms = e0.elapsed_time(e1) / decode_only_steps
            dec_graph = {"ms_per_step": round(g_ms, 3),
                         "context_tokens_per_s": cfg.context_tokens_per_step / (g_ms / 1e3),
                         "outputs_equal_eager": bool(same)}
            del graph
        except Exception as ex:  # a runtime that cannot record these launches
            dec_graph = {"error": str(ex)[:200]}

    # the unfused alternative: rebuild every attended block into a staging cache,
    # then attend over it as an uncompressed cache (one pass over all layers)
    rebuild = None
    if want_rebuild and dec_only_ms is not None:
        # staging rows: the attended blocks back to back, then (with a tail) a copy of the tail
        n_att = cfg.blocks_per_seq if sel is None else max(len(x) for x in sel)
        stg = [torch.empty((cfg.batch, H, n_att * T + cfg.tail_len, d), dtype=torch.bfloat16, device=dev)
               for _ in range(2)]
        outs2 = torch.empty((cfg.batch, Hq, d), dtype=xdt, device=dev)
        rta_kw = {}
        if sel is not None:
            rta_kw["sel"] = sel
        if cfg.tail_len:
            rta_kw.update(tail_len=[cfg.tail_len] * cfg.batch, tail_pos0=[cfg.context_len] * cfg.batch)

        def rebuild_layer(layer):
            kw = dict(rta_kw)
            if cfg.tail_len:
                kw.update(tail_k=tails[layer][0], tail_v=tails[layer][1])
            milo.reconstruct_then_attend(Q[layer], q_pos, layer_factors("k", layer), layer_factors("v", layer),
                                         cfg.blocks_per_seq, H, outs2, staging_k=stg[0], staging_v=stg[1], **kw)
        rebuild_layer(0)
        torch.cuda.synchronize()
        milo.milo_profile_read()
        milo.milo_profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for layer in range(L):
            rebuild_layer(layer)
        e1.record()
        torch.cuda.synchronize()
        rb_ms = e0.elapsed_time(e1)
        prof_rb = milo.milo_profile_read()
        milo.milo_profile_enable(False)
        rebuild = {"ms_per_step": round(rb_ms, 3), "fused_decode_ms_per_step": round(dec_only_ms, 3),
                   "slowdown_vs_fused": round(rb_ms / dec_only_ms, 3),
                   "kernels_ms_per_step": {n: round(v[1], 3) for n, v in prof_rb.items()},
                   "staging_bytes_per_layer": 2 * stg[0].numel() * stg[0].element_size()}
        del stg
        log(f"[cfg{cfg.idx}] reconstruct-then-attend: {rb_ms:.2f} ms per step vs fused decode "
            f"{dec_only_ms:.2f} ms")

    # host-offloaded cache (the pages' throughput setting): per decode step every
    # layer's attended blocks cross PCIe from pinned host memory into HBM, layer
    # l + 1's copies overlapping layer l's attention; against offloading the full
    # bf16 KV cache the same way
    offload = None
    if want_offload:
        offload = offload_measure(milo, torch, np, cfg, layer_factors, X, Q, q_pos, sel, nb_layer, fdt, xdt,
                                  dev)

    # ---------------- algorithmic work per kernel launch ----------------
    ranks = {k: F[k].rank.to(torch.int64) for k in ("k", "v")}
    sw = torch.cat([sweeps["k"], sweeps["v"]]).to(torch.float64)
    rot_mean = float(sw.abs().mean())  # plane rotations of the QR iteration per block
    # bytes per factor element (4-bit: half a byte + an fp32 scale per 32 elements;
    # 2-bit: a quarter byte + the same scales)
    fe = {"f32": 4, "bf16": 2, "i8": 1, "i4": 5 / 8, "i2": 3 / 8}[fdt]
    xe = 4 if cfg.storage == "f32" else 2
    xname = "f32" if xe == 4 else "bf16"
    tot_rank = int(ranks["k"].sum() + ranks["v"].sum())
    rank32 = int(((ranks["k"] + 31) // 32).sum() + ((ranks["v"] + 31) // 32).sum()) * 32
    ctx_tokens = cfg.context_tokens_per_step
    n_blocks_step = 2 * n_all

    # blocks attended per layer and the factor bytes they hold
    if sel is None:
        att = torch.arange(n_all, device=dev)
    else:
        ids = []
        for layer in range(L):
            for s_ in range(cfg.batch):
                for h in range(H):
                    for b in sel[s_]:
                        ids.append(layer * nb_layer + (s_ * H + h) * cfg.blocks_per_seq + b)
        att = torch.tensor(ids, device=dev)
    att_rank = int(ranks["k"][att].sum() + ranks["v"][att].sum())
    dec_bytes_all_layers = int(att_rank * (T + d) * fe)
    if fdt == "i8":
        dec_bytes_all_layers += 4 * (2 * att.numel() * T + att_rank)
    tail_bytes_all = 2 * L * cfg.batch * H * cfg.tail_len * d * xe

    work = {
        # kernel: (algorithmic amount for the whole step, unit, bound, peak)
        "gram": (n_blocks_step * T * d * xe, "GB/s", "hbm", PEAK_HBM_GBS),
        # Householder tridiagonalisation: 4 d^3 / 3 flops; the rotation kernel: Q
        # formed from its reflectors (4 d^3 / 3) and 6 flops per rotation and row;
        # the QR chain itself: about 20 flops per rotation
        "tridiag": (n_blocks_step * 4.0 * d ** 3 / 3, "TFLOP/s", "alu", PEAK_FP32_VEC_TFLOPS),
        # Jacobi (launches of few blocks): 9 d^2 (d - 1) flops a sweep, 64 x 127
        # rotations a sweep
        "jacobi": (n_blocks_step * rot_mean / (64 * 127) * 9 * d * d * (d - 1), "TFLOP/s", "alu",
                   PEAK_FP32_VEC_TFLOPS),
        "qr_chain": (n_blocks_step * 20.0 * rot_mean, "TFLOP/s", "alu", PEAK_FP32_VEC_TFLOPS),
        "qr_apply": (n_blocks_step * (4.0 * d ** 3 / 3 + 6.0 * d * rot_mean), "TFLOP/s", "alu",
                     PEAK_FP32_VEC_TFLOPS),
        # bf16 MFMA products executed: for bf16 X, V^T split in 2 bf16 terms (2
        # products); for fp32 X both in 3 terms, term pairs of order <= 2 kept (6)
        "refine": (n_blocks_step * 2.0 * T * d * d * REFINE_TERMS[xe], "TFLOP/s", "mfma",
                   PEAK_BF16_TFLOPS),
        "alloc": (n_blocks_step * d * 4, "GB/s", "hbm", PEAK_HBM_GBS),
        "project": (n_blocks_step * T * d * xe + tot_rank * (T + d) * fe + n_blocks_step * d * d * 4,
                    "GB/s", "hbm", PEAK_HBM_GBS),
        # one launch per layer: the attended blocks' factors and the tail
        "decode": (dec_bytes_all_layers + tail_bytes_all, "GB/s", "hbm", PEAK_HBM_GBS),
        "decode_combine": (L * cfg.batch * Hq * d * 4, "GB/s", "hbm", PEAK_HBM_GBS),
    }
    # MFMA work of the contractions, per step: (algorithmic flops, executed flops)
    mfma_work = {
        "gram": (n_blocks_step * 2.0 * T * d * d, n_blocks_step * 2.0 * T * d * d * GRAM_TERMS[xe]),
        "project": (2.0 * T * d * tot_rank, 2.0 * T * d * rank32 * PROJECT_TERMS[(xname, fdt)]),
        "refine": (n_blocks_step * 2.0 * T * d * d, n_blocks_step * 2.0 * T * d * d * REFINE_TERMS[xe]),
    }
    if rebuild is not None:
        # fused: the factors (and tail) once; unfused: the factors, the staging write (tail copy
        # included) and the staging read
        rebuild["bytes_per_step"] = (dec_bytes_all_layers + tail_bytes_all
                                     + 2 * L * rebuild["staging_bytes_per_layer"])
        rebuild["fused_bytes_per_step"] = dec_bytes_all_layers + tail_bytes_all
    rooflines = {}
    for name, (launches, tot_ms) in prof.items():
        if name not in work:
            continue
        amount, unit, bound, peak = work[name]
        per_launch = amount / (launches / steps)
        avg_s = tot_ms / launches / 1e3
        achieved = per_launch / avg_s / (1e9 if unit == "GB/s" else 1e12)
        src = source_hash(*KERNEL_SOURCES[name])
        # the counters were taken on the long-context workload's own factor dtype
        traffic = load_traffic(name, src) if (counters and fdt == cfg.storage) else None
        r = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
             "frac": round(achieved / peak, 4), "traffic": traffic,
             "launches_per_step": launches / steps, "avg_launch_ms": round(tot_ms / launches, 4),
             "algorithmic_per_launch": per_launch, "source_hash": src}
        if name in mfma_work:
            alg, exe = (w / (launches / steps) for w in mfma_work[name])
            m = {"peak_TFLOPs": PEAK_BF16_TFLOPS,
                 "algorithmic_flops_per_launch": alg, "algorithmic_TFLOPs": round(alg / avg_s / 1e12, 2),
                 "algorithmic_frac": round(alg / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "executed_flops_per_launch": exe, "executed_TFLOPs": round(exe / avg_s / 1e12, 2),
                 "executed_frac": round(exe / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4)}
            cnt = load_mfma(name, src) if (counters and fdt == cfg.storage) else None
            if cnt is not None:
                m.update({"counter_flops_per_launch": cnt["mfma_flops_per_launch"],
                          "counter_TFLOPs": round(cnt["mfma_flops_per_launch"] / avg_s / 1e12, 2),
                          "counter_frac": round(cnt["mfma_flops_per_launch"] / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "counter_mfma_busy_pct": cnt.get("mfma_busy_pct")})
            r["mfma"] = m
        if name in ("tridiag", "qr_apply"):
            per_blk = tridiag_executed_flops(d) if name == "tridiag" else qr_apply_executed_flops(rot_mean, d)
            exe = n_blocks_step * per_blk / (launches / steps)
            r["executed"] = {"flops_per_launch": exe, "TFLOPs": round(exe / avg_s / 1e12, 3),
                             "peak_TFLOPs": PEAK_FP32_VEC_NONPACKED_TFLOPS,
                             "frac": round(exe / avg_s / 1e12 / PEAK_FP32_VEC_NONPACKED_TFLOPS, 4)}
        rooflines[name] = r
    # decode-only rooflines (the per-token regime), same kernels
    dec_only = {}
    for name, (launches, tot_ms) in prof_dec.items():
        if name in work and name.startswith("decode"):
            amount = work[name][0]
            per_launch = amount / (launches / decode_only_steps)
            avg_s = tot_ms / launches / 1e3
            ach = per_launch / avg_s / 1e9
            dec_only[name] = {"achieved_GBs": round(ach, 1), "frac_hbm": round(ach / PEAK_HBM_GBS, 4),
                              "avg_launch_ms": round(tot_ms / launches, 4)}
    if dec_only_ms is not None:
        dec_bytes = dec_bytes_all_layers + tail_bytes_all
        dec_only["step"] = {"bytes": dec_bytes, "ms": round(dec_only_ms, 4),
                            "achieved_GBs": round(dec_bytes / dec_only_ms / 1e6, 1),
                            "frac_hbm": round(dec_bytes / dec_only_ms / 1e6 / PEAK_HBM_GBS, 4)}
    dominant = max(prof, key=lambda n: prof[n][1]) if prof else None
    roof = {k: rooflines[dominant][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")} \
        if dominant in rooflines else None
    if roof is not None:
        roof["kernel"] = dominant
        if "executed" in rooflines[dominant]:
            roof["executed"] = rooflines[dominant]["executed"]

    full_kv = 2 * n_all * T * d * 2
    factor_bytes = int(tot_rank * (T + d) * fe) + (4 * (2 * n_all * T + tot_rank) if fdt == "i8" else 0)

    cpu = None
    if want_cpu:
        cpu = cpu_baseline(cfg, fdt, X, Q, q_pos, sel, tails, nb_layer, L, ctx_tokens)

    return {
        "step_ms": step_ms,
        "config": {"workload": cfg.workload, "config_index": cfg.idx, "layers": L, "n_kv_heads": H,
                   "n_q_heads": Hq, "head_dim": d, "block_len": T, "blocks_per_seq": cfg.blocks_per_seq,
                   "batch": cfg.batch, "attended_blocks_per_seq": cfg.attended_blocks,
                   "tail_len": cfg.tail_len, "budget_frac": cfg.budget_fracs[0], "factor_dtype": fdt,
                   "context_tokens_per_step": ctx_tokens, "blocks_compressed_per_step": n_blocks_step,
                   "compress_calls_per_step": len(calls), "compress_streams": 1 if side is None else 2},
        "breakdown": {
            "compress_ms": round(comp_ms, 3), "decode_ms": round(dec_ms, 3),
            "blocks_per_s": n_blocks_step / (comp_ms / 1e3),
            "decode_context_tokens_per_s": ctx_tokens / (dec_ms / 1e3),
            "decode_only_ms_per_step": None if dec_only_ms is None else round(dec_only_ms, 3),
            "decode_only_context_tokens_per_s": None if dec_only_ms is None else ctx_tokens / (dec_only_ms / 1e3),
            "decode_only_graph": dec_graph,
            "one_stream_ms_per_step": round(one_ms, 3),
            "eig_rotations_mean": round(rot_mean, 1),
            "blocks_at_step_cap": n_bad,
            "kernels_ms_per_step": {n: round(v[1] / steps, 3) for n, v in prof.items()},
            "input_generation_s": round(gen_s, 1),
        },
        "roofline": roof,
        "rooflines": rooflines,
        "decode_only_rooflines": dec_only,
        "reconstruct_then_attend": rebuild,
        "offload": offload,
        "memory": {"full_kv_bf16_bytes": full_kv, "factor_bytes": factor_bytes,
                   "ratio": round(factor_bytes / full_kv, 4)},
        "cpu_baseline": cpu,
    }


def run_warm_cold(cfg, fdt, iters=20, copies=16):
    """Compression of a one-layer workload small enough to stay in the 256 MB
    last-level cache (MALL): 'warm' compresses the same input every iteration
    (just written, cache-resident); 'cold' cycles through `copies` copies of it
    (over 256 MB together), so every iteration reads its input from HBM.  Also
    one decode step, warm.  Per-kernel times come from HIP events on the call's
    stream; MFMA work as in run_workload."""
    import torch

    import block_wise_rank_amd as milo
    from synthetic import pool_layout
    from synthetic.planted import layer_inputs, queries

    dev = torch.device("cuda")
    T, d, H, Hq = cfg.block_len, cfg.head_dim, cfg.n_kv_heads, cfg.n_q_heads
    X = {k: layer_inputs(cfg, 0, k, device=dev) for k in ("k", "v")}
    n = X["k"].shape[0]
    cold = {k: [X[k].clone() for _ in range(copies)] for k in ("k", "v")}
    pp, bud = pool_layout(cfg)
    arena = milo.milo_arena_bytes(fdt, T, d, pp, bud)
    F = {k: milo.Factors.alloc(fdt, n, T, d, arena, device=dev) for k in ("k", "v")}
    sig = {k: torch.empty((n, d), dtype=torch.float32, device=dev) for k in ("k", "v")}
    ws = torch.empty(milo.milo_compress_workspace_bytes(n, T, d), dtype=torch.uint8, device=dev)
    xe = 4 if cfg.storage == "f32" else 2
    xname = "f32" if xe == 4 else "bf16"

    ws2 = torch.empty_like(ws)
    side = torch.cuda.Stream()
    main_stream = torch.cuda.current_stream()
    streams = {"k": main_stream, "v": main_stream}

    def comp(src):
        if streams["v"] is not main_stream:
            side.wait_stream(main_stream)
        for k in ("k", "v"):
            milo.milo_compress_blocks(src[k], pp, bud, cfg.eps2, sig[k], F[k],
                                      workspace=ws if streams[k] is main_stream else ws2, stream=streams[k])
        if streams["v"] is not main_stream:
            main_stream.wait_stream(side)

    res = {"workload": cfg.workload, "blocks_per_iteration": 2 * n, "iterations": iters,
           "input_bytes_per_iteration": 2 * X["k"].numel() * X["k"].element_size(),
           "cold_copies": copies, "cold_bytes": copies * 2 * X["k"].numel() * X["k"].element_size()}
    # warm / cold: K then V on one stream; warm_two_streams: the K and V calls on
    # two streams, so that their eigensolves (one workgroup per block, far fewer
    # blocks than CUs) run side by side
    for mode in ("warm", "cold", "warm_two_streams"):
        streams["v"] = side if mode == "warm_two_streams" else main_stream
        for i in range(3):
            comp(X if mode != "cold" else {k: cold[k][i % copies] for k in ("k", "v")})
        torch.cuda.synchronize()
        milo.milo_profile_read()
        milo.milo_profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            comp(X if mode != "cold" else {k: cold[k][i % copies] for k in ("k", "v")})
        e1.record()
        torch.cuda.synchronize()
        prof = milo.milo_profile_read()
        milo.milo_profile_enable(False)
        ms = e0.elapsed_time(e1) / iters
        ranks = torch.cat([F["k"].rank, F["v"].rank]).to(torch.int64)
        tot_rank = int(ranks.sum())
        rank32 = int(((ranks + 31) // 32).sum()) * 32
        mw = {"gram": (2 * n * 2.0 * T * d * d, 2 * n * 2.0 * T * d * d * GRAM_TERMS[xe]),
              "project": (2.0 * T * d * tot_rank, 2.0 * T * d * rank32 * PROJECT_TERMS[(xname, fdt)]),
              "refine": (2 * n * 2.0 * T * d * d, 2 * n * 2.0 * T * d * d * REFINE_TERMS[xe])}
        kern = {}
        for name, (launches, tot_ms) in prof.items():
            avg_s = tot_ms / launches / 1e3
            e = {"avg_launch_ms": round(tot_ms / launches, 4), "ms_per_iteration": round(tot_ms / iters, 4)}
            if name in mw:
                alg, exe = (w / (launches / iters) for w in mw[name])
                e.update({"algorithmic_TFLOPs": round(alg / avg_s / 1e12, 2),
                          "algorithmic_frac_bf16": round(alg / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "executed_TFLOPs": round(exe / avg_s / 1e12, 2),
                          "executed_frac_bf16": round(exe / avg_s / 1e12 / PEAK_BF16_TFLOPS, 4)})
            if name in ("gram", "refine", "project"):
                xb = n * T * d * xe  # this launch's input blocks
                e["input_GBs"] = round(xb / avg_s / 1e9, 1)
            kern[name] = e
        res[mode] = {"ms_per_iteration": round(ms, 4), "blocks_per_s": 2 * n / (ms / 1e3), "kernels": kern}
        log(f"[cfg{cfg.idx} {mode}] compress {ms:.3f} ms per iteration ({2 * n} blocks)")
    # one decode step (all blocks attended), warm
    q = queries(cfg, 0, device=dev)
    q_pos = torch.full((cfg.batch,), cfg.context_len, dtype=torch.int64, device=dev)
    out = torch.empty((cfg.batch, Hq, d), dtype=torch.float32, device=dev)
    dws = torch.empty(milo.decode_workspace_bytes(q, F["k"], F["v"], cfg.blocks_per_seq, H, out, q_pos=q_pos),
                      dtype=torch.uint8, device=dev)
    for _ in range(3):
        milo.milo_decode_attention(q, q_pos, F["k"], F["v"], cfg.blocks_per_seq, H, out, workspace=dws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        milo.milo_decode_attention(q, q_pos, F["k"], F["v"], cfg.blocks_per_seq, H, out, workspace=dws)
    e1.record()
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / iters
    res["decode_step_ms"] = round(dms, 4)
    res["decode_context_tokens_per_s"] = cfg.context_tokens_per_step / (dms / 1e3)
    return res


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return 0
    if args.ingest_stats:
        ingest_stats(args)
        return 0
    if args.ingest_traffic:
        ingest_traffic(args)
        return 0
    if args.ingest_mfma:
        ingest_mfma(args)
        return 0
    if args.filter_csv:
        import csv
        src, dst = args.filter_csv
        with open(src, newline="") as f, open(dst, "w", newline="") as g:
            rd = csv.DictReader(f)
            wr = csv.DictWriter(g, fieldnames=rd.fieldnames)
            wr.writeheader()
            for row in rd:
                if "milo::" in row.get("Kernel_Name", ""):
                    wr.writerow(row)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; "
              "rerun with --gpus 1", file=sys.stderr)
        return 2

    import torch

    from synthetic import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    cfg = CONFIGS[args.config]
    fdt = args.factor_dtype or cfg.storage
    main_res = run_workload(cfg, fdt, args.steps, args.warmup, decode_only_steps=args.decode_only_steps,
                            want_offload=not args.no_offload, want_cpu=not args.no_cpu_baseline,
                            compress_streams=args.compress_streams, compress_chunks=args.compress_chunks)
    torch.cuda.empty_cache()
    extra = {}
    for item in [x.strip() for x in args.extra.split(",") if x.strip()] if args.extra != "none" else []:
        c, _, edt = item.partition(":")
        c = int(c)
        ecfg = CONFIGS[c]
        if edt:
            # the same workload with another factor format (its offload step included)
            if edt == fdt and c == args.config:
                continue
            r = run_workload(ecfg, edt, 2, 1, decode_only_steps=10, want_rebuild=False,
                             want_offload=True, want_cpu=False, counters=False,
                             compress_streams=args.compress_streams)
            r["ms_per_step"] = round(r.pop("step_ms"), 3)
            r["value"] = ecfg.context_tokens_per_step / (r["ms_per_step"] / 1e3)
            extra[f"config{c}_{edt}"] = r
            torch.cuda.empty_cache()
            continue
        if c == args.config:
            continue
        if ecfg.layers == 1:
            extra[f"config{c}"] = run_warm_cold(ecfg, ecfg.storage)
        else:
            r = run_workload(ecfg, ecfg.storage, 3, 1, decode_only_steps=10, want_rebuild=True,
                             want_offload=False, want_cpu=False, counters=False,
                             compress_streams=args.compress_streams)
            r["ms_per_step"] = round(r.pop("step_ms"), 3)
            r["value"] = ecfg.context_tokens_per_step / (r["ms_per_step"] / 1e3)
            extra[f"config{c}"] = r
        torch.cuda.empty_cache()

    ref = hbm_reference(torch)
    annotate_reference(main_res, ref)
    for r in extra.values():
        annotate_reference(r, ref)
    step_ms = main_res.pop("step_ms")
    out = {
        "metric": METRIC,
        "value": cfg.context_tokens_per_step / (step_ms / 1e3),
        "unit": "context-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if fdt == "bf16" else fdt,
        "data": "synthetic: seeded planted-spectrum K/V blocks X = U diag(exp(-i/tau)) V^T + N(0,1e-3^2), "
                "N(0,1) queries",
        "value_definition": "context tokens attended per second of a WHOLE step = compress every K and V "
                            "block of every layer (all blocks_compressed_per_step) + one decode step of every "
                            "layer; decode alone: breakdown.decode_only_context_tokens_per_s; compression "
                            "alone: breakdown.blocks_per_s",
    }
    out.update(main_res)
    out["hbm_reference"] = ref
    out["workloads"] = extra
    print(json.dumps(out))
    return 0


def offload_measure(milo, torch, np, cfg, layer_factors, X, Q, q_pos, sel, nb_layer, fdt, xdt, dev, n_src=2):
    """Decode over all layers with the cache in pinned host memory.  n_src
    distinct layers are held on the host and cycled through (the copies do not
    depend on the bytes); two device buffers alternate, the copy stream filling
    one while the compute stream attends over the other."""
    T, d, L, H, Hq = cfg.block_len, cfg.head_dim, cfg.layers, cfg.n_kv_heads, cfg.n_q_heads
    bps = cfg.blocks_per_seq
    n_src = min(n_src, L)
    if sel is None:
        ids = list(range(nb_layer))
        sel_kw = {}
    else:
        ids = [(s_ * H + h) * bps + b for s_ in range(cfg.batch) for h in range(H) for b in sel[s_]]
        sel_kw = dict(sel_ptr=torch.tensor(np.cumsum([0] + [len(x) for x in sel]), dtype=torch.int32, device=dev),
                      sel_blk=torch.tensor(sum(sel, []), dtype=torch.int32, device=dev), sel_max=cfg.sel_blocks)
    ids_t = torch.tensor(ids, dtype=torch.int32)
    es = {"f32": 4, "bf16": 2, "i8": 1, "i4": 5 / 8, "i2": 3 / 8}[fdt]

    def layer_host_set(kind, layer):
        """A compact pinned-host copy of one layer's factor set (offsets rebased)."""
        v = layer_factors(kind, layer)
        lo = int(v.a_off.min())
        hi = int((v.b_off + (v.rank.to(torch.int64) * int(d * es))).max())
        h = milo.Factors(fdt, nb_layer, T, d, rank=v.rank.cpu().pin_memory(), a_off=(v.a_off - lo).cpu().pin_memory(),
                         b_off=(v.b_off - lo).cpu().pin_memory(), arena=v.arena[lo:hi].cpu().pin_memory())
        if fdt == "i8":
            h.a_scale, h.b_scale = v.a_scale.cpu().pin_memory(), v.b_scale.cpu().pin_memory()
        return h

    out = torch.empty((cfg.batch, Hq, d), dtype=xdt, device=dev)
    cs = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def run(fetch, attend):
        fetched = [torch.cuda.Event() for _ in range(2)]
        used = [torch.cuda.Event() for _ in range(2)]
        for layer in range(L):
            j = layer % 2
            with torch.cuda.stream(cs):
                if layer >= 2:
                    cs.wait_event(used[j])
                fetch(layer, j)
                fetched[j].record(cs)
            main.wait_event(fetched[j])
            attend(layer, j)
            used[j].record(main)

    def timed(fetch, attend):
        run(fetch, attend)  # warm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run(fetch, attend)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # compressed: the factor sets of n_src layers on the host (each with its own
    # layout, whose device copy of the metadata the device buffer takes on)
    hk = [layer_host_set("k", l) for l in range(n_src)]
    hv = [layer_host_set("v", l) for l in range(n_src)]
    meta = [(hk[i].like(dev), hv[i].like(dev)) for i in range(n_src)]
    cap_k = max(h.arena.numel() for h in hk)
    cap_v = max(h.arena.numel() for h in hv)
    dk = [milo.Factors.alloc(fdt, nb_layer, T, d, cap_k, device=dev) for _ in range(2)]
    dv = [milo.Factors.alloc(fdt, nb_layer, T, d, cap_v, device=dev) for _ in range(2)]
    for m in meta:  # the metadata sets need no arenas of their own
        m[0].arena = m[1].arena = None

    def fetch_c(layer, j):
        i = layer % n_src
        dk[j].rank, dk[j].a_off, dk[j].b_off = meta[i][0].rank, meta[i][0].a_off, meta[i][0].b_off
        dv[j].rank, dv[j].a_off, dv[j].b_off = meta[i][1].rank, meta[i][1].a_off, meta[i][1].b_off
        milo.milo_fetch_blocks(hk[i], dk[j], ids_t, stream=cs)
        milo.milo_fetch_blocks(hv[i], dv[j], ids_t, stream=cs)

    def attend_c(layer, j):
        milo.milo_decode_attention(Q[layer], q_pos, dk[j], dv[j], bps, H, out, **sel_kw)

    comp_ms = timed(fetch_c, attend_c)
    comp_bytes = 0
    for i in range(n_src):
        for h in (hk[i], hv[i]):
            r = h.rank.to(torch.int64)[ids_t.long()]
            comp_bytes += int(int(r.sum()) * (T + d) * es) + (4 * len(ids) * (T + d) if fdt == "i8" else 0)
    comp_bytes = comp_bytes * L / n_src
    del hk, hv, dk, dv, meta

    # full KV: the attended blocks' bf16 keys (pre-RoPE) and values on the host,
    # attended as an uncompressed cache (positions b * T + t as for the blocks)
    nsel = len(sel[0]) if sel is not None else bps
    if sel is not None and any(len(x) != nsel for x in sel):
        return {"compressed_ms_per_step": round(comp_ms, 3), "note": "ragged selections: full-KV side skipped"}

    def host_cache(kind, layer):
        xs = X[kind][layer * nb_layer:(layer + 1) * nb_layer].view(cfg.batch, H, bps, T, d)
        if sel is not None:
            xs = torch.stack([xs[s_][:, sel[s_]] for s_ in range(cfg.batch)])
        return xs.reshape(cfg.batch, H, nsel * T, d).to(torch.bfloat16).cpu().pin_memory()

    fk = [host_cache("k", l) for l in range(n_src)]
    fv = [host_cache("v", l) for l in range(n_src)]
    sk = [torch.empty(fk[0].shape, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    sv = [torch.empty(fv[0].shape, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    tl = torch.full((cfg.batch,), nsel * T, dtype=torch.int32, device=dev)
    tp = torch.zeros(cfg.batch, dtype=torch.int64, device=dev)
    empty = milo.Factors.alloc(fdt, 1, T, d, 256, device=dev)

    def fetch_f(layer, j):
        i = layer % n_src
        sk[j].copy_(fk[i], non_blocking=True)
        sv[j].copy_(fv[i], non_blocking=True)

    def attend_f(layer, j):
        milo.milo_decode_attention(Q[layer], q_pos, empty, empty, 0, H, out, tail_k=sk[j], tail_v=sv[j],
                                   tail_len=tl, tail_pos0=tp)

    full_ms = timed(fetch_f, attend_f)
    full_bytes = 2 * L * fk[0].numel() * 2
    del fk, fv, sk, sv
    ctx = cfg.context_tokens_per_step
    return {"compressed_ms_per_step": round(comp_ms, 3), "full_kv_ms_per_step": round(full_ms, 3),
            "speedup_vs_full_kv": round(full_ms / comp_ms, 3),
            "compressed_bytes_per_step": comp_bytes, "full_kv_bytes_per_step": full_bytes,
            "compressed_host_to_device_GBs": round(comp_bytes / comp_ms / 1e6, 1),
            "full_kv_host_to_device_GBs": round(full_bytes / full_ms / 1e6, 1),
            "compressed_context_tokens_per_s": ctx / (comp_ms / 1e3),
            "full_kv_context_tokens_per_s": ctx / (full_ms / 1e3),
            "host_layers_cycled": n_src}


def cpu_baseline(cfg, fdt, X, Q, q_pos, sel, tails, nb_layer, L, ctx_tokens, single_thread_blocks=8):
    """The oracle, as it stands, on one (sequence, layer, KV head) unit of the
    workload: the SVD of its K and V pools (the oracle's OpenMP block loop), the
    allocation and factors, and the decode of its query heads over the attended
    blocks (and tail); scaled to the whole step by the number of such units.
    Timed at all host threads (the whole pools) and at one thread (the SVD of the
    first `single_thread_blocks` blocks of each pool, scaled per block; the rest
    of the unit is single-threaded in both)."""
    import torch

    import oracle
    T, d, H = cfg.block_len, cfg.head_dim, cfg.n_kv_heads
    bps = cfg.blocks_per_seq
    Xk = X["k"][0:bps].to(torch.float64).cpu().numpy()
    Xv = X["v"][0:bps].to(torch.float64).cpu().numpy()
    q = Q[0][0:1, 0:cfg.group].to(torch.float64).cpu().numpy()
    R = cfg.budget()
    nproc = oracle.max_threads()

    t0 = time.perf_counter()
    svd_k = oracle.svd_blocks(Xk)
    svd_v = oracle.svd_blocks(Xv)
    t_svd = time.perf_counter() - t0
    t0 = time.perf_counter()
    ck = oracle.compress(Xk, [0, bps], [R], cfg.eps2, fdt, svd=svd_k)
    cv = oracle.compress(Xv, [0, bps], [R], cfg.eps2, fdt, svd=svd_v)
    blocks = list(range(bps)) if sel is None else sel[0]
    Kh = {b: oracle.reconstruct(ck.A[b], ck.B[b]) for b in blocks}
    Vh = {b: oracle.reconstruct(cv.A[b], cv.B[b]) for b in blocks}
    kw = {}
    if cfg.tail_len:
        kw = dict(tail_k=tails[0][0][0:1, 0:1].to(torch.float64).cpu().numpy(),
                  tail_v=tails[0][1][0:1, 0:1].to(torch.float64).cpu().numpy(),
                  tail_len=[cfg.tail_len], tail_pos0=[cfg.context_len])
    oracle.decode(q, [int(q_pos[0])], lambda i: Kh[i], lambda i: Vh[i], T, 1, bps,
                  sel=None if sel is None else [sel[0]], rope_base=cfg.rope_base, **kw)
    t_rest = time.perf_counter() - t0

    m = min(single_thread_blocks, bps)
    prev = oracle.set_threads(1)
    t0 = time.perf_counter()
    oracle.svd_blocks(Xk[:m])
    oracle.svd_blocks(Xv[:m])
    t_svd1 = (time.perf_counter() - t0) * bps / m
    oracle.set_threads(prev)

    units = L * cfg.batch * H
    t_all, t_one = t_svd + t_rest, t_svd1 + t_rest
    what = (f"compress its K and V pools ({2 * bps} blocks of {T}x{d}) and decode its {cfg.group} query heads "
            f"over {cfg.attended_blocks} blocks" + (f" + {cfg.tail_len}-token tail" if cfg.tail_len else ""))
    return {"value": ctx_tokens / (t_all * units), "unit": "context-tokens/s",
            "cores": nproc, "kind": "oracle",
            "sample": f"1 of {units} (layer, sequence, KV head) units: {what}; SVD on {nproc} threads "
                      f"{t_svd:.1f} s, allocation + factors + decode single-threaded {t_rest:.1f} s; "
                      f"value = step context tokens / (t x {units})",
            "sample_seconds": round(t_all, 2), "cpu_model": cpu_model(),
            "single_thread": {"value": ctx_tokens / (t_one * units), "cores": 1,
                              "sample": f"the same unit with the SVD of {m} of the {bps} blocks of each pool "
                                        f"on one thread ({t_svd1 * m / bps:.1f} s, scaled x{bps / m:g}) "
                                        f"+ the same single-threaded rest",
                              "sample_seconds": round(t_svd1 * m / bps + t_rest, 2)}}


if __name__ == "__main__":
    sys.exit(main())
