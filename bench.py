#!/usr/bin/env python3
"""Benchmark of the MILO hot path on one MI355X.

One step = one pass of the whole path over the workload's KV cache: compress
every K block and every V block of every layer (Gram -> Jacobi eigensolve ->
singular-value refinement -> rank allocation -> factors), then one decode step
of every layer over the compressed blocks.  Inputs (planted-spectrum blocks and
queries, seeded) are generated on the GPU and resident in HBM before timing.

Prints ONE JSON line.  `value` is context tokens (sum over sequences of the
tokens attended in the decode step) per second of step time; the breakdown
reports compression blocks/s and decode context-tokens/s on their own, and a
roofline entry for every kernel from per-kernel HIP-event timings taken inside
the timed steps.

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
METRIC = ("compressed-KV decode context-tokens/s (+HBM %peak); blocks/s compressed (+MFMA %)")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--factor-dtype", default=None, help="bf16 | i8 | i4 (default: the config's)")
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
    ap.add_argument("--command", action="append", default=[],
                    help="with --ingest-*: the command(s) that produced the CSV files")
    return ap.parse_args()


# kernel -> the sources that define it (the traffic records are tied to their hash)
KERNEL_SOURCES = {"gram": ["gram.hip", "common.hpp"], "jacobi": ["jacobi.hip"],
                  "refine": ["refine.hip", "common.hpp"], "alloc": ["alloc.hip"],
                  "project": ["project.hip", "common.hpp"], "reconstruct": ["reconstruct.hip", "common.hpp"],
                  "decode_blocks": ["decode.hip", "common.hpp"], "decode_tail": ["decode.hip", "common.hpp"],
                  "decode_combine": ["decode.hip", "common.hpp"], "decode_tables": ["decode.hip"]}


def kernel_key(name):
    """libmilo kernel name (as rocprofv3 prints it) -> bench kernel key."""
    for frag, key in (("gram_kernel", "gram"), ("gram_bf16_kernel", "gram"), ("jacobi_kernel", "jacobi"),
                      ("refine_kernel", "refine"), ("alloc_kernel", "alloc"), ("project_kernel", "project"),
                      ("project_bf16_kernel", "project"), ("reconstruct_kernel", "reconstruct"),
                      ("reconstruct_bf16_kernel", "reconstruct"), ("decode_combine_kernel", "decode_combine"),
                      ("decode_tables_kernel", "decode_tables")):
        if frag in name:
            return key
    if "decode_partial_kernel" in name:
        return "decode_tail" if "true>" in name else "decode_blocks"
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
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; "
              "rerun with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_wise_rank_amd as milo
    from synthetic import CONFIGS, derive_seed, pool_layout
    from synthetic.planted import layer_inputs, queries, selection, tail_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    cfg = CONFIGS[args.config]
    fdt = args.factor_dtype or cfg.storage
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
            log(f"generated layer {layer + 1}/{L} ({time.time() - t0:.1f}s)")
    Q = [queries(cfg, layer, device=dev) for layer in range(L)]
    q_pos = torch.full((cfg.batch,), cfg.context_len + cfg.tail_len, dtype=torch.int64, device=dev)
    sel = selection(cfg)
    sel_kw = {}
    if sel is not None:
        sel_kw = dict(sel_ptr=torch.tensor(np.cumsum([0] + [len(s) for s in sel]), dtype=torch.int32, device=dev),
                      sel_blk=torch.tensor(sum(sel, []), dtype=torch.int32, device=dev),
                      sel_max=cfg.sel_blocks)
    tails = []
    if cfg.tail_len:
        for layer in range(L):
            tails.append((tail_inputs(cfg, layer, "k", device=dev), tail_inputs(cfg, layer, "v", device=dev)))
        tl = torch.full((cfg.batch,), cfg.tail_len, dtype=torch.int32, device=dev)
        tp = torch.full((cfg.batch,), cfg.context_len, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    log(f"inputs ready: {2 * n_all} blocks, {2 * X['k'].numel() * X['k'].element_size() / 1e9:.1f} GB "
        f"in {gen_s:.1f}s")

    # ---------------- outputs and workspaces ----------------
    pp1, bud1 = pool_layout(cfg)
    n_pools = len(bud1) * L
    pp = [p * cfg.blocks_per_seq for p in range(n_pools + 1)]
    bud = bud1 * L
    arena_bytes = milo.milo_arena_bytes(fdt, T, d, pp, bud)
    F = {k: milo.Factors.alloc(fdt, n_all, T, d, arena_bytes, device=dev) for k in ("k", "v")}
    sigma = {k: torch.empty((n_all, d), dtype=torch.float32, device=dev) for k in ("k", "v")}
    sweeps = {k: torch.empty(n_all, dtype=torch.int32, device=dev) for k in ("k", "v")}
    ws_bytes = milo.milo_compress_workspace_bytes(n_all, T, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = [torch.empty((cfg.batch, Hq, d), dtype=xdt, device=dev) for _ in range(L)]

    def decode_layer(layer, dws):
        kw = dict(sel_kw)
        if cfg.tail_len:
            kw.update(tail_k=tails[layer][0], tail_v=tails[layer][1], tail_len=tl, tail_pos0=tp)
        milo.milo_decode_attention(Q[layer], q_pos, F["k"].view(layer * nb_layer, nb_layer),
                                   F["v"].view(layer * nb_layer, nb_layer), cfg.blocks_per_seq, H,
                                   outs[layer], workspace=dws, **kw)

    kw0 = dict(sel_kw)
    if cfg.tail_len:
        kw0.update(tail_k=tails[0][0], tail_v=tails[0][1], tail_len=tl, tail_pos0=tp)
    dws_bytes = milo.decode_workspace_bytes(Q[0], F["k"].view(0, nb_layer), F["v"].view(0, nb_layer),
                                            cfg.blocks_per_seq, H, outs[0], q_pos=q_pos, **kw0)
    dws = torch.empty(dws_bytes, dtype=torch.uint8, device=dev)

    def step(record=None):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        for kind in ("k", "v"):
            milo.milo_compress_blocks(X[kind], pp, bud, cfg.eps2, sigma[kind], F[kind],
                                      sweeps_out=sweeps[kind], workspace=ws)
        ev[1].record()
        for layer in range(L):
            decode_layer(layer, dws)
        ev[2].record()
        if record is not None:
            record.append(ev)

    # ---------------- warmup + timed steps ----------------
    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    milo.milo_profile_read()
    milo.milo_profile_enable(True)
    rec = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    prof = milo.milo_profile_read()
    milo.milo_profile_enable(False)
    comp_ms = sum(e[0].elapsed_time(e[1]) for e in rec) / args.steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in rec) / args.steps
    step_ms = wall * 1e3 / args.steps
    log(f"timed {args.steps} step(s): {step_ms:.1f} ms/step (compress {comp_ms:.1f}, decode {dec_ms:.2f})")

    # decode-only passes over the same compressed cache (the per-token regime)
    milo.milo_profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.decode_only_steps):
        for layer in range(L):
            decode_layer(layer, dws)
    e1.record()
    torch.cuda.synchronize()
    dec_only_ms = e0.elapsed_time(e1) / max(1, args.decode_only_steps)
    prof_dec = milo.milo_profile_read()
    milo.milo_profile_enable(False)

    # the unfused alternative: rebuild every attended block into a staging cache,
    # then attend over it as an uncompressed cache (one pass over all layers)
    rebuild = None
    if sel is None and not cfg.tail_len:
        stg = [torch.empty((cfg.batch, H, cfg.blocks_per_seq * T, d), dtype=torch.bfloat16, device=dev)
               for _ in range(2)]
        outs2 = torch.empty((cfg.batch, Hq, d), dtype=xdt, device=dev)

        def rebuild_layer(layer):
            milo.reconstruct_then_attend(Q[layer], q_pos, F["k"].view(layer * nb_layer, nb_layer),
                                         F["v"].view(layer * nb_layer, nb_layer), cfg.blocks_per_seq, H,
                                         outs2, staging_k=stg[0], staging_v=stg[1])
        rebuild_layer(0)
        torch.cuda.synchronize()
        milo.milo_profile_read()
        milo.milo_profile_enable(True)
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
        log(f"reconstruct-then-attend: {rb_ms:.2f} ms per step vs fused decode {dec_only_ms:.2f} ms")

    # host-offloaded cache (the pages' throughput setting): per decode step every
    # layer's attended blocks cross PCIe from pinned host memory into HBM, layer
    # l + 1's copies overlapping layer l's attention; against offloading the full
    # bf16 KV cache the same way
    offload = None
    if not args.no_offload:
        offload = offload_measure(milo, torch, np, cfg, F, X, Q, q_pos, sel, nb_layer, fdt, xdt, dev)

    # ---------------- algorithmic work per kernel launch ----------------
    ranks = {k: F[k].rank.to(torch.int64) for k in ("k", "v")}
    sw = torch.cat([sweeps["k"], sweeps["v"]]).to(torch.float64)
    sweeps_mean = float(sw.abs().mean())
    # bytes per factor element (4-bit: half a byte + an fp32 scale per 32 elements)
    fe = {"f32": 4, "bf16": 2, "i8": 1, "i4": 5 / 8}[fdt]
    xe = 4 if cfg.storage == "f32" else 2
    tot_rank = int(ranks["k"].sum() + ranks["v"].sum())
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
    q_bytes = L * cfg.batch * Hq * d * xe * 2

    work = {
        # kernel: (algorithmic amount for the whole step, unit, bound, peak)
        "gram": (n_blocks_step * T * d * xe, "GB/s", "hbm", PEAK_HBM_GBS),
        "jacobi": (n_blocks_step * sweeps_mean * 9 * d * d * (d - 1), "TFLOP/s", "alu", PEAK_FP32_VEC_TFLOPS),
        # bf16 MFMA products executed: for bf16 X, V^T split in 2 bf16 terms (2
        # products); for fp32 X both in 3 terms, term pairs of order <= 2 kept (6)
        "refine": (n_blocks_step * 2.0 * T * d * d * (2 if xe == 2 else 6), "TFLOP/s", "mfma",
                   PEAK_BF16_TFLOPS),
        "alloc": (n_blocks_step * d * 4, "GB/s", "hbm", PEAK_HBM_GBS),
        "project": (n_blocks_step * T * d * xe + tot_rank * (T + d) * fe + n_blocks_step * d * d * 4,
                    "GB/s", "hbm", PEAK_HBM_GBS),
        "decode_blocks": (dec_bytes_all_layers, "GB/s", "hbm", PEAK_HBM_GBS),
        "decode_tail": (tail_bytes_all, "GB/s", "hbm", PEAK_HBM_GBS),
        "decode_combine": (L * cfg.batch * Hq * d * 4, "GB/s", "hbm", PEAK_HBM_GBS),
    }
    if rebuild is not None:
        # fused: the factors once; unfused: the factors, the staging write, the staging read
        rebuild["bytes_per_step"] = dec_bytes_all_layers + 2 * L * rebuild["staging_bytes_per_layer"]
        rebuild["fused_bytes_per_step"] = dec_bytes_all_layers
    hashes = KERNEL_SOURCES
    rooflines = {}
    for name, (launches, tot_ms) in prof.items():
        if name not in work:
            continue
        amount, unit, bound, peak = work[name]
        per_launch = amount / (launches / args.steps)
        avg_s = tot_ms / launches / 1e3
        achieved = per_launch / avg_s / (1e9 if unit == "GB/s" else 1e12)
        src = source_hash(*hashes[name])
        # the counters were taken on the workload's own factor dtype
        traffic = load_traffic(name, src) if fdt == cfg.storage else None
        rooflines[name] = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                           "frac": round(achieved / peak, 4), "traffic": traffic,
                           "launches_per_step": launches / args.steps,
                           "avg_launch_ms": round(tot_ms / launches, 4),
                           "algorithmic_per_launch": per_launch, "source_hash": src}
    # decode-only rooflines (the per-token regime), same kernels
    dec_only = {}
    for name, (launches, tot_ms) in prof_dec.items():
        if name in work and name.startswith("decode"):
            amount = work[name][0]
            per_launch = amount / (launches / args.decode_only_steps)
            avg_s = tot_ms / launches / 1e3
            ach = per_launch / avg_s / 1e9
            dec_only[name] = {"achieved_GBs": round(ach, 1), "frac_hbm": round(ach / PEAK_HBM_GBS, 4),
                              "avg_launch_ms": round(tot_ms / launches, 4)}
    dominant = max(prof, key=lambda n: prof[n][1]) if prof else None
    roof = {k: rooflines[dominant][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")} \
        if dominant in rooflines else None
    if roof is not None:
        roof["kernel"] = dominant

    full_kv = 2 * n_all * T * d * 2
    factor_bytes = int(tot_rank * (T + d) * fe) + (4 * (2 * n_all * T + tot_rank) if fdt == "i8" else 0)

    # ---------------- CPU baseline: the oracle on a bounded sample ----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, fdt, X, Q, q_pos, sel, tails, nb_layer, L, ctx_tokens)

    out = {
        "metric": METRIC,
        "value": ctx_tokens / (step_ms / 1e3),
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
        "config": {"workload": cfg.workload, "config_index": cfg.idx, "layers": L, "n_kv_heads": H,
                   "n_q_heads": Hq, "head_dim": d, "block_len": T, "blocks_per_seq": cfg.blocks_per_seq,
                   "batch": cfg.batch, "attended_blocks_per_seq": cfg.attended_blocks,
                   "tail_len": cfg.tail_len, "budget_frac": cfg.budget_fracs[0], "factor_dtype": fdt,
                   "context_tokens_per_step": ctx_tokens, "blocks_compressed_per_step": n_blocks_step},
        "breakdown": {
            "compress_ms": round(comp_ms, 3), "decode_ms": round(dec_ms, 3),
            "blocks_per_s": n_blocks_step / (comp_ms / 1e3),
            "decode_context_tokens_per_s": ctx_tokens / (dec_ms / 1e3),
            "decode_only_ms_per_step": round(dec_only_ms, 3),
            "decode_only_context_tokens_per_s": ctx_tokens / (dec_only_ms / 1e3),
            "jacobi_sweeps_mean": round(sweeps_mean, 3),
            "kernels_ms_per_step": {n: round(v[1] / args.steps, 3) for n, v in prof.items()},
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
    print(json.dumps(out))
    return 0


def offload_measure(milo, torch, np, cfg, F, X, Q, q_pos, sel, nb_layer, fdt, xdt, dev, n_src=2):
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
    es = {"f32": 4, "bf16": 2, "i8": 1, "i4": 5 / 8}[fdt]

    def layer_host_set(f, layer):
        """A compact pinned-host copy of one layer's factor set (offsets rebased)."""
        v = f.view(layer * nb_layer, nb_layer)
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
    hk = [layer_host_set(F["k"], l) for l in range(n_src)]
    hv = [layer_host_set(F["v"], l) for l in range(n_src)]
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


def cpu_baseline(cfg, fdt, X, Q, q_pos, sel, tails, nb_layer, L, ctx_tokens):
    """The oracle, as it stands, on one (sequence, layer, KV head) of the workload:
    compress its K pool and V pool, then decode its query heads over the attended
    blocks (and tail).  Scaled to the whole step by the number of such units."""
    import numpy as np
    import torch

    import oracle
    T, d, H = cfg.block_len, cfg.head_dim, cfg.n_kv_heads
    bps = cfg.blocks_per_seq
    lo = 0  # layer 0, sequence 0, KV head 0
    Xk = X["k"][lo:lo + bps].to(torch.float64).cpu().numpy()
    Xv = X["v"][lo:lo + bps].to(torch.float64).cpu().numpy()
    q = Q[0][0:1, 0:cfg.group].to(torch.float64).cpu().numpy()
    R = cfg.budget()
    t0 = time.perf_counter()
    ck = oracle.compress(Xk, [0, bps], [R], cfg.eps2, fdt)
    cv = oracle.compress(Xv, [0, bps], [R], cfg.eps2, fdt)
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
    t = time.perf_counter() - t0
    units = L * cfg.batch * H
    return {"value": ctx_tokens / (t * units), "unit": "context-tokens/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"1 of {units} (layer, sequence, KV head) units: compress its K and V pools "
                      f"({2 * bps} blocks of {T}x{d}, SVD threaded over blocks) and decode its {cfg.group} "
                      f"query heads over {cfg.attended_blocks} blocks"
                      + (f" + {cfg.tail_len}-token tail" if cfg.tail_len else "")
                      + f" (single-threaded), {t:.1f} s; value = step context tokens / (t x {units})",
            "sample_seconds": round(t, 2)}


if __name__ == "__main__":
    sys.exit(main())
