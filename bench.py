"""Benchmark of the CSA lightning-indexer top-k on one MI355X.

One step = one csa_indexer_topk call over the whole workload (every query
row scored against every usable compressed key, chunked partition-merge
top-k, sorted outputs), inputs already resident in HBM.  Default workload:
S=65,536 queries, m=4 (T=16,384 compressed keys), H_I=64 heads, D_I=128,
k=2048, bf16 inputs q, kc ~ N(0,1)/sqrt(D_I) and w ~ N(0,1)/sqrt(H_I) drawn
from a fixed seed on the device.

Prints one JSON line: pairs/s over the whole job (K timed calls with no
per-launch instrumentation), the score kernel against the bf16 MFMA roofline
(its launch duration measured in a second run of K calls, with HIP events
that the library records around every launch on the call's stream), peak
HBM, and the CPU oracle timed on a bounded sample of the same workload's rows
on the host.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
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

import streaming_indexer_top_amd as csa  # noqa: E402
from streaming_indexer_top_amd import inputs  # noqa: E402

METRIC = "scored q-k pairs/s at S=65536 V4-Flash dims; MFMA util %; peak HBM GB"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_BUSY_PEAK = MFMA_BF16_PEAK_TFLOPS
HBM_PEAK_GBS = 8000.0
# Default timed calls: enough for about AUTO_TIMED_MS of timed work in the
# default run (every other mode takes AUTO_MIN_STEPS unless --steps is given).
AUTO_TIMED_MS = 2000.0
AUTO_MIN_STEPS = 20
AUTO_MAX_STEPS = 500
# HBM traffic of the score kernel, summarised from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE) of the default workload by --traffic-from.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_bf16_S65536_hbm_traffic.txt")
SCORE_SOURCES = ("streaming_indexer_top_amd/csrc/score_kernels.hip",
                 "streaming_indexer_top_amd/csrc/csa_internal.h")
SELECT_SOURCES = ("streaming_indexer_top_amd/csrc/select_kernels.hip",
                  "streaming_indexer_top_amd/csrc/csa_internal.h")


def pair_count(S, T, m, q_pos0=0):
    i = np.arange(S, dtype=np.int64) + q_pos0
    return int(np.minimum(T, (i + 1) // m).sum())


def source_hash(sources=SCORE_SOURCES):
    """sha256 over the code of the sources that define a kernel (// comments
    and whitespace removed, so that comment edits keep the counters valid)."""
    import re
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        code = re.sub(r"//[^\n]*", "", text)
        h.update("".join(code.split()).encode())
    return h.hexdigest()


def score_source_hash():
    return source_hash(SCORE_SOURCES)


def read_traffic():
    """Per-launch HBM bytes of the score kernel from TRAFFIC_FILE, or None when
    the file is missing or was taken from other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    kv = {a.strip(): b.strip() for a, b in kv.items()}
    if kv.get("source_sha256") != score_source_hash():
        return None
    out = {"bytes": float(kv["traffic_bytes_per_launch"]),
           "fetch": float(kv["fetch_bytes_per_launch"]),
           "write": float(kv["write_bytes_per_launch"]), "select": None}
    if kv.get("select_source_sha256") == source_hash(SELECT_SOURCES) and \
            "select_fetch_bytes_per_launch" in kv:
        out["select"] = (float(kv["select_fetch_bytes_per_launch"]),
                         float(kv["select_write_bytes_per_launch"]))
    return out


def summarize_counters(fetch_csv, write_csv, copy_bytes):
    """Summary text for TRAFFIC_FILE from the counter CSVs of two rocprofv3 runs
    of `bench.py --steps 1 --warmup 0 --no-cpu-baseline --copy-probe B` (one with
    --pmc FETCH_SIZE, one with --pmc WRITE_SIZE).  Each counter is scaled by
    what it reads for the probe's plain device copy of B bytes."""
    def load(path, counter):
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        pick = lambda tag: [float(r["Counter_Value"]) for r in rows if tag in r["Kernel_Name"]]
        copy = pick("copyBuffer")
        if len(copy) != 1:
            raise SystemExit("%s: expected one copy-probe dispatch, found %d" % (path, len(copy)))
        return pick("score_bf16_kernel"), pick("select_kernel"), copy[0]
    f_sc, f_se, f_cp = load(fetch_csv, "FETCH_SIZE")
    w_sc, w_se, w_cp = load(write_csv, "WRITE_SIZE")
    if not f_sc or len(f_sc) != len(w_sc):
        raise SystemExit("score kernel dispatches differ between the two runs")
    true_kib = copy_bytes / 1024.0
    ff, wf = true_kib / f_cp, true_kib / w_cp
    n = len(f_sc)
    fetch = sum(f_sc) * ff * 1024.0 / n
    write = sum(w_sc) * wf * 1024.0 / n
    out = [
        "source_sha256: %s" % score_source_hash(),
        "calibration_copy_bytes: %d" % copy_bytes,
        "calibration_copy_fetch_kib_raw: %.3f" % f_cp,
        "calibration_copy_write_kib_raw: %.3f" % w_cp,
        "fetch_factor: %.6f" % ff,
        "write_factor: %.6f" % wf,
        "score_launches: %d" % n,
        "score_fetch_kib_raw: %s" % " ".join("%.3f" % x for x in f_sc),
        "score_write_kib_raw: %s" % " ".join("%.3f" % x for x in w_sc),
        "fetch_bytes_per_launch: %.0f" % fetch,
        "write_bytes_per_launch: %.0f" % write,
        "traffic_bytes_per_launch: %.0f" % (fetch + write),
    ]
    if f_se and len(f_se) == len(w_se):
        m = len(f_se)
        out += [
            "select_source_sha256: %s" % source_hash(SELECT_SOURCES),
            "select_launches: %d" % m,
            "select_fetch_bytes_per_launch: %.0f" % (sum(f_se) * ff * 1024.0 / m),
            "select_write_bytes_per_launch: %.0f" % (sum(w_se) * wf * 1024.0 / m),
        ]
    return "\n".join(out) + "\n"


def summarize_mfma_busy(csv_path, match="score_bf16_kernel", xcds=8, simds=1024):
    """Summary of one rocprofv3 --pmc run with SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE over the dispatches of the kernels
    whose name contains `match` (default: the score kernel): the matrix-pipe
    busy fraction per SIMD against the GPU-busy cycles (GRBM_GUI_ACTIVE is
    summed over the XCDs), and the shader clock those cycles imply."""
    with open(csv_path) as f:
        rows = [r for r in csv.DictReader(f) if match in r["Kernel_Name"]]
    if not rows:
        raise SystemExit("%s: no dispatch of a kernel matching %r" % (csv_path, match))
    agg = {}
    ns = 0.0
    seen = set()
    for r in rows:
        agg[r["Counter_Name"]] = agg.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r["Dispatch_Id"] not in seen:
            seen.add(r["Dispatch_Id"])
            ns += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    busy = agg["SQ_VALU_MFMA_BUSY_CYCLES"]
    gpu = agg["GRBM_GUI_ACTIVE"] / xcds
    out = ["dispatches: %d" % len(seen),
           "kernel_ns_total: %.0f" % ns,
           "sq_valu_mfma_busy_cycles: %.6g" % busy,
           "grbm_gui_active_per_xcd: %.6g" % gpu,
           "mfma_busy_per_simd: %.6g" % (busy / simds),
           "mfma_busy_fraction: %.4f" % (busy / simds / gpu),
           "shader_clock_ghz: %.3f" % (gpu / ns)]
    if "SQ_BUSY_CYCLES" in agg:
        out.append("sq_busy_cycles: %.6g" % agg["SQ_BUSY_CYCLES"])
    cus = simds // 4
    if "SQ_ACTIVE_INST_VALU" in agg:
        # rocprofiler's VALUBusy for gfx9: quad-cycles summed over the SIMDs,
        # per CU, against the GPU-busy cycles.
        out.append("valu_busy_fraction: %.4f" % (agg["SQ_ACTIVE_INST_VALU"] / cus / gpu))
    for name in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAVES"):
        if name in agg:
            out.append("%s: %.6g" % (name.lower(), agg[name]))
    if "SQ_INSTS_VALU" in agg and agg.get("SQ_INSTS_MFMA"):
        # SQ_INSTS_VALU counts the MFMAs too.
        out.append("non_mfma_valu_per_mfma: %.3f"
                   % ((agg["SQ_INSTS_VALU"] - agg["SQ_INSTS_MFMA"]) / agg["SQ_INSTS_MFMA"]))
    return "\n".join(out) + "\n"


def make_inputs(cfg_n, dev):
    c = inputs.config(cfg_n)
    S, T, H, D = c["S"], c["T"], c["H"], c["D"]
    if cfg_n == 4:
        q, w, kc = inputs.bf16_mixture(S, T, H, D, seed=cfg_n, device=dev)
        dist = "q,w N(0,1) scaled; kc 64-component Gaussian mixture (spread 0.3)"
    else:
        q, w, kc = inputs.bf16_gaussian(S, T, H, D, seed=cfg_n, device=dev)
        dist = "q,kc ~ N(0,1)/sqrt(D_I), w ~ N(0,1)/sqrt(H_I)"
    return c, q, w, kc, dist


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def select_algorithmic_bytes(S, T, m, k, chunk):
    """Bytes the select stage must move for one call: the chunk scores read
    once (4 B per pair), the outputs written once (8 B per entry), and with
    several chunks the running lists read and written once per extra chunk
    (16 B per entry)."""
    i = np.arange(S, dtype=np.int64)
    n = np.minimum(T, (i + 1) // m)
    n_max = int(n.max()) if S else 0
    n_round = (n_max + 255) // 256 * 256
    c = chunk or (n_round if n_round <= 65536 else 65536)
    c = max(min(c, n_round), 1)
    extra = np.maximum((n + c - 1) // c - 1, 0)
    lists = 16 * k * int(extra.sum())
    return 4 * int(n.sum()) + 8 * S * k + lists


def cpu_baseline(q, w, kc, m, k, S, T, target_s, max_rows, seed):
    """Times the CPU oracle on sampled rows of the same workload."""
    import oracle
    oracle.build()
    threads = len(os.sched_getaffinity(0))
    kf = kc.float().cpu().numpy()

    def run(rows):
        rows = np.array(sorted(rows), dtype=np.int64)
        rt = torch.from_numpy(rows).to(q.device)
        qf = q[rt].float().cpu().numpy()
        wf = w[rt].float().cpu().numpy()
        t0 = time.perf_counter()
        res = oracle.topk(qf, wf, kf, m, k, pos=rows, nthreads=threads)
        dt = time.perf_counter() - t0
        pairs = int(np.minimum(T, (rows + 1) // m).sum())
        return rows, res, dt, pairs

    probe = inputs.sample_rows(S, m, k, 64, seed)
    _, _, dt0, pairs0 = run(probe)
    rate = pairs0 / max(dt0, 1e-9)
    mean_pairs = pair_count(S, T, m) / S
    want = int(min(max_rows, max(64, target_s * rate / max(mean_pairs, 1.0))))
    rows = inputs.sample_rows(S, m, k, want, seed)
    rows, res, dt, pairs = run(rows)
    return {
        "value": pairs / dt,
        "unit": "pairs/s",
        "cores": threads,
        "cpu": cpu_model(),
        "kind": "oracle",
        "sample": "%d query rows of the same workload (boundary rows plus seeded uniform draws), "
                  "%d valid pairs, %.2f s wall on %d host threads" % (len(rows), pairs, dt, threads),
        "seconds": dt,
        "extrapolated_full_s": pair_count(S, T, m) / (pairs / dt),
    }, rows, res


def run_sweep(args, q, w, kc, c, dev, base_alloc):
    """Top-k x chunk-size x key-tile sweep: time per call, throughput, peak HBM,
    and a bit-identity check of every setting's outputs against the first
    setting with the same k."""
    S, T, H, D, m = c["S"], c["T"], c["H"], c["D"], c["m"]
    P = pair_count(S, T, m)
    ks = [int(x) for x in args.sweep_ks.split(",")] if args.sweep_ks else [c["k"]]
    for k in ks:
        idx = torch.empty((S, k), dtype=torch.int32, device=dev)
        score = torch.empty((S, k), dtype=torch.float32, device=dev)
        ref = None
        for chunk in [int(x) for x in args.sweep_chunks.split(",")]:
            for tile in [int(x) for x in args.sweep_tiles.split(",")]:
                ws_bytes = csa.workspace_size(S, T, H, D, m, k, chunk_keys=chunk, key_tile=tile,
                                              workspace_budget=args.budget)
                torch.cuda.reset_peak_memory_stats(dev)
                workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
                kw = dict(chunk_keys=chunk, key_tile=tile, workspace_budget=args.budget,
                          workspace=workspace, out=(idx, score))
                for _ in range(args.warmup):
                    csa.topk(q, w, kc, m, k, **kw)
                torch.cuda.synchronize()
                csa.profile_collect()
                csa.profile_enable(True)
                t0 = time.perf_counter()
                for _ in range(args.steps):
                    csa.topk(q, w, kc, m, k, **kw)
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                csa.profile_enable(False)
                prof = csa.profile_collect()
                ms = (t1 - t0) * 1e3 / args.steps
                if ref is None:
                    ref = (idx.clone(), score.clone())
                    same = True
                else:
                    same = bool(torch.equal(ref[0], idx)) and bool(
                        torch.equal(ref[1].view(torch.int32), score.view(torch.int32)))
                peak = torch.cuda.max_memory_allocated(dev) - base_alloc
                print(json.dumps({
                    "workload": args.workload, "S": S, "T": T, "k": k, "chunk_keys": chunk,
                    "key_tile": tile, "ms_per_call": ms, "pairs_per_s": P / (ms * 1e-3),
                    "mfma_util_pct": 100.0 * P * 2 * H * D / (ms * 1e-3) / (MFMA_BUSY_PEAK * 1e12),
                    "score_ms": prof["score"][0] / args.steps,
                    "select_ms": prof["select"][0] / args.steps,
                    "score_launches": prof["score"][1] / args.steps,
                    "workspace_bytes": ws_bytes, "peak_hbm_gib": peak / 2 ** 30,
                    "bit_identical_to_first": same}), flush=True)
                del workspace
        del idx, score


def run_batched(args, dev):
    """B independent problems of the workload's shape (own seeded inputs each)
    in one batched call; one JSON line with the batch's pairs/s."""
    c = inputs.config(args.workload)
    S, T, H, D, m, k = c["S"], c["T"], c["H"], c["D"], c["m"], c["k"]
    B = args.batch
    probs = [inputs.bf16_gaussian(S, T, H, D, seed=100 * args.workload + b, device=dev)
             for b in range(B)]
    q, w, kc = [torch.stack([p[i] for p in probs]).contiguous() for i in range(3)]
    del probs
    idx = torch.empty((B, S, k), dtype=torch.int32, device=dev)
    score = torch.empty((B, S, k), dtype=torch.float32, device=dev)
    ws_bytes = csa.workspace_size(S, T, H, D, m, k, chunk_keys=args.chunk, key_tile=args.tile,
                                  workspace_budget=args.budget)
    workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    kw = dict(chunk_keys=args.chunk, key_tile=args.tile, workspace_budget=args.budget,
              workspace=workspace, out=(idx, score))
    for _ in range(args.warmup):
        csa.topk(q, w, kc, m, k, **kw)
    torch.cuda.synchronize()
    csa.profile_collect()
    csa.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        csa.topk(q, w, kc, m, k, **kw)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    csa.profile_enable(False)
    prof = csa.profile_collect()
    ms = (t1 - t0) * 1e3 / args.steps
    P = B * pair_count(S, T, m)
    print(json.dumps({
        "mode": "batched", "batch": B, "workload": args.workload, "S": S, "T": T, "k": k,
        "ms_per_call": ms, "pairs_per_s": P / (ms * 1e-3),
        "mfma_util_pct": 100.0 * P * 2 * H * D / (ms * 1e-3) / (MFMA_BUSY_PEAK * 1e12),
        "score_ms": prof["score"][0] / args.steps, "select_ms": prof["select"][0] / args.steps,
        "score_launches": prof["score"][1] / args.steps, "workspace_bytes": ws_bytes}),
        flush=True)


def run_attention(args, dev):
    """The composed CSA step: the indexer's top-k of the workload (W4, at
    S = 262,144, is the page's composed run) followed by the sparse attention
    over the selected entries (64 heads, 576-dim latent keys, their first 512
    dims as values); with --attn-random, the attention alone over a seeded
    uniform random selection of k entries per row.
    One JSON line: per-stage times, the attention kernel against the bf16
    MFMA peak (flops of the valid selected entries only), and peak HBM over
    inputs, outputs and workspace of both stages."""
    torch.cuda.reset_peak_memory_stats(dev)
    base_alloc = torch.cuda.memory_allocated(dev)
    if args.attn_random:
        c = inputs.config(args.workload)
        dist = "none: every row selects k uniform random entries"
    else:
        c, qi, wi, kc, dist = make_inputs(args.workload, dev)
    S, T, Hi, Di, m, k = c["S"], c["T"], c["H"], c["D"], c["m"], c["k"]
    HA, DK, DV = args.attn_heads, 576, 512
    qa, kv = inputs.attention_gaussian(S, T, HA, DK, seed=1000 + args.workload, device=dev)
    out = torch.empty((S, HA, DV), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / DK ** 0.5
    if args.attn_random:
        ws_bytes = 0
        gen = torch.Generator(device=dev)
        gen.manual_seed(2000 + args.workload)
        idx = torch.randint(0, T, (S, k), generator=gen, device=dev, dtype=torch.int32)

        def step():
            csa.sparse_attention(qa, kv, idx, DV, scale=scale, out=out)
    else:
        ws_bytes = csa.workspace_size(S, T, Hi, Di, m, k, chunk_keys=args.chunk,
                                      key_tile=args.tile, workspace_budget=args.budget)
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
        idx = torch.empty((S, k), dtype=torch.int32, device=dev)
        score = torch.empty((S, k), dtype=torch.float32, device=dev)
        kw = dict(chunk_keys=args.chunk, key_tile=args.tile, workspace_budget=args.budget,
                  workspace=workspace, out=(idx, score))

        def step():
            csa.topk(qi, wi, kc, m, k, **kw)
            csa.sparse_attention(qa, kv, idx, DV, scale=scale, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    csa.profile_collect()
    csa.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    csa.profile_enable(False)
    prof = csa.profile_collect()
    ms = (t1 - t0) * 1e3 / args.steps
    if args.attn_random:
        entries = S * k
    else:
        n = np.minimum(T, (np.arange(S, dtype=np.int64) + 1) // m)
        entries = int(np.minimum(n, k).sum())       # valid selected entries
    flops = entries * HA * (DK + DV) * 2
    att_ms = prof["attention"][0] / max(prof["attention"][1], 1)
    achieved = flops / (att_ms * 1e-3) / 1e12
    gathered = entries * DK * 2
    peak = torch.cuda.max_memory_allocated(dev) - base_alloc
    print(json.dumps({
        "mode": ("sparse attention over a random selection" if args.attn_random
                 else "composed indexer + sparse attention"), "workload": args.workload,
        "config": {"S": S, "T": T, "H_I": Hi, "D_I": Di, "m": m, "k": k,
                   "attention_heads": HA, "latent_dim": DK, "value_dim": DV,
                   "indexer_inputs": dist, "attention_inputs": "q, kv ~ N(0,1) bf16"},
        "ms_per_step": ms,
        "indexer_ms": (prof["score"][0] + prof["select"][0] + prof["merge"][0]) / args.steps,
        "attention_ms": att_ms,
        "attention_roofline": {"bound": "mfma", "achieved": achieved,
                               "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                               "flops_per_launch": flops, "valid_entries": entries,
                               "gathered_latent_gb_per_launch": gathered / 1e9,
                               "gathered_latent_gb_per_s": gathered / (att_ms * 1e-3) / 1e9},
        "peak_hbm_gib": peak / 2 ** 30, "workspace_bytes": ws_bytes,
        "steps": args.steps, "warmup": args.warmup}), flush=True)


def run_decode(args, dev):
    """R new queries at the end of the workload's sequence (q_pos0 = m*T - R,
    every query sees all T keys): the automatic plan (key splits) and the
    chunked plan (key_splits=1), one JSON line each."""
    c = inputs.config(args.workload)
    _, T, H, D, m, k = c["S"], c["T"], c["H"], c["D"], c["m"], c["k"]
    R = args.decode
    q, w, kc = inputs.bf16_gaussian(R, T, H, D, seed=1000 + args.workload, device=dev)
    q_pos0 = m * T - R
    P = pair_count(R, T, m, q_pos0)
    ref = None
    for splits in (0, 1):
        kw = dict(q_pos0=q_pos0, key_splits=splits)
        for _ in range(args.warmup):
            csa.topk(q, w, kc, m, k, **kw)
        torch.cuda.synchronize()
        csa.profile_collect()
        csa.profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            out = csa.topk(q, w, kc, m, k, **kw)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        csa.profile_enable(False)
        prof = csa.profile_collect()
        if ref is None:
            ref = out
        same = bool(torch.equal(ref[0], out[0])) and bool(
            torch.equal(ref[1].view(torch.int32), out[1].view(torch.int32)))
        ms = (t1 - t0) * 1e3 / args.steps
        graph_ms = None
        if args.graph:
            # The same call captured once in a HIP graph and replayed: no
            # per-launch host overhead (the library enqueues only kernels).
            ws_bytes = csa.workspace_size(R, T, H, D, m, k, q_pos0=q_pos0, key_splits=splits)
            ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
            gi = torch.empty((R, k), dtype=torch.int32, device=dev)
            gs = torch.empty((R, k), dtype=torch.float32, device=dev)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                csa.topk(q, w, kc, m, k, workspace=ws, out=(gi, gs), **kw)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                csa.topk(q, w, kc, m, k, workspace=ws, out=(gi, gs), **kw)
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                g.replay()
            torch.cuda.synchronize()
            graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
            same = same and bool(torch.equal(ref[0], gi)) and bool(
                torch.equal(ref[1].view(torch.int32), gs.view(torch.int32)))
        print(json.dumps({
            "mode": "decode", "plan": "key splits (auto)" if splits == 0 else "chunks only",
            "graph_replay_ms": graph_ms,
            "rows": R, "T": T, "k": k, "q_pos0": q_pos0, "ms_per_call": ms,
            "pairs_per_s": P / (ms * 1e-3),
            "mfma_util_pct": 100.0 * P * 2 * H * D / (ms * 1e-3) / (MFMA_BUSY_PEAK * 1e12),
            "kernel_ms": {kk: v[0] / args.steps for kk, v in prof.items()},
            "launches": {kk: v[1] / args.steps for kk, v in prof.items()},
            "bit_identical_to_auto": same}), flush=True)


def run_gemm_probe(args, dev):
    """A square bf16 GEMM through torch.matmul (the vendor GEMM library), timed
    with CUDA events on torch's stream: what a tuned dense contraction
    sustains on this chip under the same power limit, for comparison with the
    score kernel's fraction of the nominal peak."""
    n = args.gemm_probe
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    for _ in range(max(args.warmup, 1)):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        torch.matmul(a, b, out=c)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    print(json.dumps({"probe": "gemm_bf16", "n": n, "steps": args.steps, "ms_per_gemm": ms,
                      "tflops": tflops, "frac_of_2500": tflops / 2500.0}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed calls (default: 20; for the default run, enough calls for "
                         "about %.0f s of timed work, %d to %d)" % (AUTO_TIMED_MS / 1e3,
                                                                   AUTO_MIN_STEPS, AUTO_MAX_STEPS))
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, help="workload number 2..5")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--budget", type=int, default=0, help="workspace budget in bytes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-max-rows", type=int, default=12288)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time every (top-k x) chunk x key-tile setting (default grid: chunk "
                         "4096..65536, tile 64/128/256), one JSON line each, checking that all "
                         "settings with the same k give bit-identical outputs")
    ap.add_argument("--sweep-chunks", default="4096,8192,16384,32768,65536")
    ap.add_argument("--sweep-tiles", default="64,128,256")
    ap.add_argument("--sweep-ks", default="", help="top-k values to sweep (default: the workload's k)")
    ap.add_argument("--decode", type=int, default=0,
                    help="time this many new queries at the end of the workload's sequence "
                         "(decode shape) with and without key splits")
    ap.add_argument("--graph", action="store_true",
                    help="with --decode: also time replays of the call captured in a HIP graph")
    ap.add_argument("--batch", type=int, default=0,
                    help="time one batched call over this many independent problems of the "
                         "workload's shape (one JSON line)")
    ap.add_argument("--attention", action="store_true",
                    help="time the composed step: the workload's indexer top-k, then the sparse "
                         "attention over the selected entries (one JSON line)")
    ap.add_argument("--attn-heads", type=int, default=64, help="attention heads (32 or 64)")
    ap.add_argument("--attn-random", action="store_true",
                    help="with --attention: time the attention alone over a seeded uniform random "
                         "selection of k entries for every row (no indexer stage)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="bytes of a plain device copy run once before timing, as a known "
                         "reference for HBM traffic counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc runs "
                         "(needs --copy-probe with the probe size those runs used); no GPU")
    ap.add_argument("--mfma-busy-from", metavar="PMC_CSV",
                    help="print the MFMA-busy summary of a rocprofv3 --pmc run with "
                         "SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE; no GPU")
    ap.add_argument("--kernel-match", default="score_bf16_kernel",
                    help="with --mfma-busy-from: summarize the kernels whose name contains this")
    ap.add_argument("--gemm-probe", type=int, default=0,
                    help="time a plain library bf16 GEMM (torch.matmul, N x N x N) as a "
                         "reference for the MFMA rate this chip sustains; one JSON line")
    args = ap.parse_args()
    auto_steps = args.steps is None
    if auto_steps:
        args.steps = AUTO_MIN_STEPS

    if args.mfma_busy_from:
        sys.stdout.write(summarize_mfma_busy(args.mfma_busy_from, args.kernel_match))
        return
    if args.traffic_from:
        if not args.copy_probe:
            raise SystemExit("--traffic-from needs --copy-probe BYTES")
        sys.stdout.write(summarize_counters(args.traffic_from[0], args.traffic_from[1],
                                            args.copy_probe))
        return

    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and has no "
              "multi-GPU mode (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.gemm_probe:
        run_gemm_probe(args, dev)
        return
    csa.load_library()
    if args.attention:
        run_attention(args, dev)
        return
    if args.batch:
        run_batched(args, dev)
        return
    if args.decode:
        run_decode(args, dev)
        return

    torch.cuda.reset_peak_memory_stats(dev)
    base_alloc = torch.cuda.memory_allocated(dev)
    free_before = torch.cuda.mem_get_info(dev)[0]
    c, q, w, kc, dist = make_inputs(args.workload, dev)
    S, T, H, D, m, k = c["S"], c["T"], c["H"], c["D"], c["m"], c["k"]
    torch.cuda.synchronize()
    gen_peak = torch.cuda.max_memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)

    if args.sweep:
        run_sweep(args, q, w, kc, c, dev, base_alloc)
        return

    ws_bytes = csa.workspace_size(S, T, H, D, m, k, chunk_keys=args.chunk, key_tile=args.tile,
                                  workspace_budget=args.budget)
    workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    idx = torch.empty((S, k), dtype=torch.int32, device=dev)
    score = torch.empty((S, k), dtype=torch.float32, device=dev)
    kw = dict(chunk_keys=args.chunk, key_tile=args.tile, workspace_budget=args.budget,
              workspace=workspace, out=(idx, score))

    if args.copy_probe:
        src = torch.empty((args.copy_probe,), dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        csa.topk(q, w, kc, m, k, **kw)
    torch.cuda.synchronize()
    if auto_steps:
        # Size K from one more (untimed) call, so that the timed region is
        # long enough to be seen by a sampling monitor.
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        csa.topk(q, w, kc, m, k, **kw)
        e1.record()
        torch.cuda.synchronize()
        est = max(e0.elapsed_time(e1), 1e-3)
        args.steps = int(min(AUTO_MAX_STEPS, max(AUTO_MIN_STEPS, math.ceil(AUTO_TIMED_MS / est))))
        args.warmup += 1  # the sizing call is one more untimed call
    csa.profile_collect()  # drop anything recorded so far

    # The headline: K calls with the library's per-launch events off.  One
    # event between consecutive calls on the call stream gives per-call times
    # without a synchronisation inside the timed region.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        csa.topk(q, w, kc, m, k, **kw)
        marks[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    call_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))

    # Per-kernel launch durations: the same K calls again, with the library
    # recording HIP events around every launch on the call's stream.
    csa.profile_enable(True)
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    for i in range(args.steps):
        csa.topk(q, w, kc, m, k, **kw)
    torch.cuda.synchronize()
    tp1 = time.perf_counter()
    csa.profile_enable(False)
    prof = csa.profile_collect()

    resident = (q.numel() * q.element_size() + w.numel() * w.element_size()
                + kc.numel() * kc.element_size() + idx.numel() * 4 + score.numel() * 4)
    peak = torch.cuda.max_memory_allocated(dev) - base_alloc
    # Device memory taken since the start (hipMemGetInfo): torch's reserved
    # pool; the library itself allocates nothing.
    device_used = free_before - torch.cuda.mem_get_info(dev)[0]
    ms = (t1 - t0) * 1e3 / args.steps
    P = pair_count(S, T, m)
    flops = P * 2 * H * D
    score_ms, score_n = prof["score"]
    sel_ms, sel_n = prof["select"]
    per_launch_ms = score_ms / max(score_n, 1)
    flops_per_launch = flops / max(score_n / args.steps, 1)
    achieved = flops_per_launch / (per_launch_ms * 1e-3) / 1e12 if score_n else 0.0
    # Counter figures hold for the workload and plan they were taken on.
    traffic = None
    if args.workload == 3 and not (args.chunk or args.tile or args.budget):
        traffic = read_traffic()
    sel_launches = sel_n / args.steps
    sel_bytes = select_algorithmic_bytes(S, T, m, k, args.chunk) / max(sel_launches, 1)
    sel_launch_ms = sel_ms / max(sel_n, 1)
    sel_gbs = sel_bytes / (sel_launch_ms * 1e-3) / 1e9 if sel_n else 0.0
    sel_traffic = traffic["select"] if traffic else None

    out = {
        "metric": METRIC,
        "value": P / (ms * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "csa_indexer_topk S=%d T=%d H_I=%d D_I=%d m=%d k=%d causal bf16, %s"
                        % (S, T, H, D, m, k, dist),
            "S": S, "T": T, "H_I": H, "D_I": D, "m": m, "k": k,
            "chunk_keys": args.chunk or "auto", "key_tile": args.tile or "auto",
            "valid_pairs": P,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
            "traffic": traffic["bytes"] if traffic else None,
            "traffic_fetch_write": [traffic["fetch"], traffic["write"]] if traffic else None,
            "traffic_per": "launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a plain copy)",
            "kernel": "score_bf16_kernel",
            "launch_ms": per_launch_ms,
            "launches_per_step": score_n / args.steps,
            "flops_per_launch": flops_per_launch,
        },
        "select_roofline": {
            "bound": "hbm",
            "achieved": sel_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": sel_gbs / HBM_PEAK_GBS,
            "traffic": sum(sel_traffic) if sel_traffic else None,
            "traffic_fetch_write": list(sel_traffic) if sel_traffic else None,
            "kernel": "select_kernel",
            "launch_ms": sel_launch_ms,
            "launches_per_step": sel_launches,
            "bytes_per_launch": sel_bytes,
        },
        "call_ms": {"median": call_ms[len(call_ms) // 2], "min": call_ms[0],
                    "max": call_ms[-1]},
        "profiled_ms_per_step": (tp1 - tp0) * 1e3 / args.steps,
        "pairs_per_s_median_call": P / (call_ms[len(call_ms) // 2] * 1e-3),
        "mfma_util_pct": 100.0 * flops / (ms * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "kernel_ms_per_step": {"score": score_ms / args.steps, "select": sel_ms / args.steps,
                               "merge": prof["merge"][0] / args.steps},
        "peak_hbm_gb": peak / 1e9,
        "peak_hbm": {"total_gib": peak / 2 ** 30, "workspace_bytes": ws_bytes,
                     "resident_inputs_outputs_gib": resident / 2 ** 30,
                     "above_resident_gib": (peak - resident) / 2 ** 30,
                     "input_generation_peak_gib": gen_peak / 2 ** 30,
                     "device_memory_taken_gib": device_used / 2 ** 30,
                     "avoided_fp32_score_tensor_gib": S * H * T * 4 / 2 ** 30},
    }

    if not args.no_cpu_baseline:
        base, rows, (o_idx, o_sc) = cpu_baseline(q, w, kc, m, k, S, T, args.cpu_seconds,
                                                 args.cpu_max_rows, args.workload)
        out["cpu_baseline"] = {kk: base[kk] for kk in ("value", "unit", "cores", "kind", "sample")}
        out["cpu_baseline"]["extrapolated_full_s"] = base["extrapolated_full_s"]
        out["cpu_baseline"]["cpu"] = base["cpu"]
        out["cpu_baseline"]["gpu_over_cpu"] = out["value"] / base["value"]
        rt = torch.from_numpy(rows).to(dev)
        g_idx = idx[rt].cpu().numpy()
        n = np.minimum(T, (rows + 1) // m)
        rec = []
        for r in range(len(rows)):
            cnum = int(min(n[r], k))
            if cnum:
                rec.append(len(np.intersect1d(g_idx[r, :cnum], o_idx[r, :cnum])) / cnum)
        out["sample_recall"] = {"min": float(min(rec)), "mean": float(np.mean(rec)),
                                "rows": len(rows)}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
