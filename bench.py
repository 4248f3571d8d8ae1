#!/usr/bin/env python3
"""Benchmark of one content-routed sparse attention layer on one MI355X.

A step is one lsa_forward over the whole layer: key block summaries,
routing + top-k, and exact sparse attention (routed blocks + causal window),
on seeded synthetic inputs already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME]

Default workload: the Qwen2.5-0.5B-shaped layer at N=131072 (B=1, 14 query /
2 KV heads, D=64, block 64, top-k 16, window 512, 32 needles).  `value` is
TFLOP/s counted on the selected keys only (4*D FLOP per selected key and
query: QK^T and PV), `ms_per_step` is ms per layer.

Variant legs in the same line: consensus routing, the second-cumulant
score, two-level routing, decode, and `ties` (every key equal, so every
routing score ties: the exact routing passes' worst case).

`roofline` describes the dominant kernel (largest mean stage time, measured
with HIP events recorded between the library's kernel launches on the same
stream), `cpu_baseline` the CPU oracle timed on a bounded row sample on this
host.  `--copy-calibration` instead runs a plain copy of known size, used to
scale the FETCH_SIZE / WRITE_SIZE counters.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# HBM traffic per launch of the layer's kernels, by stage, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE runs, each scaled by the same counter's reading on
# a plain copy of known size (FETCH x 2.0, WRITE x 1.0); valid only for the
# kernel sources and compile flags they were measured with (kernel_digest).
TRAFFIC = {
    "qwen05b_n32k": {
        "csrc": "03b9e71acace6ed0", "fetch_factor": 2.0, "write_factor": 1.0,
        "kib": {
            "V transpose + bucket count": (18535.3, 8476.0),
            "bucket scan": (38.6, 96.1),
            "bucket scatter": (15687.1, 71293.6),
            "key summary": (4144.8, 528.2),
            "routed-block partials": (521557.5, 941247.9),
            "routing": (29898.7, 28672.0),
            "routing fallback": (18.0, 0.0),
            "window + merge": (530477.5, 114688.8),
        },
    },
    "qwen05b_n128k_needles": {
        "csrc": "03b9e71acace6ed0", "fetch_factor": 2.0, "write_factor": 1.0,
        "kib": {
            "V transpose + bucket count": (73833.9, 34936.0),
            "bucket scan": (347.2, 384.1),
            "bucket scatter": (120013.9, 530396.3),
            "key summary": (16433.2, 2112.2),
            "routed-block partials": (2064241.7, 3881456.8),
            "routing": (119193.1, 114688.0),
            "routing fallback": (18.0, 0.0),
            "window + merge": (2191619.8, 458757.3),
        },
    },
    "image_zorder_128x128": {
        "csrc": "03b9e71acace6ed0", "fetch_factor": 2.0, "write_factor": 1.0,
        "kib": {
            "key summary": (131153.8, 49281.8),
            "routing": (108719.1, 2048.0),
            "routing fallback": (32.2, 0.0),
            "window + merge": (212821.5, 262167.2),
        },
    },
    "qwen05b_n1m_needles": {
        "csrc": "03b9e71acace6ed0", "fetch_factor": 2.0, "write_factor": 1.0,
        "kib": {
            "V transpose + bucket count": (589931.2, 393279.9),
            "bucket scan": (347.2, 384.1),
            "bucket scatter": (989062.9, 7022027.4),
            "key summary": (131121.9, 16896.2),
            "routed-block partials": (15615502.5, 31231887.8),
            "routing": (1475803.4, 917586.2),
            "routing fallback": (186619.1, 89.2),
            "window + merge": (20101588.8, 3670079.7),
        },
    },
}


def traffic_counters(w):
    """{stage name: HBM bytes per launch} when the stored counters belong to
    this workload and to the current kernel sources, else None."""
    t = TRAFFIC.get(w.name)
    if not t or t.get("csrc") != kernel_digest():
        return None
    return {stage: fetch * 1024 * t["fetch_factor"] + write * 1024 * t["write_factor"]
            for stage, (fetch, write) in t["kib"].items()}


def kernel_sources():
    """Every kernel source and header of the library (paths relative to the
    repository), in a fixed order."""
    csrc = os.path.join(ROOT, "content_routed_block_amd", "csrc")
    return sorted(os.path.join("content_routed_block_amd", "csrc", f) for f in os.listdir(csrc)
                  if f.endswith((".hip", ".hpp")))


def kernel_digest() -> str:
    """Digest of the kernel sources and the compile flags."""
    from content_routed_block_amd import build as lsa_build
    h = hashlib.sha256()
    for f in kernel_sources():
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    h.update("\0".join(f.replace(lsa_build.ROOT, "") for f in lsa_build.FLAGS).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen05b_n128k_needles")
    ap.add_argument("--chunk", type=int, default=0,
                    help="query positions per attention chunk (0: the library's choice)")
    ap.add_argument("--top-k", type=int, default=0,
                    help="run the workload with this many routed blocks per query (1..32; "
                         "0: the workload's own); the line then names the changed workload")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the CPU-oracle sample (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--consensus-steps", type=int, default=10,
                    help="also time the layer with consensus routing (one route per KV group)")
    ap.add_argument("--cumulant-steps", type=int, default=3,
                    help="also time the layer routed by the second-cumulant score (beta = 1/sqrt(D))")
    ap.add_argument("--tree-beam", type=int, default=8,
                    help="also time the layer with two-level routing keeping this many nodes (0: skip)")
    ap.add_argument("--decode-steps", type=int, default=50,
                    help="also time single-query decode steps against the workload's cache")
    ap.add_argument("--ties-steps", type=int, default=5,
                    help="also time the layer with every key equal (every routing score ties: "
                         "the exact routing passes' worst case)")
    return ap.parse_args()


def selected_flops(w, idx_np):
    """4*D FLOP per (query, selected key): routed keys from the actual idx plus
    the causal window keys [bs*E(t), t]."""
    D = w.head_dim
    valid = (idx_np >= 0).sum(axis=-1).astype(np.int64)       # per routing row
    if w.causal:
        t = np.arange(w.seq_len, dtype=np.int64)
        E = np.maximum(0, t // w.block - w.window // w.block + 1)
        win = t - w.block * E + 1
        routed_keys = int(valid.sum()) * w.block
        window_keys = int(win.sum()) * w.batch * w.q_heads
        routed_pairs = int(valid.sum())
    else:
        routed_keys = int(valid.sum()) * w.block * w.block     # bs queries x bs keys per block
        window_keys = 0
        routed_pairs = int(valid.sum()) * w.block
    return 4 * D * routed_keys, 4 * D * window_keys, routed_pairs


def routing_candidates(w):
    if w.causal:
        t = np.arange(w.seq_len, dtype=np.int64)
        E = np.maximum(0, t // w.block - w.window // w.block + 1)
        return int(E.sum()) * w.batch * w.q_heads
    nb = w.seq_len // w.block
    return w.batch * w.q_heads * nb * nb


def host_cpu():
    """The host's CPU model and logical core counts (for the CPU baseline)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "logical_cpus": os.cpu_count()}


PARITY_GAP = 1e-3              # routing-score gap below which a row is a near tie
PARITY_MAX_ABS, PARITY_MEAN_ABS = 2e-2, 5e-3


def parity_sample(w, inp, idx_gpu, out_gpu, nrows=4000):
    """The GPU's routing and output against the CPU oracle on a seeded sample
    of routing rows plus every needle row (part of the CPU-baseline leg: the
    oracle's results for these rows are computed there anyway).

    Counts: clear_mismatches = rows whose oracle gap (k-th minus (k+1)-th
    score) exceeds 1e-3 but whose GPU set differs (must be 0); near_ties =
    rows with gap <= 1e-3; near_differing / near_invalid = near rows whose
    GPU set differs / is not a top-k within 1e-3 under the oracle's fp64
    scores; needle recall on GPU and oracle; max-abs and mean-abs output error
    against the oracle attending over the GPU's own selection."""
    import oracle
    k = w.top_k
    kbar = oracle.block_means(inp.k, w.block)
    rng = np.random.default_rng(17)
    if w.causal:
        R = w.batch * w.q_heads * w.seq_len
        rows = rng.choice(R, size=min(R, nrows), replace=False)
        needle_rows = np.array([(n.b * w.q_heads + n.h) * w.seq_len + n.t for n in inp.needles],
                               dtype=np.int64)
        rows = np.unique(np.concatenate([rows, needle_rows]))
        io, gap = oracle.route_causal(inp.q, kbar, w.block, k, w.window, rows=rows, with_gap=True)
        scores = oracle.route_scores(kbar, rows, q=inp.q, block=w.block, window=w.window, causal=1)
        t = rows % w.seq_len
        ncand = np.maximum(0, t // w.block - w.window // w.block + 1)
    else:
        nb = w.seq_len // w.block
        R = w.batch * w.q_heads * nb
        rows = np.sort(rng.choice(R, size=min(R, nrows), replace=False))
        needle_rows = np.zeros(0, np.int64)
        qbar = oracle.block_means(inp.q, w.block)
        io, gap = oracle.route_image(qbar, kbar, k, rows=rows, with_gap=True)
        scores = oracle.route_scores(kbar, rows, qbar=qbar, block=w.block, causal=0)
        ncand = np.full(rows.size, nb)
    ig = idx_gpu.reshape(-1, k)[rows]
    io = io.reshape(-1, k)
    clear = gap.reshape(-1) > PARITY_GAP
    differ = np.any(ig != io, axis=1)
    invalid = 0
    for r in np.nonzero(differ & ~clear)[0]:
        m = min(k, int(ncand[r]))
        sel = ig[r]
        chosen = sel[:m]
        ok = np.all(sel[m:] == -1) and np.all(chosen >= 0) and np.all(chosen < ncand[r]) \
            and np.all(np.diff(chosen) > 0)
        if ok:
            rest = np.setdiff1d(np.arange(int(ncand[r])), chosen)
            ok = rest.size == 0 or scores[r][chosen].min() >= scores[r][rest].max() - PARITY_GAP
        invalid += int(not ok)
    hits_g = hits_o = 0
    pos = {int(r): j for j, r in enumerate(rows)}
    for n, r in zip(inp.needles, needle_rows):
        j = pos[int(r)]
        hits_g += int(n.p // w.block in ig[j])
        hits_o += int(n.p // w.block in io[j])
    if w.causal:
        out_rows, sel = rows, ig
    else:
        bh, i = rows // nb, rows % nb
        out_rows = bh * w.seq_len + i * w.block + rng.integers(0, w.block, rows.size)
        sel = ig
    ref = oracle.attend(inp.q, inp.k, inp.v, sel, w.block, k, w.window, w.causal, rows=out_rows)
    err = np.abs(out_gpu.reshape(-1, w.head_dim)[out_rows].astype(np.float64) - ref)
    return {"rows": int(rows.size), "clear_mismatches": int(np.sum(differ & clear)),
            "near_ties": int(np.sum(~clear)), "near_differing": int(np.sum(differ & ~clear)),
            "near_invalid": invalid,
            "needles": len(inp.needles), "needle_recall_gpu": hits_g,
            "needle_recall_oracle": hits_o,
            "max_abs": float(err.max()), "mean_abs": float(err.mean()),
            "tolerance": {"gap": PARITY_GAP, "max_abs": PARITY_MAX_ABS,
                          "mean_abs": PARITY_MEAN_ABS},
            "sample": f"{rows.size} routing rows of {R} (seeded uniform sample plus every "
                      "needle row), compared with the CPU oracle"}


def cpu_baseline(w, inp, target_s):
    import oracle
    R = w.batch * w.q_heads * w.seq_len
    rng = np.random.default_rng(7)
    probe = np.sort(rng.choice(R, size=min(R, 2000), replace=False))
    t0 = time.perf_counter()
    oracle.forward(inp.q, inp.k, inp.v, w.block, w.top_k, w.window, w.causal, rows=probe)
    per_row = (time.perf_counter() - t0) / probe.size
    n = int(min(R, max(2000, target_s / max(per_row, 1e-9))))
    rows = np.sort(rng.choice(R, size=n, replace=False))
    t0 = time.perf_counter()
    _, sel = oracle.forward(inp.q, inp.k, inp.v, w.block, w.top_k, w.window, w.causal, rows=rows)
    wall = time.perf_counter() - t0
    D = w.head_dim
    routed = int((sel >= 0).sum()) * w.block
    if w.causal:
        t = rows % w.seq_len
        E = np.maximum(0, t // w.block - w.window // w.block + 1)
        win = int((t - w.block * E + 1).sum())
    else:
        win = 0
    flops = 4 * D * (routed + win)
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s (selected keys)",
            "cores": oracle.num_threads(), "kind": "oracle", **host_cpu(),
            "sample": f"{n} of {R} query rows of {w.name}, uniform without replacement; "
                      f"{wall:.1f} s wall; full layer extrapolated {wall * R / n * 1e3:.0f} ms",
            "ms_per_layer_extrapolated": wall * R / n * 1e3}


def oracle_rate(fn, n_rows):
    """Rows per second of a CPU-oracle call over n_rows sampled rows."""
    t0 = time.perf_counter()
    fn()
    wall = time.perf_counter() - t0
    return {"rows": n_rows, "s": wall, "rows_per_s": n_rows / wall}


def decode_bench(lsa, w, q, k, v, steps, inp=None):
    """One decode step (lsa_decode) for the last position of the workload's
    sequence, with the sequence as the key/value cache; steps timed between
    HIP-synchronised bracket points.  Algorithmic bytes per step: the block
    means of the eligible blocks of every KV group, plus, per query head, the
    K and V rows of its routed blocks and window."""
    import torch
    B, Hq, Hkv, N, D, bs = w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.block
    p = lsa.params(B, Hq, Hkv, N, D, bs, w.top_k, w.window, 1)
    kbar = lsa.block_summarize(p, k)
    qd = q[:, :, N - 1, :].contiguous()
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    idx = torch.empty((B, Hq, w.top_k), dtype=torch.int32, device=q.device)
    ws = torch.empty(lsa.workspace_bytes(p, lsa.OP_DECODE), dtype=torch.uint8, device=q.device)
    for _ in range(5):
        lsa.decode(p, N, qd, k, v, kbar, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        lsa.decode(p, N, qd, k, v, kbar, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    t = N - 1
    E = max(0, t // bs - w.window // bs + 1)
    used = int((idx >= 0).sum().item())
    keys = used * bs + B * Hq * (t - bs * E + 1)
    nbytes = B * Hkv * E * D * 4 + keys * D * 2 * 2
    res = {"cache_tokens": N, "us_per_step": us, "eligible_blocks": E,
            "algorithmic_bytes": nbytes, "hbm_gbs": nbytes / 1e3 / us,
            "hbm_frac": nbytes / 1e3 / us / PEAK_HBM_GBS,
            "note": "wall time per call, including launch overhead"}
    if inp is not None:
        import oracle
        rows = np.arange(B * Hq, dtype=np.int64) * N + (N - 1)
        r = oracle_rate(lambda: oracle.forward(inp.q, inp.k, inp.v, bs, w.top_k, w.window, 1,
                                               rows=rows), rows.size)
        res["cpu_oracle"] = {"kind": "oracle", "cores": oracle.num_threads(),
                             "us_per_step": r["s"] * 1e6,
                             "sample": "the step's rows: block means of the whole cache, "
                                       "routing and attention of position N-1 in every head"}
    return res


def consensus_bench(lsa, w, q, k, v, steps, inp=None):
    """The same layer with consensus routing (one route per KV group, scored
    by the sum of its query heads' scores): ms per layer, stage times and
    selected-key TFLOP/s (every query head attends through its group's
    route)."""
    import torch
    p = lsa.params(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.top_k,
                   w.window, w.causal, consensus=1)
    out = torch.empty((w.batch, w.q_heads, w.seq_len, w.head_dim), dtype=torch.float32,
                      device=q.device)
    idx = torch.empty(lsa.idx_shape(p), dtype=torch.int32, device=q.device)
    ws = torch.empty(lsa.workspace_bytes(p, lsa.OP_FORWARD), dtype=torch.uint8, device=q.device)
    for _ in range(3):
        lsa.forward(p, q, k, v, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    per_head = np.repeat(idx.cpu().numpy(), w.q_heads // w.kv_heads, axis=1)
    f_routed, f_window, _ = selected_flops(w, per_head)
    events = [lsa.StageEvents() for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        lsa.forward_profiled(p, q, k, v, events[i], out, idx, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    stage = np.array([e.stage_ms() for e in events]).mean(axis=0)
    for e in events:
        e.close()
    rep = w.q_heads // w.kv_heads
    route_ms = float(stage[1] + stage[2])
    flop = 2 * w.head_dim * routing_candidates(w) // rep   # one fp32-accurate score per candidate
    res = {"ms_per_layer": ms, "selected_tflop": (f_routed + f_window) / 1e12,
           "tflops": (f_routed + f_window) / 1e12 / (ms * 1e-3), "routing_ms": route_ms,
           "roofline": {"kernel": "routing (group rows)", "bound": "mfma",
                        "achieved": flop / 1e12 / (float(stage[1]) * 1e-3), "unit": "TFLOP/s",
                        "peak": PEAK_BF16_TFLOPS,
                        "frac": flop / 1e12 / (float(stage[1]) * 1e-3) / PEAK_BF16_TFLOPS},
           "stage_ms": {lsa.PROFILE_STAGES[i]: round(float(stage[i]), 4) for i in range(8)}}
    if inp is not None:
        import oracle
        per = w.seq_len if w.causal else w.seq_len // w.block
        G = w.batch * w.kv_heads * per
        rows = np.sort(np.random.default_rng(8).choice(G, size=min(G, 1000), replace=False))
        kbar = oracle.block_means(inp.k, w.block)
        if w.causal:
            fn = lambda: oracle.route_consensus(kbar, w.block, w.top_k, q=inp.q, window=w.window,
                                                causal=1, rows=rows)
        else:
            qbar = oracle.block_means(inp.q, w.block)
            fn = lambda: oracle.route_consensus(kbar, w.block, w.top_k, qbar=qbar, causal=0,
                                                rows=rows)
        r = oracle_rate(fn, rows.size)
        res["cpu_oracle"] = {"kind": "oracle", "cores": oracle.num_threads(),
                             "routing_rows_per_s": r["rows_per_s"],
                             "gpu_routing_rows_per_s": G / (route_ms * 1e-3),
                             "sample": f"routing of {rows.size} of {G} group rows"}
    return res


def cumulant_bench(lsa, w, q, k, v, steps, inp=None):
    """The layer routed by the second-cumulant score with beta = 1/sqrt(D):
    ms per layer, stage times, and the routing kernel against the bf16 MFMA
    peak, counting 2*D FLOP per (row, eligible key) for the raw scores whose
    per-block mean and variance form the score."""
    import torch
    beta = 1.0 / math.sqrt(w.head_dim)
    p = lsa.params(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.top_k,
                   w.window, 1, beta=beta)
    out = torch.empty((w.batch, w.q_heads, w.seq_len, w.head_dim), dtype=torch.float32,
                      device=q.device)
    idx = torch.empty(lsa.idx_shape(p), dtype=torch.int32, device=q.device)
    ws = torch.empty(lsa.workspace_bytes(p, lsa.OP_FORWARD), dtype=torch.uint8, device=q.device)
    lsa.forward(p, q, k, v, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    events = [lsa.StageEvents() for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        lsa.forward_profiled(p, q, k, v, events[i], out, idx, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    stage = np.array([e.stage_ms() for e in events]).mean(axis=0)
    for e in events:
        e.close()
    flop = 2 * w.head_dim * w.block * routing_candidates(w)
    route_ms = float(stage[1])
    res = {"beta": beta, "ms_per_layer": ms, "routing_ms": route_ms,
           "routing_tflop": flop / 1e12, "routing_tflops": flop / 1e12 / (route_ms * 1e-3),
           "routing_mfma_frac": flop / 1e12 / (route_ms * 1e-3) / PEAK_BF16_TFLOPS,
           "stage_ms": {lsa.PROFILE_STAGES[i]: round(float(stage[i]), 4) for i in range(8)}}
    if inp is not None:
        import oracle
        R = w.batch * w.q_heads * w.seq_len
        rows = np.sort(np.random.default_rng(9).choice(R, size=min(R, 200), replace=False))
        kbar = oracle.block_means(inp.k, w.block)
        r = oracle_rate(lambda: oracle.route_cumulant(inp.q, inp.k, kbar, w.block, w.top_k,
                                                      w.window, beta, rows=rows), rows.size)
        res["cpu_oracle"] = {"kind": "oracle", "cores": oracle.num_threads(),
                             "routing_rows_per_s": r["rows_per_s"],
                             "gpu_routing_rows_per_s": R / (route_ms * 1e-3),
                             "sample": f"routing of {rows.size} of {R} query rows "
                                       "(includes forming every block covariance once)"}
    return res


def tree_bench(lsa, w, q, k, v, beam, steps, inp=None):
    """The layer with two-level routing (nodes of 16 blocks, `beam` kept per
    row; in image mode the rows are the pooled query blocks): ms per layer
    and stage times (for this mode stage "routing" is the node level with
    the tail slots, and "routing fallback" is the block level over the kept
    nodes)."""
    import torch
    p = lsa.params(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.top_k,
                   w.window, w.causal, beam=beam)
    out = torch.empty((w.batch, w.q_heads, w.seq_len, w.head_dim), dtype=torch.float32,
                      device=q.device)
    idx = torch.empty(lsa.idx_shape(p), dtype=torch.int32, device=q.device)
    ws = torch.empty(lsa.workspace_bytes(p, lsa.OP_FORWARD), dtype=torch.uint8, device=q.device)
    for _ in range(2):
        lsa.forward(p, q, k, v, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    events = [lsa.StageEvents() for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        lsa.forward_profiled(p, q, k, v, events[i], out, idx, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    stage = np.array([e.stage_ms() for e in events]).mean(axis=0)
    for e in events:
        e.close()
    nb = w.seq_len // w.block
    if w.causal:
        t = np.arange(w.seq_len, dtype=np.int64)
        E = np.maximum(0, t // w.block - w.window // w.block + 1)
        per_head = w.seq_len
    else:
        E = np.full(nb, nb, dtype=np.int64)              # every query block, every key block
        per_head = nb
    S = E // 16
    heads = w.batch * w.q_heads
    scored = int((S + 16 * np.minimum(beam, S) + (E - 16 * S)).sum()) * heads
    rows = heads * per_head
    node_flop = 2 * w.head_dim * int(S.sum()) * heads
    # block level: per (row, node) pair the pair id, the gathered query row
    # (bf16, or the fp32 pooled query in image mode), 16 fp32 scores written
    # and read back, the pair position; per row its slot list and idx row
    qbytes = (2 if w.causal else 4) * w.head_dim
    pairs = int((np.minimum(beam, S) + (16 * S < E)).sum()) * heads
    blk_bytes = pairs * (4 + qbytes + 2 * 64 + 4) + rows * ((beam + 1) * 4 + w.top_k * 4)
    flat = routing_candidates(w)
    res = {"beam": beam, "ms_per_layer": ms,
           "node_level_ms": float(stage[1]), "block_level_ms": float(stage[2]),
           "routing_ms": float(stage[1] + stage[2]),
           "scores_per_layer": scored, "flat_scores_per_layer": flat,
           "node_level_roofline": {"bound": "mfma", "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS,
                                   "achieved": node_flop / 1e12 / (float(stage[1]) * 1e-3),
                                   "frac": node_flop / 1e12 / (float(stage[1]) * 1e-3)
                                   / PEAK_BF16_TFLOPS},
           "block_level_roofline": {"bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                    "bytes": blk_bytes, "pairs": pairs,
                                    "achieved": blk_bytes / 1e9 / (float(stage[2]) * 1e-3),
                                    "frac": blk_bytes / 1e9 / (float(stage[2]) * 1e-3)
                                    / PEAK_HBM_GBS},
           "stage_ms": {lsa.PROFILE_STAGES[i]: round(float(stage[i]), 4) for i in range(8)}}
    if inp is not None:
        import oracle
        sample = np.sort(np.random.default_rng(10).choice(rows, size=min(rows, 2000),
                                                          replace=False))
        kbar = oracle.block_means(inp.k, w.block)
        if w.causal:
            fn = lambda: oracle.route_tree(kbar, w.block, w.top_k, beam, q=inp.q,
                                           window=w.window, rows=sample)
        else:
            qbar = oracle.block_means(inp.q, w.block)
            fn = lambda: oracle.route_tree(kbar, w.block, w.top_k, beam, qbar=qbar, causal=0,
                                           rows=sample)
        r = oracle_rate(fn, sample.size)
        res["cpu_oracle"] = {"kind": "oracle", "cores": oracle.num_threads(),
                             "routing_rows_per_s": r["rows_per_s"],
                             "gpu_routing_rows_per_s": rows / (res["routing_ms"] * 1e-3),
                             "sample": f"routing of {sample.size} of {rows} "
                                       f"{'query rows' if w.causal else 'query blocks'}"}
    return res


def ties_bench(lsa, w, q, k, v, steps):
    """The same layer with every key replaced by the first one, so that every
    routing score ties: the survivor lists overflow and the exact routing
    passes decide every selection.  ms per layer and stage times, the counts
    of overflowing rows and routing tiles (the routing workspace's first two
    words), and whether every row took its lowest min(k, E) blocks."""
    import torch
    p = lsa.params(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.top_k,
                   w.window, w.causal)
    kt = k[:, :, :1, :].expand_as(k).contiguous()
    out = torch.empty((w.batch, w.q_heads, w.seq_len, w.head_dim), dtype=torch.float32,
                      device=q.device)
    idx = torch.empty(lsa.idx_shape(p), dtype=torch.int32, device=q.device)
    ws = torch.empty(lsa.workspace_bytes(p, lsa.OP_FORWARD), dtype=torch.uint8, device=q.device)
    for _ in range(2):
        lsa.forward(p, q, kt, v, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    events = [lsa.StageEvents() for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        lsa.forward_profiled(p, q, kt, v, events[i], out, idx, ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    stage = np.array([e.stage_ms() for e in events]).mean(axis=0)
    for e in events:
        e.close()
    got = idx.cpu().numpy().reshape(-1, w.seq_len if w.causal else w.seq_len // w.block, w.top_k)
    pos = np.arange(got.shape[1])
    E = np.maximum(0, pos // w.block - w.window // w.block + 1) if w.causal else np.full(pos.size, pos.size)
    m = np.minimum(w.top_k, E)
    slots = np.arange(w.top_k)[None, :]
    want = np.where(slots < m[:, None], slots, -1)
    wsr = torch.zeros(lsa.workspace_bytes(p, lsa.OP_ROUTE), dtype=torch.uint8, device=q.device)
    lsa.route_topk(p, q, lsa.block_summarize(p, kt), workspace=wsr)
    counts = wsr[:8].view(torch.int32).cpu().numpy()
    return {"ms_per_layer": ms, "rows": int(got.shape[0] * got.shape[1]),
            "overflow_rows": int(counts[0]), "overflow_tiles": int(counts[1]),
            "lowest_ids": bool(np.all(got == want[None])),
            "stage_ms": {lsa.PROFILE_STAGES[i]: round(float(stage[i]), 4) for i in range(8)}}


def copy_calibration():
    import torch
    n = 1 << 28                       # 256 Mi float32 = 1 GiB read + 1 GiB written
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                      "kernel": "torch.neg (elementwise)", "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards across GPUs with no exchange per (batch, KV head); "
              "this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    from content_routed_block_amd import lsa
    from content_routed_block_amd.workloads import WORKLOADS, generate

    w = WORKLOADS[args.workload]
    if args.top_k and args.top_k != w.top_k:
        import dataclasses
        w = dataclasses.replace(w, name=f"{w.name}_k{args.top_k}", top_k=args.top_k)
    inp = generate(w)
    dev = torch.device("cuda:0")

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    p = lsa.params(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.block, w.top_k,
                   w.window, w.causal, chunk=args.chunk)
    out = torch.empty((w.batch, w.q_heads, w.seq_len, w.head_dim), dtype=torch.float32, device=dev)
    rows = w.seq_len if w.causal else w.seq_len // w.block
    idx = torch.empty((w.batch, w.q_heads, rows, w.top_k), dtype=torch.int32, device=dev)
    ws = torch.empty(lsa.workspace_bytes(p, lsa.OP_FORWARD), dtype=torch.uint8, device=dev)

    for _ in range(args.warmup):
        lsa.forward(p, q, k, v, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    f_routed, f_window, routed_pairs = selected_flops(w, idx.cpu().numpy())
    f_sel = f_routed + f_window

    # the timed steps: lsa_forward as a caller runs it
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        lsa.forward(p, q, k, v, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    # stage times: the same steps again through lsa_forward_profiled (HIP
    # events recorded between the library's launches on its stream)
    events = [lsa.StageEvents() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        lsa.forward_profiled(p, q, k, v, events[i], out, idx, ws)
    torch.cuda.synchronize()
    ms_profiled = (time.perf_counter() - t0) / args.steps * 1e3
    stages = np.array([e.stage_ms() for e in events])            # [steps, 8]
    for e in events:
        e.close()
    stage_mean = stages.mean(axis=0)

    # Rooflines.  Summary: HBM-bound on its bytes.  Routing: MFMA-bound, 2*D
    # FLOP per (row, candidate block) score.  Causal attention kernels:
    # MFMA-bound on the selected-key FLOPs they compute (4*D per query and
    # selected key: the partials the routed keys, window + merge the window
    # keys).  Image-mode attention: HBM-bound on Q + K + V + idx + fp32 out.
    B, Hq, Hkv, N, D, bs = w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.block
    nb = N // bs
    rows = B * Hq * N
    kv_bytes = B * Hkv * N * D * 2                      # one of K, V
    summary_bytes = kv_bytes + B * Hkv * nb * D * 4
    cand = routing_candidates(w)
    idx_rows = rows if w.causal else B * Hq * nb
    route_bytes = B * Hq * N * D * 2 + idx_rows * w.top_k * 4 + B * Hkv * nb * D * 4
    if not w.causal:
        route_bytes += B * Hq * nb * D * 4               # pooled queries (read back)
    # the attention's algorithmic bytes: Q, K, V, idx and the fp32 output once
    attend_bytes = rows * D * 2 + 2 * kv_bytes + idx_rows * w.top_k * 4 + rows * D * 4
    work = {0: ("hbm", summary_bytes), 1: ("mfma", 2 * D * cand)}
    schedule = {}
    if w.causal:
        work[6] = ("mfma", f_routed)
        work[7] = ("mfma", f_window)
        # what the key-block-major schedule itself moves: per routed pair the
        # gathered Q row, the bf16 partial row, its log-mass and the pair id,
        # per bucket one K block and one V^T block; the merge reads the
        # partials back and streams Q, idx, K, V and the fp32 output
        buckets = B * Hkv * nb
        schedule[6] = routed_pairs * (D * 2 + D * 2 + 4 + 4) + buckets * 2 * bs * D * 2
        schedule[7] = (rows * (D * 2 + w.top_k * 4 + D * 4) + routed_pairs * (D * 2 + 4)
                       + 2 * kv_bytes)
    else:
        work[7] = ("hbm", attend_bytes)
    stage_frac = {}
    for i, (bound, amount) in work.items():
        t = stage_mean[i] * 1e-3
        name = lsa.PROFILE_STAGES[i]
        if bound == "hbm":
            ach = amount / 1e9 / t
            stage_frac[name] = {"bound": "hbm", "achieved": ach, "unit": "GB/s",
                                "peak": PEAK_HBM_GBS, "frac": ach / PEAK_HBM_GBS, "bytes": amount}
        else:
            ach = amount / 1e12 / t
            stage_frac[name] = {"bound": "mfma", "achieved": ach, "unit": "TFLOP/s",
                                "peak": PEAK_BF16_TFLOPS, "frac": ach / PEAK_BF16_TFLOPS,
                                "flop": amount}
        if i == 1:
            stage_frac[name]["hbm_frac"] = route_bytes / 1e9 / t / PEAK_HBM_GBS
        if i in schedule:
            stage_frac[name]["schedule_bytes"] = schedule[i]
            stage_frac[name]["schedule_traffic_frac"] = schedule[i] / 1e9 / t / PEAK_HBM_GBS
    dom = int(np.argmax(stage_mean))
    dom_name = lsa.PROFILE_STAGES[dom]
    d = stage_frac.get(dom_name)
    counters = traffic_counters(w)
    traffic = counters.get(dom_name) if counters else None
    roofline = {"bound": d["bound"] if d else "hbm", "achieved": d["achieved"] if d else None,
                "peak": d["peak"] if d else PEAK_HBM_GBS,
                "unit": d["unit"] if d else "GB/s", "frac": d["frac"] if d else None,
                "traffic": traffic, "kernel": dom_name, "kernel_ms": float(stage_mean[dom])}
    if d and "schedule_traffic_frac" in d:
        roofline["schedule_traffic_frac"] = d["schedule_traffic_frac"]
    attend_stages = [lsa.PROFILE_STAGES[i] for i in range(3, 8)]
    attend_traffic = None
    if counters:
        measured = sum(counters.get(n, 0.0) for n in attend_stages)
        attend_traffic = {"counter_bytes": measured, "algorithmic_bytes": attend_bytes,
                          "ratio": measured / attend_bytes,
                          "note": "HBM bytes of the attention stages from FETCH_SIZE / "
                                  "WRITE_SIZE counters over Q + K + V + idx + fp32 out"}
    breakdown = {lsa.PROFILE_STAGES[i]: round(float(stage_mean[i]), 4) for i in range(8)}
    attend_ms = float(stage_mean[3:].sum())
    # the timed steps' own selection and output, for the parity sample
    idx_host, out_host = idx.cpu().numpy(), out.cpu().numpy()

    result = {
        "metric": "sparse-attn ms/layer + selected-key TFLOP/s (%MFMA peak) at N=128K, Qwen0.5B shape",
        "value": f_sel / 1e12 / (ms * 1e-3),
        "unit": "TFLOP/s (selected keys)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded numpy PCG64; no dataset or weights)",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "seq_len": N,
                   "head_dim": D, "block": bs, "top_k": w.top_k, "window": w.window,
                   "causal": w.causal},
        "roofline": roofline,
        "layer": {"ms": ms, "ms_profiled": ms_profiled, "selected_tflop": f_sel / 1e12,
                  "mfma_frac": f_sel / 1e12 / (ms * 1e-3) / PEAK_BF16_TFLOPS,
                  "attend_ms": attend_ms,
                  "attend_mfma_frac": f_sel / 1e12 / (attend_ms * 1e-3) / PEAK_BF16_TFLOPS,
                  "attend_traffic": attend_traffic,
                  "workspace_bytes": lsa.workspace_bytes(p, lsa.OP_FORWARD),
                  "routed_pairs": routed_pairs, "stage_ms": breakdown, "stage_roofline": stage_frac},
    }
    if args.consensus_steps > 0 and w.q_heads > w.kv_heads:
        result["consensus"] = consensus_bench(lsa, w, q, k, v, args.consensus_steps,
                                              inp if args.cpu_seconds > 0 else None)
    if w.causal and args.cumulant_steps > 0 and w.seq_len <= 262144:
        result["cumulant"] = cumulant_bench(lsa, w, q, k, v, args.cumulant_steps,
                                            inp if args.cpu_seconds > 0 else None)
    if args.tree_beam > 0:
        result["tree"] = tree_bench(lsa, w, q, k, v, args.tree_beam, max(3, min(args.steps, 10)),
                                    inp if args.cpu_seconds > 0 else None)
    if w.causal and args.decode_steps > 0:
        result["decode"] = decode_bench(lsa, w, q, k, v, args.decode_steps,
                                        inp if args.cpu_seconds > 0 else None)
    if args.ties_steps > 0:
        result["ties"] = ties_bench(lsa, w, q, k, v, args.ties_steps)
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
        result["parity"] = parity_sample(w, inp, idx_host, out_host)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
