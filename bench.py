#!/usr/bin/env python3
"""Benchmark of the Pyramid Sparse Attention forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = the whole path on one batch of synthetic, seeded input already resident in HBM:
psa_build_pyramid, psa_mask (block scores, cosine check if any, threshold assignment),
psa_build_index and the level-weighted attention kernel. The pyramid and the mask are
independent and run side by side on two streams; the attention waits for both. The default workload is the
Wan2.1-1.3B-like 32k self-attention layer (12 heads, d 128, 32760 tokens padded to 32768,
query/KV blocks 128/64, sampling-mode mask with thresholds 0.5/0.7/0.8/0.9).

Prints one JSON line. `value` is whole-step throughput: executed level-weighted attention
FLOPs (4*d per executed (valid query, visible pooled key) pair) per second of step time.
`attn` gives the attention kernel alone (ms/layer, TFLOP/s, % of the 2.5 PFLOP/s dense bf16
MFMA peak, speedup over the same kernel on an all-level-0 map, and over the unpacked layout
with one logical block per hardware tile on the same map). `roofline` is for that
kernel, timed with HIP events on the stream it runs on. `bwd` times psa_attn_bwd on the same
map with a seeded output gradient (not part of `value`). `fp8` times the forward on e4m3
operands (psa_quantize_fp8 of Q, K, V; psa_attn_fwd_fp8qk with only the q . k products on fp8,
psa_attn_fwd_fp8 with the P V product too; same map; not part of `value`). `workloads` times the
attention kernel on each of the five workloads (its own inputs and map; not part of `value`).
`roofline.mfma` carries the MFMA busy fraction from the committed counter summary of the same
kernel source. `cpu_baseline` times the CPU oracle (fp64 numpy) on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, TFLOP/s
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, GB/s
METRIC = "psa_attn_fwd ms/layer + effective TFLOP/s (% bf16 MFMA peak), Wan-like 32k"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attn_fwd_bf16_traffic.txt")
ATTN_SOURCE = os.path.join(ROOT, "video_transformers_amd", "csrc", "psa_attn_bf16.hip")
# the attention's traffic also depends on the dispatch order the index builder writes
INDEX_SOURCE = os.path.join(ROOT, "video_transformers_amd", "csrc", "psa_index.hip")


def attn_sources_sha256() -> str:
    """sha256 over the attention kernel source and the index builder source, in that order:
    the counter summaries under profiles/ hold for this pair only."""
    h = hashlib.sha256()
    for path in (ATTN_SOURCE, INDEX_SOURCE):
        h.update(open(path, "rb").read())
    return h.hexdigest()


# ---------------------------------------------------------------------------------------
# work accounting (host side, from the level map)
# ---------------------------------------------------------------------------------------
def executed_pairs(level_map: np.ndarray, wl: W.Workload) -> int:
    """Number of (valid query, visible pooled key) pairs the level map executes: a pooled row j
    of level l stands for tokens [j*2^l, (j+1)*2^l) and is visible to query i iff its last
    token is < seq_valid and, when causal, <= i."""
    B, H, nqb, nkb = level_map.shape
    nv, bq = wl.seq_valid, wl.block_q
    total = 0
    kb = np.arange(nkb)
    # visible pooled rows per (kb, level) for non-causal attention
    vis = np.stack([np.clip(nv // (1 << l) - kb * (64 >> l), 0, 64 >> l) for l in range(4)], 1)
    nq = np.clip(nv - np.arange(nqb) * bq, 0, bq)
    if not wl.causal:
        for l in range(4):
            sel = (level_map == l)
            total += int(np.einsum("bhqk,k,q->", sel.astype(np.int64), vis[:, l], nq))
        return total
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                row = level_map[b, h, qb]
                lasts = []
                for l in range(4):
                    for k in np.flatnonzero(row == l):
                        j = np.arange(k * (64 >> l), (k + 1) * (64 >> l))
                        lasts.append((j + 1) * (1 << l) - 1)
                if not lasts:
                    continue
                lasts = np.sort(np.concatenate(lasts))
                qi = np.arange(qb * bq, qb * bq + nq[qb])
                lim = np.minimum(qi, nv - 1)
                total += int(np.searchsorted(lasts, lim, side="right").sum())
    return total


def dense_pairs(wl: W.Workload) -> int:
    nv = wl.seq_valid
    per_head = nv * (nv + 1) // 2 if wl.causal else nv * nv
    return wl.batch * wl.heads_q * per_head


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle, bounded sample, host cores
# ---------------------------------------------------------------------------------------
_G = {}


def _oracle_row(qb):
    import oracle
    from threadpoolctl import threadpool_limits
    g = _G
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        oracle.attention_head(g["q"], g["k"], g["v"], g["lm"], g["p"], qblocks=[qb])
        return time.perf_counter() - t


def cpu_baseline(wl: W.Workload, budget_s: float = 15.0) -> dict:
    """Times the oracle's attention on query blocks of head 0 (its own level map for that
    head) with a fork pool of one single-threaded worker per available core (at most 16)."""
    import multiprocessing as mp

    import oracle
    p = oracle.Problem.of(wl)
    q = oracle.as_f64(W.make_q(wl, [0]))[0, 0]
    k = oracle.as_f64(W.make_k(wl, [0]))[0, 0]
    v = oracle.as_f64(W.make_v(wl, [0]))[0, 0]
    if wl.map_source in ("iid", "fixed_frac"):
        lm = W.make_map(wl, [0])[0, 0]
    else:
        a = oracle.AssignParams(tuple(wl.thresholds), wl.cos_sim_min, wl.force_diag_l0,
                                wl.text_begin, wl.text_end)
        if wl.mask_mode == "sampling":
            M = oracle.mask_scores_sampling(q, k, p, wl.samples_per_qblock)
        elif wl.mask_mode == "meankey":
            M = oracle.mask_scores_meankey(q, k, p)
        else:
            M = oracle.mask_scores_antidiag(q, k, p, wl.antidiag_stride)
        sim = oracle.block_cossim(k, p) if wl.cos_sim_min > 0 else None
        lm = oracle.assign_levels(M, sim, p, a)
    _G.update(q=q, k=k, v=v, lm=lm, p=p)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t_one = _oracle_row(0)
    n_rows = int(min(wl.n_qblocks, max(workers, budget_s * workers / max(t_one, 1e-3))))
    rows = list(range(n_rows))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_row, rows, chunksize=1)
    wall = time.perf_counter() - t0
    pairs = executed_pairs(lm[None, None, :n_rows], wl.replace(heads_q=1, batch=1))
    flops = 4.0 * wl.head_dim * pairs
    return {"value": round(flops / wall / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
            "cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle attention over query blocks 0..{n_rows - 1} of head 0 "
                      f"(of {wl.heads_q} heads x {wl.n_qblocks} blocks), its own level map; "
                      f"{pairs} executed pairs in {wall:.2f} s on {workers} single-threaded "
                      f"processes"}


# ---------------------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------------------
def _traffic_from_profile(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, or None if
    the attention kernel source changed since the counters were taken or they were taken on
    another workload."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.lstrip().startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    sha = attn_sources_sha256()
    if kv.get("sources_sha256") != sha or kv.get("workload") != workload:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COUNTERS_FILE = os.path.join(ROOT, "profiles", "psa_path_wan2.1-1.3b_32k_counters.txt")
ATTN_KERNEL_BF16 = "k_attn_fwd_bf16<128, 128, true, true, 0, false>"


def _attn_counters(workload: str):
    """The bf16 attention kernel's rocprofv3 counters (mean per dispatch) from the committed
    summary, or None if the attention source changed since they were taken or the workload
    differs."""
    if workload != "wan2.1-1.3b_32k" or not os.path.exists(COUNTERS_FILE):
        return None
    sha = attn_sources_sha256()
    text = open(COUNTERS_FILE).read()
    if f"sources sha256: {sha}" not in text:
        return None
    out, cur = {}, None
    for line in text.splitlines():
        if line.startswith("#") or not line.strip():
            continue
        if not line.startswith(" "):
            cur = line.strip()
            continue
        if cur == ATTN_KERNEL_BF16:
            parts = line.split()
            try:
                out[parts[0]] = float(parts[1])
            except (IndexError, ValueError):
                pass
    return out or None


def _workload(args) -> W.Workload:
    wl = W.BY_NAME[args.workload]
    if args.mask_mode and wl.map_source == "mask":
        wl = wl.replace(mask_mode=args.mask_mode)
    return wl


def run(args) -> dict:
    import ctypes

    import torch
    import video_transformers_amd as psa

    wl = _workload(args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (t.to(dev) for t in W.make_qkv(wl))
    prob = psa.make_problem(q, k, v, block_q=wl.block_q, block_k=wl.block_k,
                            causal=wl.causal, seq_valid=wl.seq_valid)
    params = psa.MaskParams(mode=wl.mask_mode or "sampling",
                            thresholds=tuple(wl.thresholds) or (0.5, 0.7, 0.8, 0.9),
                            samples_per_qblock=wl.samples_per_qblock,
                            antidiag_stride=wl.antidiag_stride, cos_sim_min=wl.cos_sim_min,
                            force_diag_l0=wl.force_diag_l0, force_l0_begin=wl.text_begin,
                            force_l0_end=wl.text_end)
    computed_map = wl.map_source == "mask"
    drawn = None if computed_map else torch.from_numpy(W.make_map(wl)).to(dev)
    B, H, N, d = q.shape
    nqb, nkb = wl.n_qblocks, wl.n_kblocks

    # outputs and scratch allocated once
    kp = torch.empty((B, wl.heads_kv, psa.pooled_rows(prob), d), dtype=q.dtype, device=dev)
    vp = torch.empty_like(kp)
    lm_buf = torch.empty((B, H, nqb, nkb), dtype=torch.int8, device=dev)
    mass = torch.empty((B, H, nqb, nkb), dtype=torch.float32, device=dev)
    sim = (torch.empty((B, wl.heads_kv, nkb), dtype=torch.float32, device=dev)
           if wl.cos_sim_min > 0 else None)
    cp0 = params.c()
    mask_ws_bytes = psa.lib().psa_mask_workspace_bytes(prob.ref(), ctypes.byref(cp0)) if computed_map else 0
    mask_ws = torch.empty(max(mask_ws_bytes, 256), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(B * H * nqb * 5 + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(B * H * nqb * nkb, dtype=torch.int32, device=dev)
    dev_err = torch.empty(1, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    L = psa.lib()
    import ctypes
    cp = params.c()
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = ctypes.c_void_p(stream.cuda_stream)

    def check(rc, what):
        if rc != 0:
            raise psa.PsaError(rc, what)

    # The pyramid runs on a second stream beside the mask (they are independent: the pyramid
    # reads K, V and writes the pooled levels; the mask reads Q, K). The fork waits for the
    # previous step (its attention reads the pooled levels the pyramid overwrites); the
    # attention waits for the pyramid. Both streams have the default priority.
    side = torch.cuda.Stream(device=dev)
    st2 = ctypes.c_void_p(side.cuda_stream)
    fork, pyr_done = torch.cuda.Event(), torch.cuda.Event()

    def step(ev=None):
        fork.record(stream)
        side.wait_event(fork)
        if ev:
            ev[5].record(side)
        check(L.psa_build_pyramid(prob.ref(), ptr(k), ptr(v), ptr(kp), ptr(vp),
                                  psa.psa._dtype_code(kp.dtype), st2), "pyramid")
        if ev:
            ev[6].record(side)
        pyr_done.record(side)
        if ev:
            ev[1].record(stream)
        if computed_map:
            check(L.psa_mask(prob.ref(), ctypes.byref(cp), ptr(q), ptr(k), ptr(lm_buf), ptr(mass),
                             ptr(sim), ptr(mask_ws), mask_ws.numel(), st), "mask")
            lm = lm_buf
        else:
            lm = drawn
        if ev:
            ev[2].record(stream)
        check(L.psa_build_index(prob.ref(), ptr(lm), ptr(row_ptr), ptr(col_idx), ptr(dev_err), st),
              "index")
        stream.wait_event(pyr_done)
        if ev:
            ev[3].record(stream)
        check(L.psa_attn_fwd_indexed(prob.ref(), ctypes.c_float(0.0), ptr(q), ptr(k), ptr(v),
                                     ptr(kp), ptr(vp), ptr(row_ptr), ptr(col_idx), ptr(o),
                                     ptr(lse), st), "attn")
        if ev:
            ev[4].record(stream)
        return lm

    # a plain copy of known size, for scaling the HBM byte counters of a profiled run
    copy_bytes = 256 << 20
    cs = torch.empty(copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cd = torch.empty_like(cs)
    cd.copy_(cs)
    del cs, cd

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(dev_err.item()) != 0:
        raise RuntimeError("level map held invalid entries")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # pyramid (side stream), mask, index (with the wait for the pyramid), attention
    stage = np.array([[evs[i][5].elapsed_time(evs[i][6])] +
                      [evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(1, 4)]
                      for i in range(args.steps)])
    st_ms = stage.mean(axis=0)
    attn_ms = float(np.median(stage[:, 3]))
    attn_ms_mean = float(st_ms[3])

    lm_host = (lm_buf if computed_map else drawn).cpu().numpy()
    pairs = executed_pairs(lm_host, wl)
    flops = 4.0 * d * pairs
    dpairs = dense_pairs(wl)
    lv, cnt = np.unique(lm_host, return_counts=True)
    frac = {("skip" if int(a) < 0 else f"L{int(a)}"): round(float(c) / lm_host.size, 4)
            for a, c in zip(lv, cnt)}

    # the e4m3 QK^T forward on the same map, timed next to the step (same clocks)
    fp8 = None
    if not args.no_fp8 and wl.dtype == "bf16" and d == 128:
        lm_dev = lm_buf if computed_map else drawn
        fp8 = _fp8_run(wl, prob, L, ptr, st, check, q, k, v, kp, vp, lm_dev, stream, flops,
                       float(st_ms[2]), attn_ms_mean)
    # same kernel, all-level-0 map (causal: the lower triangle)
    dense_ms = float("nan")
    if not args.no_dense:
        dense_ms = _dense_run(args, wl, prob, L, ptr, st, check, q, k, v, kp, vp, o, lse,
                              row_ptr, col_idx, dev_err, stream)
    # same map, same index, one logical block per hardware tile (the unpacked ablation)
    unpacked_ms = float("nan")
    if not args.no_unpacked and wl.dtype == "bf16":
        def unpacked():
            check(L.psa_attn_fwd_unpacked(prob.ref(), ctypes.c_float(0.0), ptr(q), ptr(k), ptr(v),
                                          ptr(kp), ptr(vp), ptr(row_ptr), ptr(col_idx), ptr(o),
                                          ptr(lse), st), "attn unpacked")
        unpacked_ms = _timed_back_to_back(unpacked, stream, reps=4, warm=1)
    sustained = None
    if not args.no_sustained:
        def attn_call():
            check(L.psa_attn_fwd_indexed(prob.ref(), ctypes.c_float(0.0), ptr(q), ptr(k), ptr(v),
                                         ptr(kp), ptr(vp), ptr(row_ptr), ptr(col_idx), ptr(o),
                                         ptr(lse), st), "attn sustained")
        sustained = _sustained_attention(attn_call, stream, flops)
    meankey = None
    if (not args.no_meankey and computed_map and wl.dtype == "bf16" and wl.block_q == 128
            and nkb <= 1792):
        meankey = _meankey_run(wl, prob, params, L, ptr, st, check, q, k, v, kp, vp, stream)
    bwd = None
    if not args.no_bwd and wl.dtype == "bf16":
        bwd = _bwd_run(wl, prob, L, ptr, st, check, q, k, v, kp, vp, lm_host, o, lse, stream, flops)
    out = _report(args, wl, flops, pairs, dpairs, frac, d, B, H, N, computed_map, attn_ms,
                  attn_ms_mean, st_ms, dense_ms, wall)
    if bwd is not None:
        out["bwd"] = bwd
    if fp8 is not None:
        out["fp8"] = fp8
    if meankey is not None:
        out["meankey_fused"] = meankey
    if not args.no_workloads:
        # every workload's attention kernel, driver-observed in this same line (the step
        # above is the metric's workload; these are reported beside it)
        out["workloads"] = {w.name: _workload_attention(w, dev) for w in W.ALL}
    if sustained is not None:
        out["attn"]["sustained"] = sustained
    out["attn"]["unpacked_same_map_ms"] = None if unpacked_ms != unpacked_ms else round(unpacked_ms, 3)
    out["attn"]["speedup_vs_unpacked"] = (None if unpacked_ms != unpacked_ms
                                          else round(unpacked_ms / attn_ms_mean, 2))
    return out


def _workload_attention(wl, dev, reps: int = 10) -> dict:
    """One workload's attention on its own map (psa_mask, or the drawn map), inputs resident:
    mean of about 0.3 s (at least `reps`) of back-to-back psa_attn_fwd_indexed calls after about
    0.2 s of untimed ones (sustained attention load, unlike the step, where the pyramid and the
    mask run between attention calls), executed level-weighted FLOP over that time, and the pyramid, psa_mask and
    psa_build_index calls, each the mean of 5 back-to-back calls after its first."""
    import ctypes
    import torch
    import video_transformers_amd as psa
    L = psa.lib()
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = torch.cuda.current_stream()
    st = ctypes.c_void_p(stream.cuda_stream)
    q, k, v = (t.to(dev) for t in W.make_qkv(wl))
    prob = psa.make_problem(q, k, v, block_q=wl.block_q, block_k=wl.block_k, causal=wl.causal,
                            seq_valid=wl.seq_valid)
    drawn = None if wl.map_source == "mask" else torch.from_numpy(W.make_map(wl)).to(dev)
    kp, vp = psa.build_pyramid(k, v, prob)
    pyramid_ms = _timed_back_to_back(lambda: psa.build_pyramid(k, v, prob), stream, reps=5, warm=0)
    mask_ms = None
    if wl.map_source == "mask":
        params = psa.MaskParams(mode=wl.mask_mode, thresholds=tuple(wl.thresholds),
                                samples_per_qblock=wl.samples_per_qblock,
                                antidiag_stride=wl.antidiag_stride, cos_sim_min=wl.cos_sim_min,
                                force_diag_l0=wl.force_diag_l0, force_l0_begin=wl.text_begin,
                                force_l0_end=wl.text_end)
        lm, _, _ = psa.mask(q, k, prob, params)
        mask_ms = _timed_back_to_back(lambda: psa.mask(q, k, prob, params), stream, reps=5, warm=0)
    else:
        lm = drawn
    rp, ci, err = psa.build_index(lm, prob)
    index_ms = _timed_back_to_back(lambda: psa.build_index(lm, prob), stream, reps=5, warm=0)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def call():
        rc = L.psa_attn_fwd_indexed(prob.ref(), ctypes.c_float(0.0), ptr(q), ptr(k), ptr(v),
                                    ptr(kp), ptr(vp), ptr(rp), ptr(ci), ptr(o), ptr(lse), st)
        if rc != 0:
            raise psa.PsaError(rc, f"attn {wl.name}")
    # warm up for about 0.2 s (the clocks settle under a sustained load), then time about 0.3 s
    # of calls (at least `reps`)
    est = _timed_back_to_back(call, stream, reps=2, warm=1)
    warm = max(2, int(200.0 / max(est, 1e-3)))
    ms = _timed_back_to_back(call, stream, reps=max(reps, int(300.0 / max(est, 1e-3))), warm=warm)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"{wl.name}: level map held invalid entries")
    lm_host = lm.cpu().numpy()
    pairs = executed_pairs(lm_host, wl)
    d = wl.head_dim
    tf = 4.0 * d * pairs / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    out = {"attn_ms": round(ms, 4), "tflops_executed": round(tf, 2),
           "pct_peak": round(100 * tf / peak, 2),
           "peak": f"{'bf16' if wl.dtype == 'bf16' else 'fp32'} MFMA {peak:.1f} TFLOP/s",
           "executed_pairs": int(pairs),
           "effective_sparsity": round(1.0 - pairs / dense_pairs(wl), 4),
           "pyramid_ms": round(pyramid_ms, 4),
           "mask_ms": None if mask_ms is None else round(mask_ms, 4),
           "index_ms": round(index_ms, 4),
           "map": (f"psa_mask {wl.mask_mode}" if wl.map_source == "mask" else f"drawn ({wl.map_source})"),
           "shape": f"B{wl.batch} H{wl.heads_q}/{wl.heads_kv} N{wl.seq_len} (valid {wl.seq_valid}) "
                    f"d{d} {wl.dtype} block_q {wl.block_q}{' causal' if wl.causal else ''}"}
    del q, k, v, kp, vp, lm, rp, ci, o, lse
    torch.cuda.empty_cache()
    return out


def _smi_sample() -> dict:
    """Graphics clocks (MHz, one per XCD) and socket power (W) as amd-smi reports them now, or
    an empty dict when amd-smi is not installed or its output is not understood."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "-p"], capture_output=True, text=True, timeout=15)
    except (OSError, subprocess.SubprocessError):
        return {}
    clks = [int(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", r.stdout)]
    pw = re.findall(r"SOCKET_POWER:\s*(\d+)", r.stdout)
    out = {}
    if clks:
        out["gfx_clock_mhz"] = {"min": min(clks), "mean": round(sum(clks) / len(clks)), "max": max(clks)}
    if pw:
        out["socket_power_w"] = int(pw[0])
    return out


def _sustained_attention(fn, stream, flops: float, seconds: float = 3.0) -> dict:
    """The attention call back to back for about `seconds` (long enough for the GPU to settle
    at its power limit, as in a model's layer loop), timed over the last third in batches of
    20 calls bracketed by HIP events on the launch stream; clocks and power sampled once in
    that last third."""
    import threading
    import time

    import torch
    t0 = time.time()
    smi = {}
    sampler = None
    times = []
    while True:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(20):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        el = time.time() - t0
        if el > seconds * 2 / 3:
            times.append(ev[0].elapsed_time(ev[1]) / 20)
            if sampler is None:
                sampler = threading.Thread(target=lambda: smi.update(_smi_sample()))
                sampler.start()
        if el > seconds and sampler is not None and not sampler.is_alive():
            break
        if el > 4 * seconds:
            break
    ms = sorted(times)[len(times) // 2]
    out = {"ms_per_layer_median": round(ms, 4), "tflops_executed": round(flops / (ms * 1e-3) / 1e12, 2),
           "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
           "calls_timed": 20 * len(times),
           "note": "back-to-back calls for about 3 s; the median batch of the last third"}
    out.update(smi)
    clk = smi.get("gfx_clock_mhz")
    if clk:
        # the bf16 MFMA peak scales with the graphics clock (2.5 PFLOP/s at 2.4 GHz); under this
        # sustained load the power limit holds the clock below that
        peak_at_clock = PEAK_BF16_TFLOPS * clk["mean"] / 2400.0
        out["bf16_peak_at_mean_clock"] = round(peak_at_clock, 1)
        out["pct_of_peak_at_mean_clock"] = round(100 * flops / (ms * 1e-3) / 1e12 / peak_at_clock, 2)
    return out


def _timed_back_to_back(fn, stream, reps: int = 10, warm: int = 2) -> float:
    """Mean ms per call of `reps` calls enqueued back to back (as the step loop runs), after
    `warm` untimed calls; HIP events on the launch stream bracket the whole run."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        fn()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def _bwd_run(wl, prob, L, ptr, st, check, q, k, v, kp, vp, lm_host, o, lse, stream, fwd_flops):
    """psa_attn_bwd on the step's map, o and lse with a seeded output gradient: mean of 5 calls
    run back to back (the call builds its block index and runs its four kernels). Work is
    counted as 2.5x the forward's executed FLOPs (recomputed S, then dP, dV, dK, dQ: 10*d per
    executed pair)."""
    import ctypes
    import torch
    dev = q.device
    dout = W.make_dout(wl).to(dev)
    lm = torch.from_numpy(lm_host).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    n = L.psa_attn_bwd_workspace_bytes(prob.ref())
    ws = torch.empty(n, dtype=torch.uint8, device=dev)

    def call():
        check(L.psa_attn_bwd(prob.ref(), ctypes.c_float(0.0), ptr(q), ptr(k), ptr(v), ptr(kp),
                             ptr(vp), ptr(lm), ptr(o), ptr(lse), ptr(dout), ptr(dq), ptr(dk),
                             ptr(dv), ptr(ws), n, st), "attn bwd")
    ms = _timed_back_to_back(call, stream, reps=5)
    check(L.psa_check_status(ptr(ws), st), "attn bwd status")
    tf = 2.5 * fwd_flops / (ms * 1e-3) / 1e12
    return {"ms_per_layer": round(ms, 4), "tflops_algorithmic": round(tf, 2),
            "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "work": "2.5x the forward's executed FLOP (10*d per executed pair)",
            "workspace_bytes": n}


def _fp8_run(wl, prob, L, ptr, st, check, q, k, v, kp, vp, lm, stream, fwd_flops, index_ms,
             bf16_attn_ms):
    """The e4m3 forwards on the step's map: psa_quantize_fp8 of Q, of K with its pooled rows and
    of V with its pooled rows, then psa_attn_fwd_fp8qk (q . k on fp8, P V in bf16) and
    psa_attn_fwd_fp8 (both products on fp8); each call builds its block index, then runs the
    kernel. Means of 10 calls run back to back. A kernel's own time is estimated as its call
    minus the index build timed in the step (same map, same kernels). Bounds: fp8qk mixes two
    peaks (the q . k half of the executed FLOP, 2*d per pair, at the fp8 MFMA peak, the P V
    half at the bf16 one); fp8 puts all of it at the fp8 peak."""
    import ctypes
    import torch
    dev = q.device
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    u8 = lambda shape: torch.empty(shape, dtype=torch.uint8, device=dev)  # noqa: E731
    k8, kp8, v8, vp8, q8 = u8((B, Hkv, N, d)), u8(kp.shape), u8((B, Hkv, N, d)), u8(vp.shape), u8((B, H, N, d))
    sk = torch.empty(B * Hkv, dtype=torch.float32, device=dev)
    sv = torch.empty(B * Hkv, dtype=torch.float32, device=dev)
    sq = torch.empty(B * H, dtype=torch.float32, device=dev)
    o8 = torch.empty_like(q)
    lse8 = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    n = L.psa_attn_workspace_bytes(prob.ref())
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    kst = (ctypes.c_int64 * 3)(*k.stride()[:3])
    vst = (ctypes.c_int64 * 3)(*v.stride()[:3])
    qst = (ctypes.c_int64 * 3)(*q.stride()[:3])

    def quant_qk():
        check(L.psa_quantize_fp8(B, Hkv, N, d, ptr(k), kst, ptr(kp), ptr(k8), ptr(kp8), ptr(sk), st),
              "quantize k")
        check(L.psa_quantize_fp8(B, H, N, d, ptr(q), qst, None, ptr(q8), None, ptr(sq), st),
              "quantize q")

    def quant_v():
        check(L.psa_quantize_fp8(B, Hkv, N, d, ptr(v), vst, ptr(vp), ptr(v8), ptr(vp8), ptr(sv), st),
              "quantize v")

    def attn_qk():
        check(L.psa_attn_fwd_fp8qk(prob.ref(), ctypes.c_float(0.0), ptr(q8), ptr(sq), ptr(k8),
                                   ptr(kp8), ptr(sk), ptr(v), ptr(vp), ptr(lm), ptr(o8), ptr(lse8),
                                   ptr(ws), n, st), "attn fp8qk")

    def attn_all():
        check(L.psa_attn_fwd_fp8(prob.ref(), ctypes.c_float(0.0), ptr(q8), ptr(sq), ptr(k8),
                                 ptr(kp8), ptr(sk), ptr(v8), ptr(vp8), ptr(sv), ptr(lm), ptr(o8),
                                 ptr(lse8), ptr(ws), n, st), "attn fp8")

    qk_ms = _timed_back_to_back(quant_qk, stream)
    v_ms = _timed_back_to_back(quant_v, stream)

    def report(call_ms, bound_ms, peak):
        kern_ms = call_ms - index_ms
        tf = fwd_flops / (kern_ms * 1e-3) / 1e12
        return {"attn_call_ms": round(call_ms, 4), "attn_kernel_ms_est": round(kern_ms, 4),
                "tflops_executed": round(tf, 2),
                "speedup_vs_bf16_kernel": round(bf16_attn_ms / kern_ms, 3),
                "roofline": {"bound": "mfma", "peak": peak, "min_ms": round(bound_ms, 4),
                             "frac": round(bound_ms / kern_ms, 4)}}
    half = fwd_flops / 2
    out = {"quantize_q_k_ms": round(qk_ms, 4), "quantize_v_ms": round(v_ms, 4),
           "qk": report(_timed_back_to_back(attn_qk, stream),
                        (half / PEAK_FP8_TFLOPS + half / PEAK_BF16_TFLOPS) / 1e12 * 1e3,
                        "fp8 5000 TFLOP/s for q.k, bf16 2500 for P V"),
           "qk_pv": report(_timed_back_to_back(attn_all, stream),
                           fwd_flops / PEAK_FP8_TFLOPS / 1e12 * 1e3, "fp8 5000 TFLOP/s"),
           "quantization": "e4m3, one scale per (batch, head) for Q, K, V (pooled rows share "
                           "their head's); P relative to 2^(ceil(row max) - 7)"}
    check(L.psa_check_status(ptr(ws), st), "attn fp8 status")
    return out


def _meankey_run(wl, prob, params, L, ptr, st, check, q, k, v, kp, vp, stream):
    """Block-mean scoring, two ways, on the step's q, k, v and pyramid: psa_mask in block-mean
    mode, psa_build_index and psa_attn_fwd_indexed (three calls), against psa_attn_fwd_meankey
    (scoring, assignment and attention in one launch after the block means). Both write the map
    and the masses; means of 10 calls run back to back. The map is checked equal."""
    import ctypes
    import dataclasses
    import torch
    dev = q.device
    B, H, N, d = q.shape
    nqb, nkb = wl.n_qblocks, wl.n_kblocks
    mk = dataclasses.replace(params, mode="meankey")
    cp = mk.c()
    lm2 = torch.empty((B, H, nqb, nkb), dtype=torch.int8, device=dev)
    lmf = torch.empty_like(lm2)
    m2 = torch.empty((B, H, nqb, nkb), dtype=torch.float32, device=dev)
    mf = torch.empty_like(m2)
    sim = (torch.empty((B, wl.heads_kv, nkb), dtype=torch.float32, device=dev)
           if wl.cos_sim_min > 0 else None)
    nm = L.psa_mask_workspace_bytes(prob.ref(), ctypes.byref(cp))
    mws = torch.empty(max(nm, 256), dtype=torch.uint8, device=dev)
    nf = L.psa_attn_fwd_meankey_workspace_bytes(prob.ref())
    fws = torch.empty(max(nf, 256), dtype=torch.uint8, device=dev)
    rp = torch.empty(B * H * nqb * 5 + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(B * H * nqb * nkb, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    o2, of = torch.empty_like(q), torch.empty_like(q)
    l2 = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    lf = torch.empty_like(l2)

    def two_step():
        check(L.psa_mask(prob.ref(), ctypes.byref(cp), ptr(q), ptr(k), ptr(lm2), ptr(m2), ptr(sim),
                         ptr(mws), mws.numel(), st), "mask meankey")
        check(L.psa_build_index(prob.ref(), ptr(lm2), ptr(rp), ptr(ci), ptr(err), st), "index")
        check(L.psa_attn_fwd_indexed(prob.ref(), ctypes.c_float(0.0), ptr(q), ptr(k), ptr(v),
                                     ptr(kp), ptr(vp), ptr(rp), ptr(ci), ptr(o2), ptr(l2), st),
              "attn")

    def fused():
        check(L.psa_attn_fwd_meankey(prob.ref(), ctypes.byref(cp), ctypes.c_float(0.0), ptr(q),
                                     ptr(k), ptr(v), ptr(kp), ptr(vp), ptr(lmf), ptr(mf), ptr(of),
                                     ptr(lf), ptr(fws), fws.numel(), st), "attn meankey")
    two_ms = _timed_back_to_back(two_step, stream)
    fused_ms = _timed_back_to_back(fused, stream)
    torch.cuda.synchronize()
    same = bool(torch.equal(lm2, lmf) and torch.equal(o2, of))
    lm_host = lmf.cpu().numpy()
    pairs = executed_pairs(lm_host, wl)
    tf = 4.0 * d * pairs / (fused_ms * 1e-3) / 1e12
    return {"two_step_ms": round(two_ms, 4), "fused_ms": round(fused_ms, 4),
            "speedup": round(two_ms / fused_ms, 3), "same_map_and_output": same,
            "executed_pairs": int(pairs), "fused_tflops_executed": round(tf, 2),
            "two_step": "psa_mask (block means, scores, assignment) + psa_build_index + psa_attn_fwd_indexed",
            "fused": "psa_attn_fwd_meankey (block means, then one launch: scores, assignment, attention)"}


def _dense_run(args, wl, prob, L, ptr, st, check, q, k, v, kp, vp, o, lse, row_ptr, col_idx,
               dev_err, stream):
    import ctypes
    import torch
    B, H, N, d = q.shape
    nqb, nkb = wl.n_qblocks, wl.n_kblocks
    dev = q.device
    dense = torch.zeros((B, H, nqb, nkb), dtype=torch.int8, device=dev)
    if wl.causal:
        qb_i = torch.arange(nqb, device=dev)[:, None]
        kb_i = torch.arange(nkb, device=dev)[None, :]
        dense[:, :, kb_i.expand(nqb, nkb) * 64 > (qb_i + 1) * wl.block_q - 1] = -1
    rp_d = torch.empty_like(row_ptr)
    ci_d = torch.empty_like(col_idx)
    check(L.psa_build_index(prob.ref(), ptr(dense), ptr(rp_d), ptr(ci_d), ptr(dev_err), st), "index")
    def dense_call():
        check(L.psa_attn_fwd_indexed(prob.ref(), ctypes.c_float(0.0), ptr(q), ptr(k), ptr(v),
                                     ptr(kp), ptr(vp), ptr(rp_d), ptr(ci_d), ptr(o), ptr(lse), st),
              "attn dense")
    return _timed_back_to_back(dense_call, stream, reps=3, warm=1)


def _report(args, wl, flops, pairs, dpairs, frac, d, B, H, N, computed_map, attn_ms,
            attn_ms_mean, st_ms, dense_ms, wall):
    ms_per_step = wall * 1e3 / args.steps
    attn_tflops = flops / (attn_ms_mean * 1e-3) / 1e12
    traffic = _traffic_from_profile(wl.name)
    ctr = _attn_counters(wl.name) if wl.dtype == "bf16" else None
    mfma = None
    if ctr and "SQ_VALU_MFMA_BUSY_CYCLES" in ctr and "SQ_INSTS_MFMA" in ctr:
        # busy cycles summed over the 1024 SIMDs, against this run's kernel time at the 2.4 GHz
        # the peak is quoted at (the clock under MFMA load is lower, so this understates it)
        simd_cycles = 1024 * attn_ms_mean * 1e-3 * 2.4e9
        issued = ctr["SQ_INSTS_MFMA"] * 2 * 32 * 32 * 16
        mfma = {"busy_pct": round(100 * ctr["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles, 1),
                "issued_tflop_per_launch": round(issued / 1e12, 4),
                "issued_tflops": round(issued / (attn_ms_mean * 1e-3) / 1e12, 1),
                "executed_over_issued": round(flops / issued, 4),
                "source": os.path.relpath(COUNTERS_FILE, ROOT) + " (SQ_VALU_MFMA_BUSY_CYCLES, "
                          "SQ_INSTS_MFMA; this run's kernel time; 1024 SIMDs at 2.4 GHz)"}
        if "GRBM_GUI_ACTIVE" in ctr:
            # the same busy cycles against the cycles the GPU was active in the profiled
            # launches at the clock it actually ran (GRBM_GUI_ACTIVE sums the 8 XCDs)
            active = ctr["GRBM_GUI_ACTIVE"] / 8
            mfma["busy_pct_of_active_cycles"] = round(100 * ctr["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * active), 1)
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; clustered keys, no weights or videos)",
        "config": {"workload": wl.name, "batch": B, "heads_q": H, "heads_kv": wl.heads_kv,
                   "seq_len": N, "seq_valid": wl.seq_valid, "head_dim": d,
                   "block_q": wl.block_q, "block_k": wl.block_k, "causal": wl.causal,
                   "map": (f"psa_mask {wl.mask_mode} thresholds {list(wl.thresholds)}"
                           if computed_map else f"drawn ({wl.map_source})")},
        "attn": {"ms_per_layer_median": round(attn_ms, 4), "ms_per_layer_mean": round(attn_ms_mean, 4),
                 "tflops_executed": round(attn_tflops, 2),
                 "pct_bf16_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
                 "dense_same_kernel_ms": None if dense_ms != dense_ms else round(dense_ms, 3),
                 "speedup_vs_dense": None if dense_ms != dense_ms else round(dense_ms / attn_ms_mean, 2),
                 "dense_tflops": (None if dense_ms != dense_ms
                                  else round(4.0 * d * dpairs / (dense_ms * 1e-3) / 1e12, 2)),
                 "executed_pairs": pairs,
                 "effective_sparsity": round(1.0 - pairs / dpairs, 4),
                 "level_fractions": frac},
        "stages_ms": {"build_pyramid": round(float(st_ms[0]), 4), "mask": round(float(st_ms[1]), 4),
                      "build_index": round(float(st_ms[2]), 4), "attn_kernel": round(float(st_ms[3]), 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     # the counted bytes over this run's kernel time: what the L2s fetch from
                     # the fabric (HBM or the Infinity Cache), against the HBM peak
                     "traffic_gbs": None if traffic is None else round(traffic / (attn_ms_mean * 1e-3) / 1e9, 1),
                     "traffic_vs_hbm_peak": (None if traffic is None
                                             else round(traffic / (attn_ms_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)),
                     "mfma": mfma,
                     "kernel": "k_attn_fwd_bf16" if wl.dtype == "bf16" else "k_attn_fwd_f32",
                     "per_launch": f"{flops:.4e} executed FLOP (4*d per executed pair)"},
    }
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-sustained", action="store_true",
                    help="skip the sustained (power-limited) attention measurement")
    ap.add_argument("--workload", default=W.WAN13B_32K.name, choices=sorted(W.BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the all-level-0 comparison run (for profiling the PSA launches alone)")
    ap.add_argument("--no-unpacked", action="store_true",
                    help="skip the unpacked-layout comparison run (one logical block per tile)")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the psa_attn_bwd timing (reported beside the forward metric)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the e4m3 forward timings (reported beside the forward metric)")
    ap.add_argument("--no-meankey", action="store_true",
                    help="skip the block-mean scoring comparison (two-step against fused)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the attention timings of all five workloads (reported beside the metric)")
    ap.add_argument("--mask-mode", choices=("sampling", "antidiag", "meankey"), default=None,
                    help="score with this psa_mask mode instead of the workload's own")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(every (batch, head) is independent, so heads would shard with no exchange). "
              "Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    wl = _workload(args)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_budget)      # before the GPU is touched (fork pool)
    out = run(args)
    out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
