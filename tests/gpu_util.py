"""Shared helpers for the GPU tests: run the HIP path on seeded workload inputs and compare
with the CPU oracle. Inputs come from the workloads module only; expected values come from
the oracle only."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import video_transformers_amd as psa

DEV = "cuda"

# Parity bars. bf16 attention outputs: max-abs 2e-2 and relative L2 5e-3 (the target bar).
# float32 runs get a tighter bar (float32 MFMA and float32 pooled levels: ~1e-6 expected).
# LSE, bf16: level-0 logits are exact products of bf16 inputs accumulated in float32, but a
# pooled key is the bf16 rounding of a mean, |dK_e| <= 2^-9 |K_e|, so a logit moves by up to
# s * 2^-9 * sum_e |q_e K_e|; for unit-variance q and keys with |K_e| ~ 2 at d = 128 that is
# ~3e-2 at worst and ~2e-3 typically. The lse moves by a weighted mean of the logit errors,
# so a query that sees only a few pooled tokens (early causal rows) can reach the worst case:
# bar 3e-2. float32: 1e-5.
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
F32_MAX_ABS = 1e-4
F32_REL_L2 = 1e-5
LSE_ABS_BF16 = 3e-2
LSE_ABS_F32 = 1e-5
# Against the oracle reading whose pooled levels are the bf16 rounding of the exact means (what
# a bf16 pyramid stores and the kernel reads), the pooled keys are the same on both sides. What
# remains: the kernel forms the row sum from the bf16-rounded weights P (the same values that
# multiply V, so o stays normalised by its own weights), each within 2^-9 relative of the exact
# weight, so the sum, a weighted mean of those errors, is within 2^-9 relative and the lse
# within ln(1 + 2^-9) = 1.95e-3 (reached when one key dominates a row); float32 accumulation of
# the logits and exp2 add ~1e-6. Bar: 2e-3.
LSE_ABS_BF16_POOLED = 2e-3
# The library's certification margins per scoring mode (absolute, relative): a row whose
# float32 threshold decisions lie within them is rescored in float64.
CERT_MARGINS = {"sampling": (4e-6, 8e-6), "meankey": (4e-6, 8e-6), "antidiag": (5e-6, 3.3e-5)}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def announce(msg: str) -> None:
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def problem_for(wl: W.Workload, q, k, v) -> psa.Problem:
    return psa.make_problem(q, k, v, block_q=wl.block_q, block_k=wl.block_k, causal=wl.causal,
                            seq_valid=wl.seq_valid)


def oracle_problem(wl: W.Workload) -> oracle.Problem:
    return oracle.Problem.of(wl)


def assign_params(wl: W.Workload) -> oracle.AssignParams:
    return oracle.AssignParams(tuple(wl.thresholds), wl.cos_sim_min, wl.force_diag_l0,
                               wl.text_begin, wl.text_end)


def mask_params(wl: W.Workload) -> psa.MaskParams:
    return psa.MaskParams(mode=wl.mask_mode or "sampling",
                          thresholds=tuple(wl.thresholds) if wl.thresholds else (0.5, 0.7, 0.8, 0.9),
                          samples_per_qblock=wl.samples_per_qblock,
                          antidiag_stride=wl.antidiag_stride, cos_sim_min=wl.cos_sim_min,
                          force_diag_l0=wl.force_diag_l0, force_l0_begin=wl.text_begin,
                          force_l0_end=wl.text_end)


def oracle_map(wl: W.Workload, q, k, heads=None):
    """The level map the oracle assigns: drawn maps come from the workload's generator,
    computed maps from the oracle's own mask generator on the same inputs."""
    if wl.map_source in ("iid", "fixed_frac"):
        return W.make_map(wl, heads)
    lm, M, sim = oracle.mask(q, k, oracle_problem(wl), wl.mask_mode, assign_params(wl),
                             samples=wl.samples_per_qblock, stride=wl.antidiag_stride)
    return lm


def compare_outputs(o_gpu, o_ref, valid_rows, f32: bool):
    """(max_abs, rel_l2) over valid rows."""
    a = o_gpu[..., :valid_rows, :].double().cpu().numpy()
    r = o_ref[..., :valid_rows, :]
    diff = a - r
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(r), 1e-30))
    return max_abs, rel


def _check_lse(lse_gpu, lse_ref, valid_rows, bar, what):
    lg = lse_gpu[..., :valid_rows].double().cpu().numpy()
    lr = lse_ref[..., :valid_rows]
    both_inf = np.isneginf(lg) & np.isneginf(lr)
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), f"{what}: empty-row sets differ"
    d = np.abs(lg[~both_inf] - lr[~both_inf])
    print(f"[{what}] lse max diff {d.max(initial=0.0):.3e} (bar {bar:.0e})", flush=True)
    assert d.max(initial=0.0) <= bar, f"{what}: lse diff {d.max()} > {bar}"


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, valid_rows, f32: bool, what: str,
                    ref_pooled_bf16=None):
    """o and lse against the exact-mean oracle (o at the workload bars, lse at 3e-2 for bf16)
    and, when `ref_pooled_bf16` = (o, lse) of the oracle reading on bf16-rounded pooled levels
    is given, o at the same bars and lse at 2e-3 against that reading."""
    max_abs, rel = compare_outputs(o_gpu, o_ref, valid_rows, f32)
    bar_abs, bar_rel = (F32_MAX_ABS, F32_REL_L2) if f32 else (BF16_MAX_ABS, BF16_REL_L2)
    print(f"[{what}] max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= bar_abs, f"{what}: max abs {max_abs} > {bar_abs}"
    assert rel <= bar_rel, f"{what}: rel L2 {rel} > {bar_rel}"
    if lse_gpu is not None:
        _check_lse(lse_gpu, lse_ref, valid_rows, LSE_ABS_F32 if f32 else LSE_ABS_BF16, what)
    if ref_pooled_bf16 is not None:
        o_r, lse_r = ref_pooled_bf16
        max_abs, rel = compare_outputs(o_gpu, o_r, valid_rows, f32)
        print(f"[{what} vs bf16-pooled reading] max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
        assert max_abs <= bar_abs and rel <= bar_rel, f"{what}: o off the bf16-pooled reading"
        if lse_gpu is not None:
            _check_lse(lse_gpu, lse_r, valid_rows, LSE_ABS_BF16_POOLED,
                       what + " vs bf16-pooled reading")
    # rows past seq_valid are zero, lse -inf
    pad = o_gpu[..., valid_rows:, :]
    assert torch.count_nonzero(pad).item() == 0, f"{what}: non-zero output on pad rows"
    if lse_gpu is not None and lse_gpu.shape[-1] > valid_rows:
        assert torch.all(torch.isneginf(lse_gpu[..., valid_rows:])).item()


# Level maps are compared bit for bit, except at decisions whose float64 oracle margin is below
# ORACLE_MARGIN: a running sum that close to a threshold, two sorted masses that close
# (relative) on either side of a level change, a similarity that close to the cosine bound.
# There, the oracle's own rounding could go either way. Expected count: 0 (always printed).
ORACLE_MARGIN = 1e-12


def oracle_margin_entries(M_ref: np.ndarray, sim_ref, p: oracle.Problem, a: oracle.AssignParams,
                          eps: float = ORACLE_MARGIN, qblocks=None):
    """Boolean mask [.., NQB, NKB] of the decisions within `eps` of flipping, judged on the
    oracle's float64 values. `qblocks` restricts the scan to those query blocks."""
    t = np.array([float(np.float32(x)) for x in a.thresholds])
    B, H, nqb, nkb = M_ref.shape
    marg = np.zeros(M_ref.shape, dtype=bool)
    g = H // (sim_ref.shape[1] if sim_ref is not None else H)
    for b in range(B):
        for h in range(H):
            for qb in (range(nqb) if qblocks is None else qblocks):
                Mr = M_ref[b, h, qb]
                last = oracle.kb_diag(p, qb) if p.causal else nkb - 1
                order = sorted(range(last + 1), key=lambda kb: (-Mr[kb], kb))
                c = 0.0
                prev_level, prev_kb, prev_m = None, None, None
                for kb in order:
                    lvl = next((l for l in range(4) if c < t[l]), -1)
                    if np.min(np.abs(c - t)) < eps:
                        marg[b, h, qb, kb] = True
                    if (prev_m is not None and prev_level != lvl
                            and prev_m - Mr[kb] <= eps * prev_m):
                        marg[b, h, qb, kb] = True
                        marg[b, h, qb, prev_kb] = True
                    prev_level, prev_kb, prev_m = lvl, kb, Mr[kb]
                    c += Mr[kb]
                if sim_ref is not None and a.cos_sim_min > 0:
                    s = sim_ref[b, h // g]
                    marg[b, h, qb] |= np.abs(s - float(np.float32(a.cos_sim_min))) < eps
    return marg


def check_map(got: np.ndarray, ref: np.ndarray, marg: np.ndarray, what: str, cert=None):
    """Bit-exact map comparison but for oracle-margin entries; prints the counts."""
    diff = got != ref
    extra = f", certification: {cert[0]} rows rescored in float64, {cert[1]} left" if cert else ""
    print(f"[{what}] map entries differing {int(diff.sum())} of {diff.size}; within the oracle's "
          f"1e-12 margin {int(marg.sum())} (differing there {int((diff & marg).sum())}){extra}",
          flush=True)
    assert not np.any(diff & ~marg), f"{what}: map differs at {int((diff & ~marg).sum())} entries"
    if cert is not None:
        assert cert[1] == 0, f"{what}: {cert[1]} flagged rows left uncertified"


def order_share(wl: W.Workload) -> int:
    """XCD ranges per chunk of psa_build_index's dispatch order: the smallest f of 1, 2, 4, 8
    for which the K and V rows of all levels (N + 7N/8 rows each) of 8 / f KV heads fit in
    128 MB; 1 with a single (batch, KV head)."""
    if wl.batch * wl.heads_kv <= 1:
        return 1
    elem = 4 if wl.dtype == "f32" else 2
    per_head = (wl.seq_len + 7 * wl.seq_len // 8) * wl.head_dim * elem * 2
    f = 1
    while f < 8 and (8 // f) * per_head > (128 << 20):
        f *= 2
    return f


def chunk_slots(rows, nper, f):
    """Slot of each list position with f XCD ranges per chunk: inside a chunk, position j to
    range (first + j mod f), local slot j // f, while every range of the chunk has slots left;
    the chunk's tail then fills the ranges' remaining slots in order."""
    lens = [min(max(rows - x * nper, 0), nper) for x in range(8)]
    out = np.empty(rows, dtype=np.int64)
    for i in range(rows):
        x0 = (i // (f * nper)) * f
        j = i - x0 * nper
        m = min(lens[x0 + k] for k in range(f))
        if j < f * m:
            out[i] = (x0 + j % f) * nper + j // f
            continue
        j -= f * m
        for k in range(f):
            rem = lens[x0 + k] - m
            if j < rem:
                out[i] = (x0 + k) * nper + m + j
                break
            j -= rem
    return out


def dispatch_order(row_ptr, rows, unit, share=1):
    """The attention's dispatch order that psa_build_index writes after the CSR offsets
    (row_ptr[rows*4+1 + p] = the row of dispatch slot p), from its definition: the rows grouped
    by KV head (row // unit, unit = NQB * heads_q / heads_kv), groups ascending, and inside a
    group listed by tile count (sum over levels l of ceil(n_l / 2^l)), largest first, stably,
    over 32 buckets of the group's span of counts. With share f < 8 each XCD range of
    ceil(rows/8) positions is sorted on its own where it cuts a group; with f = 8 whole groups
    are sorted. List positions then go to slots by chunk_slots. A scheduling choice of the
    library, not part of the method: no oracle function."""
    cnt = np.diff(np.asarray(row_ptr[:rows * 4 + 1], dtype=np.int64)).reshape(rows, 4)
    tiles = sum((cnt[:, l] + (1 << l) - 1) >> l for l in range(4))
    nper = (rows + 7) // 8
    out = np.empty(rows, dtype=np.int64)
    ranges = [(0, rows)] if share == 8 else [(x * nper, min((x + 1) * nper, rows)) for x in range(8)]
    for lo, hi in ranges:
        g = lo
        while g < hi:
            g_hi = min((g // unit + 1) * unit, hi)
            t = tiles[g:g_hi]
            bucket = ((t.max() - t) * 32) // (t.max() - t.min() + 1)
            out[g:g_hi] = g + np.argsort(bucket, kind="stable")
            g = g_hi
    if share == 1:
        return out
    laid = np.empty(rows, dtype=np.int64)
    laid[chunk_slots(rows, nper, share)] = out
    return laid


def check_index(row_ptr, col_idx, rp_ref, ci_ref, unit, share=1):
    """psa_build_index's output against the oracle's CSR (bit for bit) and the dispatch order
    against its definition (bit for bit, and a permutation of the rows); unit = the rows per KV
    head (NQB * heads_q / heads_kv)."""
    rp = row_ptr.cpu().numpy() if hasattr(row_ptr, "cpu") else np.asarray(row_ptr)
    rows = (len(rp_ref) - 1) // 4
    assert len(rp) == rows * 5 + 1
    assert np.array_equal(rp[:rows * 4 + 1], rp_ref)
    ci = col_idx.cpu().numpy() if hasattr(col_idx, "cpu") else np.asarray(col_idx)
    assert np.array_equal(ci[:rp_ref[-1]], ci_ref)
    order = rp[rows * 4 + 1:]
    assert np.array_equal(np.sort(order), np.arange(rows))
    assert np.array_equal(order, dispatch_order(rp_ref, rows, unit, share))
