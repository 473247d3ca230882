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


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, valid_rows, f32: bool, what: str):
    max_abs, rel = compare_outputs(o_gpu, o_ref, valid_rows, f32)
    bar_abs, bar_rel = (F32_MAX_ABS, F32_REL_L2) if f32 else (BF16_MAX_ABS, BF16_REL_L2)
    print(f"[{what}] max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= bar_abs, f"{what}: max abs {max_abs} > {bar_abs}"
    assert rel <= bar_rel, f"{what}: rel L2 {rel} > {bar_rel}"
    if lse_gpu is not None:
        lg = lse_gpu[..., :valid_rows].double().cpu().numpy()
        lr = lse_ref[..., :valid_rows]
        both_inf = np.isneginf(lg) & np.isneginf(lr)
        assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), f"{what}: empty-row sets differ"
        d = np.abs(lg[~both_inf] - lr[~both_inf])
        bar = LSE_ABS_F32 if f32 else LSE_ABS_BF16
        assert d.max(initial=0.0) <= bar, f"{what}: lse diff {d.max()} > {bar}"
    # rows past seq_valid are zero, lse -inf
    pad = o_gpu[..., valid_rows:, :]
    assert torch.count_nonzero(pad).item() == 0, f"{what}: non-zero output on pad rows"
    if lse_gpu is not None and lse_gpu.shape[-1] > valid_rows:
        assert torch.all(torch.isneginf(lse_gpu[..., valid_rows:])).item()


def fragile_entries(M_ref: np.ndarray, sim_ref, p: oracle.Problem, a: oracle.AssignParams,
                    eps_m: float = 2e-6, eps_c: float = 2e-5, eps_s: float = 1e-6,
                    qblocks=None):
    """Boolean mask [.., NQB, NKB] of level decisions that an error of `eps` in the block
    masses (or similarities) could flip, judged on the oracle's own values: running sums within
    eps_c of a threshold, masses within eps_m of each other straddling a level change,
    similarities within eps_s of the cosine bound. Used to excuse float-rounding differences in
    end-to-end maps. `qblocks` restricts the scan to those query blocks (others stay False)."""
    t = np.array([float(np.float32(x)) for x in a.thresholds])
    B, H, nqb, nkb = M_ref.shape
    frag = np.zeros(M_ref.shape, dtype=bool)
    g = H // (sim_ref.shape[1] if sim_ref is not None else H)
    for b in range(B):
        for h in range(H):
            for qb in (range(nqb) if qblocks is None else qblocks):
                Mr = M_ref[b, h, qb]
                last = oracle.kb_diag(p, qb) if p.causal else nkb - 1
                cand = np.arange(last + 1)
                order = sorted(cand, key=lambda kb: (-Mr[kb], kb))
                c = 0.0
                prev_level, prev_kb, prev_m = None, None, None
                for kb in order:
                    lvl = next((l for l in range(4) if c < t[l]), -1)
                    near_t = np.min(np.abs(c - t)) < eps_c
                    if near_t:
                        frag[b, h, qb, kb] = True
                        if prev_kb is not None:
                            frag[b, h, qb, prev_kb] = True
                    if prev_m is not None and abs(prev_m - Mr[kb]) < eps_m and prev_level != lvl:
                        frag[b, h, qb, kb] = True
                        frag[b, h, qb, prev_kb] = True
                    prev_level, prev_kb, prev_m = lvl, kb, Mr[kb]
                    c += Mr[kb]
                if sim_ref is not None and a.cos_sim_min > 0:
                    s = sim_ref[b, h // g]
                    frag[b, h, qb] |= np.abs(s - float(np.float32(a.cos_sim_min))) < eps_s
    return frag
