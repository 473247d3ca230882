"""GPU parity of psa_attn_fwd_meankey: block-mean scoring and the threshold assignment fused into
the attention's prologue.

* Against the two-step GPU path (psa_mask in block-mean mode, then psa_attn_fwd): the same
  level map, block masses, o and lse bit for bit (same arithmetic, same order, same tiles).
* Against the oracle: the map bit for bit except at decisions within the oracle's own 1e-12
  margin (both paths certify near-threshold rows in float64), and the attention on the GPU's map
  to the bf16 bars.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import video_transformers_amd as psa
from gpu_util import (DEV, announce, assign_params, check_attention, check_map, mask_params,
                      need_gpu, oracle_margin_entries, oracle_problem, problem_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


MK = [W.small(W.WAN13B_32K).replace(name="wan2.1-1.3b-small-meankey", mask_mode="meankey"),
      W.small(W.QWEN25VL_32K).replace(name="qwen2.5-vl-7b-small-meankey", mask_mode="meankey"),
      W.small(W.COGVIDEOX5B_17K).replace(name="cogvideox-5b-small-meankey", mask_mode="meankey")]


def _both(wl, qd, kd, vd):
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    params = mask_params(wl)
    lm, M, sim = psa.mask(qd, kd, prob, params)
    o, lse = psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob)
    of, lsef, lmf, Mf = psa.attn_fwd_meankey(qd, kd, vd, kp, vp, prob, params, want_mass=True)
    torch.cuda.synchronize()
    return (lm, M, o, lse), (lmf, Mf, of, lsef)


@pytest.mark.parametrize("wl", MK, ids=[w.name for w in MK])
def test_meankey_fused_parity(wl):
    announce(f"fused block-mean scoring {wl.name}")
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    (lm, M, o, lse), (lmf, Mf, of, lsef) = _both(wl, qd, kd, vd)
    assert torch.equal(lmf, lm), "map differs from psa_mask's"
    assert torch.equal(Mf, M), "block masses differ from psa_mask's"
    assert torch.equal(of, o) and torch.equal(lsef, lse), "attention differs from psa_attn_fwd's"
    # oracle: the map rows, then the attention on the GPU's map
    p = oracle_problem(wl)
    a = assign_params(wl)
    lm_ref, M_ref, sim_ref = oracle.mask(q, k, p, "meankey", a)
    assert np.abs(Mf.double().cpu().numpy() - M_ref).max() <= 2e-6
    check_map(lmf.cpu().numpy(), lm_ref, oracle_margin_entries(M_ref, sim_ref, p, a), f"{wl.name} fused")
    o_ref, lse_ref = oracle.attention(q, k, v, lmf.cpu().numpy(), p)
    check_attention(of, lsef, o_ref, lse_ref, wl.seq_valid, False, f"{wl.name} fused")


def test_meankey_fused_fullsize_wan():
    """The Wan2.1-1.3B-like 32k layer: the fused call equals the two-step path bit for bit (the
    two-step path is held to the oracle at full size by the full-size parity tests)."""
    wl = W.WAN13B_32K.replace(name="wan2.1-1.3b_32k-meankey", mask_mode="meankey")
    announce(f"fused block-mean scoring, full size {wl.name}")
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    (lm, M, o, lse), (lmf, Mf, of, lsef) = _both(wl, qd, kd, vd)
    dm = (Mf != M)
    print(f"[{wl.name}] masses differing: {int(dm.sum())} of {M.numel()}", flush=True)
    assert torch.equal(lmf, lm) and torch.equal(Mf, M)
    assert torch.equal(of, o) and torch.equal(lsef, lse)


@pytest.mark.parametrize("d", [64, 128])
def test_meankey_fused_max_blocks(d):
    """At the fused call's limit of 1792 KV blocks (114688 tokens, GQA 2:1, 8 pad tokens), where
    the prologue's scratch (query mean, log-masses, masses, levels; a 2048-key sort) fills the
    tile buffers it borrows (at head_dim 64 to the last byte): the same map, masses, o and lse
    as the two-step path; sampled query blocks (first, middle, the ragged last) against the
    oracle's map rows and attention."""
    wl = W.WAN13B_32K.replace(name=f"meankey-1792-blocks-d{d}", heads_q=2, heads_kv=1,
                              head_dim=d, seq_len=114688, seq_valid=114680, mask_mode="meankey")
    assert wl.n_kblocks == 1792
    announce(f"fused block-mean scoring at 1792 KV blocks {wl.name}")
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    (lm, M, o, lse), (lmf, Mf, of, lsef) = _both(wl, qd, kd, vd)
    assert torch.equal(lmf, lm), "map differs from psa_mask's"
    assert torch.equal(Mf, M), "block masses differ from psa_mask's"
    assert torch.equal(of, o) and torch.equal(lsef, lse), "attention differs from psa_attn_fwd's"
    p = oracle_problem(wl)
    a = assign_params(wl)
    qbs = [0, wl.n_qblocks // 2, wl.n_qblocks - 1]
    for h in range(wl.heads_q):
        qh = oracle.as_f64(q[0, h])
        kh = oracle.as_f64(k[0, h // wl.group])
        vh = oracle.as_f64(v[0, h // wl.group])
        Mr = oracle.mask_scores_meankey(qh, kh, p, qblocks=qbs)
        lm_ref = np.stack([oracle.assign_row(Mr[qb], None, p, a, qb) for qb in qbs])
        marg = oracle_margin_entries(Mr[None, None], None, p, a, qblocks=qbs)[0, 0][qbs]
        check_map(lmf[0, h].cpu().numpy()[qbs], lm_ref, marg, f"{wl.name} head {h} qblocks {qbs}")
        assert np.abs(Mf[0, h].double().cpu().numpy()[qbs] - Mr[qbs]).max() <= 2e-6
        o_ref, lse_ref = oracle.attention_head(qh, kh, vh, lmf[0, h].cpu().numpy(), p, qblocks=qbs)
        rows = np.concatenate([np.arange(qb * wl.block_q, (qb + 1) * wl.block_q) for qb in qbs])
        valid = rows < wl.seq_valid
        og = of[0, h, rows].double().cpu().numpy()
        lg = lsef[0, h, rows].double().cpu().numpy()
        check_attention(torch.from_numpy(og[valid][None]), torch.from_numpy(lg[valid][None]),
                        o_ref[rows][valid][None], lse_ref[rows][valid][None], int(valid.sum()),
                        False, f"{wl.name} head {h} qblocks {qbs}")
