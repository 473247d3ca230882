"""Property tier: random small problems (shapes, padding, GQA ratio, causality, head dim, query
block size, level maps with every level and all-skip rows, mask modes and parameters) drawn by
hypothesis from a fixed seed, the HIP path against the CPU oracle on each.

Each example is checked to the same bars as the fixed parity tests: level maps bit for bit
but at decisions within the oracle's own 1e-12 margin, block indices bit for bit, attention
(bf16) at max-abs 2e-2 / rel-L2 5e-3 with lse 1e-3 against the bf16-pooled-level reading.
The examples are derandomized (the same every run) and bounded in size so the whole tier runs
in tens of seconds.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import workloads as W
import video_transformers_amd as psa
from gpu_util import (DEV, announce, check_attention, check_index, check_map, need_gpu, oracle_margin_entries,
                      problem_for)

pytestmark = pytest.mark.gpu

SETTINGS = dict(max_examples=12, deadline=None, derandomize=True, database=None,
                suppress_health_check=list(HealthCheck))


@st.composite
def problems(draw):
    d = draw(st.sampled_from([64, 128]))
    bq = draw(st.sampled_from([64, 128]))
    hkv = draw(st.sampled_from([1, 2]))
    g = draw(st.sampled_from([1, 2, 3]))
    nqb = draw(st.integers(1, 6))
    n = nqb * bq
    pad = 8 * draw(st.integers(0, min(n // 8 - 1, 20)))
    causal = draw(st.booleans())
    dist = draw(st.sampled_from(["normal", "clustered", "clustered_var"]))
    seed = draw(st.integers(0, 10_000))
    probs = draw(st.sampled_from([(.2, .2, .2, .2, .2), (.5, .1, .1, .1, .2), (0, .3, .3, .3, .1),
                                  (.1, 0, 0, .5, .4)]))
    return W.Workload(name="prop", seed=seed, batch=1, heads_q=hkv * g, heads_kv=hkv, head_dim=d,
                      seq_len=n, seq_valid=n - pad, block_q=bq, causal=causal, dtype="bf16",
                      k_dist=dist, map_source="iid", map_probs=probs)


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


@settings(**SETTINGS)
@given(wl=problems(), skip_row=st.booleans())
def test_prop_attention_and_index(wl, skip_row):
    announce(f"prop attention H{wl.heads_q}/{wl.heads_kv} N{wl.seq_len} nv{wl.seq_valid} "
             f"d{wl.head_dim} bq{wl.block_q} causal={wl.causal} seed={wl.seed}")
    q, k, v = W.make_qkv(wl)
    lm = W.make_map(wl)
    if skip_row:
        lm[0, 0, 0] = -1
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    lmd = torch.from_numpy(lm).to(DEV)
    row_ptr, col_idx, err = psa.build_index(lmd, prob)
    rp_ref, ci_ref = oracle.build_index(lm)
    check_index(row_ptr, col_idx, rp_ref, ci_ref, wl.n_qblocks * wl.group)
    assert err.item() == 0
    kp, vp = psa.build_pyramid(kd, vd, prob)
    o, lse = psa.attn_fwd_indexed(qd, kd, vd, kp, vp, row_ptr, col_idx, prob)
    torch.cuda.synchronize()
    p = oracle.Problem.of(wl)
    o_ref, lse_ref = oracle.attention(q, k, v, lm, p)
    rnd = oracle.attention(q, k, v, lm, p, pooled_round="bf16")
    check_attention(o, lse, o_ref, lse_ref, wl.seq_valid, False, "prop", rnd)


@settings(**SETTINGS)
@given(wl=problems(), mode=st.sampled_from(["sampling", "antidiag", "meankey"]),
       thr=st.sampled_from([(.5, .7, .8, .9), (.3, .5, .9, .95), (.6, .6, .8, 1.0)]),
       samples=st.sampled_from([1, 4, 8]), cos=st.sampled_from([0.0, 0.5, 0.8]),
       diag=st.booleans())
def test_prop_mask(wl, mode, thr, samples, cos, diag):
    announce(f"prop mask {mode} H{wl.heads_q}/{wl.heads_kv} N{wl.seq_len} nv{wl.seq_valid} "
             f"d{wl.head_dim} bq{wl.block_q} causal={wl.causal} thr={thr} S={samples} "
             f"cos={cos} seed={wl.seed}")
    q, k, v = W.make_qkv(wl)
    qd, kd = q.to(DEV), k.to(DEV)
    prob = problem_for(wl, qd, kd, kd)
    params = psa.MaskParams(mode=mode, thresholds=thr, samples_per_qblock=samples,
                            antidiag_stride=8, cos_sim_min=cos, force_diag_l0=diag)
    cert = []
    lm, M, sim = psa.mask(qd, kd, prob, params, cert_counts=cert)
    torch.cuda.synchronize()
    p = oracle.Problem.of(wl)
    a = oracle.AssignParams(thr, cos, diag)
    lm_ref, M_ref, sim_ref = oracle.mask(q, k, p, mode, a, samples=samples, stride=8)
    assert np.abs(M.double().cpu().numpy() - M_ref).max() <= 2e-6
    check_map(lm.cpu().numpy(), lm_ref, oracle_margin_entries(M_ref, sim_ref, p, a), "prop mask", cert)
