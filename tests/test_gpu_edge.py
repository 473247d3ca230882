"""GPU edge cases of the whole path, through the C ABI: empty inputs, all-padding sequences,
all-skip maps, ragged block counts (a single block; an odd number of 64-token blocks), and the
backward at its maximum row count per KV head.

Expected values: the oracle's (forward, backward, fp8 readings), or what the definitions fix
exactly (an empty softmax gives o = 0 and lse = -inf; pad query rows and rows with no visible
key have zero output and zero gradient; a query block with no valid query is all skip).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import video_transformers_amd as psa
from gpu_util import (DEV, announce, check_attention, mask_params, need_gpu, oracle_problem,
                      problem_for)
from test_gpu_bwd import _compare, _run
from test_gpu_fp8 import check_fp8pv, oracle_head_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _all_calls(wl, qd, kd, vd, lm):
    """Every forward-side call and the backward on one problem; returns the outputs."""
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    o, lse = psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob)
    bprob = psa.make_problem(qd, kd, vd, o, block_q=wl.block_q, causal=wl.causal,
                             seq_valid=wl.seq_valid)
    dq, dk, dv = psa.attn_bwd(qd, kd, vd, kp, vp, lm, o, lse, torch.ones_like(o), bprob)
    out = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    if wl.head_dim == 128:
        k8, kp8, sk = psa.quantize_fp8(kd, kp)
        v8, vp8, sv = psa.quantize_fp8(vd, vp)
        q8, _, sq = psa.quantize_fp8(qd)
        out["o8qk"], out["lse8qk"] = psa.attn_fwd_fp8qk(q8, sq, k8, kp8, sk, vd, vp, lm, prob)
        out["o8"], out["lse8"] = psa.attn_fwd_fp8(q8, sq, k8, kp8, sk, v8, vp8, sv, lm, prob)
    torch.cuda.synchronize()
    return out


def test_empty_batch():
    """Batch 0 (empty tensors, null data pointers): every call returns without error."""
    announce("empty batch")
    wl = W.small(W.QWEN25VL_32K).replace(batch=0)
    z = lambda h: torch.empty((0, h, wl.seq_len, wl.head_dim), dtype=torch.bfloat16, device=DEV)
    qd, kd, vd = z(wl.heads_q), z(wl.heads_kv), z(wl.heads_kv)
    prob = problem_for(wl, qd, kd, vd)
    lm, _, _ = psa.mask(qd, kd, prob, mask_params(wl))
    assert lm.numel() == 0
    out = _all_calls(wl, qd, kd, vd, lm)
    assert all(t.numel() == 0 for t in out.values())


def test_quantize_no_tokens():
    """seq_len 0: every head is empty, its scale is 1."""
    announce("quantize, no tokens")
    x = torch.empty((2, 3, 0, 128), dtype=torch.bfloat16, device=DEV)
    x8, _, sc = psa.quantize_fp8(x)
    torch.cuda.synchronize()
    assert x8.numel() == 0 and torch.equal(sc.cpu(), torch.ones(6))


@pytest.mark.parametrize("causal", [False, True])
def test_all_padding(causal):
    """seq_valid = 0: the mask assigns skip everywhere; with a drawn map (blocks listed at every
    level) the attention still gives o = 0, lse = -inf and zero gradients, in bf16 and fp8."""
    announce(f"all padding causal={causal}")
    wl = W.small(W.WAN13B_32K).replace(seq_len=1024, seq_valid=0, causal=causal)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    lm, _, _ = psa.mask(qd, kd, prob, mask_params(wl))
    torch.cuda.synchronize()
    assert torch.all(lm == -1).item()
    drawn = torch.from_numpy(W.make_map(wl.replace(map_source="iid", map_probs=(.2, .2, .2, .2, .2)))).to(DEV)
    out = _all_calls(wl, qd, kd, vd, drawn)
    for name in ("o", "dq", "dk", "dv", "o8qk", "o8"):
        assert torch.count_nonzero(out[name]).item() == 0, name
    for name in ("lse", "lse8qk", "lse8"):
        assert torch.all(torch.isneginf(out[name])).item(), name


def test_all_skip_map():
    """Every block skipped: o = 0, lse = -inf, zero gradients, in bf16 and fp8."""
    announce("all-skip map")
    wl = W.small(W.WAN13B_32K).replace(seq_len=1024, seq_valid=1016)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lm = torch.full((1, wl.heads_q, wl.n_qblocks, wl.n_kblocks), -1, dtype=torch.int8, device=DEV)
    out = _all_calls(wl, qd, kd, vd, lm)
    for name in ("o", "dq", "dk", "dv", "o8qk", "o8"):
        assert torch.count_nonzero(out[name]).item() == 0, name
    for name in ("lse", "lse8qk", "lse8"):
        assert torch.all(torch.isneginf(out[name])).item(), name


RAGGED = [(n, d, causal) for n in (64, 1088) for d in (64, 128) for causal in (False, True)]


@pytest.mark.parametrize("n,d,causal", RAGGED, ids=[f"n{n}-d{d}-{'causal' if c else 'full'}" for n, d, c in RAGGED])
def test_ragged_block_counts(n, d, causal):
    """One 64-token block, or 17 of them (block_q 64, GQA 4:2, 8 pad tokens, a drawn map with
    every level): forward, backward and (d = 128) both fp8 forwards against the oracle."""
    announce(f"ragged n={n} d={d} causal={causal}")
    wl = W.Workload(name="ragged", seed=91 + n + d, batch=1, heads_q=4, heads_kv=2, head_dim=d,
                    seq_len=n, seq_valid=n - 8, block_q=64, causal=causal, dtype="bf16",
                    k_dist="clustered", map_source="iid", map_probs=(0.3, 0.2, 0.2, 0.2, 0.1))
    q, k, v = W.make_qkv(wl)
    lm = W.make_map(wl)
    lm[..., 0] = 0
    p = oracle_problem(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = _all_calls(wl, qd, kd, vd, torch.from_numpy(lm).to(DEV))
    o_ref, lse_ref = oracle.attention(q, k, v, lm, p)
    check_attention(out["o"], out["lse"], o_ref, lse_ref, wl.seq_valid, False, f"ragged n{n} d{d}")
    dout = W.make_dout(wl)
    dq, dk, dv = _run(wl, q, k, v, lm, dout)
    rq, rk, rv = oracle.attention_backward(q, k, v, lm, dout, p)
    _compare("dq", dq, rq, wl.seq_valid)
    _compare("dk", dk, rk, wl.seq_valid)
    _compare("dv", dv, rv, wl.seq_valid)
    if d == 128:
        o8 = np.zeros(o_ref.shape)
        l8 = np.zeros(lse_ref.shape)
        for h in range(wl.heads_q):
            hk = h // wl.group
            qh = oracle.as_f64(q[0, h])
            s_q = oracle.fp8_scale(qh)
            s_k, k8, kp8 = oracle_head_fp8(oracle.as_f64(k[0, hk]))
            s_v, v8, vp8 = oracle_head_fp8(oracle.as_f64(v[0, hk]))
            o8[0, h], l8[0, h] = oracle.attention_fp8_head(oracle.fp8_quantize(qh, s_q), k8, kp8, v8,
                                                           vp8, s_q, s_k, s_v, lm[0, h], p)
        check_fp8pv(out["o8"], out["lse8"], o8, l8, wl.seq_valid, f"ragged n{n} fp8")


@pytest.mark.parametrize("d,heads,n,bq", [(64, 120, 4096, 64), (128, 60, 16384, 128)])
def test_bwd_row_limit(d, heads, n, bq):
    """The backward at its row limit: `heads` query heads on one KV head times their query
    blocks = 7680 (query head, query block) rows, every one listing KV block 0 at level 0 and
    block 1 at level 2, so two key-side tiles each collect all 7680 rows (at d = 128 the row list
    nearly fills what the key-side kernel's buffers leave of the LDS). dq, dk and dv against the
    oracle, every element."""
    announce(f"backward at 7680 rows per KV head, d={d}")
    wl = W.Workload(name="rowlimit", seed=313 + d, batch=1, heads_q=heads, heads_kv=1, head_dim=d,
                    seq_len=n, seq_valid=n - 8, block_q=bq, causal=False, dtype="bf16",
                    k_dist="clustered", map_source="iid", map_probs=(1.0, 0.0, 0.0, 0.0, 0.0))
    assert wl.heads_q // wl.heads_kv * wl.n_qblocks == 7680
    q, k, v = W.make_qkv(wl)
    lm = np.full((1, wl.heads_q, wl.n_qblocks, wl.n_kblocks), -1, dtype=np.int8)
    lm[..., 0] = 0
    lm[..., 1] = 2
    dout = W.make_dout(wl)
    dq, dk, dv = _run(wl, q, k, v, lm, dout)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, lm, dout, oracle_problem(wl))
    # every row sees two blocks (80 pooled keys): the few-keys bars
    _compare("dq", dq, rq, 0)
    _compare("dk", dk, rk, 0)
    _compare("dv", dv, rv, 0)
