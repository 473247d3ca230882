"""GPU parity of psa_attn_bwd (through the C ABI) against the CPU oracle's backward.

The forward runs on the GPU (its o and lse feed the backward, as in training); the oracle
recomputes everything in float64 from the same bf16 inputs, map and output gradient.

Tolerance. The kernels round P and dS to bf16 before the products that use them (relative
error <= 2^-9 each) and take D_i = dO_i . o_i from the bf16 forward output; everything else is
bf16 inputs (exact in both) with float32 accumulation. Each row of dS sums to exactly zero
(sum_j P_ij (dP_ij - D_i) = D_i - D_i), so dq_i = s sum_j dS_ij K_j is a cancelling sum: its
relative error is about 2^-9 times |(dS_ij K_j)_j| / |dq_i|, a ratio that grows when a row sees
few keys. Applying exactly these roundings to the fp64 oracle gives dq 1.2e-2 from exact at
64 tokens and <= 7e-3 from 1088 tokens on (the bf16 rounding of dS dominates; exact D changes
little). Bars: where rows see about a thousand tokens or more (every workload here, and the
ragged 1080-token case) rel-L2 <= 1e-2 per tensor and max-abs <= 2e-2 of the tensor's largest
magnitude; where they see few (64 tokens; the row-limit case, two blocks per row) rel-L2 <= 2e-2
and max-abs <= 4e-2.
Pad query rows get dq = 0 and pad tokens dk = dv = 0 exactly; two runs are bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import video_transformers_amd as psa
from gpu_util import DEV, announce, need_gpu, oracle_map, oracle_problem, problem_for

pytestmark = pytest.mark.gpu

REL_L2 = 2e-2
MAX_REL = 4e-2
# rows that see about a thousand tokens or more: the derivation's <= 7e-3 with headroom
REL_L2_LONG = 1e-2
MAX_REL_LONG = 2e-2
LONG_TOKENS = 1024


def _bars(nv):
    return (REL_L2_LONG, MAX_REL_LONG) if nv >= LONG_TOKENS else (REL_L2, MAX_REL)

BWD = [W.small(w) for w in W.ALL if w.dtype == "bf16"]
BWD.append(W.small(W.QWEN25VL_32K).replace(name="qwen2.5-vl-7b-small-bq64", block_q=64))


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _run(wl, q, k, v, lm, dout):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    lmd = torch.from_numpy(lm).to(DEV)
    o, lse = psa.attn_fwd(qd, kd, vd, kp, vp, lmd, prob)
    do = dout.to(DEV)
    bprob = psa.make_problem(qd, kd, vd, o, block_q=wl.block_q, block_k=wl.block_k,
                             causal=wl.causal, seq_valid=wl.seq_valid)
    ws = psa.attn_bwd_workspace(bprob, DEV)
    dq, dk, dv = psa.attn_bwd(qd, kd, vd, kp, vp, lmd, o, lse, do, bprob, ws=ws)
    psa.check_status(ws)
    return dq, dk, dv


def _compare(name, got, ref, nv):
    bar_rel, bar_max = _bars(nv)
    g = got.double().cpu().numpy()
    diff = g - ref
    scale = max(np.abs(ref).max(), 1e-30)
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.abs(diff).max() / scale)
    print(f"  {name}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e} max|ref|={scale:.3e} "
          f"(bars {bar_rel:.0e} / {bar_max:.0e})", flush=True)
    assert rel <= bar_rel, f"{name}: rel L2 {rel}"
    assert mx <= bar_max, f"{name}: max abs {mx} of max|ref|"


@pytest.mark.parametrize("wl", BWD, ids=[w.name for w in BWD])
def test_bwd_parity(wl):
    announce(f"backward {wl.name}: H{wl.heads_q}/{wl.heads_kv} N{wl.seq_len} d{wl.head_dim} "
             f"bq{wl.block_q} causal={wl.causal}")
    q, k, v = W.make_qkv(wl)
    lm = oracle_map(wl, q, k)
    dout = W.make_dout(wl)
    dq, dk, dv = _run(wl, q, k, v, lm, dout)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, lm, dout, oracle_problem(wl))
    nv = wl.seq_valid
    _compare("dq", dq, rq, nv)
    _compare("dk", dk, rk, nv)
    _compare("dv", dv, rv, nv)
    assert torch.count_nonzero(dq[..., nv:, :]).item() == 0
    assert torch.count_nonzero(dk[..., nv:, :]).item() == 0
    assert torch.count_nonzero(dv[..., nv:, :]).item() == 0


def test_bwd_deterministic():
    wl = W.small(W.QWEN25VL_32K)
    announce(f"backward determinism {wl.name}")
    q, k, v = W.make_qkv(wl)
    lm = oracle_map(wl, q, k)
    dout = W.make_dout(wl)
    a = _run(wl, q, k, v, lm, dout)
    b = _run(wl, q, k, v, lm, dout)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_all_l0_matches_autograd():
    """An all-level-0 map is dense attention: the gradients match torch autograd of dense
    masked attention (float32 on the GPU) to the same bars."""
    wl = W.small(W.WAN13B_32K)
    announce(f"backward all-L0 vs autograd {wl.name}")
    q, k, v = W.make_qkv(wl)
    lm = np.zeros((wl.batch, wl.heads_q, wl.n_qblocks, wl.n_kblocks), dtype=np.int8)
    dout = W.make_dout(wl)
    dq, dk, dv = _run(wl, q, k, v, lm, dout)
    nv = wl.seq_valid
    tq, tk, tv = (x.to(DEV).float().requires_grad_(True) for x in (q, k, v))
    keep = torch.arange(wl.seq_len, device=DEV)[None, :] < nv
    z = (tq @ tk.transpose(-1, -2).contiguous()) / (wl.head_dim ** 0.5)
    z = z.masked_fill(~keep, float("-inf"))
    o = torch.softmax(z, dim=-1) @ tv
    rows = (torch.arange(wl.seq_len, device=DEV) < nv)[:, None]
    (o * dout.to(DEV).float() * rows).sum().backward()
    _compare("dq", dq, tq.grad.double().cpu().numpy(), nv)
    _compare("dk", dk, tk.grad.double().cpu().numpy(), nv)
    _compare("dv", dv, tv.grad.double().cpu().numpy(), nv)


def test_bwd_token_major_layout():
    """Q, K, V, O, dO and the gradients on [batch, tokens, heads, d] storage."""
    wl = W.small(W.QWEN25VL_32K)
    announce(f"backward token-major {wl.name}")
    q, k, v = W.make_qkv(wl)
    lm = oracle_map(wl, q, k)
    dout = W.make_dout(wl)
    tm = lambda t: t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    qd, kd, vd, dod = tm(q), tm(k), tm(v), tm(dout)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    lmd = torch.from_numpy(lm).to(DEV)
    o = torch.empty_strided(qd.shape, qd.stride(), dtype=qd.dtype, device=DEV)
    oprob = psa.make_problem(qd, kd, vd, o, block_q=wl.block_q, causal=wl.causal,
                             seq_valid=wl.seq_valid)
    o, lse = psa.attn_fwd(qd, kd, vd, kp, vp, lmd, oprob, out=o)
    dq, dk, dv = psa.attn_bwd(qd, kd, vd, kp, vp, lmd, o, lse, dod, oprob)
    assert dq.stride() == qd.stride() and dk.stride() == kd.stride()
    ref = _run(wl, q, k, v, lm, dout)
    for x, y in zip((dq, dk, dv), ref):
        assert torch.equal(x.contiguous(), y)


FULL = [w for w in W.ALL if w.dtype == "bf16"]


@pytest.mark.parametrize("wl", FULL, ids=[w.name for w in FULL])
def test_bwd_fullsize(wl):
    """Full size, as the benchmark runs it. dq of sampled query blocks (first, last, middle,
    a random one) against the oracle, which computes those rows one block at a time. dk and dv
    element by element on sampled KV blocks (a middle one and the last, ragged one) of one KV
    head: only the (query head, query block) rows that list a KV block at some level reach its
    tokens, so the oracle visits just those rows of the group's query heads. Also properties
    that hold at any size: each row's P sums to 1 and a pooled row hands out exactly its
    gradient, so per KV head sum_t dv[t] = sum of dO over the rows that see a key; and
    rowsum(dS) = 0 gives sum_t dk[t] = 0."""
    announce(f"backward full size {wl.name}: H{wl.heads_q}/{wl.heads_kv} N{wl.seq_len} d{wl.head_dim}")
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    if wl.map_source == "mask":
        from gpu_util import mask_params
        lmd, _, _ = psa.mask(qd, kd, prob, mask_params(wl))
    else:
        lmd = torch.from_numpy(W.make_map(wl)).to(DEV)
    o, lse = psa.attn_fwd(qd, kd, vd, kp, vp, lmd, prob)
    dout = W.make_dout(wl)
    do = dout.to(DEV)
    bprob = psa.make_problem(qd, kd, vd, o, block_q=wl.block_q, block_k=wl.block_k,
                             causal=wl.causal, seq_valid=wl.seq_valid)
    ws = psa.attn_bwd_workspace(bprob, DEV)
    dq, dk, dv = psa.attn_bwd(qd, kd, vd, kp, vp, lmd, o, lse, do, bprob, ws=ws)
    psa.check_status(ws)
    torch.cuda.synchronize()
    lm = lmd.cpu().numpy()
    p = oracle_problem(wl)
    g = wl.group
    rng = np.random.default_rng(wl.seed)
    n = wl.n_qblocks
    for h in sorted({0, wl.heads_q - 1}):
        qbs = sorted({0, n - 1, n // 2, int(rng.integers(1, n - 1))})
        hk = h // g
        rq, _, _ = oracle.attention_backward_head(
            oracle.as_f64(q[0, h]), oracle.as_f64(k[0, hk]), oracle.as_f64(v[0, hk]), lm[0, h],
            oracle.as_f64(dout[0, h]), p, qblocks=qbs)
        rows = np.concatenate([np.arange(b * wl.block_q, (b + 1) * wl.block_q) for b in qbs])
        print(f"[{wl.name}] head {h} query blocks {qbs}", flush=True)
        _compare("dq", dq[0, h, rows], rq[rows], wl.seq_valid)
    # dk, dv of sampled KV blocks of the last KV head, from the rows that list them
    hk = wl.heads_kv - 1
    kbs = sorted({wl.n_kblocks // 2 + 1, (wl.seq_valid - 1) // 64})
    rk = np.zeros((wl.seq_len, wl.head_dim))
    rv = np.zeros_like(rk)
    kf, vf = oracle.as_f64(k[0, hk]), oracle.as_f64(v[0, hk])
    nrows = 0
    for h in range(hk * g, (hk + 1) * g):
        qbs = [qb for qb in range(n) if np.any(lm[0, h, qb, kbs] >= 0)]
        nrows += len(qbs)
        if not qbs:
            continue
        _, a_k, a_v = oracle.attention_backward_head(
            oracle.as_f64(q[0, h]), kf, vf, lm[0, h], oracle.as_f64(dout[0, h]), p, qblocks=qbs)
        rk += a_k
        rv += a_v
    toks = np.concatenate([np.arange(kb * 64, (kb + 1) * 64) for kb in kbs])
    print(f"[{wl.name}] kv head {hk} KV blocks {kbs}: {nrows} listing rows", flush=True)
    _compare("dk", dk[0, hk, toks], rk[toks], wl.seq_valid)
    _compare("dv", dv[0, hk, toks], rv[toks], wl.seq_valid)
    # sums over tokens, per KV head
    seen = torch.isfinite(lse) & (torch.arange(wl.seq_len, device=DEV) < wl.seq_valid)
    dsum = (do.float() * seen[..., None]).sum(dim=2)                      # [B, H, d]
    dsum = dsum.view(wl.batch, wl.heads_kv, g, wl.head_dim).sum(dim=2)    # [B, Hkv, d]
    vsum = dv.float().sum(dim=2)
    ksum = dk.float().sum(dim=2)
    scale_v = dsum.abs().max().item()
    err_v = (vsum - dsum).abs().max().item() / scale_v
    err_k = ksum.abs().max().item() / max(dk.float().abs().sum(dim=2).max().item(), 1e-30)
    print(f"[{wl.name}] sum dv vs sum dO: {err_v:.3e} of max|sum dO|; |sum dk| / sum|dk|: "
          f"{err_k:.3e}", flush=True)
    # bf16 gradients summed over a whole head: observed ~2e-4; a lost 2^-l factor or a
    # dropped term is O(1)
    assert err_v <= 2e-3
    assert err_k <= 2e-3
    assert torch.count_nonzero(dq[..., wl.seq_valid:, :]).item() == 0
