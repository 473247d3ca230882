"""Pins for the CPU oracle: each function returns an error magnitude that is ~0 for a correct
oracle and large when a plausible mistake is planted in it (a dropped term, a wrong sign or
index, a transposed operand). test_oracle.py asserts the errors are small; test_oracle_mutants.py
plants mistakes in the oracle (on the CPU) and asserts that some pin catches each of them.

The independent sides are library routines (torch's scaled_dot_product_attention, softmax and
logsumexp in float64 on the CPU), closed forms, invariants, and hand-derived fixtures under
tests/golden/.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x))


def rand_qkv(n=512, d=16, seed=0, nv=None, runs=1):
    """Random q, k, v [n, d] fp64; with runs > 1, k and v are constant within runs."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n // runs, d)).repeat(runs, axis=0)
    v = rng.standard_normal((n // runs, d)).repeat(runs, axis=0)
    if nv is not None:
        q[nv:] = 0
        k[nv:] = 0
        v[nv:] = 0
    return q, k, v


def sdpa(q, k, v, mask_bool, scale):
    """torch SDPA (fp64, CPU) on [n, d] rows with a [n_q, n_k] boolean keep-mask."""
    o = torch.nn.functional.scaled_dot_product_attention(
        _t(q)[None, None], _t(k)[None, None], _t(v)[None, None],
        attn_mask=_t(mask_bool)[None, None], scale=scale)
    return o[0, 0].numpy()


def torch_lse(q, k, mask_bool, scale, bias=None):
    z = scale * (_t(q) @ _t(k).T)
    if bias is not None:
        z = z + _t(bias)
    z = z.masked_fill(~_t(mask_bool), float("-inf"))
    return torch.logsumexp(z, dim=-1).numpy()


# ---------------------------------------------------------------------------------------
# P1: an all-level-0 map is dense softmax attention (also with padding and causal).
# ---------------------------------------------------------------------------------------
def pin_all_l0_dense(causal=False, nv=512):
    n, d = 512, 16
    p = oracle.Problem(seq_len=n, seq_valid=nv, head_dim=d, block_q=64, block_k=64,
                       causal=causal)
    q, k, v = rand_qkv(n, d, seed=1, nv=nv)
    lm = np.zeros((p.n_qblocks, p.n_kblocks), dtype=np.int8)
    o, lse = oracle.attention_head(q, k, v, lm, p)
    i = np.arange(n)
    keep = (i[None, :] < nv) & np.ones((n, 1), dtype=bool)
    if causal:
        keep = keep & (i[None, :] <= i[:, None])
    s = 1.0 / math.sqrt(d)
    ref = sdpa(q, k, v, keep, s)
    ref_lse = torch_lse(q, k, keep, s)
    rows = slice(0, nv)
    err = max(np.abs(o[rows] - ref[rows]).max(), np.abs(lse[rows] - ref_lse[rows]).max())
    pad_ok = np.all(o[nv:] == 0) and np.all(np.isneginf(lse[nv:]))
    return err if pad_ok else np.inf


# ---------------------------------------------------------------------------------------
# P2: a map with only {L0, skip} is block-sparse attention with a binary block mask.
# ---------------------------------------------------------------------------------------
def pin_binary_block_sparse():
    n, d, bq, bk = 512, 16, 128, 64
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=bq, block_k=bk)
    q, k, v = rand_qkv(n, d, seed=2)
    rng = np.random.default_rng(3)
    lm = np.where(rng.random((p.n_qblocks, p.n_kblocks)) < 0.5, 0, -1).astype(np.int8)
    lm[:, 0] = 0
    keep = np.repeat(np.repeat(lm == 0, bq, axis=0), bk, axis=1)
    o, lse = oracle.attention_head(q, k, v, lm, p)
    s = 1.0 / math.sqrt(d)
    ref = sdpa(q, k, v, keep, s)
    return max(np.abs(o - ref).max(), np.abs(lse - torch_lse(q, k, keep, s)).max())


# ---------------------------------------------------------------------------------------
# P3: nearest-neighbour upsampling of each pooled block back to full length, then standard
# attention, equals the level-weighted formulation (pins the 2**l weight).
# ---------------------------------------------------------------------------------------
def _upsampled_row(k, v, row_levels, bk):
    ks, vs, keep = [], [], []
    for kb, l in enumerate(row_levels):
        blk = slice(kb * bk, (kb + 1) * bk)
        if l < 0:
            ks.append(k[blk])
            vs.append(v[blk])
            keep.append(np.zeros(bk, dtype=bool))
            continue
        f = 1 << int(l)
        kp = k[blk].reshape(bk // f, f, -1).mean(axis=1)
        vp = v[blk].reshape(bk // f, f, -1).mean(axis=1)
        ks.append(np.repeat(kp, f, axis=0))
        vs.append(np.repeat(vp, f, axis=0))
        keep.append(np.ones(bk, dtype=bool))
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(keep)


def pin_upsample_equivalence(seed=4):
    n, d, bq, bk = 512, 16, 64, 64
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=bq, block_k=bk)
    q, k, v = rand_qkv(n, d, seed=seed)
    rng = np.random.default_rng(seed + 1)
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=(p.n_qblocks, p.n_kblocks))
    lm[:, 0] = 3
    o, lse = oracle.attention_head(q, k, v, lm, p)
    err = 0.0
    for qb in range(p.n_qblocks):
        qi = slice(qb * bq, (qb + 1) * bq)
        ku, vu, keep = _upsampled_row(k, v, lm[qb], bk)
        km = np.broadcast_to(keep, (bq, n))
        ref = sdpa(q[qi], ku, vu, km, 1.0 / math.sqrt(d))
        ref_lse = torch_lse(q[qi], ku, km, 1.0 / math.sqrt(d))
        err = max(err, np.abs(o[qi] - ref).max(), np.abs(lse[qi] - ref_lse).max())
    return err


# ---------------------------------------------------------------------------------------
# P4: K, V constant within runs of 2**l: level l gives the same output as level 0.
# ---------------------------------------------------------------------------------------
def pin_constant_runs(level=3):
    n, d = 512, 16
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=64)
    q, k, v = rand_qkv(n, d, seed=5, runs=1 << level)
    rng = np.random.default_rng(6)
    base = np.where(rng.random((p.n_qblocks, p.n_kblocks)) < 0.3, -1, 0).astype(np.int8)
    base[:, 1] = 0
    pooled = base.copy()
    sel = (base == 0) & (rng.random(base.shape) < 0.6)
    pooled[sel] = level
    o0, l0 = oracle.attention_head(q, k, v, base, p)
    o1, l1 = oracle.attention_head(q, k, v, pooled, p)
    return max(np.abs(o0 - o1).max(), np.abs(l0 - l1).max())


# ---------------------------------------------------------------------------------------
# P5: an all-skip row gives o = 0 and lse = -inf; other rows are unaffected.
# ---------------------------------------------------------------------------------------
def pin_all_skip_row():
    n, d = 256, 8
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=64)
    q, k, v = rand_qkv(n, d, seed=7)
    lm = np.zeros((4, 4), dtype=np.int8)
    lm[2] = -1
    o, lse = oracle.attention_head(q, k, v, lm, p)
    ok = np.all(o[128:192] == 0) and np.all(np.isneginf(lse[128:192]))
    full, fl = oracle.attention_head(q, k, v, np.zeros((4, 4), dtype=np.int8), p)
    other = np.r_[0:128, 192:256]
    return np.abs(o[other] - full[other]).max() if ok else np.inf


# ---------------------------------------------------------------------------------------
# P6: per-row weights sum to 1 including the 2**l multiplicity: the weight of a pooled
# token equals the summed weights of its 2**l upsampled copies under standard softmax.
# ---------------------------------------------------------------------------------------
def pin_weight_multiplicity():
    n, d, bk = 256, 8, 64
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=bk)
    q, k, v = rand_qkv(n, d, seed=8)
    row_levels = np.array([0, 1, 2, 3], dtype=np.int8)
    lk, lv = oracle.pyramid(k), oracle.pyramid(v)
    Kb, Vb, lvl, last = oracle.psa_oracle.gather_row_keys(lk, lv, row_levels, p)
    qi = np.arange(64)
    w = oracle.psa_oracle.attention_weights_row(q[qi], qi, Kb, lvl, last, p, p.scale)
    ku, _, _ = _upsampled_row(k, v, row_levels, bk)
    wu = torch.softmax((_t(q[qi]) @ _t(ku).T) / math.sqrt(d), dim=-1).numpy()
    # fold the upsampled weights back onto pooled tokens
    folded = []
    for kb, l in enumerate(row_levels):
        f = 1 << int(l)
        blk = wu[:, kb * bk:(kb + 1) * bk]
        folded.append(blk.reshape(64, bk // f, f).sum(axis=-1))
    folded = np.concatenate(folded, axis=1)
    return max(np.abs(w - folded).max(), np.abs(w.sum(axis=1) - 1).max())


# ---------------------------------------------------------------------------------------
# P7: pyramid. 2**l * sum(level l) == sum(level 0) per block; mean of a constant is that
# constant; progressive pooling equals direct pooling; brute-force mean on a tiny input;
# packed layout offsets.
# ---------------------------------------------------------------------------------------
def pin_pyramid():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((256, 8))
    err = 0.0
    for l in (1, 2, 3):
        pl = oracle.pool(x, l)
        f = 1 << l
        err = max(err, np.abs(f * pl.reshape(4, 64 // f, 8).sum(1)
                              - x.reshape(4, 64, 8).sum(1)).max())
    err = max(err, np.abs(oracle.pool(oracle.pool(x, 1), 1) - oracle.pool(x, 2)).max())
    err = max(err, np.abs(oracle.pool(oracle.pool(oracle.pool(x, 1), 1), 1)
                          - oracle.pool(x, 3)).max())
    c = np.full((64, 3), 1.25)
    for l in (1, 2, 3):
        err = max(err, np.abs(oracle.pool(c, l) - 1.25).max())
    tiny = rng.standard_normal((16, 2))
    p3 = oracle.pool(tiny, 3)
    for j in range(2):
        for e in range(2):
            s = 0.0
            for t in range(8):
                s += tiny[8 * j + t, e]
            err = max(err, abs(p3[j, e] - s / 8))
    packed = oracle.pack_pyramid(x)
    n = x.shape[0]
    for l in (1, 2, 3):
        off = oracle.packed_level_offset(n, l)
        err = max(err, np.abs(packed[off:off + (n >> l)] - oracle.pool(x, l)).max())
    if packed.shape[0] != 7 * n // 8:
        return np.inf
    return err


# ---------------------------------------------------------------------------------------
# P8: scoring reductions. Sampling every row (S = BQ) gives the dense softmax block mass
# averaged over the rows; antidiagonal scoring with stride 1 gives the same; stride-S
# antidiagonal orientation and the sum (not mean) of the S products; similarity special
# cases and a pure-Python pairwise brute force.
# ---------------------------------------------------------------------------------------
def _dense_block_mass(q, k, p, rows_per_block=None):
    z = (_t(q) @ _t(k).T) / math.sqrt(q.shape[1])
    n = q.shape[0]
    i = torch.arange(n)
    keep = (i[None, :] < p.seq_valid).expand(n, n)
    if p.causal:
        keep = keep & (i[None, :] <= i[:, None])
    pr = torch.softmax(z.masked_fill(~keep, float("-inf")), dim=-1).numpy()
    mass = pr.reshape(n, p.n_kblocks, p.block_k).sum(-1)
    return mass.reshape(p.n_qblocks, p.block_q, p.n_kblocks).mean(axis=1)


def pin_sampling_all_rows(causal=False):
    n, d = 512, 16
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=64,
                       causal=causal)
    q, k, _ = rand_qkv(n, d, seed=10)
    M = oracle.mask_scores_sampling(q, k, p, samples=64)
    ref = _dense_block_mass(q, k, p)
    return max(np.abs(M - ref).max(), np.abs(M.sum(1) - 1).max())


def pin_antidiag_stride1(causal=False):
    n, d = 512, 16
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=64,
                       causal=causal)
    q, k, _ = rand_qkv(n, d, seed=11)
    M = oracle.mask_scores_antidiag(q, k, p, stride=1)
    return np.abs(M - _dense_block_mass(q, k, p)).max()


def _block_constant_qk(n, d, bq, bk, seed):
    rng = np.random.default_rng(seed)
    q = np.repeat(rng.standard_normal((n // bq, d)), bq, axis=0)
    k = np.repeat(2.0 * rng.standard_normal((n // bk, d)), bk, axis=0)
    return q, k


def pin_meankey_constant_blocks():
    """Query rows constant per query block and keys constant per KV block: the block-mean
    scores are the exact attention block masses (torch softmax over all valid keys, averaged
    over the query block's rows), padded keys included in the count."""
    n, d = 512, 16
    p = oracle.Problem(seq_len=n, seq_valid=n - 24, head_dim=d, block_q=128, block_k=64)
    q, k = _block_constant_qk(n, d, 128, 64, seed=21)
    M = oracle.mask_scores_meankey(q, k, p)
    ref = _dense_block_mass(q, k, p)
    return max(np.abs(M - ref).max(), np.abs(M.sum(1) - 1).max())


def pin_meankey_causal_blocks():
    """Causal: the candidates are the KV blocks up to the last one overlapping the query
    block; with block-constant inputs the masses equal dense attention under a block-level
    causal mask (torch)."""
    n, d, bq, bk = 512, 16, 128, 64
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=bq, block_k=bk, causal=True)
    q, k = _block_constant_qk(n, d, bq, bk, seed=22)
    M = oracle.mask_scores_meankey(q, k, p)
    z = (_t(q) @ _t(k).T) / math.sqrt(d)
    i = torch.arange(n)
    keep = (i[None, :] // bk) <= (((i[:, None] // bq) + 1) * bq - 1) // bk
    pr = torch.softmax(z.masked_fill(~keep, float("-inf")), dim=-1).numpy()
    ref = pr.reshape(n, n // bk, bk).sum(-1).reshape(n // bq, bq, n // bk).mean(axis=1)
    return np.abs(M - ref).max()


def pin_antidiag_orientation_and_sum():
    """Stride 4. (a) Only q[4r+3] and k[4c] non-zero: the antidiagonal pairs exactly these
    (t = 0 term), the main diagonal would pair nothing. (b) q and k constant inside each
    4-row group: the compressed logit is 4x the token logit (a sum, not a mean)."""
    n, d, S = 256, 8, 4
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=64)
    rng = np.random.default_rng(12)
    R = n // S
    qa, ka = np.zeros((n, d)), np.zeros((n, d))
    qa[S - 1::S] = rng.standard_normal((R, d))
    ka[0::S] = rng.standard_normal((R, d))
    Ma = oracle.mask_scores_antidiag(qa, ka, p, stride=S)
    za = (_t(qa[S - 1::S]) @ _t(ka[0::S]).T) / math.sqrt(d)
    pa = torch.softmax(za, -1).numpy()
    ref_a = pa.reshape(R, p.n_kblocks, 64 // S).sum(-1).reshape(p.n_qblocks, 64 // S, -1).mean(1)
    qg = rng.standard_normal((R, d)).repeat(S, axis=0)
    kg = rng.standard_normal((R, d)).repeat(S, axis=0)
    Mb = oracle.mask_scores_antidiag(qg, kg, p, stride=S)
    zb = S * (_t(qg[::S]) @ _t(kg[::S]).T) / math.sqrt(d)
    pb = torch.softmax(zb, -1).numpy()
    ref_b = pb.reshape(R, p.n_kblocks, 64 // S).sum(-1).reshape(p.n_qblocks, 64 // S, -1).mean(1)
    return max(np.abs(Ma - ref_a).max(), np.abs(Mb - ref_b).max())


def pin_cossim():
    d = 80
    p = oracle.Problem(seq_len=64, seq_valid=64, head_dim=d, block_q=64, block_k=64)
    rng = np.random.default_rng(13)
    err = 0.0
    same = np.tile(rng.standard_normal((1, d)), (64, 1)) * rng.uniform(0.5, 2, (64, 1))
    err = max(err, abs(oracle.block_cossim(same, p)[0] - 1.0))
    eye = np.eye(d)[:64] * 3.0
    err = max(err, abs(oracle.block_cossim(eye, p)[0] - 0.0))
    x = rng.standard_normal((1, d))
    anti = np.concatenate([np.tile(x, (32, 1)), np.tile(-x, (32, 1))])
    err = max(err, abs(oracle.block_cossim(anti, p)[0] - (-1.0 / 63.0)))
    # pure-Python brute force over ordered pairs on a small block (BK = 8), one zero key
    p8 = oracle.Problem(seq_len=16, seq_valid=16, head_dim=3, block_q=8, block_k=8)
    y = rng.standard_normal((16, 3))
    y[5] = 0.0
    got = oracle.block_cossim(y, p8)
    for kb in range(2):
        tot = 0.0
        for i in range(8):
            for j in range(8):
                if i == j:
                    continue
                a, b = y[kb * 8 + i], y[kb * 8 + j]
                na = math.sqrt(sum(t * t for t in a))
                nb = math.sqrt(sum(t * t for t in b))
                if na > 0 and nb > 0:
                    tot += sum(s * t for s, t in zip(a, b)) / (na * nb)
        err = max(err, abs(got[kb] - tot / 56.0))
    return err


def pin_sample_offsets():
    ok = (oracle.sample_offsets(128, 8) == [0, 16, 32, 48, 64, 80, 96, 112]
          and oracle.sample_offsets(112, 8) == [0, 14, 28, 42, 56, 70, 84, 98]
          and oracle.sample_offsets(0, 8) == [])
    return 0.0 if ok else np.inf


# ---------------------------------------------------------------------------------------
# P9: threshold assignment against hand-derived golden rows.
# ---------------------------------------------------------------------------------------
def golden_assign_cases():
    with open(os.path.join(GOLDEN, "assign_cases.json")) as f:
        return json.load(f)["cases"]


def pin_assign_case(case):
    n = case["seq_len"]
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=8, block_q=case["block_q"],
                       block_k=64, causal=case["causal"])
    a = oracle.AssignParams(tuple(case["thresholds"]), case.get("cos_sim_min", 0.0),
                            case.get("force_diag_l0", False), case.get("force_begin", 0),
                            case.get("force_end", 0))
    sim = None
    if "sim" in case:
        sim = np.asarray(case["sim"], dtype=np.float32).astype(np.float64)
    M = np.asarray(case["M"], dtype=np.float32).astype(np.float64)
    row = oracle.assign_row(M, sim, p, a, case["qb"])
    return int(np.sum(row != np.asarray(case["expected"])))


def pin_build_index(seed=14):
    rng = np.random.default_rng(seed)
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=(2, 3, 5, 37))
    rp, ci = oracle.build_index(lm)
    rows = lm.reshape(-1, 37)
    bad = 0
    for r in range(rows.shape[0]):
        for l in range(4):
            ref = np.flatnonzero(rows[r] == l)
            got = ci[rp[r * 4 + l]:rp[r * 4 + l + 1]]
            bad += int(not np.array_equal(ref, got))
    return bad


# ---------------------------------------------------------------------------------------
# Backward pins. The gradient the oracle writes out by the chain rule is checked against
# (a) central finite differences of the oracle's own forward (the forward is pinned above;
# the difference quotient shares none of the backward's formulas), with mixed levels,
# padding, causal masking and a shared KV head; (b) torch autograd of dense masked attention
# (float64, CPU) on an all-level-0 map; (c) K, V constant within runs of 2**l: level l and
# level 0 give the same dq and the same gradient summed over each run.
# ---------------------------------------------------------------------------------------
def _bwd_problem(causal, nv, n=128, d=8):
    return oracle.Problem(seq_len=n, seq_valid=nv, head_dim=d, block_q=64, block_k=64,
                          causal=causal)


def pin_bwd_finite_difference(causal=False, nv=120, H=2, Hkv=1, seed=30, samples=12):
    n, d = 128, 8
    p = _bwd_problem(causal, nv, n, d)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, H, n, d))
    k = rng.standard_normal((1, Hkv, n, d))
    v = rng.standard_normal((1, Hkv, n, d))
    do = rng.standard_normal((1, H, n, d))
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=(1, H, p.n_qblocks, p.n_kblocks))
    lm[..., 0, 0] = 1
    lm[..., 1, 1] = 3
    lm[..., 1, 0] = 2

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, lm, p)
        return float(np.sum(np.where(np.isfinite(o), o, 0.0) * do))

    dq, dk, dv = oracle.attention_backward(q, k, v, lm, do, p)
    eps = 1e-5
    err = 0.0
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = rng.choice(x.size, size=samples, replace=False)
        for f in flat:
            idx = np.unravel_index(f, x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            err = max(err, abs(fd - g[idx]) / max(1.0, abs(fd)))
    return err


def pin_bwd_all_l0_autograd(causal=False, nv=256):
    n, d = 256, 16
    p = oracle.Problem(seq_len=n, seq_valid=nv, head_dim=d, block_q=64, block_k=64,
                       causal=causal)
    q, k, v = rand_qkv(n, d, seed=31, nv=nv)
    do = np.random.default_rng(32).standard_normal((n, d))
    do[nv:] = 0.0
    lm = np.zeros((p.n_qblocks, p.n_kblocks), dtype=np.int8)
    dq, dk, dv = oracle.attention_backward_head(q, k, v, lm, do, p)
    i = np.arange(n)
    keep = (i[None, :] < nv) & np.ones((n, 1), dtype=bool)
    if causal:
        keep = keep & (i[None, :] <= i[:, None])
    tq, tk, tv = (_t(x).clone().requires_grad_(True) for x in (q, k, v))
    z = (tq @ tk.T) / math.sqrt(d)
    z = z.masked_fill(~_t(keep), float("-inf"))
    o = torch.softmax(z, dim=-1) @ tv
    (o * _t(do)).sum().backward()
    return max(np.abs(dq - tq.grad.numpy()).max(), np.abs(dk - tk.grad.numpy()).max(),
               np.abs(dv - tv.grad.numpy()).max())


def pin_bwd_constant_runs(level=2):
    n, d = 256, 8
    f = 1 << level
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=64)
    q, k, v = rand_qkv(n, d, seed=33, runs=f)
    do = np.random.default_rng(34).standard_normal((n, d))
    rng = np.random.default_rng(35)
    base = np.where(rng.random((p.n_qblocks, p.n_kblocks)) < 0.3, -1, 0).astype(np.int8)
    base[:, 0] = 0
    pooled = base.copy()
    pooled[(base == 0) & (rng.random(base.shape) < 0.6)] = level
    g0 = oracle.attention_backward_head(q, k, v, base, do, p)
    g1 = oracle.attention_backward_head(q, k, v, pooled, do, p)
    runsum = lambda x: x.reshape(n // f, f, d).sum(axis=1)
    return max(np.abs(g0[0] - g1[0]).max(), np.abs(runsum(g0[1]) - runsum(g1[1])).max(),
               np.abs(runsum(g0[2]) - runsum(g1[2])).max())


# ---------------------------------------------------------------------------------------
# FP8 pins: the e4m3 rounding against torch's float8_e4m3fn conversion (a library routine;
# every code, plus random values across the range, ties included); the per-head scale maps
# the largest magnitude to 448 and keeps every quantized value in range, within half an e4m3
# step; attention with fp8 QK^T equals plain attention on the dequantized operands.
# ---------------------------------------------------------------------------------------
def pin_e4m3_round():
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8).view(torch.float8_e4m3fn)
    vals = codes.to(torch.float64).numpy()
    vals = vals[np.isfinite(vals)]
    err = float(np.abs(oracle.e4m3_round(vals) - vals).max())
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1e-2, 20000),
                        rng.normal(0, 1.0, 20000),
                        (vals[:-1] + np.diff(vals) / 2)[np.abs(vals[:-1]) < 440]])   # midpoints
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return max(err, float(np.abs(oracle.e4m3_round(x) - ref).max()))


def pin_fp8_scale():
    rng = np.random.default_rng(41)
    x = rng.normal(0, 3.0, (256, 64))
    s = oracle.fp8_scale(x)
    q = oracle.fp8_quantize(x, s)
    amax = np.abs(x).max()
    step = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(np.abs(x / s), 1e-300))), -6) - 3)
    bad = (np.abs(q).max() > 448) or abs(np.abs(q).max() - 448) > 1e-9 or \
        np.any(np.abs(q - x / s) > step / 2 + 1e-12) or oracle.fp8_scale(np.zeros(4)) != 1.0
    return float(bad) + abs(s * 448 - amax) / amax * 1e-3


def pin_fp8qk_reduces_to_attention(causal=False):
    n, d = 256, 16
    p = oracle.Problem(seq_len=n, seq_valid=n - 8, head_dim=d, block_q=64, causal=causal)
    rng = np.random.default_rng(42)
    q8 = oracle.e4m3_round(rng.normal(0, 8, (n, d)))
    k8 = oracle.e4m3_round(rng.normal(0, 8, (n, d)))
    v = rng.normal(0, 1, (n, d))
    s_q, s_k = 0.125, 0.0625
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=(p.n_qblocks, p.n_kblocks))
    lm[:, 0] = 0
    kp = {l: oracle.pool(k8, l) for l in (1, 2, 3)}
    o8, l8 = oracle.attention_fp8qk_head(q8, k8, kp, v, s_q, s_k, lm, p)
    o, lse = oracle.attention_head(q8 * s_q, k8 * s_k, v, lm, p)
    both = np.isfinite(lse) & np.isfinite(l8)
    same_inf = np.array_equal(np.isfinite(lse), np.isfinite(l8))
    return max(np.nanmax(np.abs(o8 - o)), np.abs(l8[both] - lse[both]).max(initial=0.0),
               0.0 if same_inf else np.inf)


def pin_fp8pv_worked_rows():
    """Hand-worked rows of attention_fp8_head. Causal, 8 valid tokens, unit query vectors,
    scale ln 2 and unit q/k scales, so the log2-unit logits are t = k8[:, 0]: key 0 at 0.5,
    key 1 at 13/64. Query 0 sees key 0 only: M = 1, 2^(0.5 - 1 + 7) = 90.51 lies between 88 and
    96 (e4m3 spacing 8 on [64, 128)) and rounds to 88; one weight, so o = s_v v8[0] and
    lse = (1 - 7 + log2 88) ln 2 = (1 + log2(11/16)) ln 2. Query 1 sees keys 0 and 1:
    (2^6.5, 2^(13/64 + 6) = 73.67) -> (88, 72); o = s_v (88 v8[0] + 72 v8[1]) / 160 and
    lse = (1 + log2(20/16)) ln 2. With v8[0] = e_0, v8[1] = -3 e_1, s_v = 3/4: query 1's o
    starts (0.4125, -1.0125). A second row puts key 1 at -6.5: 2^(-6.5 - 1 + 7) = 0.7071 rounds
    to 11/16 (spacing 1/16 on [1/2, 1)), so o = s_v (88 v8[0] + 11/16 v8[1]) / (88 + 11/16);
    relative to 2^M instead of 2^(M - 7) that weight, 2^-7.5, would fall in e4m3's subnormal
    range and round to 3 * 2^-9."""
    n, d = 64, 16
    p = oracle.Problem(seq_len=n, seq_valid=8, head_dim=d, block_q=64, causal=True)
    q8 = np.zeros((n, d))
    q8[:, 0] = 1.0
    k8 = np.zeros((n, d))
    k8[0, 0], k8[1, 0] = 0.5, 13.0 / 64.0
    k8[2:8, 0] = -2.0
    v8 = np.zeros((n, d))
    v8[0, 0], v8[1, 1] = 1.0, -3.0
    v8[2:8, 2] = 1.0
    lm = np.zeros((1, 1), dtype=np.int8)
    kp = {l: oracle.pool(k8, l) for l in (1, 2, 3)}
    vp = {l: oracle.pool(v8, l) for l in (1, 2, 3)}
    o, lse = oracle.attention_fp8_head(q8, k8, kp, v8, vp, 1.0, 1.0, 0.75, lm, p, scale=math.log(2.0))
    want0 = np.zeros(d)
    want0[0] = 0.75
    want1 = np.zeros(d)
    want1[0], want1[1] = 0.4125, -1.0125
    errs = [np.abs(o[0] - want0).max(), np.abs(o[1] - want1).max(),
            abs(lse[0] - (1 + math.log2(11 / 16)) * math.log(2)),
            abs(lse[1] - (1 + math.log2(20 / 16)) * math.log(2)),
            np.abs(o[8:]).max(), 0.0 if np.all(np.isneginf(lse[8:])) else 1.0]
    k8[1, 0] = -6.5
    o, lse = oracle.attention_fp8_head(q8, k8, kp, v8, vp, 1.0, 1.0, 0.75, lm, p, scale=math.log(2.0))
    want1 = np.zeros(d)
    want1[0], want1[1] = 0.75 * 88 / 88.6875, 0.75 * (-3) * 0.6875 / 88.6875
    errs += [np.abs(o[1] - want1).max(), abs(lse[1] - (1 - 7 + math.log2(88.6875)) * math.log(2))]
    return float(max(errs))


def pin_fp8pv_powers_of_two(causal=False):
    """Zero queries make every logit l ln 2: the p_j are powers of two, e4m3 holds them exactly,
    and attention_fp8_head must equal attention_head (pinned above) on the dequantized values
    v8 * s_v, with mixed levels, padding and (optionally) causal masking."""
    n, d = 256, 16
    p = oracle.Problem(seq_len=n, seq_valid=n - 16, head_dim=d, block_q=64, causal=causal)
    rng = np.random.default_rng(43)
    k8 = oracle.e4m3_round(rng.normal(0, 4, (n, d)))
    v8 = oracle.e4m3_round(rng.normal(0, 4, (n, d)))
    s_v = 0.3
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=(p.n_qblocks, p.n_kblocks))
    lm[:, 0] = 0
    q8 = np.zeros((n, d))
    kp = {l: oracle.pool(k8, l) for l in (1, 2, 3)}
    vp = {l: oracle.pool(v8, l) for l in (1, 2, 3)}
    o8, l8 = oracle.attention_fp8_head(q8, k8, kp, v8, vp, 0.5, 2.0, s_v, lm, p)
    o, lse = oracle.attention_head(q8, k8, v8 * s_v, lm, p)
    both = np.isfinite(lse) & np.isfinite(l8)
    same_inf = np.array_equal(np.isfinite(lse), np.isfinite(l8))
    return max(np.nanmax(np.abs(o8 - o)), np.abs(l8[both] - lse[both]).max(initial=0.0),
               0.0 if same_inf else np.inf)


# ---------------------------------------------------------------------------------------
# Sampling scores with padding: every valid row of every query block sampled exactly twice
# (S = BQ on blocks of BQ valid rows; the last block holds BQ / 2 valid rows, so the offsets
# floor(s * r / S) name each of them twice). The scores then equal the dense softmax block
# mass over the valid keys only, averaged over each block's valid rows (torch, fp64). The pad
# keys hold random non-zero values, so a pad key that stays visible takes mass.
# ---------------------------------------------------------------------------------------
def pin_sampling_padded(causal=False):
    n, d, bq = 512, 16, 64
    nv = n - bq // 2
    p = oracle.Problem(seq_len=n, seq_valid=nv, head_dim=d, block_q=bq, block_k=64,
                       causal=causal)
    q, k, _ = rand_qkv(n, d, seed=15)
    M = oracle.mask_scores_sampling(q, k, p, samples=bq)
    z = (_t(q) @ _t(k).T) / math.sqrt(d)
    i = torch.arange(n)
    keep = (i[None, :] < nv).expand(n, n)
    if causal:
        keep = keep & (i[None, :] <= i[:, None])
    pr = torch.softmax(z.masked_fill(~keep, float("-inf")), dim=-1).numpy()
    mass = pr.reshape(n, p.n_kblocks, 64).sum(-1)
    ref = np.stack([mass[qb * bq: min((qb + 1) * bq, nv)].mean(axis=0)
                    for qb in range(p.n_qblocks)])
    return max(np.abs(M - ref).max(), np.abs(M.sum(1) - 1).max())


# ---------------------------------------------------------------------------------------
# GQA grouping (4 query heads on 2 KV heads). The whole-tensor wrappers are held to
# library routines that fix the grouping independently of the oracle: torch's
# scaled_dot_product_attention with enable_gqa (query heads 2j and 2j + 1 read KV head j)
# for the all-level-0 forward, torch autograd through it for the backward (a KV head's
# gradient sums its query heads), and dense block masses from torch for the scores (sampling
# with every row, antidiagonal with stride 1). For a mixed-level map each query head is held
# to attention_head on the KV head the table KV_OF names. The similarity check is pinned by
# keys built so that KV head 0's blocks pass it (identical keys) and KV head 1's fail it
# (orthogonal keys): only query heads 0 and 1 may keep pooled levels.
# ---------------------------------------------------------------------------------------
KV_OF = (0, 0, 1, 1)


def _gqa_inputs(n=256, d=16, seed=40, nv=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 4, n, d))
    k = rng.standard_normal((1, 2, n, d))
    v = rng.standard_normal((1, 2, n, d))
    return q, k, v


def pin_gqa_attention(causal=False):
    n, d = 256, 16
    nv = n - 8
    p = oracle.Problem(seq_len=n, seq_valid=nv, head_dim=d, block_q=64, block_k=64,
                       causal=causal)
    q, k, v = _gqa_inputs(n, d)
    lm0 = np.zeros((1, 4, p.n_qblocks, p.n_kblocks), dtype=np.int8)
    o, lse = oracle.attention(q, k, v, lm0, p)
    i = torch.arange(n)
    keep = (i[None, :] < nv).expand(n, n)
    if causal:
        keep = keep & (i[None, :] <= i[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        _t(q), _t(k), _t(v), attn_mask=keep[None, None], scale=1.0 / math.sqrt(d),
        enable_gqa=True).numpy()
    err = np.abs(o[..., :nv, :] - ref[..., :nv, :]).max()
    rng = np.random.default_rng(41)
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=lm0.shape)
    for qb in range(p.n_qblocks):
        lm[..., qb, (qb * 64) // 64] = 0
    o2, l2 = oracle.attention(q, k, v, lm, p)
    for h in range(4):
        oh, lh = oracle.attention_head(q[0, h], k[0, KV_OF[h]], v[0, KV_OF[h]], lm[0, h], p)
        fin = np.isfinite(lh)
        if not np.array_equal(fin, np.isfinite(l2[0, h])):
            return np.inf
        err = max(err, np.abs(o2[0, h] - oh).max(), np.abs(l2[0, h][fin] - lh[fin]).max())
    return err


def pin_gqa_backward(causal=False):
    n, d = 128, 8
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=64,
                       causal=causal)
    q, k, v = _gqa_inputs(n, d, seed=42)
    do = np.random.default_rng(43).standard_normal(q.shape)
    lm = np.zeros((1, 4, p.n_qblocks, p.n_kblocks), dtype=np.int8)
    dq, dk, dv = oracle.attention_backward(q, k, v, lm, do, p)
    tq, tk, tv = (_t(x).clone().requires_grad_(True) for x in (q, k, v))
    i = torch.arange(n)
    keep = torch.ones(n, n, dtype=torch.bool)
    if causal:
        keep = i[None, :] <= i[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=keep[None, None], scale=1.0 / math.sqrt(d), enable_gqa=True)
    (o * _t(do)).sum().backward()
    return max(np.abs(dq - tq.grad.numpy()).max(), np.abs(dk - tk.grad.numpy()).max(),
               np.abs(dv - tv.grad.numpy()).max())


def pin_gqa_mask():
    n, d = 256, 16
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=64, block_k=64)
    q, k, _ = _gqa_inputs(n, d, seed=44)
    a = oracle.AssignParams((0.5, 0.7, 0.8, 0.9))
    err = 0.0
    z = (_t(q) @ _t(k)[:, [0, 0, 1, 1]].transpose(-1, -2)) / math.sqrt(d)
    pr = torch.softmax(z, dim=-1).numpy()[0]
    ref = pr.reshape(4, n, p.n_kblocks, 64).sum(-1).reshape(4, p.n_qblocks, 64, -1).mean(2)
    _, Ms, _ = oracle.mask(q, k, p, "sampling", a, samples=64)
    _, Ma, _ = oracle.mask(q, k, p, "antidiag", a, stride=1)
    err = max(err, np.abs(Ms[0] - ref).max(), np.abs(Ma[0] - ref).max())
    # similarity: KV head 0 blocks of identical keys (similarity 1), KV head 1 blocks of
    # independent Gaussian keys (similarity near 0); with the cosine bound 0.8 only KV head 0
    # may pool
    ks = np.zeros((1, 2, n, d))
    rng = np.random.default_rng(45)
    for kb in range(p.n_kblocks):
        ks[0, 0, kb * 64:(kb + 1) * 64] = rng.standard_normal(d)
    ks[0, 1] = rng.standard_normal((n, d))
    ac = oracle.AssignParams((0.3, 0.6, 0.8, 1.0), cos_sim_min=0.8)
    lm, _, sim = oracle.mask(q, ks, p, "sampling", ac, samples=8)
    pooled = [bool((lm[0, h] > 0).any()) for h in range(4)]
    ok = sim[0, 0].min() > 0.99 and sim[0, 1].max() < 0.5 and pooled == [True, True, False, False]
    return err if ok else np.inf


# ---------------------------------------------------------------------------------------
# bfloat16 rounding (the pooled levels a bf16 pyramid stores): bf16_round against torch's
# float32 -> bfloat16 conversion (a library routine, round to nearest even) on float32
# values: random magnitudes across the range, every midpoint between neighbouring bf16
# values of a few binades (ties), and subnormals. Then the attention reading on bf16-rounded
# pooled levels against nearest-neighbour upsampling + torch SDPA on levels rounded by torch
# (inputs chosen so that every exact mean is a float32 value, so torch rounds it once).
# ---------------------------------------------------------------------------------------
def pin_bf16_round():
    rng = np.random.default_rng(50)
    x = (rng.standard_normal(50000) * np.exp2(rng.integers(-40, 40, 50000))).astype(np.float32)
    mids = []
    for e in (-3, 0, 5):
        for m in range(128, 256):
            mids.append((2 * m + 1) * 2.0 ** (e - 8))       # halfway between m and m + 1 ulps
    sub = (rng.integers(1, 1 << 16, 2000) * 2.0 ** -149).astype(np.float32)
    xs = np.concatenate([x, np.asarray(mids, np.float32), -np.asarray(mids, np.float32), sub])
    ref = torch.from_numpy(xs).to(torch.bfloat16).double().numpy()
    got = oracle.bf16_round(xs.astype(np.float64))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 2.0 ** -140)))


def pin_bf16_pooled_attention(seed=51):
    n, d, bq, bk = 512, 16, 64, 64
    p = oracle.Problem(seq_len=n, seq_valid=n, head_dim=d, block_q=bq, block_k=bk)
    rng = np.random.default_rng(seed)
    # k, v: 10-bit integers / 64: sums of <= 8 of them and their means are float32 values
    q = rng.standard_normal((n, d))
    k = rng.integers(-512, 512, (n, d)) / 64.0
    v = rng.integers(-512, 512, (n, d)) / 64.0
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=(p.n_qblocks, p.n_kblocks))
    lm[:, 0] = 3
    o, lse = oracle.attention_head(q, k, v, lm, p, pooled_round="bf16")

    def torch_round(x):
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    err = 0.0
    for qb in range(p.n_qblocks):
        qi = slice(qb * bq, (qb + 1) * bq)
        ks, vs, keep = [], [], []
        for kb, l in enumerate(lm[qb]):
            blk = slice(kb * bk, (kb + 1) * bk)
            f = 1 << max(int(l), 0)
            kp = k[blk].reshape(bk // f, f, d).mean(axis=1)
            vp = v[blk].reshape(bk // f, f, d).mean(axis=1)
            if l > 0:
                kp, vp = torch_round(kp), torch_round(vp)
            ks.append(np.repeat(kp, f, axis=0))
            vs.append(np.repeat(vp, f, axis=0))
            keep.append(np.full(bk, l >= 0))
        ku, vu, km = np.concatenate(ks), np.concatenate(vs), np.concatenate(keep)
        km = np.broadcast_to(km, (bq, n))
        ref = sdpa(q[qi], ku, vu, km, 1.0 / math.sqrt(d))
        ref_lse = torch_lse(q[qi], ku, km, 1.0 / math.sqrt(d))
        err = max(err, np.abs(o[qi] - ref).max(), np.abs(lse[qi] - ref_lse).max())
    # the rounding must matter on these inputs (else the pin would not see it dropped)
    o_exact, _ = oracle.attention_head(q, k, v, lm, p)
    return err if np.abs(o_exact - o).max() > 1e-6 else np.inf
