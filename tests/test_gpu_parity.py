"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Reduced copies of the five workloads (same block sizes, mask mode, padding, GQA, causality,
text span) are checked element by element; they span several tiles and end in a ragged tail.
Integer outputs (block index, level maps, threshold assignment) are compared bit-exactly;
floating-point outputs against the bars in gpu_util.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import video_transformers_amd as psa
from gpu_util import (DEV, announce, assign_params, check_attention, check_index, check_map,
                      mask_params, need_gpu, oracle_map, oracle_margin_entries, oracle_problem,
                      order_share, problem_for)

pytestmark = pytest.mark.gpu

SMALL = [W.small(w) for w in W.ALL]
IDS = [w.name for w in SMALL]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _inputs(wl):
    q, k, v = W.make_qkv(wl)
    return q, k, v, q.to(DEV), k.to(DEV), v.to(DEV)


# ---------------------------------------------------------------------------------------
# pyramid
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("wl", SMALL, ids=IDS)
def test_pyramid_parity(wl):
    """float32 levels (out_dtype f32, also for bf16 inputs) against the fp64 means at the 1e-5
    bar; the bf16 levels are exactly the bf16 rounding of those float32 values; and wherever a
    bf16 level differs from the rounding of the exact mean, the exact mean lies within the
    float32 tree's error (3 roundings: 2^-22 relative) of a bf16 rounding midpoint."""
    announce(f"pyramid {wl.name}")
    q, k, v, qd, kd, vd = _inputs(wl)
    prob = problem_for(wl, qd, kd, vd)
    kp32, vp32 = psa.build_pyramid(kd, vd, prob, out_dtype=torch.float32)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    torch.cuda.synchronize()
    for name, x, xp32, xp in (("k", k, kp32, kp), ("v", v, vp32, vp)):
        ref = oracle.pack_pyramid(oracle.as_f64(x))
        got = xp32.double().cpu().numpy()
        d = np.abs(got - ref)
        print(f"[{wl.name} {name}] f32 levels: max abs {d.max():.3e} "
              f"(max |ref| {np.abs(ref).max():.3e})", flush=True)
        assert d.max() <= 1e-5 * np.abs(ref).max(), name
        assert np.linalg.norm(got - ref) <= 1e-5 * np.linalg.norm(ref), name
        if wl.dtype == "f32":
            assert torch.equal(xp, xp32), name
            continue
        assert torch.equal(xp, xp32.to(torch.bfloat16)), f"{name}: bf16 levels != RNE(f32 levels)"
        rne = oracle.bf16_round(ref)
        b = xp.double().cpu().numpy()
        off = b != rne
        # a bf16 rounding midpoint next to the exact mean: halfway between rne and its neighbour
        # on the side of b
        mid = (b + rne) / 2.0
        near = np.abs(ref - mid) <= 2.0 ** -22 * np.abs(ref)
        print(f"[{wl.name} {name}] bf16 levels differing from RNE(exact mean): {int(off.sum())} "
              f"of {off.size}", flush=True)
        assert np.all(near[off]), f"{name}: a bf16 level off RNE(mean) away from a midpoint"


# ---------------------------------------------------------------------------------------
# block index
# ---------------------------------------------------------------------------------------
# (2, 24, 64, 128) and (1, 40, 129, 258): 12288 and 20640 (row, level) counts, i.e. three whole
# scan tiles of 4096 and six with a ragged last one
@pytest.mark.parametrize("shape", [(1, 3, 16, 16), (2, 5, 65, 130), (1, 1, 1, 1), (1, 4, 33, 66),
                                   (2, 24, 64, 128), (1, 40, 129, 258)])
def test_build_index_exact(shape):
    announce(f"build_index {shape}")
    rng = np.random.default_rng(sum(shape))
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=shape,
                    p=[0.1, 0.15, 0.2, 0.05, 0.5])
    if shape[2] > 2:
        lm[0, 0, 1] = -1      # an all-skip row
        lm[0, 0, 2] = 2       # a full row at one level
    B, H, nqb, nkb = shape
    N = nkb * 64
    bq = N // nqb if N % nqb == 0 and (N // nqb) in (64, 128) else None
    if bq is None:
        pytest.skip("shape not expressible as a problem")
    q = torch.zeros((B, H, N, 64), device=DEV, dtype=torch.bfloat16)
    prob = psa.make_problem(q, q, q, block_q=bq)
    row_ptr, col_idx, err = psa.build_index(torch.from_numpy(lm).to(DEV), prob)
    rp_ref, ci_ref = oracle.build_index(lm)
    check_index(row_ptr, col_idx, rp_ref, ci_ref, nqb)
    assert err.item() == 0


def test_build_index_all_skip_many_tiles():
    """An all-skip map over six scan tiles: every row pointer is 0 (nothing listed, fewer
    listed entries than tiles)."""
    announce("build_index all skip, many tiles")
    lm = np.full((1, 40, 129, 258), -1, dtype=np.int8)
    q = torch.zeros((1, 40, 258 * 64, 64), device=DEV, dtype=torch.bfloat16)
    prob = psa.make_problem(q, q, q, block_q=128)
    row_ptr, col_idx, err = psa.build_index(torch.from_numpy(lm).to(DEV), prob)
    rows = 40 * 129
    rp = row_ptr.cpu().numpy()
    assert not np.any(rp[:rows * 4 + 1])
    assert np.array_equal(rp[rows * 4 + 1:], np.arange(rows))   # equal counts: rows in order
    assert err.item() == 0


# (N, heads_q, heads_kv, XCD ranges per chunk of the dispatch order): lengths at which the K
# and V of the KV heads in flight outgrow half the last-level cache (ragged row counts for
# f = 2 and 4)
SHARES = [(75648, 4, 2, 8), (32896, 4, 4, 2), (49280, 3, 3, 4)]


@pytest.mark.parametrize("case", SHARES, ids=[f"N{c[0]}-f{c[3]}" for c in SHARES])
def test_build_index_shared_order(case):
    """Long problems: psa_build_index lays the dispatch list over chunks of f XCD ranges
    (f = 2, 4, 8). CSR bit for bit against the oracle, the order against its definition. Only
    the map and the shape are read, so Q, K, V are zeros."""
    N, H, Hkv, f = case
    announce(f"build_index order, N {N}, f {f}")
    B, D = 1, 128
    nqb, nkb = N // 128, N // 64
    wl = W.Workload(name="shape", seed=0, batch=B, heads_q=H, heads_kv=Hkv, head_dim=D,
                    seq_len=N, seq_valid=N, block_q=128, block_k=64, dtype="bf16")
    assert order_share(wl) == f
    rng = np.random.default_rng(N)
    lm = rng.choice(np.array([0, 1, 2, 3, -1], dtype=np.int8), size=(B, H, nqb, nkb),
                    p=[0.05, 0.05, 0.05, 0.05, 0.8])
    q = torch.zeros((B, H, N, D), device=DEV, dtype=torch.bfloat16)
    k = torch.zeros((B, Hkv, N, D), device=DEV, dtype=torch.bfloat16)
    prob = psa.make_problem(q, k, k, block_q=128)
    row_ptr, col_idx, err = psa.build_index(torch.from_numpy(lm).to(DEV), prob)
    rp_ref, ci_ref = oracle.build_index(lm)
    check_index(row_ptr, col_idx, rp_ref, ci_ref, nqb * (H // Hkv), share=f)
    assert err.item() == 0


def test_build_index_flags_bad_entries():
    announce("build_index bad entries")
    lm = np.zeros((1, 2, 16, 16), dtype=np.int8)
    lm[0, 1, 3, 5] = 7
    lm[0, 0, 0, 0] = -2
    q = torch.zeros((1, 2, 1024, 64), device=DEV, dtype=torch.bfloat16)
    prob = psa.make_problem(q, q, q, block_q=64)
    row_ptr, col_idx, err = psa.build_index(torch.from_numpy(lm).to(DEV), prob)
    assert err.item() == psa.psa.PSA_ERR_BAD_LEVEL_MAP
    clean = np.where((lm < -1) | (lm > 3), -1, lm).astype(np.int8)
    rp_ref, ci_ref = oracle.build_index(clean)
    check_index(row_ptr, col_idx, rp_ref, ci_ref, 16)


def test_attn_reports_bad_level_map():
    announce("attn bad level map")
    wl = W.TINY_F32
    q, k, v, qd, kd, vd = _inputs(wl)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    lm = torch.from_numpy(W.make_map(wl)).to(DEV)
    ws = psa.attn_workspace(prob, DEV)
    psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob, ws=ws)
    psa.check_status(ws)
    lm[0, 0, 0, 1] = 9
    psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob, ws=ws)
    with pytest.raises(psa.PsaError):
        psa.check_status(ws)


# ---------------------------------------------------------------------------------------
# attention on the oracle's maps
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("wl", SMALL, ids=IDS)
def test_attention_parity(wl):
    announce(f"attention {wl.name}")
    q, k, v, qd, kd, vd = _inputs(wl)
    lm = oracle_map(wl, q, k)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    o, lse = psa.attn_fwd(qd, kd, vd, kp, vp, torch.from_numpy(lm).to(DEV), prob)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, lm, oracle_problem(wl))
    rnd = (oracle.attention(q, k, v, lm, oracle_problem(wl), pooled_round="bf16")
           if wl.dtype == "bf16" else None)
    check_attention(o, lse, o_ref, lse_ref, wl.seq_valid, wl.dtype == "f32", wl.name, rnd)


BF16_SMALL = [w for w in SMALL if w.dtype == "bf16"]


@pytest.mark.parametrize("wl", BF16_SMALL, ids=[w.name for w in BF16_SMALL])
def test_unpacked_attention_parity(wl):
    """The ablation layout (one logical block per hardware tile) computes the same attention."""
    announce(f"unpacked attention {wl.name}")
    q, k, v, qd, kd, vd = _inputs(wl)
    lm = oracle_map(wl, q, k)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    row_ptr, col_idx, err = psa.build_index(torch.from_numpy(lm).to(DEV), prob)
    o, lse = psa.attn_fwd_unpacked(qd, kd, vd, kp, vp, row_ptr, col_idx, prob)
    torch.cuda.synchronize()
    assert err.item() == 0
    o_ref, lse_ref = oracle.attention(q, k, v, lm, oracle_problem(wl))
    check_attention(o, lse, o_ref, lse_ref, wl.seq_valid, False, wl.name + " unpacked")


def test_unpacked_attention_rejects_f32():
    announce("unpacked attention f32")
    wl = W.TINY_F32
    q, k, v, qd, kd, vd = _inputs(wl)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    row_ptr, col_idx, err = psa.build_index(torch.from_numpy(W.make_map(wl)).to(DEV), prob)
    with pytest.raises(psa.PsaError) as ei:
        psa.attn_fwd_unpacked(qd, kd, vd, kp, vp, row_ptr, col_idx, prob)
    assert ei.value.status == psa.psa.PSA_ERR_UNSUPPORTED


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,bq", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_attention_shapes(causal, dtype, d, bq):
    """Every kernel instantiation, with padding, GQA and maps holding every level, including
    pooled levels on causal diagonal blocks and all-skip rows."""
    announce(f"attention d={d} bq={bq} {dtype} causal={causal}")
    wl = W.Workload(name="shape", seed=77, batch=2, heads_q=4, heads_kv=2, head_dim=d,
                    seq_len=1024, seq_valid=1000, block_q=bq, causal=causal, dtype=dtype,
                    k_dist="clustered", map_source="iid", map_probs=(0.2, 0.2, 0.2, 0.2, 0.2))
    q, k, v, qd, kd, vd = _inputs(wl)
    lm = W.make_map(wl)
    lm[0, 1, 2] = -1
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    o, lse = psa.attn_fwd(qd, kd, vd, kp, vp, torch.from_numpy(lm).to(DEV), prob)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, lm, oracle_problem(wl))
    rnd = (oracle.attention(q, k, v, lm, oracle_problem(wl), pooled_round="bf16")
           if dtype == "bf16" else None)
    check_attention(o, lse, o_ref, lse_ref, wl.seq_valid, dtype == "f32", f"shape d{d} bq{bq}", rnd)


TOKEN_MAJOR = [W.small(W.WAN13B_32K), W.small(W.QWEN25VL_32K)]


@pytest.mark.parametrize("wl", TOKEN_MAJOR, ids=[w.name for w in TOKEN_MAJOR])
def test_path_on_token_major_layout(wl):
    """Q, K, V as [batch, tokens, heads, d] storage viewed as [batch, heads, tokens, d] (token
    stride heads*d): the pyramid, the mask and the attention (the general-stride kernels)."""
    announce(f"path on a token-major layout {wl.name}")
    q, k, v = W.make_qkv(wl)
    def token_major(t):
        return t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    qd, kd, vd = token_major(q), token_major(k), token_major(v)
    assert qd.stride(2) == wl.heads_q * wl.head_dim and kd.stride(2) == wl.heads_kv * wl.head_dim
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    cert = []
    lm, M, sim = psa.mask(qd, kd, prob, mask_params(wl), cert_counts=cert)
    o, lse = psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob)
    torch.cuda.synchronize()
    assert o.stride() == qd.stride()
    p = oracle_problem(wl)
    lm_ref, M_ref, sim_ref = oracle.mask(q, k, p, wl.mask_mode, assign_params(wl),
                                         samples=wl.samples_per_qblock, stride=wl.antidiag_stride)
    assert np.abs(M.double().cpu().numpy() - M_ref).max() <= 2e-6
    check_map(lm.cpu().numpy(), lm_ref, oracle_margin_entries(M_ref, sim_ref, p, assign_params(wl)),
              f"{wl.name} token-major", cert)
    o_ref, lse_ref = oracle.attention(q, k, v, lm.cpu().numpy(), p)
    check_attention(o, lse, o_ref, lse_ref, wl.seq_valid, False, f"{wl.name} token-major")
    # the attention on this layout equals the attention on the contiguous copies
    qc, kc, vc = qd.contiguous(), kd.contiguous(), vd.contiguous()
    prob_c = problem_for(wl, qc, kc, vc)
    kpc, vpc = psa.build_pyramid(kc, vc, prob_c)
    assert torch.equal(kpc, kp) and torch.equal(vpc, vp)
    oc, _ = psa.attn_fwd(qc, kc, vc, kpc, vpc, lm, prob_c)
    assert torch.equal(oc, o.contiguous())


def test_attention_all_l0_matches_sdpa():
    """An all-L0 map is dense attention: compare with torch SDPA (float32, on the GPU)."""
    announce("attention all-L0 vs SDPA")
    wl = W.small(W.WAN13B_32K).replace(seq_valid=2048)
    q, k, v, qd, kd, vd = _inputs(wl)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    lm = torch.zeros((1, wl.heads_q, wl.n_qblocks, wl.n_kblocks), dtype=torch.int8, device=DEV)
    o, _ = psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob)
    ref = torch.nn.functional.scaled_dot_product_attention(qd.float(), kd.float(), vd.float())
    err = (o.float() - ref).abs().max().item()
    assert err < 2e-2, err


def test_attention_pad_keys_do_not_leak():
    """Large values in the pad rows of K and V must not reach any output."""
    announce("attention pad leak")
    wl = W.small(W.WAN14B_720P_75K)
    q, k, v = W.make_qkv(wl)
    k2, v2 = k.clone(), v.clone()
    k2[..., wl.seq_valid:, :] = 1e3
    v2[..., wl.seq_valid:, :] = 1e3
    lm = W.make_map(wl)
    qd = q.to(DEV)
    outs = []
    for kk, vv in ((k, v), (k2, v2)):
        kd, vd = kk.to(DEV), vv.to(DEV)
        prob = problem_for(wl, qd, kd, vd)
        kp, vp = psa.build_pyramid(kd, vd, prob)
        o, _ = psa.attn_fwd(qd, kd, vd, kp, vp, torch.from_numpy(lm).to(DEV), prob)
        outs.append(o)
    assert torch.equal(outs[0], outs[1])


def test_attention_deterministic():
    announce("attention determinism")
    wl = W.small(W.QWEN25VL_32K)
    q, k, v, qd, kd, vd = _inputs(wl)
    lm = torch.from_numpy(W.make_map(wl.replace(map_source="iid",
                                                map_probs=(.3, .2, .2, .1, .2)))).to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    o1, l1 = psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob)
    o2, l2 = psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------------------
# threshold assignment, exact
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("causal,force_diag,span,cos,nv", [
    (False, False, (0, 0), 0.0, 4096),
    (True, True, (0, 0), 0.8, 4096),
    (False, True, (3000, 3300), 0.8, 4096),
    (False, False, (0, 0), 0.0, 3712),     # last query block all padding
    (True, False, (100, 900), 0.5, 4096),
])
def test_mask_assign_exact(causal, force_diag, span, cos, nv):
    """Dyadic masses (multiples of 2^-20 summing to 1, with ties) make every running sum exact,
    so the level maps must agree bit for bit."""
    announce(f"mask_assign causal={causal} diag={force_diag} span={span} cos={cos} nv={nv}")
    B, H, Hkv, N, bq = 1, 4, 2, 4096, 128
    nqb, nkb = N // bq, N // 64
    rng = np.random.default_rng(5)
    counts = np.stack([rng.multinomial(1 << 20, rng.dirichlet(np.full(nkb, 0.3)))
                       for _ in range(B * H * nqb)])
    M = (counts / float(1 << 20)).astype(np.float32).reshape(B, H, nqb, nkb)
    sim = rng.integers(0, 1 << 10, size=(B, Hkv, nkb)).astype(np.float32) / (1 << 10)
    sim[..., ::7] = np.float32(0.8)                          # exactly at the bound
    thr = (0.5, 0.7, 0.8, 0.9)
    p = oracle.Problem(seq_len=N, seq_valid=nv, head_dim=64, block_q=bq, causal=causal)
    a = oracle.AssignParams(thr, cos, force_diag, span[0], span[1])
    ref = np.stack([np.stack([oracle.assign_levels(M[b, h].astype(np.float64),
                                                   sim[b, h // (H // Hkv)].astype(np.float64) if cos > 0 else None,
                                                   p, a) for h in range(H)]) for b in range(B)])
    qd = torch.zeros((B, H, N, 64), device=DEV, dtype=torch.bfloat16)
    kd = torch.zeros((B, Hkv, N, 64), device=DEV, dtype=torch.bfloat16)
    prob = psa.make_problem(qd, kd, kd, block_q=bq, causal=causal, seq_valid=nv)
    mp = psa.MaskParams(thresholds=thr, cos_sim_min=cos, force_diag_l0=force_diag,
                        force_l0_begin=span[0], force_l0_end=span[1])
    got = psa.mask_assign(torch.from_numpy(M).to(DEV), torch.from_numpy(sim).to(DEV), prob, mp)
    assert np.array_equal(got.cpu().numpy(), ref)


# ---------------------------------------------------------------------------------------
# mask generator end to end
# ---------------------------------------------------------------------------------------
MASKED = [w for w in SMALL if w.map_source == "mask"]
# the antidiagonal scorer's general path (compressed columns not a whole number of 128-column
# tiles) next to its fast path above
MASKED.append(W.small(W.QWEN25VL_32K).replace(name="qwen2.5-vl-7b-small-1536", seq_len=1536,
                                                  seq_valid=1536))
# a last tile of compressed columns that is partial (2176 / 8 = 272 columns = 4.25 tiles of 64),
# with padding: a regression case for the general path's last tile
MASKED.append(W.small(W.QWEN25VL_32K).replace(name="qwen2.5-vl-7b-small-partial-tile", seq_len=2176,
                                                  seq_valid=2168))
# block-mean scoring on the sampling workloads' inputs, non-causal with padding and causal
MASKED.append(W.small(W.WAN13B_32K).replace(name="wan2.1-1.3b-small-meankey", mask_mode="meankey"))
MASKED.append(W.small(W.QWEN25VL_32K).replace(name="qwen2.5-vl-7b-small-meankey", mask_mode="meankey"))


@pytest.mark.parametrize("wl", MASKED, ids=[w.name for w in MASKED])
def test_mask_parity(wl):
    announce(f"mask {wl.name}")
    q, k, v, qd, kd, vd = _inputs(wl)
    p = oracle_problem(wl)
    a = assign_params(wl)
    lm_ref, M_ref, sim_ref = oracle.mask(q, k, p, wl.mask_mode, a, samples=wl.samples_per_qblock,
                                         stride=wl.antidiag_stride)
    prob = problem_for(wl, qd, kd, vd)
    cert = []
    lm, M, sim = psa.mask(qd, kd, prob, mask_params(wl), cert_counts=cert)
    torch.cuda.synchronize()
    Mg = M.double().cpu().numpy()
    dM = np.abs(Mg - M_ref)
    big = M_ref > 1e-3
    rel = (dM[big] / M_ref[big]).max(initial=0.0)
    print(f"[{wl.name}] mass max abs diff {dM.max():.3e}, max rel diff (masses > 1e-3) {rel:.3e}",
          flush=True)
    assert dM.max() <= 2e-6
    if sim_ref is not None:
        ds = np.abs(sim.double().cpu().numpy() - sim_ref)
        print(f"[{wl.name}] sim max abs diff {ds.max():.3e}", flush=True)
        assert ds.max() <= 1e-6
    check_map(lm.cpu().numpy(), lm_ref, oracle_margin_entries(M_ref, sim_ref, p, a), wl.name, cert)


# ---------------------------------------------------------------------------------------
# float64 certification of near-threshold rows, forced
# ---------------------------------------------------------------------------------------
def _prefix_sums(Mr, last):
    """Exclusive cumulative masses of one row in the assignment's order (mass descending, ties
    by block index)."""
    order = sorted(range(last + 1), key=lambda kb: (-float(Mr[kb]), kb))
    return np.cumsum([0.0] + [float(Mr[kb]) for kb in order])[:-1]


def _near_thresholds(rows_c, delta):
    """Four increasing thresholds, the l-th `delta` above an exclusive cumulative mass in the
    l-th quarter of (0.3, 0.97) of row l of `rows_c` (else of row 0)."""
    edges = np.linspace(0.3, 0.97, 5)
    t = []
    for l in range(4):
        for c in (rows_c[l], rows_c[0]):
            inside = c[(c > edges[l]) & (c < edges[l + 1] - 2 * delta)]
            if inside.size:
                t.append(float(np.float32(inside[inside.size // 2] + delta)))
                break
        else:
            raise AssertionError("row too concentrated for the test")
    assert all(t[i] < t[i + 1] for i in range(3))
    return tuple(t)


_QW = W.small(W.QWEN25VL_32K)
FORCED = [
    # sampling, every query block of head 0 a copy of the first: all its rows flagged
    ("sampling-repeated", W.small(W.WAN13B_32K).replace(seq_valid=2048), True, 1.5e-6),
    # antidiagonal S = 8, 16 compressed rows per query block (the float64 MFMA rescoring)
    ("antidiag-s8-repeated", _QW.replace(causal=False, force_diag_l0=False), True, 2e-6),
    # antidiagonal S = 4 with 64-row query blocks (16 compressed rows again)
    ("antidiag-s4-repeated", _QW.replace(causal=False, force_diag_l0=False, block_q=64,
                                         antidiag_stride=4), True, 2e-6),
    # causal antidiagonal S = 8: each threshold next to a cumulative mass of another query block
    ("antidiag-s8-causal", _QW, False, 2e-6),
    # block-mean scoring (float64 key sums per KV block), also through the fused attention
    ("meankey-repeated", W.small(W.WAN13B_32K).replace(seq_valid=2048, mask_mode="meankey"), True,
     1.5e-6),
]


@pytest.mark.parametrize("case", FORCED, ids=[c[0] for c in FORCED])
def test_certification_forced(case):
    """Thresholds placed `delta` above cumulative masses of chosen rows (inside the float32 margin
    that flags a row for float64 rescoring, far outside the oracle's own 1e-12 margin): the
    flagged rows are rescored in float64 and the map must equal the oracle's bit for bit. With
    every query block of head 0 a copy of the first (non-causal), all of head 0's rows are
    flagged."""
    name, wl, repeated, delta = case
    announce(f"forced certification {name}")
    q, k, v = W.make_qkv(wl)
    if repeated:
        B, H, N, D = q.shape
        q = q.clone()
        q[:, 0] = q[:, 0, :wl.block_q].repeat(1, N // wl.block_q, 1)
    p = oracle_problem(wl)
    a0 = assign_params(wl)
    _, M_ref, sim_ref = oracle.mask(q, k, p, wl.mask_mode, a0, samples=wl.samples_per_qblock,
                                    stride=wl.antidiag_stride)
    nq = p.n_qblocks
    rows = (nq - 1,) * 4 if repeated else (nq - 1, nq - 3, nq // 2 + 1, nq // 2 - 1)
    t = _near_thresholds([_prefix_sums(M_ref[0, 0, r], oracle.kb_diag(p, r) if p.causal else
                                       p.n_kblocks - 1) for r in rows], delta)
    wl_t = wl.replace(thresholds=t)
    a = assign_params(wl_t)
    lm_ref = np.stack([np.stack([oracle.assign_levels(M_ref[b, h], None if sim_ref is None else
                                                      sim_ref[b, h // (q.shape[1] // k.shape[1])], p, a)
                                 for h in range(q.shape[1])]) for b in range(q.shape[0])])
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl_t, qd, kd, vd)
    cert = []
    lm, M, sim = psa.mask(qd, kd, prob, mask_params(wl_t), cert_counts=cert)
    torch.cuda.synchronize()
    need = p.n_qblocks if repeated else 4
    print(f"[{name}] thresholds {t}: {cert[0]} rows rescored in float64 (at least {need} expected)",
          flush=True)
    assert cert[1] == 0 and cert[0] >= need
    check_map(lm.cpu().numpy(), lm_ref, oracle_margin_entries(M_ref, sim_ref, p, a), name, cert)
    if wl.mask_mode == "meankey":
        # the fused call certifies the same rows in its prologue: the same map and masses
        kp, vp = psa.build_pyramid(kd, vd, prob)
        _, _, lmf, Mf = psa.attn_fwd_meankey(qd, kd, vd, kp, vp, prob, mask_params(wl_t),
                                             want_mass=True)
        torch.cuda.synchronize()
        assert torch.equal(lmf, lm) and torch.equal(Mf, M), "fused call differs from psa_mask"
