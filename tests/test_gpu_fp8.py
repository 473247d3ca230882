"""GPU parity of the fp8 QK^T reading: psa_quantize_fp8 and psa_attn_fwd_fp8qk against the
oracle's fp8_scale / fp8_quantize / attention_fp8qk_head.

* Quantization is integer output decided in float64 on both sides: scales and codes must agree
  bit for bit (codes compared as e4m3 values; no NaN code may appear).
* The attention kernel alone runs on the oracle's own codes and scales (uploaded), so it is
  compared with the oracle on identical fp8 operands, to the bf16 attention bars (P and V are
  bf16 as in the bf16 path; the q8 . k8 products are exact and summed in float32).
* The whole GPU chain (pyramid, quantization, attention) is compared with the oracle run on its
  own quantization of the same bf16 inputs. The pooled K that the GPU quantizes is its bf16
  pyramid output; the oracle's is the float64 mean rounded to bf16 (round to nearest even).
  The two differ in a few pooled values by one bf16 ulp (the pairwise float32 tree), which can
  move an e4m3 code by one step; the test counts those codes (at most 1e-3 of them) and holds
  the outputs to the same bars.
The pooled levels enter the quantizer as bf16 values: the tensors the pyramid stores.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import video_transformers_amd as psa
from gpu_util import DEV, announce, check_attention, need_gpu, oracle_map, oracle_problem, problem_for

pytestmark = pytest.mark.gpu

NAN_CODES = (0x7F, 0xFF)


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def bf16_rne(x):
    """float64 values rounded once to the nearest bf16 (8 significant bits), ties to even."""
    x = np.asarray(x, dtype=np.float64)
    m, ex = np.frexp(np.abs(x))          # |x| = m 2^ex, m in [0.5, 1)
    q = np.ldexp(1.0, ex - 8)            # spacing of the binade [2^(ex-1), 2^ex)
    return np.sign(x) * np.round(np.abs(x) / q) * q


def decode(codes: torch.Tensor) -> np.ndarray:
    c = codes.cpu()
    assert not any(torch.any(c == n).item() for n in NAN_CODES), "NaN e4m3 code written"
    return c.view(torch.float8_e4m3fn).float().double().numpy()


def encode(values: np.ndarray) -> torch.Tensor:
    """e4m3 values (exactly representable) -> their codes, as uint8."""
    t = torch.from_numpy(np.ascontiguousarray(values)).to(torch.float32).to(torch.float8_e4m3fn)
    assert np.array_equal(t.float().double().numpy(), values), "value not representable in e4m3"
    return t.view(torch.uint8)


def oracle_head_fp8(kh: np.ndarray):
    """(s, level-0 values, {l: pooled values}) of one K head in the oracle's reading."""
    s = oracle.fp8_scale(kh)
    lk = oracle.pyramid(kh)
    return s, oracle.fp8_quantize(kh, s), {l: oracle.fp8_quantize(bf16_rne(lk[l]), s)
                                           for l in range(1, oracle.NUM_LEVELS)}


def pack_levels(levels):
    return np.concatenate([levels[l] for l in range(1, oracle.NUM_LEVELS)], axis=0)


# ---------------------------------------------------------------------------------------
# quantization
# ---------------------------------------------------------------------------------------
def every_bf16_upto(amax: float, n: int) -> torch.Tensor:
    """Every bf16 value v with |v| <= amax (both signs, amax itself included), zero-padded to
    n values."""
    bits = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    pos = bits[bits.float() <= amax].float()
    vals = torch.cat([pos, -pos])
    assert vals.numel() <= n and float(pos.max()) == amax
    out = torch.zeros(n)
    out[:vals.numel()] = vals
    return out


# amax values whose scale amax / 448 makes a float32 estimate of x / s round to the wrong code
# for some bf16 x (found by enumerating the bf16 amax values in [2^-8, 2^8])
AMAX_ESTIMATE_MISSES = (0.00396728515625, 0.00408935546875, 0.0045166015625)


def test_quantize_every_bf16_value():
    """Heads holding every finite bf16 up to their amax: amax 448 (scale exactly 1; every e4m3
    value and every midpoint between two of them appear), the same values times 2^-20 (scale
    exactly 2^-20, same codes; values below 2^-100 left out so that the product stays exact),
    an all-zero head (scale 1, all codes zero), amax values whose scale defeats a float32
    estimate of the quotient, and amax 448 * 2^-120 (scale 2^-120, below the float32 path's
    range)."""
    announce("quantize_fp8 every bf16 value")
    N, D = 272, 128
    head = every_bf16_upto(448.0, N * D)
    big = torch.where(head.abs() >= 2.0 ** -100, head, torch.zeros_like(head))
    heads = [head, big * 2.0 ** -20, torch.zeros(N * D)]
    heads += [every_bf16_upto(a, N * D) for a in AMAX_ESTIMATE_MISSES]
    heads.append(every_bf16_upto(448.0 * 2.0 ** -120, N * D))
    x = torch.stack(heads).view(1, len(heads), N, D).to(torch.bfloat16)
    assert torch.equal(x[0, 1].float().flatten() * 2.0 ** 20, big)
    x8, _, sc = psa.quantize_fp8(x.to(DEV))
    torch.cuda.synchronize()
    got_s = sc.cpu().numpy()
    got = decode(x8)
    for h in range(len(heads)):
        xh = oracle.as_f64(x[0, h])
        s = oracle.fp8_scale(xh)
        assert np.float32(s) == got_s[h], (h, s, got_s[h])
        ref = oracle.fp8_quantize(xh, s)
        assert np.array_equal(got[0, h], ref), (h, int(np.sum(got[0, h] != ref)))
    assert got_s[0] == 1.0 and got_s[1] == 2.0 ** -20 and got_s[2] == 1.0
    assert got_s[-1] == 2.0 ** -120
    assert np.count_nonzero(got[0, 2]) == 0


QUANT = [W.small(W.WAN13B_32K), W.small(W.QWEN25VL_32K), W.small(W.WAN14B_720P_75K)]


@pytest.mark.parametrize("token_major", [False, True])
@pytest.mark.parametrize("wl", QUANT, ids=[w.name for w in QUANT])
def test_quantize_exact(wl, token_major):
    """Q (level 0) and K with its pooled levels, per head, on the workload's bf16 inputs
    (token-major: [batch, tokens, heads, d] storage viewed as [batch, heads, tokens, d])."""
    announce(f"quantize_fp8 {wl.name} token_major={token_major}")
    q, k, _ = W.make_qkv(wl)
    def dev(t):
        if token_major:
            return t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
        return t.to(DEV)
    B, Hkv = wl.batch, wl.heads_kv
    kp_in = np.stack([np.stack([pack_levels({l: bf16_rne(x) for l, x in
                                             oracle.pyramid(oracle.as_f64(k[b, h])).items() if l})
                                for h in range(Hkv)]) for b in range(B)])
    kp_dev = torch.from_numpy(kp_in).to(torch.float32).to(torch.bfloat16).to(DEV)
    assert np.array_equal(kp_dev.double().cpu().numpy(), kp_in)
    q8, none, sq = psa.quantize_fp8(dev(q))
    k8, kp8, sk = psa.quantize_fp8(dev(k), kp_dev)
    torch.cuda.synchronize()
    assert none is None
    gq, gk, gkp = decode(q8), decode(k8), decode(kp8)
    sq, sk = sq.cpu().numpy(), sk.cpu().numpy()
    for b in range(B):
        for h in range(wl.heads_q):
            qh = oracle.as_f64(q[b, h])
            s = oracle.fp8_scale(qh)
            assert np.float32(s) == sq[b * wl.heads_q + h]
            assert np.array_equal(gq[b, h], oracle.fp8_quantize(qh, s)), ("q", b, h)
        for h in range(Hkv):
            kh = oracle.as_f64(k[b, h])
            s = oracle.fp8_scale(kh)
            assert np.float32(s) == sk[b * Hkv + h]
            assert np.array_equal(gk[b, h], oracle.fp8_quantize(kh, s)), ("k", b, h)
            assert np.array_equal(gkp[b, h], oracle.fp8_quantize(kp_in[b, h], s)), ("kp", b, h)


# ---------------------------------------------------------------------------------------
# attention on fp8 operands
# ---------------------------------------------------------------------------------------
ATTN = [W.small(W.WAN13B_32K), W.small(W.WAN14B_720P_75K), W.small(W.QWEN25VL_32K),
        W.small(W.QWEN25VL_32K).replace(name="qwen2.5-vl-7b-small-bq64", block_q=64)]


def _oracle_fp8_inputs(wl, q, k):
    """Per-head oracle quantization: (s_q [B,H], q8 [B,H,N,d], s_k [B,Hkv], k8, kp8 levels)."""
    B, H, Hkv = wl.batch, wl.heads_q, wl.heads_kv
    sq = np.zeros((B, H))
    q8 = np.zeros(q.shape)
    for b in range(B):
        for h in range(H):
            qh = oracle.as_f64(q[b, h])
            sq[b, h] = oracle.fp8_scale(qh)
            q8[b, h] = oracle.fp8_quantize(qh, sq[b, h])
    sk = np.zeros((B, Hkv))
    k8 = np.zeros(k.shape)
    kp8 = [[None] * Hkv for _ in range(B)]
    for b in range(B):
        for h in range(Hkv):
            sk[b, h], k8[b, h], kp8[b][h] = oracle_head_fp8(oracle.as_f64(k[b, h]))
    return sq, q8, sk, k8, kp8


def _oracle_fp8_attention(wl, q8, sq, k8, kp8, sk, v, lm):
    p = oracle_problem(wl)
    g = wl.group
    o = np.zeros(q8.shape)
    lse = np.zeros(q8.shape[:3])
    for b in range(wl.batch):
        for h in range(wl.heads_q):
            hk = h // g
            o[b, h], lse[b, h] = oracle.attention_fp8qk_head(
                q8[b, h], k8[b, hk], kp8[b][hk], oracle.as_f64(v[b, hk]), sq[b, h], sk[b, hk],
                lm[b, h], p)
    return o, lse


@pytest.mark.parametrize("wl", ATTN, ids=[w.name for w in ATTN])
def test_fp8qk_kernel_parity(wl):
    """The attention kernel on the oracle's own e4m3 codes and scales."""
    announce(f"fp8qk kernel {wl.name}")
    q, k, v = W.make_qkv(wl)
    lm = oracle_map(wl, q, k)
    sq, q8, sk, k8, kp8 = _oracle_fp8_inputs(wl, q, k)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    _, vp = psa.build_pyramid(kd, vd, prob)
    kp8_packed = np.stack([np.stack([pack_levels(kp8[b][h]) for h in range(wl.heads_kv)])
                           for b in range(wl.batch)])
    o, lse = psa.attn_fwd_fp8qk(encode(q8).to(DEV), torch.from_numpy(sq.ravel()).float().to(DEV),
                                encode(k8).to(DEV), encode(kp8_packed).to(DEV),
                                torch.from_numpy(sk.ravel()).float().to(DEV), vd, vp,
                                torch.from_numpy(lm).to(DEV), prob)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle_fp8_attention(wl, q8, np.float32(sq).astype(np.float64), k8, kp8,
                                           np.float32(sk).astype(np.float64), v, lm)
    check_attention(o, lse, o_ref, lse_ref, wl.seq_valid, False, f"{wl.name} fp8qk kernel")


def _gpu_fp8_path(wl, qd, kd, vd, lm_dev, prob):
    kp, vp = psa.build_pyramid(kd, vd, prob)
    k8, kp8, sk = psa.quantize_fp8(kd, kp)
    q8, _, sq = psa.quantize_fp8(qd)
    o, lse = psa.attn_fwd_fp8qk(q8, sq, k8, kp8, sk, vd, vp, lm_dev, prob)
    return kp8, o, lse


@pytest.mark.parametrize("wl", ATTN, ids=[w.name for w in ATTN])
def test_fp8qk_path_parity(wl):
    """Pyramid, quantization and attention on the GPU against the oracle's fp8 reading."""
    announce(f"fp8qk path {wl.name}")
    q, k, v = W.make_qkv(wl)
    lm = oracle_map(wl, q, k)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    kp8, o, lse = _gpu_fp8_path(wl, qd, kd, vd, torch.from_numpy(lm).to(DEV), prob)
    torch.cuda.synchronize()
    sq, q8, sk, k8, kp8_ref = _oracle_fp8_inputs(wl, q, k)
    got = decode(kp8)
    ref = np.stack([np.stack([pack_levels(kp8_ref[b][h]) for h in range(wl.heads_kv)])
                    for b in range(wl.batch)])
    moved = float(np.mean(got != ref))
    print(f"[{wl.name}] pooled e4m3 codes that differ: {moved:.2e}", flush=True)
    assert moved <= 1e-3
    o_ref, lse_ref = _oracle_fp8_attention(wl, q8, sq, k8, kp8_ref, sk, v, lm)
    check_attention(o, lse, o_ref, lse_ref, wl.seq_valid, False, f"{wl.name} fp8qk path")
    # how far the fp8 reading lies from the exact (unquantized) attention: reported, with a
    # loose bound that only catches a broken scale or operand
    o_exact, _ = oracle.attention(q, k, v, lm, oracle_problem(wl))
    n = wl.seq_valid
    a = o[..., :n, :].double().cpu().numpy()
    rel = np.linalg.norm(a - o_exact[..., :n, :]) / np.linalg.norm(o_exact[..., :n, :])
    print(f"[{wl.name}] fp8 QK^T vs exact attention: rel L2 {rel:.3e}", flush=True)
    assert rel < 0.1


def test_fp8qk_token_major_v_and_rejects_d64():
    """V in a token-major layout (general-stride V loads beside contiguous fp8 K) gives the
    same output as contiguous V; head_dim 64 has no fp8 kernel."""
    announce("fp8qk token-major V, d64 rejected")
    wl = W.small(W.QWEN25VL_32K)
    q, k, v = W.make_qkv(wl)
    lm = torch.from_numpy(W.make_map(wl.replace(map_source="iid",
                                                map_probs=(.3, .2, .2, .1, .2)))).to(DEV)
    qd, kd = q.to(DEV), k.to(DEV)
    vc = v.to(DEV)
    vt = v.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    outs = []
    for vd in (vc, vt):
        prob = problem_for(wl, qd, kd, vd)
        _, o, lse = _gpu_fp8_path(wl, qd, kd, vd, lm, prob)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    wl64 = W.small(W.COGVIDEOX5B_17K)
    q, k, v = W.make_qkv(wl64)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl64, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    k8, kp8, sk = psa.quantize_fp8(kd, kp)
    q8, _, sq = psa.quantize_fp8(qd)
    with pytest.raises(psa.PsaError) as ei:
        lm64 = W.make_map(wl64.replace(map_source="iid", map_probs=(.3, .2, .2, .1, .2)))
        psa.attn_fwd_fp8qk(q8, sq, k8, kp8, sk, vd, vp, torch.from_numpy(lm64).to(DEV), prob)
    assert ei.value.status == psa.psa.PSA_ERR_UNSUPPORTED


def test_fp8qk_deterministic():
    announce("fp8qk determinism")
    wl = W.small(W.WAN13B_32K)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lm = torch.from_numpy(W.make_map(wl.replace(map_source="iid",
                                                map_probs=(.3, .2, .2, .1, .2)))).to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    r1 = _gpu_fp8_path(wl, qd, kd, vd, lm, prob)
    r2 = _gpu_fp8_path(wl, qd, kd, vd, lm, prob)
    assert all(torch.equal(a, b) for a, b in zip(r1, r2))


def test_fp8qk_fullsize_wan():
    """The Wan2.1-1.3B-like 32k layer at full size, with the mask's own map, in the launch
    configuration the benchmark times; sampled heads and query blocks (first, middle, last
    with its pad rows, one drawn) against the oracle's fp8 reading on the GPU map rows."""
    wl = W.WAN13B_32K
    announce(f"fp8qk full size {wl.name}")
    from gpu_util import mask_params
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    lm, _, _ = psa.mask(qd, kd, prob, mask_params(wl))
    kp8, o, lse = _gpu_fp8_path(wl, qd, kd, vd, lm, prob)
    torch.cuda.synchronize()
    lm = lm.cpu().numpy()
    p = oracle_problem(wl)
    n = wl.n_qblocks
    rng = np.random.default_rng(wl.seed)
    for h in (0, wl.heads_q - 1):
        qh, kh, vh = (oracle.as_f64(t[0, h]) for t in (q, k, v))
        s_q = oracle.fp8_scale(qh)
        s_k, k8h, kp8h = oracle_head_fp8(kh)
        qbs = sorted({0, n // 2, n - 1, int(rng.integers(1, n - 1))})
        o_ref, lse_ref = oracle.attention_fp8qk_head(oracle.fp8_quantize(qh, s_q), k8h, kp8h, vh,
                                                     s_q, s_k, lm[0, h], p, qblocks=qbs)
        rows = np.concatenate([np.arange(qb * wl.block_q, (qb + 1) * wl.block_q) for qb in qbs])
        valid = rows[rows < wl.seq_valid]
        og = o[0, h, valid].double().cpu().numpy()
        d = og - o_ref[valid]
        rel = np.linalg.norm(d) / np.linalg.norm(o_ref[valid])
        mx = np.abs(d).max()
        ld = np.abs(lse[0, h, valid].double().cpu().numpy() - lse_ref[valid]).max()
        print(f"[{wl.name}] head {h} blocks {qbs}: max_abs={mx:.3e} rel_l2={rel:.3e} "
              f"lse={ld:.3e}", flush=True)
        assert mx <= 2e-2 and rel <= 5e-3 and ld <= 3e-2
        pad = rows[rows >= wl.seq_valid]
        assert torch.count_nonzero(o[0, h, pad]).item() == 0


# ---------------------------------------------------------------------------------------
# attention with the P V product on e4m3 operands as well
# ---------------------------------------------------------------------------------------
# Bars. P is rounded to e4m3 on both sides from values computed in different precisions (fp32
# logits and exp2 on the GPU, fp64 in the oracle); a value within rounding of an e4m3 midpoint
# can land on either neighbouring code. One code step moves that weight w_j by at most w_j / 8,
# so o_i by at most w_j / 8 * |v_j - o_i| and the lse by at most ln(1 + 1/8) = 0.118. Such
# flips are sparse (a pair's value must lie within ~2^-22 relative of a midpoint), so the
# relative L2 bar stays that of bf16 (5e-3); max-abs allows a flip on a key of weight 0.05
# at |v_j - o_i| = 8 (N(0,1) values): 5e-2; lse 0.125.
FP8PV_MAX_ABS = 5e-2
FP8PV_REL_L2 = 5e-3
FP8PV_LSE = 0.125


def check_fp8pv(o, lse, o_ref, lse_ref, nv, what):
    a = o[..., :nv, :].double().cpu().numpy()
    r = o_ref[..., :nv, :]
    mx = float(np.abs(a - r).max())
    rel = float(np.linalg.norm(a - r) / np.linalg.norm(r))
    lg = lse[..., :nv].double().cpu().numpy()
    lr = lse_ref[..., :nv]
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), f"{what}: empty-row sets differ"
    ld = float(np.abs(np.where(np.isneginf(lr), 0.0, lg - lr)).max(initial=0.0))
    print(f"[{what}] max_abs={mx:.3e} rel_l2={rel:.3e} lse={ld:.3e}", flush=True)
    assert mx <= FP8PV_MAX_ABS and rel <= FP8PV_REL_L2 and ld <= FP8PV_LSE, what
    assert torch.count_nonzero(o[..., nv:, :]).item() == 0, f"{what}: non-zero pad rows"
def _oracle_v_fp8(wl, v):
    """Per-KV-head oracle quantization of V and its pooled levels (the pyramid's bf16 means)."""
    B, Hkv = wl.batch, wl.heads_kv
    sv = np.zeros((B, Hkv))
    v8 = np.zeros(v.shape)
    vp8 = [[None] * Hkv for _ in range(B)]
    for b in range(B):
        for h in range(Hkv):
            sv[b, h], v8[b, h], vp8[b][h] = oracle_head_fp8(oracle.as_f64(v[b, h]))
    return sv, v8, vp8


def _oracle_fp8pv_attention(wl, q8, sq, k8, kp8, sk, v8, vp8, sv, lm, qblocks=None, heads=None):
    p = oracle_problem(wl)
    g = wl.group
    o = np.zeros(q8.shape)
    lse = np.zeros(q8.shape[:3])
    for b in range(wl.batch):
        for h in (range(wl.heads_q) if heads is None else heads):
            hk = h // g
            o[b, h], lse[b, h] = oracle.attention_fp8_head(
                q8[b, h], k8[b, hk], kp8[b][hk], v8[b, hk], vp8[b][hk], sq[b, h], sk[b, hk],
                sv[b, hk], lm[b, h], p, qblocks=qblocks)
    return o, lse


def _packed_levels(wl, levels):
    return np.stack([np.stack([pack_levels(levels[b][h]) for h in range(wl.heads_kv)])
                     for b in range(wl.batch)])


@pytest.mark.parametrize("wl", ATTN, ids=[w.name for w in ATTN])
def test_fp8_kernel_parity(wl):
    """The fp8 Q K^T + P V kernel on the oracle's own e4m3 codes and scales."""
    announce(f"fp8 kernel {wl.name}")
    q, k, v = W.make_qkv(wl)
    lm = oracle_map(wl, q, k)
    sq, q8, sk, k8, kp8 = _oracle_fp8_inputs(wl, q, k)
    sv, v8, vp8 = _oracle_v_fp8(wl, v)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x).ravel()).float().to(DEV)
    o, lse = psa.attn_fwd_fp8(encode(q8).to(DEV), up(sq), encode(k8).to(DEV),
                              encode(_packed_levels(wl, kp8)).to(DEV), up(sk), encode(v8).to(DEV),
                              encode(_packed_levels(wl, vp8)).to(DEV), up(sv),
                              torch.from_numpy(lm).to(DEV), prob)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle_fp8pv_attention(wl, q8, sq, k8, kp8, sk, v8, vp8, sv, lm)
    check_fp8pv(o, lse, o_ref, lse_ref, wl.seq_valid, f"{wl.name} fp8 kernel")


def _gpu_fp8pv_path(qd, kd, vd, lm_dev, prob):
    kp, vp = psa.build_pyramid(kd, vd, prob)
    k8, kp8, sk = psa.quantize_fp8(kd, kp)
    v8, vp8, sv = psa.quantize_fp8(vd, vp)
    q8, _, sq = psa.quantize_fp8(qd)
    o, lse = psa.attn_fwd_fp8(q8, sq, k8, kp8, sk, v8, vp8, sv, lm_dev, prob)
    return o, lse


@pytest.mark.parametrize("wl", ATTN, ids=[w.name for w in ATTN])
def test_fp8_path_parity(wl):
    """Pyramid, quantization of Q, K and V, and the fp8 attention on the GPU against the
    oracle's fp8 reading of the same bf16 inputs."""
    announce(f"fp8 path {wl.name}")
    q, k, v = W.make_qkv(wl)
    lm = oracle_map(wl, q, k)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    o, lse = _gpu_fp8pv_path(qd, kd, vd, torch.from_numpy(lm).to(DEV), prob)
    torch.cuda.synchronize()
    sq, q8, sk, k8, kp8 = _oracle_fp8_inputs(wl, q, k)
    sv, v8, vp8 = _oracle_v_fp8(wl, v)
    o_ref, lse_ref = _oracle_fp8pv_attention(wl, q8, sq, k8, kp8, sk, v8, vp8, sv, lm)
    check_fp8pv(o, lse, o_ref, lse_ref, wl.seq_valid, f"{wl.name} fp8 path")
    o_exact, _ = oracle.attention(q, k, v, lm, oracle_problem(wl))
    n = wl.seq_valid
    a = o[..., :n, :].double().cpu().numpy()
    rel = np.linalg.norm(a - o_exact[..., :n, :]) / np.linalg.norm(o_exact[..., :n, :])
    print(f"[{wl.name}] fp8 Q K^T and P V vs exact attention: rel L2 {rel:.3e}", flush=True)
    assert rel < 0.12


def test_fp8_deterministic_and_rejects_d64():
    announce("fp8 determinism, d64 rejected")
    wl = W.small(W.QWEN25VL_32K)
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lm = torch.from_numpy(W.make_map(wl.replace(map_source="iid",
                                                map_probs=(.3, .2, .2, .1, .2)))).to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    r1 = _gpu_fp8pv_path(qd, kd, vd, lm, prob)
    r2 = _gpu_fp8pv_path(qd, kd, vd, lm, prob)
    assert all(torch.equal(a, b) for a, b in zip(r1, r2))
    wl64 = W.small(W.COGVIDEOX5B_17K)
    q, k, v = W.make_qkv(wl64)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl64, qd, kd, vd)
    lm64 = torch.from_numpy(W.make_map(wl64.replace(map_source="iid",
                                                    map_probs=(.3, .2, .2, .1, .2)))).to(DEV)
    with pytest.raises(psa.PsaError) as ei:
        _gpu_fp8pv_path(qd, kd, vd, lm64, prob)
    assert ei.value.status == psa.psa.PSA_ERR_UNSUPPORTED


def test_fp8_fullsize_wan():
    """The fp8 Q K^T + P V path on the full Wan2.1-1.3B-like 32k layer with the mask's own
    map; sampled heads and query blocks against the oracle's fp8 reading on the GPU map rows."""
    wl = W.WAN13B_32K
    announce(f"fp8 full size {wl.name}")
    from gpu_util import mask_params
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    lm, _, _ = psa.mask(qd, kd, prob, mask_params(wl))
    o, lse = _gpu_fp8pv_path(qd, kd, vd, lm, prob)
    torch.cuda.synchronize()
    lm = lm.cpu().numpy()
    p = oracle_problem(wl)
    n = wl.n_qblocks
    rng = np.random.default_rng(wl.seed + 1)
    for h in (0, wl.heads_q - 1):
        qh, kh, vh = (oracle.as_f64(t[0, h]) for t in (q, k, v))
        s_q = oracle.fp8_scale(qh)
        s_k, k8h, kp8h = oracle_head_fp8(kh)
        s_v, v8h, vp8h = oracle_head_fp8(vh)
        qbs = sorted({0, n // 2, n - 1, int(rng.integers(1, n - 1))})
        o_ref, lse_ref = oracle.attention_fp8_head(oracle.fp8_quantize(qh, s_q), k8h, kp8h, v8h,
                                                   vp8h, s_q, s_k, s_v, lm[0, h], p, qblocks=qbs)
        rows = np.concatenate([np.arange(qb * wl.block_q, (qb + 1) * wl.block_q) for qb in qbs])
        valid = rows[rows < wl.seq_valid]
        og = o[0, h, valid].double().cpu().numpy()
        d = og - o_ref[valid]
        rel = np.linalg.norm(d) / np.linalg.norm(o_ref[valid])
        mx = np.abs(d).max()
        ld = np.abs(lse[0, h, valid].double().cpu().numpy() - lse_ref[valid]).max()
        print(f"[{wl.name}] fp8 head {h} blocks {qbs}: max_abs={mx:.3e} rel_l2={rel:.3e} "
              f"lse={ld:.3e}", flush=True)
        assert mx <= FP8PV_MAX_ABS and rel <= FP8PV_REL_L2 and ld <= FP8PV_LSE
        pad = rows[rows >= wl.seq_valid]
        assert torch.count_nonzero(o[0, h, pad]).item() == 0
