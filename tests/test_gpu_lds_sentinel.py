"""LDS sentinel: every kernel of the path starts on LDS that a diagnostic fill left holding a
NaN pattern (psa_debug_fill_lds right before each call), and must give outputs bit-identical
to the same calls started on LDS filled with zeros. A kernel that read an LDS word it had not
written first (an unloaded tile row, a stale list entry, a scratch word of the prologue) would
carry the pattern into its results: NaN through the MFMA products and sums, or a different
value. The path here: pyramid, mask (each scoring mode), block index, bf16 attention, the
unpacked layout, block-mean fused attention, backward, both fp8 forwards.
"""
import pytest
import torch

import workloads as W
import video_transformers_amd as psa
from gpu_util import DEV, announce, mask_params, need_gpu, problem_for

pytestmark = pytest.mark.gpu

NAN = 0x7FC00000
ALL_ONES = 0xFFFFFFFF   # a NaN with every payload bit set

CASES = [W.small(W.WAN13B_32K), W.small(W.COGVIDEOX5B_17K), W.small(W.QWEN25VL_32K),
         W.small(W.WAN14B_720P_75K)]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _path(wl, qd, kd, vd, pattern):
    """Every call of the path, each enqueued right after an LDS fill with `pattern`."""
    fill = lambda: psa.debug_fill_lds(pattern)  # noqa: E731
    out = {}
    prob = problem_for(wl, qd, kd, vd)
    fill()
    kp, vp = psa.build_pyramid(kd, vd, prob)
    out["kp"], out["vp"] = kp, vp
    if wl.map_source == "mask":
        fill()
        lm, M, sim = psa.mask(qd, kd, prob, mask_params(wl))
        out["map"], out["mass"] = lm, M
        fill()
        mk = mask_params(wl)
        mk.mode = "meankey"
        if wl.block_q == 128:
            of, lf, lmf, Mf = psa.attn_fwd_meankey(qd, kd, vd, kp, vp, prob, mk, want_mass=True)
            out.update(o_mk=of, lse_mk=lf, map_mk=lmf, mass_mk=Mf)
    else:
        lm = torch.from_numpy(W.make_map(wl)).to(DEV)
    fill()
    rp, ci, err = psa.build_index(lm, prob)
    out["row_ptr"] = rp
    fill()
    o, lse = psa.attn_fwd_indexed(qd, kd, vd, kp, vp, rp, ci, prob)
    out["o"], out["lse"] = o, lse
    fill()
    ou, lu = psa.attn_fwd_unpacked(qd, kd, vd, kp, vp, rp, ci, prob)
    out["o_unpacked"], out["lse_unpacked"] = ou, lu
    do = W.make_dout(wl).to(DEV)
    bprob = psa.make_problem(qd, kd, vd, o, block_q=wl.block_q, block_k=wl.block_k,
                             causal=wl.causal, seq_valid=wl.seq_valid)
    fill()
    out["dq"], out["dk"], out["dv"] = psa.attn_bwd(qd, kd, vd, kp, vp, lm, o, lse, do, bprob)
    if wl.head_dim == 128:
        q8, _, sq = psa.quantize_fp8(qd)
        k8, kp8, sk = psa.quantize_fp8(kd, kp)
        v8, vp8, sv = psa.quantize_fp8(vd, vp)
        fill()
        out["o8qk"], out["lse8qk"] = psa.attn_fwd_fp8qk(q8, sq, k8, kp8, sk, vd, vp, lm, prob)
        fill()
        out["o8"], out["lse8"] = psa.attn_fwd_fp8(q8, sq, k8, kp8, sk, v8, vp8, sv, lm, prob)
    torch.cuda.synchronize()
    assert err.item() == 0
    return out


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_lds_sentinel(wl):
    announce(f"LDS sentinel {wl.name}")
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref = _path(wl, qd, kd, vd, 0)
    for pattern in (NAN, ALL_ONES):
        got = _path(wl, qd, kd, vd, pattern)
        for name, x in ref.items():
            y = got[name]
            if x.dtype.is_floating_point:
                assert not torch.isnan(y).any().item(), f"{name}: NaN after an LDS fill"
            assert torch.equal(x, y), f"{name}: differs after an LDS fill with {pattern:#x}"
