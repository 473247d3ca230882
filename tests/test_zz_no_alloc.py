"""The allocation-free attention entry point (psa_attn_fwd_noalloc), through the C ABI, against
the existing entry point (psa_attn_fwd, which builds its block index in a caller workspace):
two calls in a row on one GPU, the second on a smaller problem than the first, each compared
with psa_attn_fwd on the same inputs bit for bit (the same kernels run on the same index; the
bar is exact equality, stricter than the attention's float bars). The second call's index
overwrites the first's in the shared scratch, so any state carried from the first call would
show. Also: an invalid map entry sets the caller's error word."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
import video_transformers_amd as psa
from gpu_util import DEV, announce, need_gpu, oracle_map, problem_for

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _case(wl):
    q, k, v = W.make_qkv(wl)
    lm = torch.from_numpy(oracle_map(wl, q, k)).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    prob = problem_for(wl, qd, kd, vd)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    return qd, kd, vd, kp, vp, lm, prob


def _noalloc(qd, kd, vd, kp, vp, lm, prob):
    """One call through the C ABI; every output preallocated here, none by the library."""
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=DEV)
    err = torch.full((1,), 123, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = psa.lib().psa_attn_fwd_noalloc(prob.ref(), ctypes.c_float(0.0), ptr(qd), ptr(kd), ptr(vd),
                                        ptr(kp), ptr(vp), ptr(lm), ptr(o), ptr(lse), ptr(err), st)
    assert rc == 0, psa.lib().psa_status_string(rc)
    torch.cuda.synchronize()
    return o, lse, int(err.item())


def test_noalloc_matches_attn_fwd_then_smaller():
    big = W.small(W.WAN14B_720P_75K)                  # 2 heads x 4096 tokens, drawn map
    small = W.small(W.QWEN25VL_32K).replace(seq_len=1024, seq_valid=1016)   # GQA, causal
    assert big.heads_q * big.n_qblocks * big.n_kblocks > small.heads_q * small.n_qblocks * small.n_kblocks
    for wl in (big, small):
        announce(f"allocation-free attention {wl.name}: H{wl.heads_q}/{wl.heads_kv} N{wl.seq_len}")
        qd, kd, vd, kp, vp, lm, prob = _case(wl)
        o, lse, err = _noalloc(qd, kd, vd, kp, vp, lm, prob)
        o_ref, lse_ref = psa.attn_fwd(qd, kd, vd, kp, vp, lm, prob)
        torch.cuda.synchronize()
        assert err == 0
        assert torch.equal(o, o_ref), "o differs from psa_attn_fwd's"
        assert torch.equal(lse, lse_ref), "lse differs from psa_attn_fwd's"


def test_noalloc_reports_bad_map_entry():
    wl = W.small(W.WAN13B_32K)
    announce("allocation-free attention, an invalid map entry")
    qd, kd, vd, kp, vp, lm, prob = _case(wl)
    lm[0, 0, 1, 3] = 7
    _, _, err = _noalloc(qd, kd, vd, kp, vp, lm, prob)
    assert err == psa.psa.PSA_ERR_BAD_LEVEL_MAP
    lm[0, 0, 1, 3] = 0
    _, _, err = _noalloc(qd, kd, vd, kp, vp, lm, prob)
    assert err == 0
