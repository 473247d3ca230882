"""Host-side checks of the C ABI (no GPU): the library loads, exports every function that
include/psa.h declares, and rejects bad arguments with the documented status before touching
the device."""
import ctypes
import os
import re

import pytest
import torch

import video_transformers_amd as psa
from video_transformers_amd import psa as P

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "psa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(psa_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_header_lists_the_binding_exports():
    assert declared_functions() == sorted(psa.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = psa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def _prob(**kw):
    q = torch.zeros(1, 2, 1024, 64)
    p = psa.make_problem(q, q, q, block_q=64)
    for k, v in kw.items():
        setattr(p.c, k, v)
    return p


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, P.PSA_ERR_UNSUPPORTED),
    ("block_k", 32, P.PSA_ERR_UNSUPPORTED),
    ("block_q", 256, P.PSA_ERR_UNSUPPORTED),
    ("dtype", 7, P.PSA_ERR_UNSUPPORTED),
    ("seq_valid", 1020, P.PSA_ERR_UNSUPPORTED),     # padding not a multiple of 8
    ("seq_valid", 2000, P.PSA_ERR_INVALID_ARG),     # beyond seq_len
    ("seq_len", 1088 + 8, P.PSA_ERR_UNSUPPORTED),   # not a multiple of block_q
    ("heads_kv", 3, P.PSA_ERR_INVALID_ARG),         # heads_q % heads_kv
    ("heads_q", 0, P.PSA_ERR_INVALID_ARG),
])
def test_problem_checks(field, value, status):
    p = _prob(**{field: value})
    L = psa.lib()
    assert L.psa_pooled_rows(p.ref()) == -1
    assert L.psa_attn_workspace_bytes(p.ref()) == 0
    dummy = ctypes.c_void_p(256)
    rc = L.psa_attn_fwd(p.ref(), 0.0, dummy, dummy, dummy, dummy, dummy, dummy, dummy, None,
                        dummy, 1 << 20, None)
    assert rc == status
    assert L.psa_build_pyramid(p.ref(), dummy, dummy, dummy, dummy, P.PSA_BF16, None) == status


def test_pyramid_out_dtype_checks():
    """out_dtype: the problem's dtype or float32; a bf16 level of a float32 problem is
    unsupported, anything else is an invalid argument (nothing is launched)."""
    L = psa.lib()
    d = ctypes.c_void_p(256)
    pb = _prob(dtype=P.PSA_BF16)
    pf = _prob(dtype=P.PSA_F32)
    assert L.psa_build_pyramid(pb.ref(), d, d, d, d, 7, None) == P.PSA_ERR_INVALID_ARG
    assert L.psa_build_pyramid(pb.ref(), d, d, d, d, -1, None) == P.PSA_ERR_INVALID_ARG
    assert L.psa_build_pyramid(pf.ref(), d, d, d, d, P.PSA_BF16, None) == P.PSA_ERR_UNSUPPORTED
    assert L.psa_build_pyramid(pb.ref(), None, d, d, d, P.PSA_F32, None) == P.PSA_ERR_INVALID_ARG
    assert L.psa_build_pyramid(pf.ref(), d, d, d, None, P.PSA_F32, None) == P.PSA_ERR_INVALID_ARG


def test_bad_stride_rejected():
    p = _prob()
    p.c.k_stride[2] = 60   # not a multiple of 8
    assert psa.lib().psa_pooled_rows(p.ref()) == -1


def test_null_pointer_and_workspace_checks():
    p = _prob()
    L = psa.lib()
    d = ctypes.c_void_p(256)
    assert L.psa_attn_fwd(p.ref(), 0.0, None, d, d, d, d, d, d, None, d, 1 << 20, None) == P.PSA_ERR_INVALID_ARG
    need = L.psa_attn_workspace_bytes(p.ref())
    assert need > 0
    assert L.psa_attn_fwd(p.ref(), 0.0, d, d, d, d, d, d, d, None, d, need - 1, None) == P.PSA_ERR_WORKSPACE
    assert L.psa_attn_fwd(p.ref(), 0.0, d, d, d, d, d, d, d, None, None, need, None) == P.PSA_ERR_WORKSPACE
    misaligned = ctypes.c_void_p(264)
    assert L.psa_attn_fwd(p.ref(), 0.0, misaligned, d, d, d, d, d, d, None, d, need, None) == P.PSA_ERR_INVALID_ARG
    assert L.psa_build_index(p.ref(), None, d, d, d, None) == P.PSA_ERR_INVALID_ARG
    assert L.psa_check_status(None, None) == P.PSA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(thresholds=(0.5, 0.4, 0.8, 0.9)), P.PSA_ERR_INVALID_ARG),   # decreasing
    (dict(thresholds=(0.0, 0.7, 0.8, 0.9)), P.PSA_ERR_INVALID_ARG),   # t0 <= 0
    (dict(thresholds=(0.5, 0.7, 0.8, 1.5)), P.PSA_ERR_INVALID_ARG),   # > 1
    (dict(samples_per_qblock=0), P.PSA_ERR_INVALID_ARG),
    (dict(samples_per_qblock=65), P.PSA_ERR_INVALID_ARG),             # > block_q (64)
    (dict(samples_per_qblock=12), P.PSA_ERR_UNSUPPORTED),             # not a power of two
    (dict(samples_per_qblock=64), P.PSA_ERR_UNSUPPORTED),             # > 32
    (dict(mode="antidiag", antidiag_stride=3), P.PSA_ERR_UNSUPPORTED),
    (dict(mode="antidiag", antidiag_stride=16), P.PSA_ERR_UNSUPPORTED),
    (dict(force_l0_begin=10, force_l0_end=5000), P.PSA_ERR_INVALID_ARG),
])
def test_mask_param_checks(kw, status):
    p = _prob(dtype=P.PSA_BF16)
    mp = psa.MaskParams(**kw).c()
    L = psa.lib()
    d = ctypes.c_void_p(256)
    assert L.psa_mask_workspace_bytes(p.ref(), ctypes.byref(mp)) == 0
    assert L.psa_mask(p.ref(), ctypes.byref(mp), d, d, d, d, d, d, 1 << 20, None) == status
    assert L.psa_mask_assign(p.ref(), ctypes.byref(mp), d, d, d, None) == status


def test_mask_workspace_per_mode():
    """Every scoring mode is accepted and sizes its workspace: the log-masses (scoring rows x
    blocks, float32; for block means also the query and key means), then the certification
    area: the counters (256 bytes), the flagged-row list, the batches of flagged rows (16 int32
    slots per certifiable row) and the float64 log-masses of the certifiable rows (all 32 rows
    of this small problem: scoring rows per query block x blocks x 8 bytes each), plus the
    float64 similarities when the cosine check is on."""
    p = _prob(dtype=P.PSA_BF16)
    L = psa.lib()
    B, H, Hkv, N, D = 1, 2, 2, 1024, 64   # the _prob() shape
    nqb, nkb = N // 64, N // 64
    R = B * H * nqb
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    sizes = {}
    for mode in ("sampling", "antidiag", "meankey"):
        mp = psa.MaskParams(mode=mode, samples_per_qblock=8, antidiag_stride=8).c()
        sizes[mode] = L.psa_mask_workspace_bytes(p.ref(), ctypes.byref(mp))
    cert = lambda rq: 256 + a256(R * 4) + a256(R * 16 * 4) + R * rq * nkb * 8  # noqa: E731
    assert sizes["sampling"] == a256(B * H * nkb * nqb * 8 * 4) + cert(8)
    assert sizes["antidiag"] == a256(B * H * nkb * (N // 8) * 4) + cert(64 // 8)
    assert sizes["meankey"] >= B * H * nkb * nqb * 4 + B * H * nqb * D * 4 + B * Hkv * nkb * D * 4 + cert(1)
    mp = psa.MaskParams(mode="antidiag", antidiag_stride=8, cos_sim_min=0.8).c()
    assert (L.psa_mask_workspace_bytes(p.ref(), ctypes.byref(mp))
            == sizes["antidiag"] + a256(B * Hkv * nkb * 8))
    with pytest.raises(ValueError):
        psa.MaskParams(mode="bogus").c()


def test_mask_needs_bf16():
    p = _prob()   # float32 problem
    mp = psa.MaskParams().c()
    d = ctypes.c_void_p(256)
    assert psa.lib().psa_mask(p.ref(), ctypes.byref(mp), d, d, d, d, d, d, 0, None) == P.PSA_ERR_UNSUPPORTED


def test_status_strings():
    L = psa.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.psa_status_string(code).startswith(b"PSA_")
    assert L.psa_last_hip_error() == 0


def test_attn_bwd_host_checks():
    L = psa.lib()
    d = ctypes.c_void_p(256)
    args13 = lambda **o: [o.get(n, d) for n in ("q", "k", "v", "kp", "vp", "map", "o", "lse",
                                                 "do", "dq", "dk", "dv", "ws")]
    # f32 problems have no backward
    p32 = _prob()
    need32 = L.psa_attn_bwd_workspace_bytes(p32.ref())
    assert need32 > L.psa_attn_workspace_bytes(p32.ref())
    assert L.psa_attn_bwd(p32.ref(), 0.0, *args13(), need32, None) == P.PSA_ERR_UNSUPPORTED
    p = _prob(dtype=P.PSA_BF16)
    need = L.psa_attn_bwd_workspace_bytes(p.ref())
    # per-row lse2 and D, and the f32 gradients of all N + 7N/8 rows of K and V
    rows, grows = 2 * 1024, 2 * (1024 + 896)
    assert need >= 2 * rows * 4 + 2 * grows * 64 * 4 + L.psa_attn_workspace_bytes(p.ref())
    assert L.psa_attn_bwd(p.ref(), 0.0, *args13(), need - 1, None) == P.PSA_ERR_WORKSPACE
    assert L.psa_attn_bwd(p.ref(), 0.0, *args13(ws=None), need, None) == P.PSA_ERR_WORKSPACE
    for name in ("q", "lse", "do", "dq", "dk", "dv", "map"):
        assert L.psa_attn_bwd(p.ref(), 0.0, *args13(**{name: None}), need, None) == P.PSA_ERR_INVALID_ARG, name
    assert L.psa_attn_bwd(p.ref(), 0.0, *args13(dk=ctypes.c_void_p(264)), need, None) == P.PSA_ERR_INVALID_ARG
    assert L.psa_attn_bwd(p.ref(), float("nan"), *args13(), need, None) == P.PSA_ERR_INVALID_ARG
    # the key-side kernel's row list: at most 7680 (query head, query block) rows per KV head
    big = _prob(dtype=P.PSA_BF16, heads_q=32, heads_kv=1, seq_len=16384, seq_valid=16384)
    assert L.psa_attn_bwd(big.ref(), 0.0, *args13(), 1 << 40, None) == P.PSA_ERR_UNSUPPORTED


def test_quantize_fp8_host_checks():
    L = psa.lib()
    d = ctypes.c_void_p(256)
    st = lambda *v: (ctypes.c_int64 * 3)(*v)
    ok = st(2 * 1024 * 128, 1024 * 128, 128)
    q = lambda B=1, H=2, N=1024, D=128, x=d, s=ok, xp=None, x8=d, x8p=None, sc=d: \
        L.psa_quantize_fp8(B, H, N, D, x, s, xp, x8, x8p, sc, None)
    assert q(H=0) == P.PSA_ERR_INVALID_ARG
    assert q(N=-8) == P.PSA_ERR_INVALID_ARG
    assert q(N=1020) == P.PSA_ERR_UNSUPPORTED          # pooled rows need N % 8 == 0
    assert q(D=100) == P.PSA_ERR_UNSUPPORTED
    assert q(B=300, H=300) == P.PSA_ERR_UNSUPPORTED   # grid y holds the heads
    assert q(s=st(0, 1024 * 128, 128)) == P.PSA_ERR_INVALID_ARG
    assert q(s=st(2 * 1024 * 128, 1024 * 128, 64)) == P.PSA_ERR_INVALID_ARG   # row stride < d
    assert q(x=None) == P.PSA_ERR_INVALID_ARG
    assert q(sc=None) == P.PSA_ERR_INVALID_ARG
    assert q(xp=d) == P.PSA_ERR_INVALID_ARG            # pooled input without pooled output
    assert q(x8p=d) == P.PSA_ERR_INVALID_ARG
    assert q(x=ctypes.c_void_p(264)) == P.PSA_ERR_INVALID_ARG   # 16-byte alignment
    assert q(x8=ctypes.c_void_p(260)) == P.PSA_ERR_INVALID_ARG  # 8-byte alignment
    assert q(sc=ctypes.c_void_p(258)) == P.PSA_ERR_INVALID_ARG


def test_attn_fwd_fp8qk_host_checks():
    L = psa.lib()
    d = ctypes.c_void_p(256)
    args11 = lambda **o: [o.get(n, d) for n in ("q8", "qs", "k8", "kp8", "ks", "v", "vp", "map",
                                                 "o", "lse", "ws")]
    q = torch.zeros(1, 2, 1024, 128)
    p = psa.make_problem(q, q, q, block_q=64)
    p.c.dtype = P.PSA_BF16
    need = L.psa_attn_workspace_bytes(p.ref())
    call = lambda prob, n=need, sc=0.0, **o: L.psa_attn_fwd_fp8qk(prob.ref(), sc, *args11(**o), n, None)
    assert call(p, n=need - 1) == P.PSA_ERR_WORKSPACE
    assert call(p, ws=None) == P.PSA_ERR_WORKSPACE
    for name in ("q8", "qs", "k8", "kp8", "ks", "v", "vp", "map", "o"):
        assert call(p, **{name: None}) == P.PSA_ERR_INVALID_ARG, name
    assert call(p, k8=ctypes.c_void_p(264)) == P.PSA_ERR_INVALID_ARG
    assert call(p, sc=float("inf")) == P.PSA_ERR_INVALID_ARG
    p.c.dtype = P.PSA_F32
    assert call(p) == P.PSA_ERR_UNSUPPORTED
    p64 = _prob(dtype=P.PSA_BF16)                      # head_dim 64: no fp8 kernel
    assert call(p64, n=1 << 30) == P.PSA_ERR_UNSUPPORTED


def test_attn_fwd_fp8_host_checks():
    L = psa.lib()
    d = ctypes.c_void_p(256)
    names = ("q8", "qs", "k8", "kp8", "ks", "v8", "vp8", "vs", "map", "o", "lse", "ws")
    args = lambda **o: [o.get(n, d) for n in names]
    q = torch.zeros(1, 2, 1024, 128)
    p = psa.make_problem(q, q, q, block_q=64)
    p.c.dtype = P.PSA_BF16
    need = L.psa_attn_workspace_bytes(p.ref())
    call = lambda prob, n=need, sc=0.0, **o: L.psa_attn_fwd_fp8(prob.ref(), sc, *args(**o), n, None)
    assert call(p, n=need - 1) == P.PSA_ERR_WORKSPACE
    assert call(p, ws=None) == P.PSA_ERR_WORKSPACE
    for name in ("q8", "qs", "k8", "kp8", "ks", "v8", "vp8", "vs", "map", "o"):
        assert call(p, **{name: None}) == P.PSA_ERR_INVALID_ARG, name
    assert call(p, v8=ctypes.c_void_p(264)) == P.PSA_ERR_INVALID_ARG
    assert call(p, vs=ctypes.c_void_p(258)) == P.PSA_ERR_INVALID_ARG
    assert call(p, sc=float("nan")) == P.PSA_ERR_INVALID_ARG
    p.c.dtype = P.PSA_F32
    assert call(p) == P.PSA_ERR_UNSUPPORTED
    assert call(_prob(dtype=P.PSA_BF16), n=1 << 30) == P.PSA_ERR_UNSUPPORTED   # head_dim 64


@pytest.mark.parametrize("field,value", [("batch", 0), ("seq_len", 0)])
def test_empty_problems_do_nothing(field, value):
    """No batch or no tokens: every call returns PSA_OK without touching its (null) pointers."""
    L = psa.lib()
    q = torch.zeros(1, 2, 1024, 128)
    p = psa.make_problem(q, q, q, block_q=128)
    p.c.dtype = P.PSA_BF16
    setattr(p.c, field, value)
    if field == "seq_len":
        p.c.seq_valid = 0
    n = None
    mp = psa.MaskParams().c()
    assert L.psa_build_pyramid(p.ref(), n, n, n, n, P.PSA_BF16, n) == P.PSA_OK
    assert L.psa_mask(p.ref(), ctypes.byref(mp), n, n, n, n, n, n, 0, n) == P.PSA_OK
    assert L.psa_mask_assign(p.ref(), ctypes.byref(mp), n, n, n, n) == P.PSA_OK
    assert L.psa_build_index(p.ref(), n, n, n, n, n) == P.PSA_OK
    assert L.psa_attn_fwd(p.ref(), 0.0, *[n] * 9, 0, n) == P.PSA_OK
    assert L.psa_attn_fwd_indexed(p.ref(), 0.0, *[n] * 10) == P.PSA_OK
    assert L.psa_attn_fwd_unpacked(p.ref(), 0.0, *[n] * 10) == P.PSA_OK
    assert L.psa_attn_bwd(p.ref(), 0.0, *[n] * 13, 0, n) == P.PSA_OK
    assert L.psa_attn_fwd_fp8qk(p.ref(), 0.0, *[n] * 11, 0, n) == P.PSA_OK
    assert L.psa_attn_fwd_fp8(p.ref(), 0.0, *[n] * 12, 0, n) == P.PSA_OK
    mk = psa.MaskParams(mode="meankey").c()
    assert L.psa_attn_fwd_meankey(p.ref(), ctypes.byref(mk), 0.0, *[n] * 10, 0, n) == P.PSA_OK
    if field == "batch":
        st = (ctypes.c_int64 * 3)(2 * 1024 * 128, 1024 * 128, 128)
        assert L.psa_quantize_fp8(0, 2, 1024, 128, n, st, n, n, n, n, n) == P.PSA_OK


def test_attn_fwd_meankey_host_checks():
    L = psa.lib()
    d = ctypes.c_void_p(256)
    q = torch.zeros(1, 2, 1024, 128)
    p = psa.make_problem(q, q, q, block_q=128)
    p.c.dtype = P.PSA_BF16
    need = L.psa_attn_fwd_meankey_workspace_bytes(p.ref())
    # query and key block means, block similarities
    assert need >= (2 * 8 * 128 + 16 * 128 + 16) * 4
    mk = psa.MaskParams(mode="meankey").c()
    call = lambda prob, params=mk, n=need, sc=0.0, **o: L.psa_attn_fwd_meankey(
        prob.ref(), ctypes.byref(params), sc,
        *[o.get(x, d) for x in ("q", "k", "v", "kp", "vp", "map", "mass", "o", "lse", "ws")], n, None)
    assert call(p, n=need - 1) == P.PSA_ERR_WORKSPACE
    assert call(p, ws=None) == P.PSA_ERR_WORKSPACE
    for name in ("q", "k", "v", "kp", "vp", "o"):
        assert call(p, **{name: None}) == P.PSA_ERR_INVALID_ARG, name
    assert call(p, params=psa.MaskParams(mode="sampling").c()) == P.PSA_ERR_INVALID_ARG
    assert call(p, sc=float("inf")) == P.PSA_ERR_INVALID_ARG
    p64 = psa.make_problem(q, q, q, block_q=64)
    p64.c.dtype = P.PSA_BF16
    assert call(p64, n=1 << 30) == P.PSA_ERR_UNSUPPORTED          # block_q 64
    big = psa.make_problem(torch.zeros(1, 1, 64 * 1800, 64), torch.zeros(1, 1, 64 * 1800, 64),
                           torch.zeros(1, 1, 64 * 1800, 64), block_q=128)
    big.c.dtype = P.PSA_BF16
    assert call(big, n=1 << 40) == P.PSA_ERR_UNSUPPORTED          # more than 1792 KV blocks
    p.c.dtype = P.PSA_F32
    assert call(p, n=1 << 30) == P.PSA_ERR_UNSUPPORTED


def _big(nkb, block_q=128):
    q = torch.zeros(1, 1, 64, 128)
    p = psa.make_problem(q, q, q, block_q=64)
    p.c.seq_len = p.c.seq_valid = nkb * 64
    p.c.block_q = block_q
    for st in (p.c.q_stride, p.c.k_stride, p.c.v_stride, p.c.o_stride):
        st[0] = st[1] = nkb * 64 * 128
        st[2] = 128
    p.c.dtype = P.PSA_BF16
    return p


# sampling, 8 samples: 8 * 2048 + 37 * NKB <= 65536 up to NKB = 1328 (block_q 64 keeps every
# NKB a whole number of query blocks); antidiagonal, stride 8, block_q 128 (16 scoring rows):
# 8 * 1024 + 69 * NKB <= 65536 up to NKB = 831, i.e. 830 with whole 128-token query blocks
@pytest.mark.parametrize("mode,nkb,bq,ok", [("sampling", 1328, 64, True), ("sampling", 1329, 64, False),
                                            ("antidiag", 830, 128, True), ("antidiag", 832, 128, False)])
def test_mask_assignment_lds_limit(mode, nkb, bq, ok):
    """psa_mask refuses, before enqueueing anything, a problem whose per-row assignment would
    not fit 64 KB of LDS (sort keys, masses, staged log-masses, levels)."""
    p = _big(nkb, bq)
    mp = psa.MaskParams(mode=mode).c()
    L = psa.lib()
    d = ctypes.c_void_p(256)
    rc = L.psa_mask(p.ref(), ctypes.byref(mp), d, d, d, d, d, d, 0, None)
    # within the limit the call gets as far as the workspace check (none given)
    assert rc == (P.PSA_ERR_WORKSPACE if ok else P.PSA_ERR_UNSUPPORTED)


def test_attention_block_limit():
    """The attention calls refuse seq_len/64 > 16384 (a row's block list is staged in LDS)."""
    L = psa.lib()
    d = ctypes.c_void_p(256)
    for nkb, want in ((16385, P.PSA_ERR_UNSUPPORTED), (16384, P.PSA_ERR_WORKSPACE)):
        p = _big(nkb)
        assert L.psa_attn_fwd(p.ref(), 0.0, d, d, d, d, d, d, d, None, d, 0, None) == want


def test_noalloc_host_checks():
    """The allocation-free attention: the fixed scratch's size, a problem whose block index does
    not fit it (PSA_ERR_SCRATCH), a missing output or error word (PSA_ERR_INVALID_ARG), an empty
    problem (PSA_OK); nothing is launched in any of these."""
    L = psa.lib()
    cap = L.psa_attn_fwd_noalloc_max_bytes()
    assert cap == 128 << 20
    d = ctypes.c_void_p(256)
    p = _prob(dtype=P.PSA_BF16)
    assert L.psa_attn_fwd_noalloc(p.ref(), 0.0, d, d, d, d, d, d, d, None, None, None) == P.PSA_ERR_INVALID_ARG
    assert L.psa_attn_fwd_noalloc(p.ref(), 0.0, d, d, d, d, d, d, None, None, d, None) == P.PSA_ERR_INVALID_ARG
    # 40 heads x 1024 query blocks x 2048 KV blocks: a 335 MB index
    big = torch.zeros(1, 40, 131072, 64)
    pb = psa.make_problem(big, big, big, block_q=128)
    pb.c.dtype = P.PSA_BF16
    assert L.psa_attn_fwd_noalloc(pb.ref(), 0.0, d, d, d, d, d, d, d, None, d, None) == P.PSA_ERR_SCRATCH
    pe = _prob(dtype=P.PSA_BF16)
    pe.c.batch = 0
    n = None
    assert L.psa_attn_fwd_noalloc(pe.ref(), 0.0, *[n] * 9, n) == P.PSA_OK
    assert b"SCRATCH" in L.psa_status_string(P.PSA_ERR_SCRATCH)
