"""Thin ctypes binding of libpsa (include/psa.h): argument marshalling only.

Every step of the Pyramid Sparse Attention forward path runs in the library's HIP kernels;
torch supplies device memory and the current HIP stream and nothing else. If the library is
not built, every entry point raises (there is no fallback).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PSA_LIBRARY selects another build of the same library (the host-sanitized one the CPU tests
# run the argument checks under); by default the in-tree libpsa.so.
LIB_PATH = os.environ.get("PSA_LIBRARY") or os.path.join(_HERE, "libpsa.so")

PSA_OK = 0
PSA_ERR_INVALID_ARG = -1
PSA_ERR_UNSUPPORTED = -2
PSA_ERR_WORKSPACE = -3
PSA_ERR_HIP = -4
PSA_ERR_BAD_LEVEL_MAP = -5
PSA_ERR_SCRATCH = -6
PSA_F32 = 0
PSA_BF16 = 1
PSA_MASK_SAMPLING = 0
PSA_MASK_ANTIDIAG = 1
PSA_MASK_MEANKEY = 2
_MODES = {"sampling": PSA_MASK_SAMPLING, "antidiag": PSA_MASK_ANTIDIAG, "meankey": PSA_MASK_MEANKEY}
SKIP = -1

# every symbol include/psa.h declares
EXPORTS = ("psa_pooled_rows", "psa_build_pyramid", "psa_mask_workspace_bytes", "psa_mask",
           "psa_mask_assign", "psa_mask_certified_rows", "psa_build_index", "psa_attn_workspace_bytes", "psa_attn_fwd",
           "psa_attn_fwd_indexed", "psa_attn_fwd_unpacked", "psa_attn_bwd_workspace_bytes",
           "psa_attn_bwd", "psa_quantize_fp8", "psa_attn_fwd_fp8qk", "psa_attn_fwd_fp8",
           "psa_attn_fwd_meankey_workspace_bytes", "psa_attn_fwd_meankey", "psa_check_status",
           "psa_status_string", "psa_last_hip_error", "psa_debug_fill_lds",
           "psa_attn_fwd_noalloc", "psa_attn_fwd_noalloc_max_bytes")


class PsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().psa_status_string(status).decode()
        if status == PSA_ERR_HIP:
            msg += f" (hipError_t {lib().psa_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


class CProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
                ("heads_kv", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("seq_valid", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3)]


class CMaskParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("thresholds", ctypes.c_float * 4),
                ("samples_per_qblock", ctypes.c_int32), ("antidiag_stride", ctypes.c_int32),
                ("cos_sim_min", ctypes.c_float), ("force_diag_l0", ctypes.c_int32),
                ("force_l0_begin", ctypes.c_int32), ("force_l0_end", ctypes.c_int32)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Loads libpsa.so once (after torch, so both bind the same HIP runtime)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m video_transformers_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, V, I32, I64, SZ = (ctypes.POINTER(CProblem), ctypes.c_void_p, ctypes.c_int,
                              ctypes.c_int64, ctypes.c_size_t)
        MP = ctypes.POINTER(CMaskParams)
        L.psa_pooled_rows.argtypes, L.psa_pooled_rows.restype = [P], I64
        L.psa_build_pyramid.argtypes, L.psa_build_pyramid.restype = [P, V, V, V, V, I32, V], I32
        L.psa_mask_workspace_bytes.argtypes, L.psa_mask_workspace_bytes.restype = [P, MP], SZ
        L.psa_mask.argtypes, L.psa_mask.restype = [P, MP, V, V, V, V, V, V, SZ, V], I32
        L.psa_mask_assign.argtypes, L.psa_mask_assign.restype = [P, MP, V, V, V, V], I32
        L.psa_mask_certified_rows.argtypes = [P, MP, V, ctypes.POINTER(I32), V]
        L.psa_mask_certified_rows.restype = I32
        L.psa_build_index.argtypes, L.psa_build_index.restype = [P, V, V, V, V, V], I32
        L.psa_attn_workspace_bytes.argtypes, L.psa_attn_workspace_bytes.restype = [P], SZ
        L.psa_attn_fwd.argtypes = [P, ctypes.c_float, V, V, V, V, V, V, V, V, V, SZ, V]
        L.psa_attn_fwd.restype = I32
        L.psa_attn_fwd_indexed.argtypes = [P, ctypes.c_float, V, V, V, V, V, V, V, V, V, V]
        L.psa_attn_fwd_indexed.restype = I32
        L.psa_attn_fwd_unpacked.argtypes = [P, ctypes.c_float, V, V, V, V, V, V, V, V, V, V]
        L.psa_attn_fwd_unpacked.restype = I32
        L.psa_attn_bwd_workspace_bytes.argtypes = [P]
        L.psa_attn_bwd_workspace_bytes.restype = SZ
        L.psa_attn_bwd.argtypes = [P, ctypes.c_float] + [V] * 13 + [SZ, V]
        L.psa_attn_bwd.restype = I32
        L.psa_quantize_fp8.argtypes = [I32, I32, I32, I32, V, ctypes.POINTER(I64), V, V, V, V, V]
        L.psa_quantize_fp8.restype = I32
        L.psa_attn_fwd_fp8qk.argtypes = [P, ctypes.c_float] + [V] * 11 + [SZ, V]
        L.psa_attn_fwd_fp8qk.restype = I32
        L.psa_attn_fwd_fp8.argtypes = [P, ctypes.c_float] + [V] * 12 + [SZ, V]
        L.psa_attn_fwd_fp8.restype = I32
        L.psa_attn_fwd_meankey_workspace_bytes.argtypes = [P]
        L.psa_attn_fwd_meankey_workspace_bytes.restype = SZ
        L.psa_attn_fwd_meankey.argtypes = [P, MP, ctypes.c_float] + [V] * 10 + [SZ, V]
        L.psa_attn_fwd_meankey.restype = I32
        L.psa_check_status.argtypes, L.psa_check_status.restype = [V, V], I32
        L.psa_status_string.argtypes, L.psa_status_string.restype = [I32], ctypes.c_char_p
        L.psa_last_hip_error.argtypes, L.psa_last_hip_error.restype = [], I32
        L.psa_debug_fill_lds.argtypes, L.psa_debug_fill_lds.restype = [ctypes.c_uint32, V], I32
        L.psa_attn_fwd_noalloc.argtypes = [P, ctypes.c_float] + [V] * 9 + [V]
        L.psa_attn_fwd_noalloc.restype = I32
        L.psa_attn_fwd_noalloc_max_bytes.argtypes, L.psa_attn_fwd_noalloc_max_bytes.restype = [], SZ
        _LIB = L
    return _LIB


def _check(rc: int, where: str) -> None:
    if rc != PSA_OK:
        raise PsaError(rc, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return PSA_BF16
    if dt == torch.float32:
        return PSA_F32
    raise TypeError(f"unsupported dtype {dt}")


@dataclasses.dataclass
class Problem:
    """A psa_problem built from Q [B,H,N,d], K/V [B,Hkv,N,d] (and O) tensors."""
    c: CProblem

    @property
    def n_qblocks(self) -> int:
        return self.c.seq_len // self.c.block_q

    @property
    def n_kblocks(self) -> int:
        return self.c.seq_len // self.c.block_k

    def ref(self):
        return ctypes.byref(self.c)


def make_problem(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 o: Optional[torch.Tensor] = None, *, block_q: int, block_k: int = 64,
                 causal: bool = False, seq_valid: Optional[int] = None) -> Problem:
    for name, t in (("q", q), ("k", k), ("v", v)) + ((("o", o),) if o is not None else ()):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be [batch, heads, tokens, head_dim] with a contiguous head_dim")
    B, H, N, d = q.shape
    o = q if o is None else o
    c = CProblem()
    c.batch, c.heads_q, c.heads_kv, c.seq_len = B, H, k.shape[1], N
    c.seq_valid = N if seq_valid is None else int(seq_valid)
    c.head_dim, c.block_q, c.block_k = d, block_q, block_k
    c.causal = 1 if causal else 0
    c.dtype = _dtype_code(q.dtype)
    for arr, t in ((c.q_stride, q), (c.k_stride, k), (c.v_stride, v), (c.o_stride, o)):
        arr[0], arr[1], arr[2] = t.stride(0), t.stride(1), t.stride(2)
    return Problem(c)


@dataclasses.dataclass
class MaskParams:
    mode: str = "sampling"                 # "sampling" | "antidiag" | "meankey"
    thresholds: Sequence[float] = (0.5, 0.7, 0.8, 0.9)
    samples_per_qblock: int = 8
    antidiag_stride: int = 8
    cos_sim_min: float = 0.0
    force_diag_l0: bool = False
    force_l0_begin: int = 0
    force_l0_end: int = 0

    def c(self) -> CMaskParams:
        m = CMaskParams()
        if self.mode not in _MODES:
            raise ValueError(f"unknown mask mode {self.mode!r}")
        m.mode = _MODES[self.mode]
        for i, t in enumerate(self.thresholds):
            m.thresholds[i] = float(t)
        m.samples_per_qblock = self.samples_per_qblock
        m.antidiag_stride = self.antidiag_stride
        m.cos_sim_min = float(self.cos_sim_min)
        m.force_diag_l0 = 1 if self.force_diag_l0 else 0
        m.force_l0_begin = self.force_l0_begin
        m.force_l0_end = self.force_l0_end
        return m


def pooled_rows(prob: Problem) -> int:
    n = lib().psa_pooled_rows(prob.ref())
    if n < 0:
        raise PsaError(PSA_ERR_INVALID_ARG, "psa_pooled_rows")
    return n


def build_pyramid(k: torch.Tensor, v: torch.Tensor, prob: Problem,
                  out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None, stream=None,
                  out_dtype: Optional[torch.dtype] = None):
    """Levels 1..3 of K and V packed as [B, Hkv, 7N/8, d] (level l at row N - 2N/2^l), in
    `out_dtype` (default: the input dtype; torch.float32 gives the unrounded levels)."""
    B, Hkv, _, d = k.shape
    if out is None:
        dt = k.dtype if out_dtype is None else out_dtype
        shape = (B, Hkv, pooled_rows(prob), d)
        out = (torch.empty(shape, dtype=dt, device=k.device),
               torch.empty(shape, dtype=dt, device=v.device))
    kp, vp = out
    _check(lib().psa_build_pyramid(prob.ref(), _ptr(k), _ptr(v), _ptr(kp), _ptr(vp),
                                   _dtype_code(kp.dtype), _stream(stream)), "psa_build_pyramid")
    return kp, vp


def mask(q: torch.Tensor, k: torch.Tensor, prob: Problem, params: MaskParams, stream=None,
         cert_counts: Optional[list] = None):
    """Returns (level_map int8 [B,H,NQB,NKB], block_mass f32 [B,H,NQB,NKB], block_sim or None).
    With a list `cert_counts`, the call's certification counters are appended to it (rows
    rescored in float64, flagged rows left uncertified); reading them synchronizes the stream."""
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    nqb, nkb = prob.n_qblocks, prob.n_kblocks
    cp = params.c()
    lm = torch.empty((B, H, nqb, nkb), dtype=torch.int8, device=q.device)
    mass = torch.empty((B, H, nqb, nkb), dtype=torch.float32, device=q.device)
    sim = (torch.empty((B, Hkv, nkb), dtype=torch.float32, device=q.device)
           if params.cos_sim_min > 0 else None)
    nbytes = lib().psa_mask_workspace_bytes(prob.ref(), ctypes.byref(cp))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().psa_mask(prob.ref(), ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(lm), _ptr(mass),
                          _ptr(sim), _ptr(ws), nbytes, _stream(stream)), "psa_mask")
    if cert_counts is not None:
        c = (ctypes.c_int32 * 2)()
        _check(lib().psa_mask_certified_rows(prob.ref(), ctypes.byref(cp), _ptr(ws), c,
                                             _stream(stream)), "psa_mask_certified_rows")
        cert_counts.extend([int(c[0]), int(c[1])])
    return lm, mass, sim


def mask_assign(block_mass: torch.Tensor, block_sim: Optional[torch.Tensor], prob: Problem,
                params: MaskParams, stream=None) -> torch.Tensor:
    cp = params.c()
    lm = torch.empty(block_mass.shape, dtype=torch.int8, device=block_mass.device)
    _check(lib().psa_mask_assign(prob.ref(), ctypes.byref(cp), _ptr(block_mass), _ptr(block_sim),
                                 _ptr(lm), _stream(stream)), "psa_mask_assign")
    return lm


def build_index(level_map: torch.Tensor, prob: Problem, stream=None):
    """Returns (row_ptr int32 [R*5+1]: the CSR offsets [R*4+1] then the attention's dispatch
    order [R], col_idx int32 [R*NKB] (prefix valid), dev_err int32 [1])."""
    rows = level_map.numel() // prob.n_kblocks
    dev = level_map.device
    row_ptr = torch.empty(rows * 5 + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(rows * prob.n_kblocks, 1), dtype=torch.int32, device=dev)
    dev_err = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().psa_build_index(prob.ref(), _ptr(level_map), _ptr(row_ptr), _ptr(col_idx),
                                 _ptr(dev_err), _stream(stream)), "psa_build_index")
    return row_ptr, col_idx, dev_err


def attn_workspace(prob: Problem, device) -> torch.Tensor:
    n = lib().psa_attn_workspace_bytes(prob.ref())
    if n == 0:
        raise PsaError(PSA_ERR_INVALID_ARG, "psa_attn_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_fwd(q, k, v, k_pooled, v_pooled, level_map, prob: Problem, *, scale: float = 0.0,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             want_lse: bool = True, ws: Optional[torch.Tensor] = None, stream=None):
    """Level-weighted attention. Returns (o, lse or None). `out` must match the problem's
    o_stride (make_problem(..., o=out)); by default o is allocated with q's strides."""
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if ws is None:
        ws = attn_workspace(prob, q.device)
    _check(lib().psa_attn_fwd(prob.ref(), ctypes.c_float(scale), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(k_pooled), _ptr(v_pooled), _ptr(level_map), _ptr(out),
                              _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)), "psa_attn_fwd")
    return out, lse


def attn_fwd_indexed(q, k, v, k_pooled, v_pooled, row_ptr, col_idx, prob: Problem, *,
                     scale: float = 0.0, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_lse: bool = True, stream=None):
    """attn_fwd on an index from build_index. Returns (o, lse or None)."""
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check(lib().psa_attn_fwd_indexed(prob.ref(), ctypes.c_float(scale), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(k_pooled), _ptr(v_pooled), _ptr(row_ptr),
                                      _ptr(col_idx), _ptr(out), _ptr(lse), _stream(stream)),
           "psa_attn_fwd_indexed")
    return out, lse


def attn_fwd_unpacked(q, k, v, k_pooled, v_pooled, row_ptr, col_idx, prob: Problem, *,
                      scale: float = 0.0, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, want_lse: bool = True, stream=None):
    """attn_fwd_indexed with one logical block per hardware tile (the ablation baseline of the
    block-tile packing). Returns (o, lse or None)."""
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check(lib().psa_attn_fwd_unpacked(prob.ref(), ctypes.c_float(scale), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(k_pooled), _ptr(v_pooled), _ptr(row_ptr),
                                       _ptr(col_idx), _ptr(out), _ptr(lse), _stream(stream)),
           "psa_attn_fwd_unpacked")
    return out, lse


def attn_bwd_workspace(prob: Problem, device) -> torch.Tensor:
    n = lib().psa_attn_bwd_workspace_bytes(prob.ref())
    if n == 0:
        raise PsaError(PSA_ERR_INVALID_ARG, "psa_attn_bwd_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_bwd(q, k, v, k_pooled, v_pooled, level_map, o, lse, dout, prob: Problem, *,
             scale: float = 0.0, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None, stream=None):
    """Backward of attn_fwd: returns (dq, dk, dv). o and dout share the problem's o_stride
    (make_problem(..., o=o)); dq/dk/dv default to q's/k's/v's strides."""
    if dout.stride() != o.stride():
        raise ValueError("dout must have the same strides as o")
    if dq is None:
        dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if dk is None:
        dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    if dv is None:
        dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device)
    if ws is None:
        ws = attn_bwd_workspace(prob, q.device)
    _check(lib().psa_attn_bwd(prob.ref(), ctypes.c_float(scale), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(k_pooled), _ptr(v_pooled), _ptr(level_map), _ptr(o),
                              _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                              ws.numel(), _stream(stream)), "psa_attn_bwd")
    return dq, dk, dv


def quantize_fp8(x: torch.Tensor, x_pooled: Optional[torch.Tensor] = None, stream=None):
    """Per-head e4m3 codes of a bf16 [B, Hx, N, d] tensor (and of its packed pooled rows, same
    scale). Returns (x8 [B,Hx,N,d] uint8, x8_pooled or None, scale [B*Hx] float32); the codes
    view as torch.float8_e4m3fn."""
    if x.dtype != torch.bfloat16 or x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("x must be bf16 [B, Hx, N, d] with a contiguous last axis")
    B, Hx, N, d = x.shape
    x8 = torch.empty((B, Hx, N, d), dtype=torch.uint8, device=x.device)
    x8p = None
    if x_pooled is not None:
        if x_pooled.dtype != torch.bfloat16 or not x_pooled.is_contiguous():
            raise ValueError("x_pooled must be contiguous bf16")
        x8p = torch.empty(x_pooled.shape, dtype=torch.uint8, device=x.device)
    scale = torch.empty(B * Hx, dtype=torch.float32, device=x.device)
    st = (ctypes.c_int64 * 3)(*x.stride()[:3])
    _check(lib().psa_quantize_fp8(B, Hx, N, d, _ptr(x), st, _ptr(x_pooled), _ptr(x8), _ptr(x8p),
                                  _ptr(scale), _stream(stream)), "psa_quantize_fp8")
    return x8, x8p, scale


def attn_fwd_fp8qk(q8, q_scale, k8, k8_pooled, k_scale, v, v_pooled, level_map, prob: Problem, *,
                   scale: float = 0.0, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                   ws: Optional[torch.Tensor] = None, stream=None):
    """attn_fwd with the q . k products on e4m3 operands from quantize_fp8 (q8, k8, k8_pooled
    contiguous uint8). `prob` is the bf16 problem of Q, K, V (its o_stride applies to out).
    Returns (o, lse or None)."""
    for t in (q8, k8, k8_pooled):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("q8, k8, k8_pooled must be contiguous uint8 codes")
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    if lse is None and want_lse:
        lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    if ws is None:
        ws = attn_workspace(prob, q8.device)
    _check(lib().psa_attn_fwd_fp8qk(prob.ref(), ctypes.c_float(scale), _ptr(q8), _ptr(q_scale),
                                    _ptr(k8), _ptr(k8_pooled), _ptr(k_scale), _ptr(v),
                                    _ptr(v_pooled), _ptr(level_map), _ptr(out), _ptr(lse),
                                    _ptr(ws), ws.numel(), _stream(stream)), "psa_attn_fwd_fp8qk")
    return out, lse


def attn_fwd_fp8(q8, q_scale, k8, k8_pooled, k_scale, v8, v8_pooled, v_scale, level_map,
                 prob: Problem, *, scale: float = 0.0, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                 ws: Optional[torch.Tensor] = None, stream=None):
    """attn_fwd_fp8qk with the P V product on e4m3 operands too (v8, v8_pooled from
    quantize_fp8 of V and its pooled rows). Returns (o, lse or None)."""
    for t in (q8, k8, k8_pooled, v8, v8_pooled):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("q8, k8, k8_pooled, v8, v8_pooled must be contiguous uint8 codes")
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    if lse is None and want_lse:
        lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    if ws is None:
        ws = attn_workspace(prob, q8.device)
    _check(lib().psa_attn_fwd_fp8(prob.ref(), ctypes.c_float(scale), _ptr(q8), _ptr(q_scale),
                                  _ptr(k8), _ptr(k8_pooled), _ptr(k_scale), _ptr(v8),
                                  _ptr(v8_pooled), _ptr(v_scale), _ptr(level_map), _ptr(out),
                                  _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)), "psa_attn_fwd_fp8")
    return out, lse


def attn_fwd_meankey(q, k, v, k_pooled, v_pooled, prob: Problem, params: MaskParams, *,
                     scale: float = 0.0, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_map: bool = True,
                     want_mass: bool = False, ws: Optional[torch.Tensor] = None, stream=None):
    """Block-mean scoring fused into the attention (params.mode must be "meankey"). Returns
    (o, lse, level_map or None, block_mass or None)."""
    dev = q.device
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=dev)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    shape = (q.shape[0], q.shape[1], prob.n_qblocks, prob.n_kblocks)
    lm = torch.empty(shape, dtype=torch.int8, device=dev) if want_map else None
    mass = torch.empty(shape, dtype=torch.float32, device=dev) if want_mass else None
    if ws is None:
        n = lib().psa_attn_fwd_meankey_workspace_bytes(prob.ref())
        if n == 0:
            raise PsaError(PSA_ERR_INVALID_ARG, "psa_attn_fwd_meankey_workspace_bytes")
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
    cp = params.c()
    _check(lib().psa_attn_fwd_meankey(prob.ref(), ctypes.byref(cp), ctypes.c_float(scale), _ptr(q),
                                      _ptr(k), _ptr(v), _ptr(k_pooled), _ptr(v_pooled), _ptr(lm),
                                      _ptr(mass), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                      _stream(stream)), "psa_attn_fwd_meankey")
    return out, lse, lm, mass


def check_status(ws: torch.Tensor, stream=None) -> None:
    _check(lib().psa_check_status(_ptr(ws), _stream(stream)), "psa_check_status")


def forward(q, k, v, *, block_q: int, params: MaskParams, causal: bool = False,
            seq_valid: Optional[int] = None, scale: float = 0.0):
    """The whole path: pyramid, mask, attention. Returns (o, lse, level_map)."""
    prob = make_problem(q, k, v, block_q=block_q, causal=causal, seq_valid=seq_valid)
    kp, vp = build_pyramid(k, v, prob)
    lm, _, _ = mask(q, k, prob, params)
    o, lse = attn_fwd(q, k, v, kp, vp, lm, prob, scale=scale)
    return o, lse, lm


def debug_fill_lds(pattern: int, stream=None) -> None:
    """Diagnostics: fill every CU's LDS with the 32-bit `pattern` on the stream."""
    _check(lib().psa_debug_fill_lds(ctypes.c_uint32(pattern & 0xffffffff), _stream(stream)),
           "psa_debug_fill_lds")


def attn_fwd_noalloc(q, k, v, k_pooled, v_pooled, level_map, prob: Problem, *, scale: float = 0.0,
                     out: torch.Tensor, lse: Optional[torch.Tensor], dev_err: torch.Tensor,
                     stream=None) -> None:
    """psa_attn_fwd without a workspace: the block index lives in the library's fixed per-GPU
    scratch array. Every output (o, lse, the int32 device error word) is caller-provided; the
    call allocates nothing."""
    _check(lib().psa_attn_fwd_noalloc(prob.ref(), ctypes.c_float(scale), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(k_pooled), _ptr(v_pooled), _ptr(level_map), _ptr(out),
                                      _ptr(lse), _ptr(dev_err), _stream(stream)),
           "psa_attn_fwd_noalloc")
