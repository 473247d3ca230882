"""Seeded synthetic inputs for the Pyramid Sparse Attention (PSA) forward path.

This module holds workload shapes, seeds and random draws only. It contains none of the
method's arithmetic (no pooling, scoring, level assignment or attention), so that both the
HIP path's callers (tests, benchmark) and the CPU oracle can consume the same inputs without
sharing any method code.

Shapes follow the video-DiT and VLM attention layers the PSA pages evaluate on (PSA summary
article at rg.mbintangr.com, "Results": Wan2.1, CogVideoX-5B and Qwen2.5-VL-7B). No model
weights or videos are used: every tensor is drawn from a seeded generator with the structure
described per workload (clustered keys so that block importance is non-uniform).

Random streams. Every tensor slice is drawn from its own PCG64 stream keyed by
(workload seed, tensor code, batch index, head index), so any head can be regenerated on its
own (the oracle checks sampled heads of the full-size workloads without materialising all
of them). Draws are made in float32 and rounded to bfloat16 with round-to-nearest-even (torch's
conversion) when the workload is bf16; the rounded tensors are the canonical inputs for both
sides. Rows at or beyond ``seq_valid`` are zero.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

SKIP = -1

# tensor codes for the per-slice streams
_T_Q, _T_K, _T_V, _T_MAP, _T_DO = 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_len: int            # padded length N (multiple of block_q and block_k)
    seq_valid: int          # valid tokens Nv <= N; (N - Nv) % 8 == 0
    block_q: int
    block_k: int = 64
    causal: bool = False
    dtype: str = "bf16"     # "f32" | "bf16"
    k_dist: str = "normal"  # "normal" | "clustered" | "clustered_var"
    # where the level map comes from: "iid" / "fixed_frac" (drawn here) or "mask" (computed)
    map_source: str = "mask"
    map_probs: tuple = ()   # iid: P(L0..L3, skip); fixed_frac: fractions of L0..L3 per row
    force_diag_l0: bool = False
    # mask parameters (map_source == "mask")
    mask_mode: Optional[str] = None   # "sampling" | "antidiag" | "meankey"
    thresholds: tuple = ()
    samples_per_qblock: int = 8
    antidiag_stride: int = 8
    cos_sim_min: float = 0.0          # <= 0 disables the similarity check
    text_begin: int = 0               # token span [begin, end) forced to L0 both ways
    text_end: int = 0
    description: str = ""

    # ---- derived sizes -------------------------------------------------------------------
    @property
    def n_qblocks(self) -> int:
        return self.seq_len // self.block_q

    @property
    def n_kblocks(self) -> int:
        return self.seq_len // self.block_k

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _rng(seed: int, tensor: int, b: int, h: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(tensor, b, h))
    return np.random.Generator(np.random.PCG64(ss))


def _finish(x: np.ndarray, wl: Workload) -> torch.Tensor:
    x[wl.seq_valid:] = 0.0
    return torch.from_numpy(x).to(wl.torch_dtype)


def make_q_head(wl: Workload, b: int, h: int) -> torch.Tensor:
    """Q[b, h] ~ N(0, 1), shape [N, d]."""
    rng = _rng(wl.seed, _T_Q, b, h)
    return _finish(rng.standard_normal((wl.seq_len, wl.head_dim), dtype=np.float32), wl)


def make_v_head(wl: Workload, b: int, h: int) -> torch.Tensor:
    """V[b, kv head h] ~ N(0, 1), shape [N, d]."""
    rng = _rng(wl.seed, _T_V, b, h)
    return _finish(rng.standard_normal((wl.seq_len, wl.head_dim), dtype=np.float32), wl)


def make_k_head(wl: Workload, b: int, h: int) -> torch.Tensor:
    """K[b, kv head h], shape [N, d].

    normal:        N(0, 1).
    clustered:     per 64-token block a centre c ~ N(0, 2^2)^d plus token noise N(0, 0.5^2)^d.
    clustered_var: as clustered but the noise deviation is drawn per block from U(0.1, 1.0).
    Tokens in the text span [text_begin, text_end) are N(0, 1) in every mode.
    Draw order inside the stream: centres, noise, per-block deviations.
    """
    rng = _rng(wl.seed, _T_K, b, h)
    n, d, bk = wl.seq_len, wl.head_dim, wl.block_k
    if wl.k_dist == "normal":
        x = rng.standard_normal((n, d), dtype=np.float32)
    else:
        nkb = n // bk
        centres = 2.0 * rng.standard_normal((nkb, d), dtype=np.float32)
        noise = rng.standard_normal((n, d), dtype=np.float32)
        if wl.k_dist == "clustered":
            sigma = np.full((nkb,), 0.5, dtype=np.float32)
        elif wl.k_dist == "clustered_var":
            sigma = rng.uniform(0.1, 1.0, size=nkb).astype(np.float32)
        else:
            raise ValueError(wl.k_dist)
        x = (np.repeat(centres, bk, axis=0)
             + noise * np.repeat(sigma, bk)[:, None]).astype(np.float32)
        if wl.text_end > wl.text_begin:
            t = rng.standard_normal((wl.text_end - wl.text_begin, d), dtype=np.float32)
            x[wl.text_begin:wl.text_end] = t
    return _finish(x, wl)


def _stack(wl: Workload, fn, heads: int, head_ids: Optional[Sequence[int]]) -> torch.Tensor:
    hs = range(heads) if head_ids is None else head_ids
    out = torch.empty((wl.batch, len(hs), wl.seq_len, wl.head_dim), dtype=wl.torch_dtype)
    for b in range(wl.batch):
        for i, h in enumerate(hs):
            out[b, i] = fn(wl, b, h)
    return out


def make_q(wl: Workload, heads: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Q as [B, H, N, d] (or only the listed heads), CPU tensor in the workload dtype."""
    return _stack(wl, make_q_head, wl.heads_q, heads)


def make_k(wl: Workload, heads: Optional[Sequence[int]] = None) -> torch.Tensor:
    return _stack(wl, make_k_head, wl.heads_kv, heads)


def make_v(wl: Workload, heads: Optional[Sequence[int]] = None) -> torch.Tensor:
    return _stack(wl, make_v_head, wl.heads_kv, heads)


def make_qkv(wl: Workload):
    return make_q(wl), make_k(wl), make_v(wl)


def make_dout_head(wl: Workload, b: int, h: int) -> torch.Tensor:
    """The output gradient dO[b, h] ~ N(0, 1), shape [N, d] (pad rows zero)."""
    rng = _rng(wl.seed, _T_DO, b, h)
    return _finish(rng.standard_normal((wl.seq_len, wl.head_dim), dtype=np.float32), wl)


def make_dout(wl: Workload, heads: Optional[Sequence[int]] = None) -> torch.Tensor:
    """dO as [B, H, N, d], for the backward."""
    return _stack(wl, make_dout_head, wl.heads_q, heads)


def diag_blocks(wl: Workload, qb: int) -> range:
    """KV blocks whose token range overlaps the token range of query block qb."""
    lo = (qb * wl.block_q) // wl.block_k
    hi = ((qb + 1) * wl.block_q - 1) // wl.block_k
    return range(lo, hi + 1)


def make_map_head(wl: Workload, b: int, h: int) -> np.ndarray:
    """Level map [NQB, NKB] int8 for one (b, h) when the workload draws it directly.

    iid:        every entry drawn independently with P(L0..L3, skip) = map_probs.
    fixed_frac: per row, n_l = round(frac_l * NKB) blocks at level l (l = 0..3), the rest skip;
                blocks are ranked by a seeded uniform key with the diagonal blocks first, so
                the diagonal counts toward L0.
    force_diag_l0 sets the diagonal blocks to L0 afterwards (iid) or by construction.
    """
    rng = _rng(wl.seed, _T_MAP, b, h)
    nqb, nkb = wl.n_qblocks, wl.n_kblocks
    if wl.map_source == "iid":
        vals = np.array([0, 1, 2, 3, SKIP], dtype=np.int8)
        m = rng.choice(vals, size=(nqb, nkb), p=np.asarray(wl.map_probs, dtype=np.float64))
        m = m.astype(np.int8)
        if wl.force_diag_l0:
            for qb in range(nqb):
                for kb in diag_blocks(wl, qb):
                    m[qb, kb] = 0
        return m
    if wl.map_source == "fixed_frac":
        counts = [int(round(f * nkb)) for f in wl.map_probs]
        key = rng.random((nqb, nkb))
        for qb in range(nqb):
            for kb in diag_blocks(wl, qb):
                key[qb, kb] = -1.0
        order = np.argsort(key, axis=1, kind="stable")
        m = np.full((nqb, nkb), SKIP, dtype=np.int8)
        start = 0
        rows = np.arange(nqb)[:, None]
        for lvl, c in enumerate(counts):
            m[rows, order[:, start:start + c]] = lvl
            start += c
        return m
    raise ValueError(f"workload {wl.name} computes its map with the mask generator")


def make_map(wl: Workload, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    hs = range(wl.heads_q) if heads is None else heads
    out = np.empty((wl.batch, len(hs), wl.n_qblocks, wl.n_kblocks), dtype=np.int8)
    for b in range(wl.batch):
        for i, h in enumerate(hs):
            out[b, i] = make_map_head(wl, b, h)
    return out


# ----------------------------------------------------------------------------------------
# The five workloads. Names say what they are; sizes are the attention layer's.
# ----------------------------------------------------------------------------------------

TINY_F32 = Workload(
    name="tiny_f32_1k", seed=1001, batch=1, heads_q=2, heads_kv=2, head_dim=64,
    seq_len=1024, seq_valid=1024, block_q=64, block_k=64, dtype="f32", k_dist="normal",
    map_source="iid", map_probs=(0.15, 0.15, 0.15, 0.15, 0.40), force_diag_l0=True,
    description="tiny fp32 PSA forward, B1 H2 N1024 d64, iid level map")

WAN13B_32K = Workload(
    name="wan2.1-1.3b_32k", seed=1002, batch=1, heads_q=12, heads_kv=12, head_dim=128,
    seq_len=32768, seq_valid=21 * 30 * 52, block_q=128, block_k=64, dtype="bf16",
    k_dist="clustered", map_source="mask", mask_mode="sampling",
    thresholds=(0.5, 0.7, 0.8, 0.9), samples_per_qblock=8,
    description="Wan2.1-1.3B-like self-attention, 21x30x52=32760 tokens padded to 32768, "
                "sampling-mode mask")

COGVIDEOX5B_17K = Workload(
    name="cogvideox-5b_17k", seed=1003, batch=1, heads_q=48, heads_kv=48, head_dim=64,
    seq_len=17792, seq_valid=17776, block_q=128, block_k=64, dtype="bf16",
    k_dist="clustered", map_source="mask", mask_mode="sampling",
    thresholds=(0.6, 0.75, 0.85, 0.92), samples_per_qblock=8,
    text_begin=17550, text_end=17776,
    description="CogVideoX-5B-like joint attention, 17550 video + 226 text tokens padded to "
                "17792, text blocks forced to L0")

WAN14B_720P_75K = Workload(
    name="wan2.1-14b-720p_75k", seed=1004, batch=1, heads_q=40, heads_kv=40, head_dim=128,
    seq_len=75648, seq_valid=21 * 45 * 80, block_q=128, block_k=64, dtype="bf16",
    k_dist="clustered", map_source="fixed_frac", map_probs=(0.05, 0.05, 0.05, 0.05),
    force_diag_l0=True,
    description="Wan2.1-14B-720p-like self-attention, 75600 tokens padded to 75648, "
                "5/5/5/5/80 level map")

QWEN25VL_32K = Workload(
    name="qwen2.5-vl-7b_32k_causal", seed=1005, batch=1, heads_q=28, heads_kv=4, head_dim=128,
    seq_len=32768, seq_valid=32768, block_q=128, block_k=64, causal=True, dtype="bf16",
    k_dist="clustered_var", map_source="mask", mask_mode="antidiag",
    thresholds=(0.6, 0.8, 0.9, 0.95), antidiag_stride=8, cos_sim_min=0.8,
    force_diag_l0=True,
    description="Qwen2.5-VL-7B-like causal video prefill, GQA 28:4, antidiagonal mask with "
                "cosine check")

ALL = (TINY_F32, WAN13B_32K, COGVIDEOX5B_17K, WAN14B_720P_75K, QWEN25VL_32K)
BY_NAME = {w.name: w for w in ALL}


def small(wl: Workload) -> Workload:
    """A reduced copy of a full-size workload with the same structure (block sizes, mask mode,
    padding, GQA, causal, text span) that the oracle finishes in seconds."""
    if wl is TINY_F32 or wl.name == TINY_F32.name:
        return wl
    if wl.name == WAN13B_32K.name:
        return wl.replace(name=wl.name + "-small", heads_q=2, heads_kv=2,
                          seq_len=2048, seq_valid=2040)
    if wl.name == COGVIDEOX5B_17K.name:
        # video 1814 + text 226 = 2040 valid, padded to 2048 (pad 8)
        return wl.replace(name=wl.name + "-small", heads_q=2, heads_kv=2,
                          seq_len=2048, seq_valid=2040, text_begin=1814, text_end=2040)
    if wl.name == WAN14B_720P_75K.name:
        return wl.replace(name=wl.name + "-small", heads_q=2, heads_kv=2,
                          seq_len=4096, seq_valid=4048)
    if wl.name == QWEN25VL_32K.name:
        return wl.replace(name=wl.name + "-small", heads_q=4, heads_kv=2,
                          seq_len=2048, seq_valid=2048)
    raise KeyError(wl.name)
