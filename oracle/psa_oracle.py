"""CPU oracle for the Pyramid Sparse Attention (PSA) path, forward and backward — fp64, numpy.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The product path (the HIP library and its Python binding) never imports,
links or calls it, and this module imports nothing from the product path: the two share no
code. It is deliberately plain and slow: one (batch, head, query block) row at a time, fp64
throughout, no blocking, fusion or reordering beyond what each definition states.

Sources (PSA: Pyramid Sparse Attention for Efficient Video Understanding and Generation,
arXiv 2512.04025, as described on the web pages):
  [ART]  summary article at rg.mbintangr.com, sections "Problem", "Method", "Results"
  [SKILL] skill summary at skillsmp.com, sections "Core Technique", "Implementation"
  [NEWS] news summary at euno.news, section "Methodology" (items 2 and 4)
  [ABS]  the paper's abstract (chatpaper.ai and mlsanity.com pages)

Where the pages leave a step open, the reading taken is stated in the function's docstring
(and listed with the rest of the design notes). Pins that tie each function to something other
than itself live in tests/test_oracle.py. The pages print no worked example for the mask
generator, so its functions (mask_scores_sampling, mask_scores_antidiag, mask_scores_meankey,
block_cossim, assign_levels) are pinned by special cases that reduce them to a plain definition
(every query row sampled gives the dense block mass; stride 1 gives the full logits; constant
key blocks give the exact block-mean logit), by brute force (the similarity over all key
pairs equals its closed form) and by hand-computed assignment cases, not by values printed on
the pages.

Notation: N padded length, Nv valid length, d head dim, BQ/BK query/KV block size,
NQB = N/BQ, NKB = N/BK, level l in {0,1,2,3}, skip = -1, s = 1/sqrt(d).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

SKIP = -1
NUM_LEVELS = 4
LN2 = math.log(2.0)


@dataclasses.dataclass(frozen=True)
class Problem:
    seq_len: int
    seq_valid: int
    head_dim: int
    block_q: int
    block_k: int = 64
    causal: bool = False

    @property
    def n_qblocks(self) -> int:
        return self.seq_len // self.block_q

    @property
    def n_kblocks(self) -> int:
        return self.seq_len // self.block_k

    @property
    def scale(self) -> float:
        # [NEWS] "Methodology" item 4: the result is standard scaled dot-product attention,
        # so the softmax scale is 1/sqrt(d).
        return 1.0 / math.sqrt(self.head_dim)

    @staticmethod
    def of(wl) -> "Problem":
        return Problem(wl.seq_len, wl.seq_valid, wl.head_dim, wl.block_q, wl.block_k, wl.causal)


def as_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (fp32 or bf16) or array to a float64 ndarray."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------------------
# 1. KV pyramid
# ----------------------------------------------------------------------------------------

def pool(x: np.ndarray, level: int) -> np.ndarray:
    """Level-`level` KV: the mean of each run of 2**level consecutive tokens (axis -2).

    [SKILL] "Core Technique"/"Implementation": level l holds the KV average-pooled by 2**l,
    each level pooled straight from the full-resolution KV. [ART] "Method" builds the same
    levels "progressively" by 1D mean pooling; the two agree in exact arithmetic (pinned).
    """
    f = 1 << level
    n = x.shape[-2]
    if n % f:
        raise ValueError("sequence length must be a multiple of the pool factor")
    return x.reshape(*x.shape[:-2], n // f, f, x.shape[-1]).mean(axis=-2)


def pyramid(x: np.ndarray, pooled_round: Optional[str] = None) -> Dict[int, np.ndarray]:
    """All levels 0..3 of one tensor (K or V); level 0 is the input itself. With
    pooled_round="bf16" the pooled levels (1..3) are the exact means rounded once to bfloat16
    (bf16_round): the levels a bf16 pyramid stores for the attention to read."""
    out = {l: (x if l == 0 else pool(x, l)) for l in range(NUM_LEVELS)}
    if pooled_round == "bf16":
        out = {l: (v if l == 0 else bf16_round(v)) for l, v in out.items()}
    elif pooled_round is not None:
        raise ValueError(pooled_round)
    return out


def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value of float64 x, ties to even (bfloat16: 8 exponent bits with bias
    127, 7 stored mantissa bits, subnormals below 2^-126). Written from the format: in the
    binade [2^E, 2^(E+1)), E >= -126, the spacing is 2^(E-7); below 2^-126 it is 2^-133.
    Finite inputs whose rounding stays below the largest finite bfloat16 only."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    q = np.ldexp(1.0, (e - 7.0).astype(np.int64))
    r = np.round(a / q) * q   # np.round: ties to even
    return np.sign(x) * r


def packed_level_offset(seq_len: int, level: int) -> int:
    """Row offset of level l (l >= 1) in the packed [.., 7N/8, d] pooled tensor:
    level 1 at 0, level 2 at N/2, level 3 at 3N/4 (sum of the sizes of the finer levels)."""
    return sum(seq_len >> j for j in range(1, level))


def pack_pyramid(x: np.ndarray) -> np.ndarray:
    """Levels 1..3 of x concatenated along the token axis: [.., 7N/8, d]."""
    return np.concatenate([pool(x, l) for l in range(1, NUM_LEVELS)], axis=-2)


def pooled_last_token(level: int, rows: np.ndarray) -> np.ndarray:
    """Index of the last full-resolution token inside pooled row(s) `rows` of level l."""
    return (np.asarray(rows) + 1) * (1 << level) - 1


# ----------------------------------------------------------------------------------------
# 2. Mask generator: block importance
# ----------------------------------------------------------------------------------------

def _valid_rows_in_qblock(p: Problem, qb: int) -> int:
    return int(np.clip(p.seq_valid - qb * p.block_q, 0, p.block_q))


def sample_offsets(rows_valid: int, samples: int) -> List[int]:
    """Sampled query rows of a block with `rows_valid` valid rows: floor(s * r / S), s < S.
    (Our reading of [ART] "Method" "sampling-based strategy": deterministic strided rows.)"""
    if rows_valid <= 0:
        return []
    return [(s * rows_valid) // samples for s in range(samples)]


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row softmax with -inf entries excluded; an all -inf row gives zeros."""
    m = np.max(z, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(z - m)
    den = e.sum(axis=-1, keepdims=True)
    return np.divide(e, den, out=np.zeros_like(e), where=den > 0)


def mask_scores_sampling(q: np.ndarray, k: np.ndarray, p: Problem, samples: int,
                         qblocks: Optional[Iterable[int]] = None) -> np.ndarray:
    """Block importance M[qb, kb] for one (batch, head) from sampled query rows.

    [ART] "Method": for video generation the multi-level mask generator estimates the
    importance of each query/key block pair with a sampling-based strategy. Our reading: take
    S sampled rows of the query block (sample_offsets), compute their softmax over all valid
    full-resolution keys (scale s; keys >= Nv masked; causal keys > row masked), and average
    the probability mass each KV block receives over the S rows. Every row of M sums to 1
    (0 for a query block with no valid rows). q: [N, d]; k: [N, d] of the matching KV head.
    """
    nqb, nkb = p.n_qblocks, p.n_kblocks
    M = np.zeros((nqb, nkb), dtype=np.float64)
    qbs = range(nqb) if qblocks is None else qblocks
    keys = np.arange(p.seq_len)
    for qb in qbs:
        offs = sample_offsets(_valid_rows_in_qblock(p, qb), samples)
        if not offs:
            continue
        rows = qb * p.block_q + np.asarray(offs)
        z = p.scale * (q[rows] @ k.T)                       # [S, N]
        vis = keys[None, :] < p.seq_valid
        if p.causal:
            vis = vis & (keys[None, :] <= rows[:, None])
        z = np.where(vis, z, -np.inf)
        prob = _softmax_rows(z)
        mass = prob.reshape(len(rows), nkb, p.block_k).sum(axis=-1)
        M[qb] = mass.mean(axis=0)
    return M


def mask_scores_antidiag(q: np.ndarray, k: np.ndarray, p: Problem, stride: int,
                         qblocks: Optional[Iterable[int]] = None) -> np.ndarray:
    """Block importance M[qb, kb] for one (batch, head) by antidiagonal scoring.

    [ART] "Method": for video understanding the mask generator scores blocks along
    antidiagonals (the method the pages cite as XAttention). Our reading, with stride S:
      compressed logit A[r, c] = s * sum_{t<S} q[r*S + S-1-t] . k[c*S + t]
    (the S products along the antidiagonal of the S x S sub-tile, summed, not averaged);
    compressed row r / column c is valid iff all its tokens are < Nv; causal: c <= r.
    P = softmax of A over the valid columns of each row. M[qb, kb] is the mass of the
    columns of kb, averaged over the valid compressed rows of qb (so rows of M sum to 1).
    """
    S = stride
    n, d = q.shape
    R = n // S
    qs = q.reshape(R, S, d)[:, ::-1, :].reshape(R, S * d)    # row r: q[rS+S-1], ..., q[rS]
    ks = k.reshape(R, S, d).reshape(R, S * d)                 # col c: k[cS], ..., k[cS+S-1]
    A = p.scale * (qs @ ks.T)
    idx = np.arange(R)
    valid = (idx * S + S - 1) < p.seq_valid
    vis = valid[None, :] & valid[:, None]
    if p.causal:
        vis = vis & (idx[None, :] <= idx[:, None])
    P = _softmax_rows(np.where(vis, A, -np.inf))
    rq, ck = p.block_q // S, p.block_k // S
    nqb, nkb = p.n_qblocks, p.n_kblocks
    M = np.zeros((nqb, nkb), dtype=np.float64)
    qbs = range(nqb) if qblocks is None else qblocks
    for qb in qbs:
        rows = slice(qb * rq, (qb + 1) * rq)
        nv = int(valid[rows].sum())
        if nv == 0:
            continue
        colmass = P[rows].sum(axis=0).reshape(nkb, ck).sum(axis=-1)
        M[qb] = colmass / nv
    return M


def mask_scores_meankey(q: np.ndarray, k: np.ndarray, p: Problem,
                        qblocks: Optional[Iterable[int]] = None) -> np.ndarray:
    """Block importance M[qb, kb] for one (batch, head) from block means.

    [SKILL] "Implementation" (block importance scoring): a query is scored against the mean
    key of each KV block. Our reading, turned into the block masses the threshold rule needs:
    q_bar = mean of the query block's valid rows, k_bar = mean of the KV block's valid keys,
    z_kb = s * q_bar . k_bar + ln(n_kb) with n_kb the block's valid keys (a block of n
    identical keys k_bar carries n times the weight of one), M[qb] = softmax of z over the
    candidate blocks (causal: kb up to the last block overlapping the query block). A query
    block with no valid rows gets M = 0. When every query block's rows are equal and every
    KV block's keys are equal, this is exactly the sampling-mode mass (non-causal).
    """
    nqb, nkb = p.n_qblocks, p.n_kblocks
    M = np.zeros((nqb, nkb), dtype=np.float64)
    nv = np.clip(p.seq_valid - np.arange(nkb) * p.block_k, 0, p.block_k)
    kbar = np.zeros((nkb, k.shape[1]))
    for kb in range(nkb):
        if nv[kb] > 0:
            kbar[kb] = k[kb * p.block_k: kb * p.block_k + nv[kb]].mean(axis=0)
    qbs = range(nqb) if qblocks is None else qblocks
    for qb in qbs:
        rv = _valid_rows_in_qblock(p, qb)
        if rv == 0:
            continue
        qbar = q[qb * p.block_q: qb * p.block_q + rv].mean(axis=0)
        last = kb_diag(p, qb) if p.causal else nkb - 1
        cand = np.arange(nkb) <= last
        ok = cand & (nv > 0)
        z = np.full(nkb, -np.inf)
        z[ok] = p.scale * (kbar[ok] @ qbar) + np.log(nv[ok])
        M[qb] = _softmax_rows(z[None, :])[0]
    return M


def block_cossim(k: np.ndarray, p: Problem) -> np.ndarray:
    """Intra-block key similarity sim[kb] for one (batch, KV head).

    [ART] "Method"/"Results": pooling is allowed only when the block passes an intra-block
    similarity check (a cosine-similarity constraint). Our reading: the mean cosine
    similarity over all ordered pairs (i, j), i != j, of the block's valid level-0 keys: the
    full matrix of pairwise cosines is formed and its off-diagonal entries averaged. A zero
    key has cosine 0 with everything. A block with fewer than two valid keys has similarity 1.
    """
    nkb, bk = p.n_kblocks, p.block_k
    sim = np.ones((nkb,), dtype=np.float64)
    for kb in range(nkb):
        lo = kb * bk
        nv = int(np.clip(p.seq_valid - lo, 0, bk))
        if nv < 2:
            continue
        x = k[lo:lo + nv]
        nrm = np.linalg.norm(x, axis=1)
        xh = np.divide(x, nrm[:, None], out=np.zeros_like(x), where=nrm[:, None] > 0)
        cos = xh @ xh.T                                   # [nv, nv] pairwise cosines
        off = ~np.eye(nv, dtype=bool)
        sim[kb] = cos[off].sum() / (nv * (nv - 1))
    return sim


# ----------------------------------------------------------------------------------------
# 3. Threshold assignment of levels
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class AssignParams:
    thresholds: Tuple[float, float, float, float]
    cos_sim_min: float = 0.0          # <= 0 disables the similarity fallback
    force_diag_l0: bool = False
    force_begin: int = 0              # token span [begin, end) forced to L0 both ways
    force_end: int = 0


def kb_diag(p: Problem, qb: int) -> int:
    """Last KV block that overlaps query block qb (the causal frontier)."""
    return ((qb + 1) * p.block_q - 1) // p.block_k


def _overlaps(lo: int, hi: int, b: int, e: int) -> bool:
    return lo < e and b < hi


def assign_row(M: np.ndarray, sim: Optional[np.ndarray], p: Problem, a: AssignParams,
               qb: int) -> np.ndarray:
    """Levels of one query block's row of KV blocks.

    [ART] "Method": important blocks get finer levels, less important ones coarser levels,
    the least important are skipped; "Results": the generation rule is threshold based and
    pooling is subject to a cosine-similarity constraint. Our reading:
      1. candidates: every kb (causal: kb <= kb_diag); a query block without valid rows is
         all skip;
      2. sort candidates by M descending, ties by kb ascending;
      3. exclusive cumulative mass c (fp64, in that order); level = min{l : c < t_l}, else
         skip (thresholds are taken at float32 precision, as the library receives them);
      4. overrides, in order: causal kb > kb_diag -> skip; forced L0 (the diagonal blocks
         if flagged; any block pair touching the forced token span, in either direction);
         similarity fallback: a pooled level (1..3) on a block with sim < cos_sim_min -> L0.
    """
    nkb = p.n_kblocks
    t = [float(np.float32(x)) for x in a.thresholds]
    row = np.full((nkb,), SKIP, dtype=np.int8)
    if _valid_rows_in_qblock(p, qb) == 0:
        return row
    last = kb_diag(p, qb) if p.causal else nkb - 1
    cand = list(range(last + 1))
    order = sorted(cand, key=lambda kb: (-float(M[kb]), kb))
    c = 0.0
    for kb in order:
        lvl = SKIP
        for l in range(NUM_LEVELS):
            if c < t[l]:
                lvl = l
                break
        row[kb] = lvl
        c += float(M[kb])
    # overrides
    if p.causal:
        row[last + 1:] = SKIP
    qlo, qhi = qb * p.block_q, (qb + 1) * p.block_q
    for kb in range(last + 1):
        klo, khi = kb * p.block_k, (kb + 1) * p.block_k
        forced = False
        if a.force_diag_l0 and _overlaps(qlo, qhi, klo, khi):
            forced = True
        if a.force_end > a.force_begin and (_overlaps(qlo, qhi, a.force_begin, a.force_end)
                                            or _overlaps(klo, khi, a.force_begin, a.force_end)):
            forced = True
        if forced:
            row[kb] = 0
        elif (a.cos_sim_min > 0 and sim is not None and row[kb] > 0
              and float(sim[kb]) < float(np.float32(a.cos_sim_min))):
            row[kb] = 0
    return row


def assign_levels(M: np.ndarray, sim: Optional[np.ndarray], p: Problem,
                  a: AssignParams) -> np.ndarray:
    """Level map [NQB, NKB] int8 for one (batch, head): assign_row for every query block."""
    return np.stack([assign_row(M[qb], sim, p, a, qb) for qb in range(p.n_qblocks)])


# ----------------------------------------------------------------------------------------
# 4. Block index
# ----------------------------------------------------------------------------------------

def build_index(level_map: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """CSR over (row, level) keys of a level map [..., NQB, NKB] flattened row-major to
    R rows: row_ptr[R*4 + 1] and col_idx listing, per row and level 0..3, the kb with that
    level in ascending order. Entries outside {-1, 0, 1, 2, 3} are rejected."""
    m = np.asarray(level_map)
    nkb = m.shape[-1]
    rows = m.reshape(-1, nkb)
    bad = ~np.isin(rows, [SKIP, 0, 1, 2, 3])
    if bad.any():
        raise ValueError("level map holds values outside {-1, 0, 1, 2, 3}")
    row_ptr = [0]
    cols: List[int] = []
    for r in range(rows.shape[0]):
        for l in range(NUM_LEVELS):
            sel = [kb for kb in range(nkb) if rows[r, kb] == l]
            cols.extend(sel)
            row_ptr.append(len(cols))
    return np.asarray(row_ptr, dtype=np.int64), np.asarray(cols, dtype=np.int64)


# ----------------------------------------------------------------------------------------
# 5. Adaptive Pyramid Attention
# ----------------------------------------------------------------------------------------

def gather_row_keys(levels_k: Dict[int, np.ndarray], levels_v: Dict[int, np.ndarray],
                    row_levels: np.ndarray, p: Problem):
    """The pooled keys/values one query block reads: for every kb with level l >= 0, the
    64/2**l rows of level l that cover kb. Returns (K̄, V̄, level per key, last token per key)."""
    ks, vs, lv, last = [], [], [], []
    for kb in range(p.n_kblocks):
        l = int(row_levels[kb])
        if l < 0:
            continue
        per = p.block_k >> l
        rows = np.arange(kb * per, (kb + 1) * per)
        ks.append(levels_k[l][rows])
        vs.append(levels_v[l][rows])
        lv.append(np.full(per, l))
        last.append(pooled_last_token(l, rows))
    if not ks:
        d = levels_k[0].shape[-1]
        return (np.zeros((0, d)), np.zeros((0, d)), np.zeros(0, dtype=int),
                np.zeros(0, dtype=int))
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(lv), np.concatenate(last)


def attention_weights_row(q_rows: np.ndarray, query_idx: np.ndarray, Kb, lv, last,
                          p: Problem, scale: float) -> np.ndarray:
    """Softmax weights of each query over its gathered pooled keys.

    [ART] "Method": each KV block is read at its assigned level and a scaling factor keeps the
    probability distribution consistent. Our reading: a pooled token of level l stands for 2**l
    tokens, so its logit gets + l*ln2 (weight 2**l); this equals nearest-neighbour upsampling
    of the pooled block followed by standard attention ([NEWS] "Methodology" item 4). A pooled
    token is visible to query i iff its last constituent token is < Nv and (causal) <= i.
    Rows with no visible key get all-zero weights.
    """
    z = scale * (q_rows @ Kb.T) + lv[None, :] * LN2
    vis = last[None, :] < p.seq_valid
    if p.causal:
        vis = vis & (last[None, :] <= query_idx[:, None])
    z = np.where(vis, z, -np.inf)
    return _softmax_rows(z)


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, level_map: np.ndarray,
                   p: Problem, scale: Optional[float] = None,
                   qblocks: Optional[Iterable[int]] = None,
                   pooled_round: Optional[str] = None) -> Tuple[np.ndarray, np.ndarray]:
    """PSA forward for one (batch, head). q: [N, d]; k, v: [N, d] of its KV head (level 0);
    level_map: [NQB, NKB]. Returns (o [N, d], lse [N]) in fp64. For each valid query i:
      z_j = s * q_i . K̄_j + l_j * ln2,  o_i = sum_j softmax(z)_j V̄_j,  lse_i = logsumexp(z).
    Query rows >= Nv, and rows with no visible key, give o = 0 and lse = -inf. Rows of query
    blocks not listed in `qblocks` are left as NaN. pooled_round="bf16" reads the pooled
    levels as a bf16 pyramid stores them (each exact mean rounded once to bfloat16); the rest
    of the arithmetic stays fp64.
    """
    sc = p.scale if scale is None else scale
    return _attention_from_levels(q, pyramid(k, pooled_round), pyramid(v, pooled_round),
                                  level_map, p, sc, qblocks)


def _attention_from_levels(q: np.ndarray, lk: Dict[int, np.ndarray], lvv: Dict[int, np.ndarray],
                           level_map: np.ndarray, p: Problem, sc: float,
                           qblocks: Optional[Iterable[int]] = None):
    """The body of attention_head on prepared key/value levels (logit scale sc)."""
    n, d = q.shape
    o = np.full((n, d), np.nan)
    lse = np.full((n,), np.nan)
    qbs = range(p.n_qblocks) if qblocks is None else qblocks
    for qb in qbs:
        qi = np.arange(qb * p.block_q, (qb + 1) * p.block_q)
        Kb, Vb, lv, last = gather_row_keys(lk, lvv, level_map[qb], p)
        if Kb.shape[0] == 0:
            o[qi] = 0.0
            lse[qi] = -np.inf
            continue
        z = sc * (q[qi] @ Kb.T) + lv[None, :] * LN2
        vis = last[None, :] < p.seq_valid
        if p.causal:
            vis = vis & (last[None, :] <= qi[:, None])
        z = np.where(vis, z, -np.inf)
        w = _softmax_rows(z)
        o[qi] = w @ Vb
        m = np.max(z, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            lse_b = np.where(np.isfinite(m),
                             m + np.log(np.sum(np.exp(z - np.where(np.isfinite(m), m, 0.0)[:, None]),
                                               axis=1)),
                             -np.inf)
        lse[qi] = lse_b
        pad = qi >= p.seq_valid
        o[qi[pad]] = 0.0
        lse[qi[pad]] = -np.inf
    return o, lse


# ----------------------------------------------------------------------------------------
# 5b. FP8 (e4m3) operands for the QK^T product (and for P V)
# ----------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_round(x) -> np.ndarray:
    """Nearest e4m3 value (OCP FP8 E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits, subnormals down to 2^-9, largest finite 448), ties to even. |x| must not exceed
    464, the midpoint above 448 (which still rounds to 448). Written from the format: in the
    binade [2^E, 2^(E+1)), E >= -6, the spacing is 2^(E-3); below 2^-6 it is 2^-9."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 464.0):
        raise ValueError("value beyond the e4m3 range")
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    q = 2.0 ** (e - 3.0)
    return np.sign(x) * (np.round(a / q) * q)   # np.round: ties to even


def fp8_scale(x) -> float:
    """The per-(batch, head) scale of the fp8 reading: s = amax / 448 rounded to float32
    (amax over the head's level-0 rows, exact for bf16 inputs); an all-zero head gets 1.
    [ABS] and [NEWS] "Practical": the block-tile design suits FP16/FP8; the pages give no
    recipe, this one is the plainest (one scale per head, shared by the pooled levels, whose
    means never exceed the head's amax)."""
    amax = float(np.max(np.abs(np.asarray(x, dtype=np.float64)))) if np.size(x) else 0.0
    if amax == 0.0:
        return 1.0
    return float(np.float32(np.float32(amax) / np.float32(E4M3_MAX)))


def fp8_quantize(x, s: float) -> np.ndarray:
    """x / s rounded to e4m3 (values, not codes); the fp8 operand is this value, and it
    stands for (value * s)."""
    return e4m3_round(np.asarray(x, dtype=np.float64) / s)


def attention_fp8qk_head(q8: np.ndarray, k8: np.ndarray, kp8_levels: Dict[int, np.ndarray],
                         v: np.ndarray, s_q: float, s_k: float, level_map: np.ndarray, p: Problem,
                         scale: Optional[float] = None, qblocks: Optional[Iterable[int]] = None):
    """attention_head with the QK^T product taken on the fp8 operands: q8, k8 (level 0) and
    kp8_levels[l] (the pooled levels, quantized with the same scale s_k) are e4m3 values;
    logits are scale * s_q * s_k * (q8 . k8) + l ln 2 (exact), V and the rest as in
    attention_head."""
    sc = p.scale if scale is None else scale
    lk = {0: k8}
    lk.update(kp8_levels)
    lvv = pyramid(v)
    return _attention_from_levels(q8, lk, lvv, level_map, p, sc * s_q * s_k, qblocks)


def attention_fp8_head(q8: np.ndarray, k8: np.ndarray, kp8_levels: Dict[int, np.ndarray],
                       v8: np.ndarray, vp8_levels: Dict[int, np.ndarray], s_q: float, s_k: float,
                       s_v: float, level_map: np.ndarray, p: Problem,
                       scale: Optional[float] = None, qblocks: Optional[Iterable[int]] = None):
    """attention_fp8qk_head with the P V product on e4m3 operands as well ([ABS], [NEWS]
    "Practical": FP8 arithmetic on the block-tile kernel; the pages give no recipe). V and its
    pooled levels are e4m3 values with one scale s_v per head (v8 stands for v8 * s_v). For
    each valid query, in log2 units t_j = z_j / ln 2 (z_j as in attention_fp8qk_head):
      M = ceil(max_j t_j), an integer;  P8_j = e4m3(2^(t_j - M + 7));
      o = s_v * sum_j P8_j v8_j / sum_j P8_j;  lse = (M - 7 + log2 sum_j P8_j) * ln 2.
    The weights that multiply V are the quantized P8_j, normalised by their own sum. The
    reference 2^(M - 7) puts the largest weight in (64, 128], so every weight down to 2^-13 of
    it stays in e4m3's normal range (>= 2^-6; below, the subnormal spacing 2^-9 would cost
    relative precision). Rounding commutes with scaling by a power of two in the normal range,
    so any integer reference between M - 8 and M - 7 gives the same codes there. Rows with no
    visible key and pad rows give o = 0 and lse = -inf."""
    sc = p.scale if scale is None else scale
    lk = {0: k8}
    lk.update(kp8_levels)
    lvv = {0: v8}
    lvv.update(vp8_levels)
    n, d = q8.shape
    o = np.full((n, d), np.nan)
    lse = np.full((n,), np.nan)
    for qb in (range(p.n_qblocks) if qblocks is None else qblocks):
        qi = np.arange(qb * p.block_q, (qb + 1) * p.block_q)
        Kb, Vb, lv, last = gather_row_keys(lk, lvv, level_map[qb], p)
        o[qi] = 0.0
        lse[qi] = -np.inf
        if Kb.shape[0] == 0:
            continue
        t = (sc * s_q * s_k * (q8[qi] @ Kb.T) + lv[None, :] * LN2) / LN2
        vis = np.broadcast_to(last[None, :] < p.seq_valid, t.shape)
        if p.causal:
            vis = vis & (last[None, :] <= qi[:, None])
        for r in range(qi.size):
            if qi[r] >= p.seq_valid or not np.any(vis[r]):
                continue
            tr = t[r][vis[r]]
            M = math.ceil(float(np.max(tr)))
            P8 = e4m3_round(2.0 ** (tr - M + 7))
            l8 = float(np.sum(P8))
            o[qi[r]] = s_v * (P8 @ Vb[vis[r]]) / l8
            lse[qi[r]] = (M - 7 + math.log2(l8)) * LN2
    return o, lse


# ----------------------------------------------------------------------------------------
# 6. Backward of the Adaptive Pyramid Attention
# ----------------------------------------------------------------------------------------

def attention_backward_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, level_map: np.ndarray,
                            do: np.ndarray, p: Problem, scale: Optional[float] = None,
                            qblocks: Optional[Iterable[int]] = None):
    """Gradients of the PSA forward of one (batch, head) with respect to q, k and v (level 0),
    given the output gradient do [N, d]. Returns (dq [N, d], dk [N, d], dv [N, d]) in fp64.

    [NEWS] "Methodology" item 4: pooling is deterministic, so gradients flow through every
    level and the whole layer trains end to end. This function is the chain rule of
    attention_head written out, one query block at a time:
      P = softmax(z) over the gathered pooled keys (z as in attention_head),
      dV̄ = P^T dO,  dP = dO V̄^T,  D_i = sum_j P_ij dP_ij,  dz = P * (dP - D),
      dq = s dz K̄,  dK̄ = s dz^T q;
    each gathered pooled row's gradient is added to its level's pooled row, and a pooled row
    of level l, the mean of 2**l consecutive tokens, hands 2**-l of its gradient to each of
    them. Pad query rows and rows with no visible key have a constant output (zero): they
    contribute nothing. With `qblocks`, only those query blocks are visited: their dq rows
    are exact, other dq rows stay zero, and dk, dv hold only those blocks' contributions.
    """
    sc = p.scale if scale is None else scale
    lk, lvv = pyramid(k), pyramid(v)
    n, d = q.shape
    gk = {l: np.zeros_like(lk[l]) for l in range(NUM_LEVELS)}
    gv = {l: np.zeros_like(lvv[l]) for l in range(NUM_LEVELS)}
    dq = np.zeros((n, d))
    for qb in (range(p.n_qblocks) if qblocks is None else qblocks):
        qi = np.arange(qb * p.block_q, (qb + 1) * p.block_q)
        qi = qi[qi < p.seq_valid]
        if qi.size == 0:
            continue
        Kb, Vb, lv, last = gather_row_keys(lk, lvv, level_map[qb], p)
        if Kb.shape[0] == 0:
            continue
        # which pooled row of which level each gathered key is
        src_l, src_r = [], []
        for kb in range(p.n_kblocks):
            l = int(level_map[qb, kb])
            if l < 0:
                continue
            per = p.block_k >> l
            src_l.append(np.full(per, l))
            src_r.append(np.arange(kb * per, (kb + 1) * per))
        src_l, src_r = np.concatenate(src_l), np.concatenate(src_r)
        P = attention_weights_row(q[qi], qi, Kb, lv, last, p, sc)
        dO = do[qi]
        dP = dO @ Vb.T
        D = np.sum(P * dP, axis=1)
        dz = P * (dP - D[:, None])
        dq[qi] = sc * (dz @ Kb)
        dKb = sc * (dz.T @ q[qi])
        dVb = P.T @ dO
        for l in range(NUM_LEVELS):
            sel = src_l == l
            np.add.at(gk[l], src_r[sel], dKb[sel])
            np.add.at(gv[l], src_r[sel], dVb[sel])
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    for l in range(NUM_LEVELS):
        tok = np.arange(n)
        dk += gk[l][tok >> l] * 2.0 ** -l
        dv += gv[l][tok >> l] * 2.0 ** -l
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# Whole-tensor wrappers ([B, H, N, d] inputs, GQA: KV head = h // (H / Hkv))
# ----------------------------------------------------------------------------------------

def attention(q, k, v, level_map, p: Problem, scale: Optional[float] = None,
              pooled_round: Optional[str] = None):
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, H = q.shape[:2]
    g = H // k.shape[1]
    o = np.empty_like(q)
    lse = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, h // g], v[b, h // g],
                                                level_map[b, h], p, scale,
                                                pooled_round=pooled_round)
    return o, lse


def attention_backward(q, k, v, level_map, do, p: Problem, scale: Optional[float] = None):
    """(dq [B,H,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d]): per-head gradients; a KV head's gradient
    is the sum over the query heads that share it."""
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    B, H = q.shape[:2]
    g = H // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            a, bk, bv = attention_backward_head(q[b, h], k[b, h // g], v[b, h // g],
                                                level_map[b, h], do[b, h], p, scale)
            dq[b, h] = a
            dk[b, h // g] += bk
            dv[b, h // g] += bv
    return dq, dk, dv


def mask(q, k, p: Problem, mode: str, a: AssignParams, samples: int = 8, stride: int = 8):
    """Full mask generator: (level map [B,H,NQB,NKB], M [B,H,NQB,NKB], sim [B,Hkv,NKB] or None)."""
    q, k = as_f64(q), as_f64(k)
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    g = H // Hkv
    sim = None
    if a.cos_sim_min > 0:
        sim = np.stack([np.stack([block_cossim(k[b, h], p) for h in range(Hkv)])
                        for b in range(B)])
    M = np.empty((B, H, p.n_qblocks, p.n_kblocks))
    lm = np.empty(M.shape, dtype=np.int8)
    for b in range(B):
        for h in range(H):
            if mode == "sampling":
                M[b, h] = mask_scores_sampling(q[b, h], k[b, h // g], p, samples)
            elif mode == "antidiag":
                M[b, h] = mask_scores_antidiag(q[b, h], k[b, h // g], p, stride)
            elif mode == "meankey":
                M[b, h] = mask_scores_meankey(q[b, h], k[b, h // g], p)
            else:
                raise ValueError(mode)
            lm[b, h] = assign_levels(M[b, h], None if sim is None else sim[b, h // g], p, a)
    return lm, M, sim
