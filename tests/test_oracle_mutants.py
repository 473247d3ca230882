"""Plant plausible mistakes in the CPU oracle (on the CPU, in a private copy of its source)
and check that at least one pin catches each one. This guards the pins themselves: a pin set
that a dropped term, a flipped sign, a wrong index or a transposed operand slips through is
not pinning the oracle."""
import importlib.util
import os
import sys
import types

import numpy as np
import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "psa_oracle.py")

ALL_PINS = {
    "p1": lambda: max(pins.pin_all_l0_dense(False, 512), pins.pin_all_l0_dense(False, 488),
                      pins.pin_all_l0_dense(True, 512)),
    "p2": pins.pin_binary_block_sparse,
    "p3": pins.pin_upsample_equivalence,
    "p4": lambda: max(pins.pin_constant_runs(l) for l in (1, 2, 3)),
    "p5": pins.pin_all_skip_row,
    "p6": pins.pin_weight_multiplicity,
    "p7": pins.pin_pyramid,
    "p8s": lambda: max(pins.pin_sampling_all_rows(False), pins.pin_sampling_all_rows(True)),
    "p8s_pad": lambda: max(pins.pin_sampling_padded(False), pins.pin_sampling_padded(True)),
    "gqa": lambda: max(pins.pin_gqa_attention(False), pins.pin_gqa_attention(True),
                       pins.pin_gqa_mask()),
    "gqa_bwd": lambda: max(pins.pin_gqa_backward(False), pins.pin_gqa_backward(True)),
    "p8a": lambda: max(pins.pin_antidiag_stride1(False), pins.pin_antidiag_stride1(True),
                       pins.pin_antidiag_orientation_and_sum()),
    "p8c": pins.pin_cossim,
    "p8m": lambda: max(pins.pin_meankey_constant_blocks(), pins.pin_meankey_causal_blocks()),
    "p9": lambda: sum(pins.pin_assign_case(c) for c in pins.golden_assign_cases()),
    "idx": pins.pin_build_index,
    # (pin, tolerance): the finite-difference quotient is good to ~1e-10 relative
    "pbwd_fd": (lambda: max(pins.pin_bwd_finite_difference(False, 120, 2, 1),
                            pins.pin_bwd_finite_difference(True, 128, 2, 2)), 1e-6),
    "pbwd_l0": lambda: max(pins.pin_bwd_all_l0_autograd(False, 232),
                           pins.pin_bwd_all_l0_autograd(True, 256)),
    "pbwd_runs": lambda: max(pins.pin_bwd_constant_runs(l) for l in (1, 3)),
    "pfp8": lambda: max(pins.pin_e4m3_round(), pins.pin_fp8_scale(),
                        pins.pin_fp8qk_reduces_to_attention(True)),
    "pbf16": lambda: max(pins.pin_bf16_round(), pins.pin_bf16_pooled_attention()),
    "pfp8pv": lambda: max(pins.pin_fp8pv_worked_rows(), pins.pin_fp8pv_powers_of_two(True)),
}


def _pin(entry):
    return entry if isinstance(entry, tuple) else (entry, 1e-9)

MUTANTS = [
    ("bias_sign", "lv[None, :] * LN2\n        vis", "lv[None, :] * -LN2\n        vis"),
    ("bias_dropped", "lv[None, :] * LN2\n        vis", "lv[None, :] * 0.0\n        vis"),
    ("scale_dropped", "return 1.0 / math.sqrt(self.head_dim)", "return 1.0"),
    ("pv_uses_keys", "o[qi] = w @ Vb", "o[qi] = w @ Kb"),
    ("last_token_off_by_one", "return (np.asarray(rows) + 1) * (1 << level) - 1",
     "return (np.asarray(rows) + 1) * (1 << level)"),
    ("pool_wrong_axis", "n // f, f, x.shape[-1]).mean(axis=-2)",
     "n // f, f, x.shape[-1]).mean(axis=-1)[..., None].repeat(x.shape[-1], -1)"),
    ("pad_keys_visible", "vis = last[None, :] < p.seq_valid\n        if p.causal",
     "vis = last[None, :] < p.seq_len\n        if p.causal"),
    ("antidiag_no_reverse", "qs = q.reshape(R, S, d)[:, ::-1, :]", "qs = q.reshape(R, S, d)[:, :, :]"),
    ("antidiag_mean", "A = p.scale * (qs @ ks.T)", "A = p.scale * (qs @ ks.T) / S"),
    ("sampling_pad_keys_visible", "vis = keys[None, :] < p.seq_valid", "vis = keys[None, :] < p.seq_len"),
    ("gqa_modulo_attention", "attention_head(q[b, h], k[b, h // g], v[b, h // g],",
     "attention_head(q[b, h], k[b, h % k.shape[1]], v[b, h % k.shape[1]],"),
    ("gqa_modulo_backward", "attention_backward_head(q[b, h], k[b, h // g], v[b, h // g],",
     "attention_backward_head(q[b, h], k[b, h % k.shape[1]], v[b, h % k.shape[1]],"),
    ("gqa_modulo_backward_sum", "dk[b, h // g] += bk\n            dv[b, h // g] += bv",
     "dk[b, h % k.shape[1]] += bk\n            dv[b, h % k.shape[1]] += bv"),
    ("gqa_modulo_mask_sampling", "mask_scores_sampling(q[b, h], k[b, h // g], p, samples)",
     "mask_scores_sampling(q[b, h], k[b, h % Hkv], p, samples)"),
    ("gqa_modulo_mask_antidiag", "mask_scores_antidiag(q[b, h], k[b, h // g], p, stride)",
     "mask_scores_antidiag(q[b, h], k[b, h % Hkv], p, stride)"),
    ("gqa_modulo_mask_sim", "None if sim is None else sim[b, h // g], p, a)",
     "None if sim is None else sim[b, h % Hkv], p, a)"),
    ("sampling_no_causal", "vis = vis & (keys[None, :] <= rows[:, None])", "vis = vis"),
    ("cossim_keeps_diagonal", "sim[kb] = cos[off].sum()", "sim[kb] = cos.sum()"),
    ("meankey_no_count", "p.scale * (kbar[ok] @ qbar) + np.log(nv[ok])", "p.scale * (kbar[ok] @ qbar)"),
    ("meankey_key_sum", "kbar[kb] = k[kb * p.block_k: kb * p.block_k + nv[kb]].mean(axis=0)",
     "kbar[kb] = k[kb * p.block_k: kb * p.block_k + nv[kb]].sum(axis=0)"),
    ("meankey_no_causal", "last = kb_diag(p, qb) if p.causal else nkb - 1\n        cand",
     "last = nkb - 1\n        cand"),
    ("assign_le", "if c < t[l]:", "if c <= t[l]:"),
    ("assign_tie_reversed", "key=lambda kb: (-float(M[kb]), kb)", "key=lambda kb: (-float(M[kb]), -kb)"),
    ("assign_inclusive_cumsum", "for kb in order:\n        lvl = SKIP",
     "for kb in order:\n        c += float(M[kb])\n        lvl = SKIP"),
    ("cos_fallback_inclusive", "float(sim[kb]) < float(np.float32(a.cos_sim_min))",
     "float(sim[kb]) <= float(np.float32(a.cos_sim_min))"),
    ("bwd_no_rowsum_term", "dz = P * (dP - D[:, None])", "dz = P * dP"),
    ("bwd_pool_unweighted", "dk += gk[l][tok >> l] * 2.0 ** -l", "dk += gk[l][tok >> l]"),
    ("bwd_dk_unscaled", "dKb = sc * (dz.T @ q[qi])", "dKb = dz.T @ q[qi]"),
    ("bwd_dv_from_dz", "dVb = P.T @ dO", "dVb = dz.T @ dO"),
    ("bwd_dq_uses_values", "dq[qi] = sc * (dz @ Kb)", "dq[qi] = sc * (dz @ Vb)"),
    ("bwd_gqa_overwrites", "dk[b, h // g] += bk", "dk[b, h // g] = bk"),
    ("bwd_pool_wrong_row", "dv += gv[l][tok >> l] * 2.0 ** -l", "dv += gv[l][np.minimum(tok >> (l - 1 if l else 0), tok.size - 1)] * 2.0 ** -l"),
    ("bf16_ties_away", "r = np.round(a / q) * q   # np.round: ties to even", "r = np.floor(a / q + 0.5) * q"),
    ("bf16_eight_mantissa_bits", "q = np.ldexp(1.0, (e - 7.0).astype(np.int64))",
     "q = np.ldexp(1.0, (e - 8.0).astype(np.int64))"),
    ("bf16_no_subnormals", "e = np.maximum(e, -126.0)", "e = np.maximum(e, -1260.0)"),
    ("bf16_pooled_not_rounded", "out = {l: (v if l == 0 else bf16_round(v)) for l, v in out.items()}",
     "out = {l: v for l, v in out.items()}"),
    ("bf16_level0_rounded", "out = {l: (v if l == 0 else bf16_round(v)) for l, v in out.items()}",
     "out = {l: bf16_round(v) for l, v in out.items()}"),
    ("e4m3_ties_away", "return np.sign(x) * (np.round(a / q) * q)",
     "return np.sign(x) * (np.floor(a / q + 0.5) * q)"),
    ("e4m3_no_subnormals", "e = np.maximum(e, -6.0)", "e = np.maximum(e, -60.0)"),
    ("e4m3_four_mantissa_bits", "q = 2.0 ** (e - 3.0)", "q = 2.0 ** (e - 4.0)"),
    ("fp8_scale_unscaled", "return _attention_from_levels(q8, lk, lvv, level_map, p, sc * s_q * s_k, qblocks)",
     "return _attention_from_levels(q8, lk, lvv, level_map, p, sc * s_q, qblocks)"),
    ("fp8pv_p_unquantized", "P8 = e4m3_round(2.0 ** (tr - M + 7))", "P8 = 2.0 ** (tr - M + 7)"),
    ("fp8pv_sum_unquantized", "l8 = float(np.sum(P8))", "l8 = float(np.sum(2.0 ** (tr - M + 7)))"),
    ("fp8pv_reference_at_max", "P8 = e4m3_round(2.0 ** (tr - M + 7))", "P8 = e4m3_round(2.0 ** (tr - M)) * 128.0"),
    ("fp8pv_reference_not_integer", "M = math.ceil(float(np.max(tr)))", "M = float(np.max(tr))"),
    ("fp8pv_v_unscaled", "o[qi[r]] = s_v * (P8 @ Vb[vis[r]]) / l8", "o[qi[r]] = (P8 @ Vb[vis[r]]) / l8"),
    ("index_descending", "sel = [kb for kb in range(nkb) if rows[r, kb] == l]",
     "sel = [kb for kb in reversed(range(nkb)) if rows[r, kb] == l]"),
]


def _mutant_module(old, new, monkeypatch):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("psa_oracle_mutant")
    mod.__file__ = SRC
    monkeypatch.setitem(sys.modules, "psa_oracle_mutant", mod)
    exec(compile(src.replace(old, new), SRC, "exec"), mod.__dict__)
    mod.psa_oracle = mod
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_catches_mutant(monkeypatch, name, old, new):
    mod = _mutant_module(old, new, monkeypatch)
    monkeypatch.setattr(pins, "oracle", mod)
    caught = []
    for pin, entry in ALL_PINS.items():
        fn, tol = _pin(entry)
        try:
            with np.errstate(all="ignore"):
                err = fn()
        except Exception:
            err = np.inf
        if not (err < tol):
            caught.append(pin)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    mod = _mutant_module("SKIP = -1\n", "SKIP = -1\n", monkeypatch)
    monkeypatch.setattr(pins, "oracle", mod)
    for pin, entry in ALL_PINS.items():
        fn, tol = _pin(entry)
        assert fn() < tol, pin
