"""The CPU oracle against its pins (no GPU). See tests/pins.py for what each pin compares."""
import numpy as np
import pytest

import oracle
import pins

TOL = 1e-12


@pytest.mark.parametrize("causal,nv", [(False, 512), (False, 488), (True, 512)])
def test_p1_all_l0_is_dense_attention(causal, nv):
    assert pins.pin_all_l0_dense(causal=causal, nv=nv) < TOL


def test_p2_binary_block_sparse():
    assert pins.pin_binary_block_sparse() < TOL


@pytest.mark.parametrize("seed", [4, 40])
def test_p3_upsample_equivalence(seed):
    assert pins.pin_upsample_equivalence(seed) < TOL


@pytest.mark.parametrize("level", [1, 2, 3])
def test_p4_constant_runs(level):
    assert pins.pin_constant_runs(level) < TOL


def test_p5_all_skip_row():
    assert pins.pin_all_skip_row() < TOL


def test_p6_weight_multiplicity():
    assert pins.pin_weight_multiplicity() < TOL


def test_p7_pyramid():
    assert pins.pin_pyramid() < TOL


@pytest.mark.parametrize("causal", [False, True])
def test_p8_sampling_all_rows(causal):
    assert pins.pin_sampling_all_rows(causal) < TOL


@pytest.mark.parametrize("causal", [False, True])
def test_p8_sampling_padded(causal):
    assert pins.pin_sampling_padded(causal) < TOL


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_attention_grouping(causal):
    assert pins.pin_gqa_attention(causal) < TOL


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_grouping(causal):
    assert pins.pin_gqa_backward(causal) < TOL


def test_gqa_mask_grouping():
    assert pins.pin_gqa_mask() < TOL


@pytest.mark.parametrize("causal", [False, True])
def test_p8_antidiag_stride1(causal):
    assert pins.pin_antidiag_stride1(causal) < TOL


def test_p8_antidiag_orientation_and_sum():
    assert pins.pin_antidiag_orientation_and_sum() < TOL


def test_p8_meankey_constant_blocks():
    assert pins.pin_meankey_constant_blocks() < TOL


def test_p8_meankey_causal_blocks():
    assert pins.pin_meankey_causal_blocks() < TOL


def test_p8_cossim():
    assert pins.pin_cossim() < TOL


def test_sample_offsets():
    assert pins.pin_sample_offsets() == 0


@pytest.mark.parametrize("case", pins.golden_assign_cases(), ids=lambda c: c["name"])
def test_p9_assign_golden(case):
    assert pins.pin_assign_case(case) == 0


def test_build_index_matches_nonzero():
    assert pins.pin_build_index() == 0


def test_build_index_rejects_bad_values():
    lm = np.zeros((1, 1, 2, 4), dtype=np.int8)
    lm[0, 0, 1, 2] = 5
    with pytest.raises(ValueError):
        oracle.build_index(lm)


def test_antidiag_rows_sum_to_one_with_padding():
    rng = np.random.default_rng(0)
    n, nv, d = 512, 384, 8
    p = oracle.Problem(seq_len=n, seq_valid=nv, head_dim=d, block_q=128, block_k=64)
    q = rng.standard_normal((n, d)); k = rng.standard_normal((n, d))
    q[nv:] = 0; k[nv:] = 0
    M = oracle.mask_scores_antidiag(q, k, p, stride=8)
    assert np.allclose(M[:3].sum(1), 1.0, atol=1e-12)
    assert np.all(M[3] == 0)            # query block 3 = tokens 384..511 is all pad
    assert np.all(M[:, 6:] == 0)        # KV blocks 6, 7 = tokens 384..511 are all pad


def test_padded_query_block_is_all_skip():
    p = oracle.Problem(seq_len=256, seq_valid=128, head_dim=8, block_q=64, block_k=64)
    M = np.zeros((4, 4))
    lm = oracle.assign_levels(M, None, p, oracle.AssignParams((0.5, 0.7, 0.8, 0.9)))
    assert np.all(lm[2:] == -1)
    assert np.all(lm[:2, 0] == 0)


def test_causal_pooled_visibility_uses_last_token():
    """A pooled token on the causal diagonal is visible to query i iff its last constituent
    token is <= i: query 7 sees the level-3 token covering 0..7, query 6 does not."""
    d = 4
    p = oracle.Problem(seq_len=64, seq_valid=64, head_dim=d, block_q=64, block_k=64,
                       causal=True)
    rng = np.random.default_rng(1)
    q = rng.standard_normal((64, d)); k = rng.standard_normal((64, d)); v = rng.standard_normal((64, d))
    o, lse = oracle.attention_head(q, k, v, np.array([[3]], dtype=np.int8), p)
    assert np.all(np.isneginf(lse[:7])) and np.all(o[:7] == 0)
    assert np.allclose(o[7], v[:8].mean(0), atol=1e-14)


@pytest.mark.parametrize("causal,nv,H,Hkv", [(False, 120, 2, 1), (True, 128, 2, 2), (True, 112, 1, 1)])
def test_pbwd_finite_difference(causal, nv, H, Hkv):
    assert pins.pin_bwd_finite_difference(causal, nv, H, Hkv) < 1e-6


@pytest.mark.parametrize("causal,nv", [(False, 256), (False, 232), (True, 256)])
def test_pbwd_all_l0_is_dense_autograd(causal, nv):
    assert pins.pin_bwd_all_l0_autograd(causal, nv) < 1e-10


@pytest.mark.parametrize("level", [1, 2, 3])
def test_pbwd_constant_runs(level):
    assert pins.pin_bwd_constant_runs(level) < 1e-10


def test_pfp8_e4m3_round_is_torch_e4m3():
    assert pins.pin_e4m3_round() == 0.0


def test_pfp8_scale():
    assert pins.pin_fp8_scale() < 1e-9


@pytest.mark.parametrize("causal", [False, True])
def test_pfp8_qk_reduces_to_attention(causal):
    assert pins.pin_fp8qk_reduces_to_attention(causal) < 1e-12


def test_pfp8_pv_worked_rows():
    assert pins.pin_fp8pv_worked_rows() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_pfp8_pv_powers_of_two(causal):
    assert pins.pin_fp8pv_powers_of_two(causal) < 1e-12


def test_bf16_round_matches_torch():
    assert pins.pin_bf16_round() == 0.0


def test_bf16_pooled_attention_reading():
    assert pins.pin_bf16_pooled_attention() < TOL
