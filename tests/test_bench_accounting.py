"""The benchmark's work accounting (host logic, no GPU): the executed (valid query, visible
pooled key) pairs that every TFLOP/s figure is computed from, against a brute-force count of
the same definition. A pooled row j of level l stands for tokens [j 2^l, (j + 1) 2^l) (PSA
summary article at rg.mbintangr.com, "Method": keys and values mean-pooled by 2^l); it is
visible to query i iff its last token is below seq_valid and, when causal, not after i."""
import numpy as np
import pytest

import bench
import workloads as W


def _brute(lm, wl):
    B, H, nqb, nkb = lm.shape
    nv, bq = wl.seq_valid, wl.block_q
    total = 0
    for b in range(B):
        for h in range(H):
            for qb in range(nqb):
                for i in range(qb * bq, min(qb * bq + bq, nv)):
                    for kb in range(nkb):
                        l = int(lm[b, h, qb, kb])
                        if l < 0:
                            continue
                        rows = 64 >> l
                        for j in range(kb * rows, (kb + 1) * rows):
                            last = ((j + 1) << l) - 1
                            if last <= nv - 1 and (not wl.causal or last <= i):
                                total += 1
    return total


CASES = [(causal, bq, nv) for causal in (False, True) for bq in (64, 128) for nv in (512, 504, 389)]


@pytest.mark.parametrize("causal,bq,nv", CASES)
def test_executed_pairs_brute_force(causal, bq, nv):
    wl = W.Workload(name="acct", seed=7, batch=1, heads_q=2, heads_kv=2, head_dim=64, seq_len=512,
                    seq_valid=nv, block_q=bq, causal=causal, map_source="iid")
    rng = np.random.default_rng(nv * 3 + bq + causal)
    lm = rng.choice([-1, 0, 1, 2, 3], size=(1, 2, 512 // bq, 8)).astype(np.int8)
    assert bench.executed_pairs(lm, wl) == _brute(lm, wl)


@pytest.mark.parametrize("causal", [False, True])
def test_all_level0_is_dense_and_all_skip_is_empty(causal):
    wl = W.Workload(name="acct", seed=7, batch=2, heads_q=3, heads_kv=3, head_dim=64, seq_len=1024,
                    seq_valid=1000, block_q=128, causal=causal, map_source="iid")
    shape = (2, 3, 1024 // 128, 1024 // 64)
    assert bench.executed_pairs(np.zeros(shape, np.int8), wl) == bench.dense_pairs(wl)
    assert bench.executed_pairs(np.full(shape, -1, np.int8), wl) == 0


def test_one_pooled_block():
    """One level-3 block listed for one full query block: 8 pooled keys for each of its queries."""
    wl = W.Workload(name="acct", seed=7, batch=1, heads_q=1, heads_kv=1, head_dim=64, seq_len=512,
                    seq_valid=512, block_q=128, map_source="iid")
    lm = np.full((1, 1, 4, 8), -1, np.int8)
    lm[0, 0, 1, 5] = 3
    assert bench.executed_pairs(lm, wl) == 128 * 8
