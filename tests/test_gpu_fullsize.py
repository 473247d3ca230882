"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times, and at
the largest sizes psa_mask accepts.

The whole path runs on the full tensors exactly as the benchmark's step does
(psa_build_pyramid, psa_mask or the drawn map, psa_build_index, psa_attn_fwd_indexed, on one
stream, into preallocated buffers). The oracle cannot run a full layer in seconds, so it
checks outputs it can compute one by one, on sampled heads and query blocks:
  * pooled K/V rows of the sampled KV heads (every level);
  * float32 pooled rows (out_dtype float32) at the 1e-5 bar, and the bf16 levels the
    attention reads;
  * mask rows: block masses, similarities and the level map row of each sampled query block,
    recomputed by the oracle from the same inputs (bit for bit but at decisions within the
    oracle's own 1e-12 margin; near-threshold rows are certified in float64 on the GPU);
  * the attention output and lse of every query of each sampled block, on the oracle's own
    level map row, against the exact-mean reading and the bf16-pooled-level reading (lse 1e-3).
Sampled blocks include the first block, the last one (ragged: it holds the pad rows) and, for
the causal workload, blocks whose diagonal split the query block.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
import video_transformers_amd as psa
from gpu_util import (CERT_MARGINS, DEV, announce, assign_params, check_attention, check_map,
                      dispatch_order, mask_params, need_gpu, oracle_margin_entries, order_share)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()


def _sampled_heads(wl):
    H = wl.heads_q
    return sorted({0, H // 2, H - 1})


def _sampled_qblocks(wl, h):
    n = wl.n_qblocks
    rng = np.random.default_rng(wl.seed * 131 + h)
    picks = {0, n - 1, n // 2, int(rng.integers(1, max(2, n - 1)))}
    if wl.text_end > wl.text_begin:
        picks.add(wl.text_begin // wl.block_q)        # a block holding text queries
    return sorted(picks)


def _run_path(wl, qd, kd, vd):
    """One step of the path, as the benchmark launches it. Returns every output."""
    prob = psa.make_problem(qd, kd, vd, block_q=wl.block_q, block_k=wl.block_k,
                            causal=wl.causal, seq_valid=wl.seq_valid)
    kp, vp = psa.build_pyramid(kd, vd, prob)
    M = sim = None
    cert = []
    if wl.map_source == "mask":
        lm, M, sim = psa.mask(qd, kd, prob, mask_params(wl), cert_counts=cert)
    else:
        lm = torch.from_numpy(W.make_map(wl)).to(DEV)
    row_ptr, col_idx, err = psa.build_index(lm, prob)
    o, lse = psa.attn_fwd_indexed(qd, kd, vd, kp, vp, row_ptr, col_idx, prob)
    torch.cuda.synchronize()
    assert err.item() == 0
    # the dispatch order at full size: a permutation, from its definition bit for bit
    rows = lm.numel() // prob.n_kblocks
    rp = row_ptr.cpu().numpy()
    assert np.array_equal(np.sort(rp[rows * 4 + 1:]), np.arange(rows))
    assert np.array_equal(rp[rows * 4 + 1:], dispatch_order(rp, rows, wl.n_qblocks * wl.group, order_share(wl)))
    return kp, vp, lm, M, sim, o, lse, cert


# the five workloads, plus block-mean scoring on the Wan-like 32k layer, plus two layers at the
# largest NKB whose per-row assignment fits its 64 KB of LDS (sampling with 8 samples: 1328
# blocks; antidiagonal with stride 8 and 128-token query blocks: 830 blocks, which also runs
# the general antidiagonal scorer: N / 8 is not a whole number of 128-column tiles)
FULL = list(W.ALL) + [
    W.WAN13B_32K.replace(name="wan2.1-1.3b_32k-meankey", mask_mode="meankey"),
    W.WAN13B_32K.replace(name="wan-like-sampling-nkb1328", heads_q=2, heads_kv=2, seq_len=1328 * 64,
                         seq_valid=1328 * 64 - 8, block_q=64),
    W.QWEN25VL_32K.replace(name="qwen-like-antidiag-nkb830", heads_q=2, heads_kv=1, seq_len=830 * 64,
                           seq_valid=830 * 64),
]


@pytest.mark.parametrize("wl", FULL, ids=[w.name for w in FULL])
def test_fullsize_sampled_parity(wl):
    announce(f"full size {wl.name}: B{wl.batch} H{wl.heads_q}/{wl.heads_kv} N{wl.seq_len} "
             f"d{wl.head_dim}")
    q, k, v = W.make_qkv(wl)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kp, vp, lm, M, sim, o, lse, cert = _run_path(wl, qd, kd, vd)
    if cert:
        print(f"[{wl.name}] certification: {cert[0]} rows rescored in float64, {cert[1]} left "
              f"(of {wl.batch * wl.heads_q * wl.n_qblocks})", flush=True)
        assert cert[1] == 0
    kp32 = vp32 = None
    if wl.dtype == "bf16":
        prob = psa.make_problem(qd, kd, vd, block_q=wl.block_q, block_k=wl.block_k,
                                causal=wl.causal, seq_valid=wl.seq_valid)
        kp32, vp32 = psa.build_pyramid(kd, vd, prob, out_dtype=torch.float32)
        assert torch.equal(kp32.to(torch.bfloat16), kp) and torch.equal(vp32.to(torch.bfloat16), vp)
    p = oracle.Problem.of(wl)
    a = assign_params(wl)
    g = wl.group
    f32 = wl.dtype == "f32"
    compared = skipped = 0
    for h in _sampled_heads(wl):
        hk = h // g
        qh = oracle.as_f64(q[0, h])
        kh = oracle.as_f64(k[0, hk])
        vh = oracle.as_f64(v[0, hk])
        qbs = _sampled_qblocks(wl, h)

        # pyramid rows of this KV head
        ref = oracle.pack_pyramid(kh)
        got = kp[0, hk].double().cpu().numpy()
        tol = 1e-5 * np.abs(ref).max() if f32 else None
        for name, r, gt, g32 in (("k", ref, got, kp32), ("v", oracle.pack_pyramid(vh),
                                 vp[0, hk].double().cpu().numpy(), vp32)):
            if f32:
                assert np.abs(gt - r).max() <= tol, f"pooled {name} head {hk}"
            else:
                assert np.all(np.abs(gt - r) <= np.abs(r) * 2.0 ** -7 + 1e-30), \
                    f"pooled {name} head {hk}: beyond one bf16 ulp of the exact mean"
                x32 = g32[0, hk].double().cpu().numpy()
                assert np.abs(x32 - r).max() <= 1e-5 * np.abs(r).max(), f"f32 pooled {name} head {hk}"
                assert np.linalg.norm(x32 - r) <= 1e-5 * np.linalg.norm(r), f"f32 pooled {name} head {hk}"

        # the level map rows the oracle assigns
        lm_ref = np.full((p.n_qblocks, p.n_kblocks), oracle.SKIP, dtype=np.int8)
        marg = np.zeros_like(lm_ref, dtype=bool)
        lm_gpu = lm[0, h].cpu().numpy()
        if wl.map_source == "mask":
            if wl.mask_mode == "sampling":
                Mr = oracle.mask_scores_sampling(qh, kh, p, wl.samples_per_qblock, qblocks=qbs)
            elif wl.mask_mode == "meankey":
                Mr = oracle.mask_scores_meankey(qh, kh, p, qblocks=qbs)
            else:
                Mr = oracle.mask_scores_antidiag(qh, kh, p, wl.antidiag_stride, qblocks=qbs)
            simr = oracle.block_cossim(kh, p) if wl.cos_sim_min > 0 else None
            Mg = M[0, h].double().cpu().numpy()
            dM = np.abs(Mg[qbs] - Mr[qbs]).max()
            print(f"[{wl.name}] head {h}: block mass max abs diff {dM:.3e}", flush=True)
            assert dM <= 2e-6
            # the premise of the certification margins (absolute, relative): a row's running
            # sums are off by at most its summed absolute mass error, which must stay below the
            # absolute margin, and two masses can trade places only within the sum of their
            # relative errors, each of which must stay below half the relative margin
            m_abs, m_rel = CERT_MARGINS[wl.mask_mode]
            row_abs = np.abs(Mg[qbs] - Mr[qbs]).sum(-1).max()
            big = Mr[qbs] > 1e-9
            rel = (np.abs(Mg[qbs] - Mr[qbs])[big] / Mr[qbs][big]).max()
            print(f"[{wl.name}] head {h}: summed abs mass error per row <= {row_abs:.3e} "
                  f"(margin {m_abs:g}), relative <= {rel:.3e} (half margin {m_rel / 2:g})", flush=True)
            assert row_abs < m_abs and rel < m_rel / 2
            if simr is not None:
                ds = np.abs(sim[0, hk].double().cpu().numpy() - simr).max()
                print(f"[{wl.name}] kv head {hk}: similarity max abs diff {ds:.3e}", flush=True)
                assert ds <= 1e-6
            for qb in qbs:
                lm_ref[qb] = oracle.assign_row(Mr[qb], simr, p, a, qb)
            marg = oracle_margin_entries(Mr[None, None], None if simr is None else simr[None, None],
                                         p, a, qblocks=qbs)[0, 0]
        else:
            lm_ref = W.make_map(wl, [h])[0, 0]
        check_map(lm_gpu[qbs], lm_ref[qbs], marg[qbs], f"{wl.name} head {h} qblocks {qbs}")

        # attention of the sampled blocks on the oracle's map rows (a row may differ only at a
        # decision within the oracle's own 1e-12 margin: such a block is counted, not compared)
        agree = [qb for qb in qbs if np.array_equal(lm_gpu[qb], lm_ref[qb])]
        skipped += len(qbs) - len(agree)
        if not agree:
            continue
        o_ref, lse_ref = oracle.attention_head(qh, kh, vh, lm_ref, p, qblocks=agree)
        rnd = None
        if not f32:
            o_r, lse_r = oracle.attention_head(qh, kh, vh, lm_ref, p, qblocks=agree,
                                               pooled_round="bf16")
        rows = np.concatenate([np.arange(qb * wl.block_q, (qb + 1) * wl.block_q) for qb in agree])
        valid = rows < wl.seq_valid
        og = o[0, h, rows].double().cpu().numpy()
        lg = lse[0, h, rows].double().cpu().numpy()
        if not f32:
            rnd = (o_r[rows][valid][None], lse_r[rows][valid][None])
        check_attention(torch.from_numpy(og[valid][None]), torch.from_numpy(lg[valid][None]),
                        o_ref[rows][valid][None], lse_ref[rows][valid][None],
                        int(valid.sum()), f32, f"{wl.name} head {h} qblocks {agree}", rnd)
        assert np.all(og[~valid] == 0.0), "pad query rows must be zero"
        assert np.all(np.isneginf(lg[~valid]))
        compared += len(agree)
    print(f"[{wl.name}] compared {compared} query blocks, {skipped} left out (map row differing "
          f"within the oracle's 1e-12 margin)", flush=True)
    assert compared > 0
