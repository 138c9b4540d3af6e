"""The five DSA / CSA workloads at full size through dsa_forward, against the fp64 oracle.

dsa_forward runs in the launch configuration the benchmark times; the oracle recomputes sampled
query rows one by one (all rows where it is cheap): indexer scores, the top-k set (ties within
1e-4 relative of the k-th score allowed) and attention re-evaluated on the GPU's validated set.
"Sharp" variants (q, kv ~ N(0,1), scale 4/sqrt(D_K)) give the attention bound teeth.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DeviceWorkload, check_attention, check_compressed, check_scores,
                      check_topk, log, score_mass, to_host, visible)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.empty_cache()


def _sample_rows(c, n, always=()):
    rows = [(b, t) for b in range(c.B) for t in range(c.T)]
    if len(rows) <= n:
        return rows
    rng = np.random.default_rng(c.seed)
    pick = {rows[i] for i in rng.choice(len(rows), n, replace=False)}
    pick |= {(0, t) for t in always if t < c.T}
    pick |= {rows[0], rows[-1]}
    return sorted(pick)


def _run(c, n_sample=16, always=(), bf16_scale_allowance=False):
    wl = synth.make_workload(c)
    dw = DeviceWorkload(wl)
    f = dw.forward(keep_scores=True, keep_idx=True)
    log(f"[{c.name}] dsa_forward B={c.B} T={c.T} N={c.N} k={c.top_k} m={c.m} W={c.W}")
    f.run()
    torch.cuda.synchronize()
    rows = _sample_rows(c, n_sample, always)
    run = oracle.QueryRunner(wl)
    if c.compress:
        # the call pooled kv_raw itself: its entries within one ulp of the fp64 means, then the
        # attention is compared on those bytes (as for HCA)
        check_compressed(dw, run)
    swaps, worst_s, worst_a = 0, 0.0, (0.0, 0.0)
    for b, t in rows:
        sc = to_host(f.scores[b, t])
        ix = to_host(f.idx[b, t])
        out = oracle.decode(to_host(f.out[b, t]))
        lse = to_host(f.lse[b, t])
        ref_sc = run.scores(b, t)
        nv = visible(wl, b, t)
        what = f"{c.name} b={b} t={t}"
        worst_s = max(worst_s, check_scores(sc, ref_sc, nv, what=what))
        swaps += check_topk(ix, ref_sc, nv, c.top_k, what=what)
        ro, rl = run.attend(b, t, ix)
        mx, s = check_attention(out, lse, ro, rl, what=what,
                                bf16_scale_allowance=bf16_scale_allowance)
        worst_a = max(worst_a, (mx, s))
    log(f"[{c.name}] rows={len(rows)} score rel err {worst_s:.2e}, tie swaps {swaps}, "
        f"attention max abs err {worst_a[0]:.3e} (max|ref| {worst_a[1]:.3e})")
    del f, dw


def test_tiny():
    _run(synth.CONFIGS["tiny"])
    _run(synth.CONFIGS["tiny"].sharp())


def test_decode():
    _run(synth.CONFIGS["decode"])
    _run(synth.CONFIGS["decode"].sharp())


def test_decode_fp8_indexer():
    _run(synth.CONFIGS["decode_fp8"])
    _run(synth.CONFIGS["decode_fp8"].sharp())


def test_prefill_fp8_indexer():
    _run(synth.CONFIGS["prefill_fp8"], n_sample=12, always=(0, 2047, 2048, 32767))


def test_csa_decode_fp4():
    _run(synth.CONFIGS["csa_decode"])
    _run(synth.CONFIGS["csa_decode"].sharp())


def test_prefill():
    _run(synth.CONFIGS["prefill"], n_sample=16, always=(0, 1, 2046, 2047, 2048, 2049, 32767))


def test_prefill_sharp_8k():
    c = synth.CONFIGS["prefill"].with_(T=8192, N=8192).sharp()
    _run(c, n_sample=12, always=(0, 2047, 2048, 8191))


def test_csa_prefill():
    _run(synth.CONFIGS["csa_prefill"], n_sample=12)


def test_csa_prefill_sharp_small():
    c = synth.CONFIGS["csa_prefill"].with_(N=8192, T=2048, pos0=32768 - 2048).sharp()
    _run(c, n_sample=12)


def _run_fused(c, periodic=0):
    """dsa_forward on few query rows with N <= 32768, where the attention kernel selects the
    top-k itself. The selection is checked exactly against the oracle's top-k over the GPU's own
    fp32 scores (the same decision in the same precision: the set is unique, exact ties go to the
    lowest index), the row in ascending index order with -1 padding, and attention against the
    oracle. periodic > 0 repeats the indexer keys with that period, so whole groups of entries
    tie at the k-th score."""
    wl = synth.make_workload(c)
    if periodic:
        k = wl.k_I()
        wl._cache["k_I"] = np.ascontiguousarray(np.tile(k[:, :periodic], (1, -(-c.N // periodic), 1))[:, :c.N])
    dw = DeviceWorkload(wl)
    f = dw.forward(keep_scores=True, keep_idx=True)
    log(f"[{c.name}] fused dsa_forward B={c.B} T={c.T} N={c.N} k={c.top_k} m={c.m} W={c.W} "
        f"periodic={periodic}")
    f.run()
    torch.cuda.synchronize()
    run = oracle.QueryRunner(wl)
    worst = 0.0
    for b in range(c.B):
        for t in range(c.T):
            what = f"{c.name} b={b} t={t}"
            sc = to_host(f.scores[b, t])
            ix = to_host(f.idx[b, t])
            nv = visible(wl, b, t)
            cnt = min(nv, c.top_k)
            ref, rcnt = oracle.topk_row(sc[:nv].astype(np.float64), nv, c.top_k)
            assert rcnt == cnt
            assert np.array_equal(ix[:cnt], ref[:cnt]), f"{what}: selection differs"
            assert (ix[cnt:] == -1).all(), f"{what}: padding"
            if b == 0 or t % 7 == 0:
                worst = max(worst, check_scores(sc, run.scores(b, t), nv, what=what))
                out = oracle.decode(to_host(f.out[b, t]))
                ro, rl = run.attend(b, t, ix)
                check_attention(out, to_host(f.lse[b, t]), ro, rl, what=what)
    log(f"[{c.name}] fused selection exact on {c.B * c.T} rows, score rel err {worst:.2e}")
    del f, dw


def test_fused_selection_ragged():
    # 96 rows at positions 100..2967 of a 3001-entry context: rows up to 2047 keep everything
    c = synth.CONFIGS["decode"].with_(B=2, T=48, N=3001, pos0=100, pos_stride=61, name="fused")
    _run_fused(c)
    _run_fused(c.with_(name="fused_ties", seed=7), periodic=97)


def test_fused_selection_csa_window():
    # CSA blocks (m=4, mxfp4 keys) with a 128-token raw window; N=5003 is not a multiple of 4
    p0 = 4 * 3000
    c = synth.CONFIGS["csa_decode"].with_(B=2, T=40, N=5003, pos0=p0, pos_stride=203,
                                          raw_base=p0 - 127, n_raw=203 * 39 + 128,
                                          name="fused_csa")
    _run_fused(c)


# ------------------------------------------------------------ heavily compressed attention ----

def _run_hca(c, n_sample=16):
    """hca_forward against the oracle's dense composition (every visible block + window)."""
    wl = synth.make_workload(c)
    dw = DeviceWorkload(wl)
    f = dw.hca()
    log(f"[{c.name}] hca_forward B={c.B} T={c.T} N={c.N} m={c.m} W={c.W} compress={c.compress}")
    f.run()
    torch.cuda.synchronize()
    run = oracle.QueryRunner(wl)
    if c.compress:
        check_compressed(dw, run)
    worst = (0.0, 0.0)
    for b, t in _sample_rows(c, n_sample):
        r = run.run_dense(b, t)
        out = oracle.decode(to_host(f.out[b, t]))
        worst = max(worst, check_attention(out, to_host(f.lse[b, t]), r["out"], r["lse"],
                                           what=f"{c.name} b={b} t={t} n_vis={r['n_vis']}"))
    log(f"[{c.name}] attention max abs err {worst[0]:.3e} (max|ref| {worst[1]:.3e})")
    del f, dw


def test_hca_decode():
    _run_hca(synth.CONFIGS["hca_decode"])
    _run_hca(synth.CONFIGS["hca_decode"].sharp())


def test_hca_prefill():
    _run_hca(synth.CONFIGS["hca_prefill"], n_sample=12)
    _run_hca(synth.CONFIGS["hca_prefill"].with_(T=1024, pos0=131072 - 1024).sharp(), n_sample=12)


# ------------------------------------------------------------- head weights of either sign ----
# The head weights come from a learned projection, so their sign is free: scores of either sign,
# top-k thresholds below zero, and rows of exact +-0 scores (a zero key row scores exactly 0 for
# every query; a zero weight row scores 0 everywhere). Each shape below reaches one selection
# kernel: <= 128 rows with N <= 32768 the fused selection inside the attention kernel, more
# rows the register radix select, N > 32768 the chunk filter + candidate select (MXFP4 keys).

def _plant_special_rows(wl):
    """Rewrite the host inputs (before upload; the oracle sees the same bytes):
      sequence 1: every weight negative, every 7th key zero (fewer zero keys than k: all of them
                  are selected, at the top of a row of negative scores);
      sequence 2: every weight zero (the whole row scores exactly 0: the first k are taken);
      sequence 3: every weight negative and the first 3000 keys zero (a tie at 0 across more
                  entries than k: the lowest zero-key indices are taken);
      sequence 4: half of the weights -0.0, the rest negative (scores of -0 and +0 rank equal);
      sequence 5 (bf16 keys): key s scaled by 1 + 3 s / N, so scores grow along the row and the
                  top k crowd into its last entries.
    Sequences beyond B are skipped."""
    c = wl.cfg
    w = wl.w().copy()
    k = wl.k_I()
    if isinstance(k, tuple):
        k = (k[0].copy(), k[1])
        codes = k[0]
    else:
        k = k.copy()
        codes = k
    if c.B > 1:
        w[1] = -np.abs(w[1])
        codes[1, ::7] = 0
    if c.B > 2:
        w[2] = 0.0
    if c.B > 3:
        w[3] = -np.abs(w[3])
        codes[3, :3000] = 0
    if c.B > 4:
        w[4] = -np.abs(w[4])
        w[4, :, : c.H_I // 2] = -0.0
    if c.B > 5 and not isinstance(k, tuple):
        f = (k[5].astype(np.uint32) << 16).view(np.float32)
        f = f * (1.0 + 3.0 * np.arange(c.N, dtype=np.float32) / c.N)[:, None]
        u = f.view(np.uint32)
        k[5] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # RNE to bf16
    wl._cache["w"] = np.ascontiguousarray(w, np.float32)
    wl._cache["k_I"] = k


def _run_exact_selection(c, n_attend=8):
    """dsa_forward with every row's selection checked exactly: the oracle's top-k over the GPU's
    own fp32 scores (the same decision in the same precision, so the set is unique; exact ties
    go to the lowest index), count and -1 padding; the scores of sampled rows against the
    oracle's, and attention on the GPU's set for sampled rows."""
    wl = synth.make_workload(c)
    _plant_special_rows(wl)
    dw = DeviceWorkload(wl)
    f = dw.forward(keep_scores=True, keep_idx=True)
    log(f"[{c.name}] dsa_forward B={c.B} T={c.T} N={c.N} k={c.top_k} m={c.m} W={c.W} "
        f"w ~ U({c.w_lo}, 1) with planted rows")
    f.run()
    torch.cuda.synchronize()
    run = oracle.QueryRunner(wl)
    rows = [(b, t) for b in range(c.B) for t in range(c.T)]
    check = set(_sample_rows(c, n_attend)) | {(b, 0) for b in range(min(c.B, 5))}
    worst, worst_b, negative_tau, zero_tau = 0.0, 0.0, 0, 0
    for b, t in rows:
        what = f"{c.name} b={b} t={t}"
        sc = to_host(f.scores[b, t])
        ix = to_host(f.idx[b, t])
        nv = visible(wl, b, t)
        cnt = min(nv, c.top_k)
        ref, rcnt = oracle.topk_row(sc[:nv].astype(np.float64), nv, c.top_k)
        assert rcnt == cnt
        assert np.array_equal(np.sort(ix[:cnt]), ref[:cnt]), f"{what}: selection differs"
        assert (ix[cnt:] == -1).all(), f"{what}: padding"
        if nv > c.top_k:
            tau = sc[ref[:cnt]].min()
            negative_tau += int(tau < 0)
            zero_tau += int(tau == 0)
        if (b, t) in check:
            mass = score_mass(wl, b, t)
            e = check_scores(sc, run.scores(b, t), nv, what=what, mass=mass,
                             dims=(c.H_I, c.D_I))
            if mass is None:
                worst = max(worst, e)
            else:
                worst_b = max(worst_b, e)
            out = oracle.decode(to_host(f.out[b, t]))
            ro, rl = run.attend(b, t, ix)
            check_attention(out, to_host(f.lse[b, t]), ro, rl, what=what)
    log(f"[{c.name}] selection exact on {len(rows)} rows ({negative_tau} with a negative and "
        f"{zero_tau} with a zero threshold), score rel err {worst:.2e} (positive weights), "
        f"largest error / fp32 accumulation bound {worst_b:.2e} (mixed signs)")
    assert negative_tau > 0 and zero_tau > 0
    del f, dw


def test_mixed_sign_weights_fused_decode():
    # the decode workload's shape (16 rows, N = 8192): selection inside the attention kernel
    _run_exact_selection(synth.CONFIGS["decode"].with_(w_lo=-1.0, name="decode_mixed_w"))


def test_mixed_sign_weights_prefill_rows():
    # 5 x 60 = 300 rows in one call: the register radix select of topk_select
    c = synth.CONFIGS["decode"].with_(B=5, T=60, N=3500, pos0=100, pos_stride=57, top_k=1024,
                                      w_lo=-1.0, name="prefill_rows_mixed_w")
    _run_exact_selection(c, n_attend=12)


def test_mixed_sign_weights_sampled_rows():
    # 6 x 40 rows over 5000 .. 19430 visible entries (> 4096: the streaming top-k's sampled
    # threshold; the planted rows of ties and the rising row take its exact fallback)
    c = synth.CONFIGS["decode"].with_(B=6, T=40, N=20000, pos0=5000, pos_stride=370, top_k=1024,
                                      w_lo=-1.0, name="sampled_rows_mixed_w")
    _run_exact_selection(c, n_attend=10)


@pytest.mark.parametrize("k_dt", ["mxfp4", "mxfp8"])
def test_mixed_sign_weights_indexer_segments(k_dt):
    # >= 2^20 keys per call over N > 32768 blocks: the decode indexer's epilogue writes the
    # top-k's candidate segments itself (its chunks are interleaved, so ties at the threshold
    # go through the exact fallback); visibility from 25000 to all 40000 blocks
    c = synth.CONFIGS["csa_decode"].with_(B=5, T=6, N=40000, pos0=100003, pos_stride=12000, W=0,
                                          n_raw=0, raw_base=0, k_dt=k_dt, w_lo=-1.0,
                                          name=f"indexer_segments_{k_dt}_mixed_w")
    _run_exact_selection(c, n_attend=6)


def test_mixed_sign_weights_csa_decode_fp4():
    # MXFP4 keys over N = 40000 blocks (> 32768): chunk filter + candidate select, CSA window
    p = 4 * 40000 - 1
    c = synth.CONFIGS["csa_decode"].with_(B=5, N=40000, pos0=p, raw_base=p + 1 - 128, w_lo=-1.0,
                                          name="csa_decode_mixed_w")
    _run_exact_selection(c)
