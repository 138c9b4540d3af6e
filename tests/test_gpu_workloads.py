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
from gpu_util import (DeviceWorkload, check_attention, check_scores, check_topk, log, to_host)

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


def _run(c, n_sample=16, always=()):
    wl = synth.make_workload(c)
    dw = DeviceWorkload(wl)
    f = dw.forward(keep_scores=True, keep_idx=True)
    log(f"[{c.name}] dsa_forward B={c.B} T={c.T} N={c.N} k={c.top_k} m={c.m} W={c.W}")
    f.run()
    torch.cuda.synchronize()
    rows = _sample_rows(c, n_sample, always)
    run = oracle.QueryRunner(wl)
    swaps, worst_s, worst_a = 0, 0.0, (0.0, 0.0)
    for b, t in rows:
        sc = to_host(f.scores[b, t])
        ix = to_host(f.idx[b, t])
        out = oracle.decode(to_host(f.out[b, t]))
        lse = to_host(f.lse[b, t])
        ref_sc = run.scores(b, t)
        nv = oracle.n_vis(int(wl.q_pos()[b, t]), c.m, c.N)
        what = f"{c.name} b={b} t={t}"
        worst_s = max(worst_s, check_scores(sc, ref_sc, nv, what=what))
        swaps += check_topk(ix, ref_sc, nv, c.top_k, what=what)
        ro, rl = run.attend(b, t, ix)
        mx, s = check_attention(out, lse, ro, rl, what=what)
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
