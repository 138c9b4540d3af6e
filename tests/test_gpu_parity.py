"""GPU parity of each C-ABI call against the fp64 oracle, on the same seeded inputs.

Sizes span several tiles with ragged tails and run in seconds; the full-size workloads are in
test_gpu_workloads.py. Every call goes through the C ABI (lightning_indexer_top_03_amd).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (DeviceWorkload, check_attention, check_compressed, check_scores,
                      check_topk, log, to_dev, to_host, visible)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import lightning_indexer_top_03_amd as dsa


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _cfg(base, **kw):
    return synth.CONFIGS[base].with_(**kw)


# --------------------------------------------------------------------------- compression ----

@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_compress_mean(dt):
    c = _cfg("csa_prefill", B=2, N=1000, n_raw=4003, dt=dt, name="compress_" + dt)
    raw = synth.normal(c.seed, synth.TID_KV, (2, 4003, 576), 1.0 / 24, dt)
    log(f"[compress {dt}] n_raw=4003 m=4")
    out = to_host(dsa.kv_compress_mean(to_dev(raw), 4))
    torch.cuda.synchronize()
    assert out.shape == (2, 1000, 576)
    for b in range(2):
        ref = oracle.compress_mean(raw[b], 4)
        got = oracle.decode(out[b])
        if dt == "f32":
            # fp32 sum of m terms, then one division: error <= ~m ulps of sum |x| / m
            mag = oracle.compress_mean(np.abs(raw[b]).astype(np.float32), 4)
            assert (np.abs(got - ref) <= 2.0 ** -21 * mag + 1e-30).all()
        else:
            # one RNE rounding of an fp32 sum: within one bf16 ulp of the exact mean
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
            assert (np.abs(got - ref) <= ulp).all()
            assert (np.abs(got - ref) <= 0.5 * ulp * (1 + 1e-6)).mean() > 0.999


# ------------------------------------------------------------------------------- indexer ----

def _run_indexer(c, label):
    wl = synth.make_workload(c)
    k = wl.k_I()
    kdev = (to_dev(k[0]), to_dev(k[1])) if c.k_dt in ("mxfp4", "mxfp8") else to_dev(k)
    q = wl.q_I()
    qdev = (to_dev(q[0]), to_dev(q[1])) if c.qi_dt == "mxfp8" else to_dev(q)
    log(f"[indexer {label}] B={c.B} T={c.T} N={c.N} q_I={c.qi_dt or c.dt} k_dt={c.k_dt}")
    sc = dsa.indexer_scores(qdev, to_dev(wl.w()), kdev, to_dev(wl.q_pos()), m=c.m)
    torch.cuda.synchronize()
    sc = to_host(sc)
    run = oracle.QueryRunner(wl)
    worst = 0.0
    rows = [(b, t) for b in range(c.B) for t in range(c.T)]
    if len(rows) > 48:
        rng = np.random.default_rng(0)
        pick = rng.choice(len(rows), 40, replace=False)
        rows = sorted({rows[i] for i in pick} | {rows[0], rows[-1]})
    for b, t in rows:
        ref = run.scores(b, t)
        nv = visible(wl, b, t)
        worst = max(worst, check_scores(sc[b, t], ref, nv, what=f"{label} b={b} t={t}"))
    log(f"[indexer {label}] max rel err {worst:.2e}")
    return sc


def test_indexer_decode_bf16_ragged():
    # decode-shaped (MFMA streaming kernel): ragged N, a partially visible row
    c = _cfg("decode", B=3, N=3001, name="idx_decode")
    c = c.with_(pos0=3000)
    _run_indexer(c, "decode")
    _run_indexer(c.with_(pos0=1234, name="idx_decode_partial"), "decode-partial")


def test_indexer_prefill_bf16_causal():
    # prefill-shaped (MFMA, keys in registers, queries through LDS): causal triangle, ragged
    c = _cfg("prefill", B=2, T=700, N=700, name="idx_prefill")
    _run_indexer(c, "prefill")
    # N % 4 != 0: score rows are not 16-byte aligned (per-element stores); queries start
    # mid-sequence so a key block is visible to some rows of a query block and not others
    _run_indexer(_cfg("prefill", B=1, T=333, N=1001, pos0=600, name="idx_prefill_odd"),
                 "prefill-odd")


def test_indexer_prefill_csa_blocks():
    c = _cfg("csa_prefill", B=1, T=300, N=900, pos0=3300, pos_stride=2, compress=False,
             n_raw=0, W=0, name="idx_csa")
    _run_indexer(c, "csa")


def test_indexer_mxfp4_keys():
    c = _cfg("csa_decode", B=2, N=5003, pos0=4 * 5003 - 1, name="idx_fp4")
    _run_indexer(c, "mxfp4")
    _run_indexer(c.with_(pos0=4 * 4000 + 2, name="idx_fp4_partial"), "mxfp4-partial")


def test_indexer_mxfp8_keys_and_queries():
    # fp8 keys against bf16 queries (two-part split) and against fp8 queries (one MFMA / step),
    # ragged N, positions before and past the end of the keys
    c = _cfg("decode", B=3, N=5003, pos0=4999, k_dt="mxfp8", name="idx_fp8")
    _run_indexer(c, "mxfp8-keys")
    _run_indexer(c.with_(qi_dt="mxfp8", pos0=3001, name="idx_fp8q"), "mxfp8-both")
    # fp8 queries against FP4 blocks (CSA), many rows in one call
    _run_indexer(_cfg("csa_decode", B=1, T=96, N=3001, pos0=4 * 2900, pos_stride=5,
                      qi_dt="mxfp8", name="idx_fp8q_fp4k"), "mxfp8-q-fp4-k")
    _run_indexer(_cfg("decode", B=1, T=70, N=2100, pos0=2030, qi_dt="mxfp8", k_dt="mxfp8",
                      name="idx_fp8_rows"), "mxfp8-rows")
    # causal prefill with fp8 queries and keys: several key blocks, ragged tail
    _run_indexer(_cfg("prefill", T=2100, N=2100, qi_dt="mxfp8", k_dt="mxfp8",
                      name="idx_fp8_prefill"), "mxfp8-prefill")
    # the scalar kernel (4 heads x 32 dims)
    _run_indexer(_cfg("tiny", dt="bf16", k_dt="mxfp8", name="tiny_fp8"), "tiny-fp8")
    _run_indexer(_cfg("tiny", dt="bf16", k_dt="mxfp8", qi_dt="mxfp8", name="tiny_fp8q"),
                 "tiny-fp8-both")


def test_indexer_generic_fp32_and_small_heads():
    _run_indexer(synth.CONFIGS["tiny"], "tiny-f32")
    _run_indexer(_cfg("tiny", dt="bf16", k_dt="bf16", name="tiny_bf16"), "tiny-bf16")
    _run_indexer(_cfg("tiny", dt="bf16", k_dt="mxfp4", name="tiny_fp4"), "tiny-fp4")


# --------------------------------------------------------------------------------- top-k ----

def _topk_case(label, n_rows, N, k, m=1, ties=False, pos=None, seed=0, order=None):
    rng = np.random.default_rng(seed)
    s = synth.normal(50 + seed, 1, (n_rows, N), 1.0, "f32")
    if ties:
        s = (np.round(s * 8) / 8).astype(np.float32)
        s[0, : N // 2] = 0.5  # one row with a very wide tie
    if order == "sorted":
        # row 0 ascending, row 1 descending, row 2 constant: the top k crowd into one end of
        # the row (or tie everywhere), which defeats any per-chunk shortcut
        s[0] = np.sort(s[0])
        s[1] = np.sort(s[1])[::-1]
        s[2] = 1.25
    if pos is None:
        pos = rng.integers(0, N * m, n_rows).astype(np.int32)
        pos[0] = N * m - 1
    pos = pos.reshape(n_rows, 1).astype(np.int32)
    log(f"[topk {label}] rows={n_rows} N={N} k={k} m={m} ties={ties}")
    idx = to_host(dsa.topk_select(to_dev(s.reshape(n_rows, 1, N)), to_dev(pos), k, m=m))
    torch.cuda.synchronize()
    for r in range(n_rows):
        nv = oracle.n_vis(int(pos[r, 0]), m, N)
        ref, cnt = oracle.topk_row(s[r].astype(np.float64), nv, k)
        got = idx[r, 0]
        # same fp32 values on both sides: the set is unique (lowest index wins exact ties)
        assert np.array_equal(np.sort(got[got >= 0]), ref[ref >= 0]), f"{label} row {r}"
        assert (got < 0).sum() == k - cnt
        # every path (streaming, filtered long rows, their exact fallbacks) writes the selection
        # in ascending index order, so the result does not depend on timing
        v = got[got >= 0]
        assert (np.diff(v) > 0).all(), f"{label} row {r}: not in ascending index order"


def test_topk_exact_sets():
    _topk_case("decode", 16, 8192, 2048)
    _topk_case("ragged", 9, 3001, 512, seed=1)
    _topk_case("small-k", 5, 777, 7, seed=2)
    _topk_case("keep-all", 4, 1500, 2048, seed=3)
    _topk_case("csa", 6, 4000, 1024, m=4, seed=4)
    _topk_case("long", 2, 262144, 1024, seed=5)


def test_topk_long_rows():
    # rows longer than 32768 entries: filtered candidates per 4096-entry chunk, then a select
    # over the candidates, with the exact whole-row select as fallback
    _topk_case("long-mixed-nvis", 7, 40000, 1000, seed=7,
               pos=np.array([39999, 999, 1000, 1001, 20000, 32768, 36863], np.int32))
    _topk_case("long-m4", 3, 70001, 1024, m=4, seed=8)
    _topk_case("long-ties", 3, 50000, 1024, ties=True, seed=9)
    _topk_case("long-sorted", 3, 65536, 1024, seed=10, pos=np.full(3, 65535, np.int32))
    _topk_case("long-k4096", 2, 300000, 4096, seed=11)


def test_topk_stream_fallback():
    # prefill-length rows (the streaming select): ascending / descending / constant rows put
    # more than a wave's candidate segment into one quarter of the row, so the exact whole-row
    # fallback runs; an odd row length takes the unaligned loads
    _topk_case("stream-sorted", 3, 32768, 2048, seed=12, order="sorted",
               pos=np.full(3, 32767, np.int32))
    _topk_case("stream-odd", 4, 30001, 2048, seed=13, order="sorted",
               pos=np.array([30000, 30000, 30000, 17000], np.int32))
    _topk_case("stream-ties", 4, 32768, 2048, ties=True, seed=14)


def test_topk_ties_take_lowest_index():
    _topk_case("ties", 8, 5000, 1000, ties=True, seed=6)
    # all-equal row: exactly the first k indices
    s = np.zeros((1, 1, 3000), np.float32)
    s[0, 0, ::2] = -0.0  # -0 ranks equal to +0
    idx = to_host(dsa.topk_select(to_dev(s), to_dev(np.array([[2999]], np.int32)), 100))
    assert np.array_equal(np.sort(idx[0, 0]), np.arange(100))


# ----------------------------------------------------------------------------- attention ----

def _attend_case(c, label, seed=0, frac_masked=0.05):
    wl = synth.make_workload(c)
    rng = np.random.default_rng(seed)
    B, T, k = c.B, c.T, c.top_k
    pos = wl.q_pos()
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            nv = visible(wl, b, t)
            n = min(k, nv)
            sel = rng.choice(nv, n, replace=False).astype(np.int32)
            drop = rng.random(n) < frac_masked
            sel[drop] = -1
            idx[b, t, :n] = sel
            rng.shuffle(idx[b, t])
    kv = wl.kv() if not c.compress else None
    raw = wl.kv_raw()
    base, n_raw = wl.raw_extent()
    log(f"[attend {label}] B={B} T={T} N={c.N} k={k} W={c.W} dt={c.dt}")
    sink = wl.sink()
    out, lse = dsa.sparse_mla_attend(to_dev(wl.q()), to_dev(kv), to_dev(idx), to_dev(pos), c.D_V,
                                     c.softmax_scale, kv_raw=to_dev(raw) if raw is not None else None,
                                     raw_base=base, W=c.W, m=c.m,
                                     sink=to_dev(sink) if sink is not None else None)
    torch.cuda.synchronize()
    out, lse = oracle.decode(to_host(out)), to_host(lse)
    worst = (0.0, 0.0)
    for b in range(B):
        for t in range(T):
            ro, rl = oracle.attend_row(wl.q()[b, t], kv[b], idx[b, t], c.D_V, c.softmax_scale,
                                       p=int(pos[b, t]), W=c.W,
                                       kv_raw=raw[b] if raw is not None else None, raw_base=base,
                                       sink=None if sink is None else sink.astype(np.float64))
            mx, sc = check_attention(out[b, t], lse[b, t], ro, rl, what=f"{label} b={b} t={t}")
            worst = max(worst, (mx, sc))
    log(f"[attend {label}] max abs err {worst[0]:.3e} (max|ref| {worst[1]:.3e})")


def test_attend_decode_split():
    c = _cfg("decode", B=4, N=3001, pos0=3000, name="att_decode")
    _attend_case(c, "decode")
    _attend_case(c.sharp(), "decode-sharp", seed=1)


def test_attend_prefill_many_rows_ragged_k():
    # enough rows for the no-split plan; k not a multiple of the 32-entry tile
    c = _cfg("decode", B=1, T=300, N=2000, top_k=1000, pos0=1700, name="att_rows")
    _attend_case(c.sharp(), "rows-sharp", seed=2)


def test_attend_window_csa():
    c = _cfg("csa_decode", B=2, N=2500, pos0=4 * 2500 - 1, n_raw=128,
             raw_base=4 * 2500 - 128, name="att_win")
    _attend_case(c, "window")
    _attend_case(c.sharp(), "window-sharp", seed=3)
    # window clipped at position 0 and partly outside kv_raw
    c2 = _cfg("csa_decode", B=1, N=100, pos0=40, n_raw=30, raw_base=20, top_k=64, name="att_clip")
    _attend_case(c2.sharp(), "window-clip", seed=4)


def test_attend_generic_fp32():
    _attend_case(synth.CONFIGS["tiny"], "tiny-f32")
    _attend_case(synth.CONFIGS["tiny"].sharp(), "tiny-f32-sharp", seed=5)
    _attend_case(_cfg("tiny", dt="bf16", name="tiny_bf16").sharp(), "tiny-bf16-sharp", seed=6)


def test_generic_kernels_at_their_limits():
    # the generic indexer at H_I x D_I = 8192 (its LDS bound) and the generic attention at
    # D_K = 1024 (DSA_MAX_DK) with k = 4096 (DSA_MAX_TOPK)
    for H_I, D_I, dt, k_dt in ((8, 1024, "f32", "f32"), (1, 8192, "bf16", "bf16"),
                               (64, 128, "f32", "f32"), (8, 1024, "bf16", "mxfp4")):
        _run_indexer(_cfg("tiny", B=2, T=5, N=700, H_I=H_I, D_I=D_I, dt=dt, k_dt=k_dt, pos0=300,
                          pos_stride=97, name=f"ix_limit_{H_I}x{D_I}_{k_dt}"), f"limit {H_I}x{D_I}")
    for dt, D_V in (("f32", 1024), ("bf16", 1024), ("bf16", 8)):
        c = _cfg("decode", B=2, T=2, N=5000, H=2, D_K=1024, D_V=D_V, dt=dt, top_k=4096,
                 pos0=4500, pos_stride=400, scale=1.0 / 32, name=f"att_limit_{dt}_{D_V}")
        _attend_case(c, f"limit D_K 1024 D_V {D_V} {dt}")
        _attend_case(c.sharp(), f"limit D_K 1024 D_V {D_V} {dt} sharp", seed=1)


def test_attend_all_masked_row_gives_zero():
    c = _cfg("decode", B=1, N=500, top_k=64, pos0=499, name="att_empty")
    wl = synth.make_workload(c)
    idx = np.full((1, 1, 64), -1, np.int32)
    out, lse = dsa.sparse_mla_attend(to_dev(wl.q()), to_dev(wl.kv()), to_dev(idx),
                                     to_dev(wl.q_pos()), 512, c.softmax_scale)
    torch.cuda.synchronize()
    assert (to_host(out.float()) == 0).all()
    assert np.isneginf(to_host(lse)).all()


# ------------------------------------------------------------ heavily compressed attention ----

def _hca_case(c):
    wl = synth.make_workload(c)
    dw = DeviceWorkload(wl)
    f = dw.hca()
    log(f"[hca {c.name}] B={c.B} T={c.T} N={c.N} m={c.m} W={c.W} dt={c.dt} compress={c.compress}")
    f.run()
    torch.cuda.synchronize()
    run = oracle.QueryRunner(wl)
    if c.compress:
        check_compressed(dw, run)
    for b in range(c.B):
        for t in range(c.T):
            r = run.run_dense(b, t)
            out = to_host(f.out[b, t])
            out = oracle.decode(out) if c.dt == "bf16" else out.astype(np.float64)
            # sharp rows whose output reaches several units carry the bar for the bf16 rounding
            # of P and of the stored output, as in the sweeps (see check_attention)
            check_attention(out, to_host(f.lse[b, t]), r["out"], r["lse"],
                            what=f"hca {c.name} b={b} t={t} n_vis={r['n_vis']}",
                            bf16_scale_allowance=c.name.endswith("_sharp") and c.dt == "bf16")
    del f, dw


def test_hca_ragged_window_and_compress():
    base = synth.CONFIGS["hca_decode"]
    # stored blocks; positions from before the first complete block (window only) to past N
    _hca_case(base.with_(B=2, T=7, N=300, m=8, pos0=3, pos_stride=397, raw_base=0, n_raw=2386,
                         name="hca_small").sharp())
    # few rows split the entry list; many rows do not
    _hca_case(base.with_(B=1, T=3, N=2900, m=8, W=0, pos0=8 * 2900 - 3, n_raw=0, raw_base=0,
                         name="hca_nowin"))
    # the most splits the merge takes (32), the last one ragged
    _hca_case(base.with_(B=1, T=2, N=5000, m=8, W=0, pos0=8 * 5000 - 9, n_raw=0, raw_base=0,
                         name="hca_32split"))
    # blocks produced from raw rows in the same call, 140 query rows; the sharp variant has no
    # window: with one, its N(0,1) raw rows outweigh the 16-token means and the outputs reach
    # ~4, where bf16 output rounding alone (up to 1.6e-2) uses up most of the 2e-2 bound
    hp = synth.CONFIGS["hca_prefill"].with_(T=140, N=40, m=16, pos0=16 * 40 - 140, n_raw=640,
                                            name="hca_compress")
    _hca_case(hp)
    _hca_case(hp.with_(W=0).sharp())
    # fp32 (scalar kernel)
    _hca_case(base.with_(B=2, T=5, N=77, m=4, H=8, D_K=64, D_V=48, dt="f32", k_dt="f32",
                         pos0=1, pos_stride=71, raw_base=0, n_raw=300, name="hca_f32"))
