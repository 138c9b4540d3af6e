"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked values
(tests/golden/*.json, each citing its passage), closed forms, library routines the method reduces
to in special cases (numpy matmul / argpartition / mean, torch scaled_dot_product_attention in
fp64), and invariants. They are chosen so that a dropped term, a wrong sign or index, or a
transposed operand in any oracle step fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _num(x):
    return float(x)


# ---------------------------------------------------------------- stored-value decoding ----

def test_bf16_decode_golden():
    g = _load("bf16.json")
    for hexbits, val in g["decode"]:
        got = oracle.decode(np.array([int(hexbits, 16)], np.uint16))[0]
        want = _num(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), hexbits


def test_mxfp4_golden_table_and_bytes():
    g = _load("h4_mxfp4.json")
    for code, val in enumerate(g["e2m1"]):
        got = oracle.e2m1(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for byte, val in g["e8m0"].items():
        assert oracle.e8m0(int(byte)) == val
    assert math.isnan(oracle.e8m0(0xFF))
    for case in g["bytes"]:
        codes = np.zeros((1, 16), np.uint8)
        codes[0, 0] = case["byte"]
        scales = np.full((1, 1), case["scale"], np.uint8)
        row = oracle.decode_mxfp4(codes, scales)[0]
        assert row[0] == case["values"][0] and math.copysign(1, row[0]) == math.copysign(1, case["values"][0])
        assert row[1] == case["values"][1]


def test_mxfp4_exhaustive_codes_times_scales():
    """All 16 codes x 255 finite scales: value = e2m1 table entry * 2^(s-127)."""
    table = _load("h4_mxfp4.json")["e2m1"]
    # byte j: low nibble (element 2j) = code j, high nibble (element 2j+1) = code 15 - j
    codes = np.zeros((255, 16), np.uint8)
    for j in range(16):
        lo, hi = j, 15 - j
        codes[:, j] = lo | (hi << 4)
    scales = np.repeat(np.arange(255, dtype=np.uint8)[:, None], 1, axis=1)
    vals = oracle.decode_mxfp4(codes, scales)
    for s in range(255):
        for j in range(16):
            assert vals[s, 2 * j] == table[j] * 2.0 ** (s - 127)
            assert vals[s, 2 * j + 1] == table[15 - j] * 2.0 ** (s - 127)


def test_mxfp4_scale_per_32_elements():
    codes = np.full((1, 32), 0x22, np.uint8)  # every element = 1.0 * scale
    scales = np.array([[127, 128]], np.uint8)
    v = oracle.decode_mxfp4(codes, scales)[0]
    assert (v[:32] == 1.0).all() and (v[32:] == 2.0).all()


# --------------------------------------------------------------------- indexer scores ----

def _h1():
    g = _load("h1_indexer.json")
    k = np.array(g["k_I"], np.float64)
    q = np.array(g["q_I"], np.float64)
    w = np.array(g["w"], np.float32)
    return g, k, q, w


def test_e4m3_every_code_matches_torch_float8():
    """OCP e4m3 (E4M3FN) decoding against torch's own float8_e4m3fn dtype, all 256 codes."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3(int(c)) for c in codes])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(got[fin]))  # -0 for 0x80


def test_e8m0_matches_torch_float8_e8m0():
    b = np.arange(255, dtype=np.uint8)  # 0xFF is NaN
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(ref, np.array([oracle.e8m0(int(x)) for x in b]))


def test_mxfp8_hand_bytes_and_one_scale_per_32():
    # 0x38 = +1.0, 0xFE = -448 (largest finite), 0x01 = 2^-9 (smallest subnormal)
    codes = np.array([[0x38] * 32 + [0xFE] * 31 + [0x01]], np.uint8)
    scales = np.array([[127, 130]], np.uint8)  # 2^0, 2^3
    row = oracle.decode_mxfp8(codes, scales)[0]
    assert (row[:32] == 1.0).all() and (row[32:63] == -448.0 * 8).all()
    assert row[63] == 2.0 ** -9 * 8


def test_mxfp8_quantiser_rounds_like_torch():
    """The generator's e4m3 rounding (RNE, saturating at 448) against torch's cast, on random
    values, exact ties between neighbouring codes and the saturation edge."""
    rng = np.random.default_rng(3)
    grid = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ties = (grid[1:] + grid[:-1]) / 2
    x = np.concatenate([rng.standard_normal(4000) * 50, ties, -ties, [447.0, 448.0, 460.0, 463.9]])
    for i in range(0, x.size - x.size % 32, 32):
        blk = x[i:i + 32].copy()
        blk[0] = 300.0  # pin the block scale to 2^0 so that codes are e4m3 of the values
        codes, sc = synth.mxfp8_block(blk)
        assert sc == 127
        ref = torch.from_numpy(blk).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, ref), (blk, codes, ref)


def test_scores_mxfp8_paths_equal_decoded_values():
    kc, ks = synth.normal_mxfp8(7, 2, 64, 128)
    qc, qs = synth.normal_mxfp8(7, 1, 4, 128)
    w = synth.uniform(7, 3, (4,), 0.0, 1.0)
    got = oracle.scores_row(qc, w, kc, 60, k_scale=ks, q_scale=qs)
    ref = oracle.scores_row(oracle.decode_mxfp8(qc, qs), w, oracle.decode_mxfp8(kc, ks), 60)
    np.testing.assert_array_equal(got, ref)
    assert np.isneginf(got[60:]).all()


def test_h1_scores_and_masking():
    g, k, q, w = _h1()
    for case in g["cases"]:
        nv = oracle.n_vis(case["p"], case["m"], k.shape[0])
        sc = oracle.scores_row(q, w, k, nv)
        want = np.array([_num(x) for x in case["scores"]])
        assert np.array_equal(sc, want), case


def test_h1_negative_w_applies_after_relu():
    g, k, q, _ = _h1()
    c = g["negative_w"]
    sc = oracle.scores_row(q, np.array(c["w"], np.float32), k, oracle.n_vis(c["p"], 1, 4))
    assert np.array_equal(sc, np.array(c["scores"]))


def test_h1_topk():
    g, k, q, w = _h1()
    for case in g["cases"]:
        nv = oracle.n_vis(case["p"], case["m"], k.shape[0])
        sc = oracle.scores_row(q, w, k, nv)
        for kk, want in case["topk"].items():
            idx, cnt = oracle.topk_row(sc, nv, int(kk))
            assert idx.tolist() == want, (case, kk)
            assert cnt == sum(1 for x in want if x >= 0)


def test_scores_reduce_to_gemm_with_one_head_and_positive_dots():
    """H_I = 1, w = 1 and all dot products positive: I = K q (a plain matrix-vector product)."""
    rng = np.random.default_rng(0)
    k = rng.uniform(0.1, 1.0, (300, 24))
    q = rng.uniform(0.1, 1.0, (1, 24))
    sc = oracle.scores_row(q, np.ones(1, np.float32), k, 300)
    np.testing.assert_allclose(sc, k @ q[0], rtol=1e-13)


def test_scores_sum_over_heads_and_transposition():
    """Heads with disjoint supports and positive dots: I = sum_j w_j (K q_j) -- distinguishes
    k_I[s] . q_I[j] from any transposed pairing (H_I != D_I)."""
    rng = np.random.default_rng(1)
    k = rng.uniform(0.1, 1.0, (50, 8))
    q = rng.uniform(0.1, 1.0, (3, 8))
    w = np.array([0.25, 2.0, 0.5], np.float32)
    sc = oracle.scores_row(q, w, k, 50)
    np.testing.assert_allclose(sc, (k @ q.T) @ w.astype(np.float64), rtol=1e-13)


def test_scores_negated_query_gives_zero():
    """All dots positive; negating the single head makes every ReLU zero."""
    rng = np.random.default_rng(2)
    k = rng.uniform(0.1, 1.0, (40, 16))
    q = rng.uniform(0.1, 1.0, (1, 16))
    sc = oracle.scores_row(-q, np.ones(1, np.float32), k, 40)
    assert (sc == 0.0).all()


def test_scores_mxfp4_path_equals_decoded_keys():
    codes, sc = synth.normal_mxfp4(7, 2, 64, 128)
    q = synth.normal(7, 1, (4, 128), 1.0, "bf16")
    w = synth.uniform(7, 3, (4,), 0.0, 1.0)
    dec = oracle.decode_mxfp4(codes, sc)
    a = oracle.scores_row(q, w, codes, 50, k_scale=sc)
    b = oracle.scores_row(q, w, dec, 50)
    assert np.array_equal(a, b)
    assert np.isneginf(a[50:]).all()


@pytest.mark.parametrize("p,m,N,want", [(0, 1, 10, 1), (9, 1, 10, 10), (20, 1, 10, 10),
                                         (2, 4, 10, 0), (3, 4, 10, 1), (6, 4, 10, 1),
                                         (7, 4, 10, 2), (1048575, 4, 262144, 262144), (-1, 1, 5, 0)])
def test_n_vis(p, m, N, want):
    assert oracle.n_vis(p, m, N) == want


# ------------------------------------------------------------------------------ top-k ----

def test_topk_matches_argpartition_on_untied_scores():
    rng = np.random.default_rng(3)
    s = rng.standard_normal(5000)
    idx, cnt = oracle.topk_row(s, 4000, 300)
    want = np.sort(np.argpartition(-s[:4000], 300)[:300])
    assert cnt == 300 and np.array_equal(idx, want)


def test_topk_invariants_brute_force():
    rng = np.random.default_rng(4)
    for trial in range(20):
        n = int(rng.integers(1, 400))
        k = int(rng.integers(1, 300))
        s = np.round(rng.standard_normal(n) * 4) / 4  # many exact ties
        idx, cnt = oracle.topk_row(s, n, k)
        sel = idx[idx >= 0]
        assert cnt == min(n, k) == sel.size
        assert np.unique(sel).size == sel.size and (np.diff(sel) > 0).all()
        assert (idx[cnt:] == -1).all()
        rest = np.setdiff1d(np.arange(n), sel)
        if rest.size:
            assert s[sel].min() >= s[rest].max()
            # ties at the threshold are resolved toward the lower index
            tau = s[sel].min()
            tied_out = rest[s[rest] == tau]
            tied_in = sel[s[sel] == tau]
            if tied_out.size:
                assert tied_in.max() < tied_out.min()
        # brute force: stable sort by descending score
        order = sorted(range(n), key=lambda i: (-s[i], i))[:k]
        assert np.array_equal(sel, np.sort(order))


def test_topk_masked_entries_never_selected():
    s = np.array([5.0, 1.0, 2.0, 100.0, 100.0])
    idx, cnt = oracle.topk_row(s, 3, 2)
    assert idx.tolist() == [0, 2]


# -------------------------------------------------------------------------- attention ----

def test_h2_attention_golden():
    g = _load("h2_attention.json")
    q = np.array(g["q"], np.float64)
    kv = np.array(g["kv"], np.float64)
    for case in g["cases"]:
        out, lse = oracle.attend_row(q, kv, np.array(case["idx"], np.int32), g["D_V"], g["scale"])
        assert out[0, 0] == pytest.approx(case["out"], abs=1e-14), case
        want = _num(case["lse"])
        if math.isinf(want):
            assert math.isinf(lse[0]) and lse[0] < 0
        else:
            assert lse[0] == pytest.approx(want, abs=1e-14)


def _dense_sdpa(q, kv, D_V, scale, mask):
    """torch fp64 SDPA with MQA kv expanded over heads. q [H, D_K], kv [n, D_K], mask [n] bool."""
    qt = torch.from_numpy(q)[None, :, None, :]            # [1, H, 1, D_K]
    kt = torch.from_numpy(kv)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(kv[:, :D_V]))[None, None].expand(1, q.shape[0], -1, -1)
    m = torch.from_numpy(mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0, :, 0].numpy()


def test_dense_reduction_when_k_covers_context():
    """k >= n_vis: DSA reduces to plain causal MQA attention (torch SDPA, fp64)."""
    rng = np.random.default_rng(5)
    H, D_K, D_V, N, k = 6, 40, 24, 37, 64
    kv = rng.standard_normal((N, D_K))
    for p in (0, 5, 36):
        q = rng.standard_normal((H, D_K))
        nv = oracle.n_vis(p, 1, N)
        idx, _ = oracle.topk_row(rng.standard_normal(N), nv, k)
        out, lse = oracle.attend_row(q, kv, idx, D_V, 0.3)
        mask = np.arange(N) <= p
        np.testing.assert_allclose(out, _dense_sdpa(q, kv, D_V, 0.3, mask), rtol=1e-12, atol=1e-12)
        z = 0.3 * q @ kv[: p + 1].T
        np.testing.assert_allclose(lse, np.log(np.exp(z).sum(1)), rtol=1e-12)


def test_sparse_equals_dense_over_the_selected_subset():
    """Attention over idx equals dense attention masked to exactly those entries."""
    rng = np.random.default_rng(6)
    H, D_K, D_V, N = 4, 32, 16, 100
    kv = rng.standard_normal((N, D_K))
    q = rng.standard_normal((H, D_K))
    sel = np.sort(rng.choice(N, 17, replace=False)).astype(np.int32)
    idx = np.concatenate([sel[::-1], -np.ones(5, np.int32)])  # order and padding do not matter
    out, _ = oracle.attend_row(q, kv, idx, D_V, 0.2)
    mask = np.zeros(N, bool)
    mask[sel] = True
    np.testing.assert_allclose(out, _dense_sdpa(q, kv, D_V, 0.2, mask), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_selected_values():
    rng = np.random.default_rng(7)
    kv = rng.standard_normal((50, 12))
    idx = np.array([3, 7, 7, 20, -1], np.int32)  # duplicates count twice
    out, lse = oracle.attend_row(np.zeros((2, 12)), kv, idx, 5, 1.0)
    np.testing.assert_allclose(out[0], kv[[3, 7, 7, 20], :5].mean(0), rtol=1e-13)
    assert lse[0] == pytest.approx(math.log(4))


def test_attention_bf16_rows_decoded_exactly():
    q = synth.normal(9, 4, (3, 64), 0.5, "bf16")
    kv = synth.normal(9, 5, (20, 64), 0.5, "bf16")
    idx = np.arange(20, dtype=np.int32)
    a, la = oracle.attend_row(q, kv, idx, 48, 0.125)
    b, lb = oracle.attend_row(oracle.decode(q), oracle.decode(kv), idx, 48, 0.125)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_attention_mxfp8_cache_equals_decoded_rows():
    # an MXFP8 latent cache (codes, scales): the same attention as over its exactly decoded rows,
    # for masked slots, repeated entries and an entry of the last row
    codes, sc = synth.normal_mxfp8(13, 5, 40, 64, 1.0)
    q = synth.normal(13, 4, (4, 64), 1.0, "bf16")
    idx = np.array([3, -1, 17, 3, 39, 0, -1], np.int32)
    a, la = oracle.attend_row(q, (codes, sc), idx, 48, 0.125)
    b, lb = oracle.attend_row(q, oracle.decode_mxfp8(codes, sc), idx, 48, 0.125)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-13)
    e, le = oracle.attend_row(q, (codes, sc), np.full(5, -1, np.int32), 48, 0.125)
    assert (e == 0).all() and np.isneginf(le).all()


def test_attention_mxfp8_constant_rows_closed_form():
    # every code 0x38 (e4m3 1.0) and scale 2^(e - 127): each selected row is the constant
    # 2^(e - 127); a zero query averages them
    codes = np.full((6, 32), 0x38, np.uint8)
    sc = np.array([[127], [128], [126], [130], [127], [125]], np.uint8)
    idx = np.array([1, 3, -1, 5], np.int32)
    out, lse = oracle.attend_row(np.zeros((2, 32)), (codes, sc), idx, 16, 1.0)
    want = (2.0 + 8.0 + 0.25) / 3
    np.testing.assert_allclose(out, want, rtol=1e-15)
    np.testing.assert_allclose(lse, math.log(3), rtol=1e-15)


def test_attention_mxfp4_cache_equals_decoded_rows():
    # an MXFP4 latent cache (e2m1 pairs [N, D_K/2], scales): the same attention as over its
    # exactly decoded rows
    codes, sc = synth.normal_mxfp4(17, 5, 40, 64, 1.0)
    q = synth.normal(17, 4, (4, 64), 1.0, "bf16")
    idx = np.array([3, -1, 17, 3, 39, 0, -1], np.int32)
    a, la = oracle.attend_row(q, (codes, sc), idx, 48, 0.125)
    b, lb = oracle.attend_row(q, oracle.decode_mxfp4(codes, sc), idx, 48, 0.125)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=0, atol=1e-13)


def test_attention_mxfp4_constant_rows_closed_form():
    # every code pair 0x22 (e2m1 1.0, 1.0) and scale 2^(e - 127): each selected row is the
    # constant 2^(e - 127); a zero query averages them; with a sign bit on the high nibbles
    # (0xa2: 1.0, -1.0) the odd columns flip sign
    sc = np.array([[127], [128], [126], [130], [127], [125]], np.uint8)
    idx = np.array([1, 3, -1, 5], np.int32)
    out, lse = oracle.attend_row(np.zeros((2, 32)), (np.full((6, 16), 0x22, np.uint8), sc), idx,
                                 16, 1.0)
    want = (2.0 + 8.0 + 0.25) / 3
    np.testing.assert_allclose(out, want, rtol=1e-15)
    np.testing.assert_allclose(lse, math.log(3), rtol=1e-15)
    out, _ = oracle.attend_row(np.zeros((2, 32)), (np.full((6, 16), 0xa2, np.uint8), sc), idx,
                               16, 1.0)
    np.testing.assert_allclose(out[:, 0::2], want, rtol=1e-15)
    np.testing.assert_allclose(out[:, 1::2], -want, rtol=1e-15)


# -------------------------------------------------------------------------------- CSA ----

def test_h3_csa_golden():
    g = _load("h3_csa.json")
    raw = np.array(g["kv_raw"], np.float64)
    comp = oracle.compress_mean(raw, g["m"])
    assert np.array_equal(comp, np.array(g["compressed"]))
    for case in g["cases"]:
        assert oracle.n_vis(case["p"], g["m"], comp.shape[0]) == case["n_vis"]
        out, _ = oracle.attend_row(np.array(case["q"]), comp, np.array(case["idx"], np.int32),
                                   g["D_V"], 1.0, p=case["p"], W=case["W"], kv_raw=raw, raw_base=0)
        assert out[0, 0] == pytest.approx(case["out"], abs=1e-14), case


def test_h5_hca_golden():
    g = _load("h5_hca.json")
    raw = np.array(g["kv_raw"], np.float64)
    comp = oracle.compress_mean(raw, g["m"])
    np.testing.assert_allclose(comp, np.array(g["compressed"]), rtol=0, atol=1e-15)
    for case in g["cases"]:
        nv = oracle.n_vis(case["p"], g["m"], comp.shape[0])
        assert nv == case["n_vis"]
        idx = oracle.dense_entries(nv, comp.shape[0])
        assert list(idx[:nv]) == list(range(nv)) and (idx[nv:] == -1).all()
        out, lse = oracle.attend_row(np.array(g["q"]), comp, idx, g["D_V"], g["scale"],
                                     p=case["p"], W=case["W"], kv_raw=raw, raw_base=0)
        assert out[0, 0] == pytest.approx(case["out"], abs=1e-12), case
        if nv == 0 and case["W"] == 0:
            assert lse[0] == -np.inf


def test_hca_reduces_to_dense_attention_over_compressed_sequence():
    """HCA with no window = causal MQA attention over the mean-pooled sequence (torch SDPA, fp64),
    masked to the complete blocks."""
    rng = np.random.default_rng(12)
    H, D_K, D_V, m, n_raw = 5, 24, 16, 8, 203
    raw = rng.standard_normal((n_raw, D_K))
    comp = raw[: n_raw // m * m].reshape(-1, m, D_K).mean(axis=1)  # pooling written out here
    N = comp.shape[0]
    for p in (7, 8, 100, n_raw - 1):
        q = rng.standard_normal((H, D_K))
        nv = oracle.n_vis(p, m, N)
        out, _ = oracle.attend_row(q, oracle.compress_mean(raw, m),
                                   oracle.dense_entries(nv, N), D_V, 0.4)
        mask = np.arange(N) < (p + 1) // m
        np.testing.assert_allclose(out, _dense_sdpa(q, comp, D_V, 0.4, mask), rtol=1e-12, atol=1e-12)


def test_compress_identity_constant_and_mean():
    rng = np.random.default_rng(8)
    raw = rng.standard_normal((41, 9))
    assert np.array_equal(oracle.compress_mean(raw, 1), raw)
    np.testing.assert_allclose(oracle.compress_mean(raw, 4), raw[:40].reshape(10, 4, 9).mean(1),
                               rtol=1e-14)
    c = oracle.compress_mean(np.full((16, 3), 2.75), 4)
    assert (c == 2.75).all() and c.shape == (4, 3)


def test_window_only_is_banded_dense_attention():
    """No selected entries + window W: plain sliding-window attention (torch SDPA, band mask)."""
    rng = np.random.default_rng(9)
    H, D_K, D_V, n, W = 3, 16, 8, 30, 5
    raw = rng.standard_normal((n, D_K))
    for p in (0, 3, 29):
        q = rng.standard_normal((H, D_K))
        out, _ = oracle.attend_row(q, None, -np.ones(4, np.int32), D_V, 0.5, p=p, W=W,
                                   kv_raw=raw, raw_base=0)
        mask = (np.arange(n) <= p) & (np.arange(n) > p - W)
        np.testing.assert_allclose(out, _dense_sdpa(q, raw, D_V, 0.5, mask), rtol=1e-12, atol=1e-12)


def test_window_respects_raw_base_and_joins_blocks():
    """kv_raw holding only the window rows (raw_base > 0) gives the same result as the full raw
    sequence; blocks and window rows share one softmax."""
    rng = np.random.default_rng(10)
    D_K, D_V, m, W = 8, 4, 4, 6
    raw = rng.standard_normal((64, D_K))
    comp = oracle.compress_mean(raw, m)
    q = rng.standard_normal((2, D_K))
    p = 61
    idx = np.array([0, 5, 9], np.int32)
    a, la = oracle.attend_row(q, comp, idx, D_V, 0.7, p=p, W=W, kv_raw=raw, raw_base=0)
    b, lb = oracle.attend_row(q, comp, idx, D_V, 0.7, p=p, W=W, kv_raw=raw[56:], raw_base=56)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    ents = np.concatenate([comp[idx], raw[p - W + 1:p + 1]])
    mask = np.ones(len(ents), bool)
    np.testing.assert_allclose(a, _dense_sdpa(q, ents, D_V, 0.7, mask), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ end to end on the tiny run ----

def test_tiny_workload_end_to_end_invariants():
    wl = synth.make_workload("tiny")
    run = oracle.QueryRunner(wl)
    c = wl.cfg
    for t in range(c.T):
        r = run.run(0, t)
        p = 240 + t
        assert r["n_vis"] == p + 1
        sel = r["idx"][r["idx"] >= 0]
        assert sel.size == c.top_k and sel.max() <= p
        assert np.isneginf(r["scores"][p + 1:]).all()
        rest = np.setdiff1d(np.arange(p + 1), sel)
        assert r["scores"][sel].min() >= r["scores"][rest].max()
        assert np.isfinite(r["out"]).all() and r["out"].shape == (c.H, c.D_V)


# ------------------------------------------------------------------ attention sink, ragged ----

def test_h6_sink_golden():
    g = json.load(open(os.path.join(GOLD, "h6_sink.json")))
    q = np.array(g["q"], np.float64)
    kv = np.array(g["kv"], np.float64)
    for c in g["cases"]:
        sink = np.array([float(c["sink"])], np.float64)
        out, lse = oracle.attend_row(q, kv, np.array(c["idx"], np.int32), g["D_V"], g["scale"],
                                     sink=sink)
        assert abs(out[0, 0] - c["out"]) < 1e-12, c
        assert abs(lse[0] - float(c["lse"])) < 1e-12, c


def test_sink_invariants():
    # a sink logit equal to the entries' own log-sum-exp takes half of every head's mass: the
    # output halves and lse grows by ln 2; a sink of -inf is no sink at all
    rng = np.random.default_rng(11)
    H, D_K, D_V, N = 5, 16, 12, 40
    q = rng.standard_normal((H, D_K))
    kv = rng.standard_normal((N, D_K))
    idx = rng.choice(N, 25, replace=False).astype(np.int32)
    out0, lse0 = oracle.attend_row(q, kv, idx, D_V, 0.3)
    out1, lse1 = oracle.attend_row(q, kv, idx, D_V, 0.3, sink=lse0)
    assert np.allclose(out1, out0 / 2, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse1, lse0 + np.log(2.0), rtol=1e-12)
    out2, lse2 = oracle.attend_row(q, kv, idx, D_V, 0.3, sink=np.full(H, -np.inf))
    assert np.array_equal(out2, out0) and np.array_equal(lse2, lse0)
    # against the definition written with numpy: softmax over [z, s] with a zero value row
    z = 0.3 * q @ kv[idx].T
    s = rng.standard_normal(H) * 3
    out3, lse3 = oracle.attend_row(q, kv, idx, D_V, 0.3, sink=s)
    zz = np.concatenate([z, s[:, None]], axis=1)
    w = np.exp(zz - zz.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    vals = np.concatenate([kv[idx, :D_V], np.zeros((1, D_V))], axis=0)
    assert np.allclose(out3, w @ vals, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse3, np.log(np.exp(zz).sum(1)), rtol=1e-12)


@pytest.mark.parametrize("p,m,N,L,want", [(99, 1, 200, 50, 50), (99, 1, 200, 150, 100),
                                          (99, 4, 200, 10, 10), (99, 4, 200, 30, 25),
                                          (7, 1, 5, 100, 5), (10, 1, 20, 0, 0), (-1, 1, 20, 9, 0)])
def test_n_vis_ragged(p, m, N, L, want):
    assert oracle.n_vis(p, m, N, seq_len=L) == want


def test_ragged_scores_and_topk_equal_a_shorter_context():
    # a sequence holding L entries scores and selects exactly as the same query over a context
    # truncated to L entries
    rng = np.random.default_rng(5)
    H_I, D_I, N, L, k = 3, 8, 60, 37, 10
    qI = rng.standard_normal((H_I, D_I))
    w = rng.uniform(-1, 1, H_I).astype(np.float32)
    kI = rng.standard_normal((N, D_I))
    nv = oracle.n_vis(N - 1, 1, N, seq_len=L)
    assert nv == L
    sc = oracle.scores_row(qI, w, kI, nv)
    sc_short = oracle.scores_row(qI, w, kI[:L].copy(), oracle.n_vis(L - 1, 1, L))
    assert np.array_equal(sc[:L], sc_short) and np.isneginf(sc[L:]).all()
    assert np.array_equal(oracle.topk_row(sc, nv, k)[0], oracle.topk_row(sc_short, L, k)[0])
