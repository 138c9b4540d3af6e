"""Helpers of the GPU parity tests: device copies of seeded workloads and the parity checks.

The checks compare the HIP path with the fp64 oracle at the tolerances the path is held to:
  scores     |I_gpu - I_ref| <= 1e-3 |I_ref| + 1e-6 max_s |I_ref|; masked entries exactly -inf.
             Rows with head weights of either sign add the error bound of fp32 accumulation,
             (D_I + H_I + 2) 2^-24 sum_j |w_j| sum_d |q_I[j,d] k_I[s,d]| (recursive summation of
             the products of each dot, then of the weighted heads): a score that cancels to
             near zero cannot be held to a bound relative to itself
  top-k      the same set, except entries whose oracle score lies within 1e-4 |tau| of the
             oracle's k-th largest score tau (ties); count = min(k, n_vis); -1 padding
  attention  max |out_gpu - out_ref| <= 2e-2 (acceptance) and <= 2e-2 max |out_ref| (so that
             the bound has teeth at small output scales); |lse_gpu - lse_ref| <= 2e-3
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import synth

SCORE_RTOL = 1e-3
SCORE_FLOOR = 1e-6
TIE_RTOL = 1e-4
ATT_ABS = 2e-2
ATT_REL = 2e-2
LSE_ABS = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dt: str | None = None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host numpy in its stored form (bf16 as uint16 bit patterns)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceWorkload:
    """Device tensors of a synth.Workload, in the layouts of include/dsa.h."""

    def __init__(self, wl: synth.Workload, q_chunk_rows: int = 4096):
        c = wl.cfg
        self.wl, self.cfg = wl, c
        t0 = time.time()
        self.q_pos = to_dev(wl.q_pos())
        if not c.dense:  # HCA has no indexer
            q = wl.q_I()
            self.q_I = (to_dev(q[0]), to_dev(q[1])) if c.qi_dt == "mxfp8" else to_dev(q)
            self.w = to_dev(wl.w())
            k = wl.k_I()
            self.k_I = (to_dev(k[0]), to_dev(k[1])) if c.k_dt in ("mxfp4", "mxfp8") else to_dev(k)
        rows = c.B * c.T
        if rows * c.H * c.D_K > (1 << 28):
            # generate q in chunks straight into the device tensor
            tdt = torch.bfloat16 if c.dt == "bf16" else torch.float32
            self.q = torch.empty((c.B, c.T, c.H, c.D_K), dtype=tdt, device="cuda")
            qf = self.q.view(rows, c.H, c.D_K)
            for r0 in range(0, rows, q_chunk_rows):
                n = min(q_chunk_rows, rows - r0)
                qf[r0:r0 + n] = to_dev(wl.q_chunk(r0, n))
        else:
            self.q = to_dev(wl.q())
        raw = wl.kv_raw()
        self.kv_raw = to_dev(raw) if raw is not None else None
        self.raw_base, self.n_raw = wl.raw_extent()
        if c.compress:
            tdt = torch.bfloat16 if c.dt == "bf16" else torch.float32
            self.kv = torch.empty((c.B, c.N, c.D_K), dtype=tdt, device="cuda")
        else:
            kv = wl.kv()
            self.kv = ((to_dev(kv[0]), to_dev(kv[1])) if c.kv_dt in ("mxfp8", "mxfp4")
                       else to_dev(kv))
        lens, sink = wl.seq_len(), wl.sink()
        self.seq_len = to_dev(lens) if lens is not None else None
        self.sink = to_dev(sink) if sink is not None else None
        torch.cuda.synchronize()
        log(f"[{c.name}] inputs on device in {time.time() - t0:.1f}s")

    def forward(self, keep_scores=True, keep_idx=True):
        import lightning_indexer_top_03_amd as dsa
        c = self.cfg
        scores = (torch.empty((c.B, c.T, c.N), dtype=torch.float32, device="cuda")
                  if keep_scores else None)
        idx = torch.empty((c.B, c.T, c.top_k), dtype=torch.int32, device="cuda") if keep_idx else None
        f = dsa.Forward(self.q_I, self.w, self.k_I, self.q, self.kv, self.q_pos, c.top_k, c.D_V,
                        c.softmax_scale, m=c.m, W=c.W, kv_raw=self.kv_raw,
                        raw_base=self.raw_base, compress=c.compress, scores=scores, idx=idx,
                        seq_len=self.seq_len, sink=self.sink)
        return f


    def hca(self):
        import lightning_indexer_top_03_amd as dsa
        c = self.cfg
        return dsa.HcaForward(self.q, self.kv, self.q_pos, c.D_V, c.softmax_scale, c.m, W=c.W,
                              kv_raw=self.kv_raw, raw_base=self.raw_base, compress=c.compress,
                              seq_len=self.seq_len, sink=self.sink)


def _decoded_keys(wl, b):
    """Sequence b's indexer keys as fp64 [N, D_I] (cached on the workload)."""
    cache = wl._cache.setdefault("_keys_f64", {})
    if b not in cache:
        c = wl.cfg
        k = wl.k_I()
        if c.k_dt == "mxfp4":
            cache[b] = oracle.decode_mxfp4(k[0][b], k[1][b])
        elif c.k_dt == "mxfp8":
            cache[b] = oracle.decode_mxfp8(k[0][b], k[1][b])
        else:
            cache[b] = oracle.decode(k[b])
    return cache[b]


def score_mass(wl, b, t):
    """sum_j |w_j| sum_d |q_I[j,d] k_I[s,d]| for every key s of query (b, t), or None when the
    row's weights are all +0 or positive (then every term of the score is >= 0 and the bound
    relative to the score itself already covers fp32 accumulation)."""
    c = wl.cfg
    w = np.asarray(wl.w()[b, t], np.float64)
    if not np.signbit(w).any():
        return None
    if c.qi_dt == "mxfp8":
        qc, qs = wl.q_I()
        q = oracle.decode_mxfp8(qc[b, t], qs[b, t])
    else:
        q = oracle.decode(wl.q_I()[b, t] if "q_I" in wl._cache else wl.q_I_rows(b, t))
    u = np.abs(q).T @ np.abs(w)  # [D_I]
    return np.abs(_decoded_keys(wl, b)) @ u


def visible(wl, b: int, t: int) -> int:
    """Entries query (b, t) of a workload sees: its position's causal count, capped by the
    sequence's length in a ragged batch (the oracle's n_vis with seq_len)."""
    c = wl.cfg
    lens = wl.seq_len()
    return oracle.n_vis(int(wl.q_pos()[b, t]), c.m, c.N,
                        seq_len=None if lens is None else int(lens[b]))


def _abs_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| with equal values (the same infinity included) at 0; a NaN on either side is an
    infinite difference."""
    with np.errstate(invalid="ignore"):
        d = np.abs(a - b)
    d = np.where(a == b, 0.0, d)
    return np.where(np.isnan(d), np.inf, d)


def check_scores(gpu: np.ndarray, ref: np.ndarray, n_vis: int, full_row: bool = True, what="",
                 mass=None, dims=(64, 128)):
    """mass: score_mass of the row (mixed-sign weights), dims: (H_I, D_I). Returns the largest
    relative error, or with mass the largest error as a fraction of the fp32 bound."""
    g = gpu.astype(np.float64)
    if full_row:
        assert np.isneginf(g[n_vis:]).all(), f"{what}: masked scores must be -inf"
    r = ref[:n_vis]
    gv = g[:n_vis]
    if n_vis == 0:
        return 0.0
    tol = SCORE_RTOL * np.abs(r) + SCORE_FLOOR * np.abs(r).max()
    if mass is not None:
        bound = (dims[0] + dims[1] + 2) * 2.0 ** -24 * mass[:n_vis]
        err = _abs_diff(gv, r)
        assert (err <= tol + bound).all(), (
            f"{what}: scores beyond the fp32 accumulation bound, first s="
            f"{np.nonzero(err > tol + bound)[0][0]}")
        return float((err / np.maximum(bound, 1e-300)).max())
    err = _abs_diff(gv, r)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (f"{what}: {bad.size} scores out of tolerance, first s={bad[0]} "
                           f"gpu={gv[bad[0]]} ref={r[bad[0]]}")
    return float((err / np.maximum(np.abs(r), 1e-30)).max())


def check_topk(gpu_idx: np.ndarray, ref_scores: np.ndarray, n_vis: int, k: int, what=""):
    """Returns the number of tie swaps relative to the oracle's set."""
    sel = gpu_idx[gpu_idx >= 0]
    cnt = min(k, n_vis)
    assert sel.size == cnt, f"{what}: selected {sel.size}, want {cnt}"
    assert (gpu_idx[gpu_idx < 0] == -1).all()
    assert np.unique(sel).size == sel.size, f"{what}: duplicate indices"
    assert (sel < n_vis).all(), f"{what}: index beyond the visible range"
    if n_vis <= k:
        assert np.array_equal(np.sort(sel), np.arange(n_vis)), f"{what}: keep-all rule"
        return 0
    ref_idx, _ = oracle.topk_row(ref_scores, n_vis, k)
    tau = ref_scores[ref_idx].min()
    a, b = set(sel.tolist()), set(ref_idx.tolist())
    swaps = (a - b) | (b - a)
    for s in swaps:
        assert abs(ref_scores[s] - tau) <= TIE_RTOL * abs(tau), (
            f"{what}: entry {s} (score {ref_scores[s]}) differs from the oracle's set, tau={tau}")
    return len(a - b)


def check_attention(gpu_out: np.ndarray, gpu_lse, ref_out: np.ndarray, ref_lse, what="",
                    bf16_scale_allowance=False):
    """max-abs bar 2e-2 (and 2e-2 of max|ref|). bf16_scale_allowance: for sharp inputs whose
    outputs reach several units, the bar grows by the two bf16 roundings on the path, P and the
    stored output (unit roundoff 2^-8 each, relative to max|ref|): at |out| ~ 4.5 they alone
    come to ~3.5e-2, past the bare 2e-2 that is stated for the configurations' scale."""
    d = np.abs(gpu_out.astype(np.float64) - ref_out)
    mx = float(d.max())
    scale = float(np.abs(ref_out).max())
    abs_tol = ATT_ABS + (2 * 2.0 ** -8 * scale if bf16_scale_allowance else 0.0)
    assert mx <= abs_tol, f"{what}: max abs error {mx} (max|ref| {scale})"
    assert mx <= ATT_REL * max(scale, 1e-30), f"{what}: max abs error {mx} vs max|ref| {scale}"
    if gpu_lse is not None:
        fin = np.isfinite(ref_lse)
        assert (np.isfinite(gpu_lse) == fin).all(), f"{what}: lse finiteness"
        if fin.any():
            le = float(np.abs(gpu_lse[fin] - ref_lse[fin]).max())
            assert le <= LSE_ABS, f"{what}: lse error {le}"
    return mx, scale


def check_compressed(dw, run) -> None:
    """Chained check of a call that compresses kv_raw itself: the GPU's pooled entries must lie
    within one bf16 ulp of the oracle's fp64 means (rounding a mean to the stored dtype is the
    only difference the step allows), and the runner then attends over those validated bytes,
    so the attention comparison is not charged with the storage rounding of the cache."""
    c = dw.cfg
    for b in range(c.B):
        ref = oracle.compress_mean(dw.wl.kv_raw()[b], c.m)
        got = to_host(dw.kv[b])
        got = oracle.decode(got) if c.dt == "bf16" else got.astype(np.float64)
        if c.dt == "bf16":
            ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
            assert (np.abs(got - ref) <= ulp).all(), f"{c.name} b={b}: compressed entries"
        else:
            mag = oracle.compress_mean(np.abs(dw.wl.kv_raw()[b]).astype(np.float32), c.m)
            assert (np.abs(got - ref) <= 2.0 ** -20 * mag + 1e-30).all(), f"{c.name} b={b}"
        run._kvc[b] = got


def bf16_decode(a: np.ndarray) -> np.ndarray:
    """Stored values -> fp64 through the oracle's exact decoder."""
    return oracle.decode(np.ascontiguousarray(a))
