"""Plain fp64 CPU oracle of the DSA / CSA hot path - TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. It shares no code with the GPU library (``lightning_indexer_top_03_amd``) and never
imports it; both consume the same stored bytes written by the seeded generator (``synth``).

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over keys / heads); this module only
marshals numpy arrays and composes the steps per query:
  n_vis -> scores -> top-k -> attention over (selected entries u raw window).
See ``oracle.c`` for the definitions and the passages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, MXFP4, F64, MXFP8 = 0, 1, 2, 3, 4
_DT = {"f32": F32, "bf16": BF16, "mxfp4": MXFP4, "f64": F64, "mxfp8": MXFP8}


def build(force: bool = True) -> str:
    """Compile liboracle.so (gcc, -O2, OpenMP). Plain C, no BLAS."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = dbl
        L.orc_e2m1_to_double.argtypes = [i32]
        L.orc_e2m1_to_double.restype = dbl
        L.orc_e4m3_to_double.argtypes = [i32]
        L.orc_e4m3_to_double.restype = dbl
        L.orc_e8m0_to_double.argtypes = [i32]
        L.orc_e8m0_to_double.restype = dbl
        L.orc_decode.argtypes = [i32, vp, i64, vp]
        L.orc_decode_mxfp4_row.argtypes = [vp, vp, i32, vp]
        L.orc_decode_mxfp8_row.argtypes = [vp, vp, i32, vp]
        L.orc_compress_mean.argtypes = [i64, i32, i32, i32, vp, vp]
        L.orc_n_vis.argtypes = [i64, i32, i64]
        L.orc_n_vis.restype = i64
        L.orc_n_vis_len.argtypes = [i64, i32, i64, i64]
        L.orc_n_vis_len.restype = i64
        L.orc_scores_row.argtypes = [i32, i32, i64, i64, i32, vp, vp, vp, i32, vp, vp, vp]
        L.orc_topk_row.argtypes = [vp, i64, i32, vp]
        L.orc_topk_row.restype = i32
        L.orc_attend_row.argtypes = [i32, i32, i32, i32, vp, i32, vp, vp, i32, i32, vp, i64,
                                     i64, i64, i32, dbl, vp, vp, vp]
        L.orc_max_threads.restype = i32
        for f in ("orc_decode", "orc_decode_mxfp4_row", "orc_decode_mxfp8_row",
                  "orc_compress_mean", "orc_scores_row",
                  "orc_attend_row"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dt_of(a: np.ndarray, hint: Optional[str] = None) -> int:
    if hint is not None:
        return _DT[hint]
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"no stored dtype for {a.dtype}")


# ---- single steps ---------------------------------------------------------------------------

def decode(a: np.ndarray) -> np.ndarray:
    """Stored f32 / bf16(uint16) / f64 values -> fp64 (exact)."""
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, np.float64)
    lib().orc_decode(_dt_of(a), _p(a), a.size, _p(out))
    return out


def decode_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows (codes [..., D/2], scales [..., D/32]) -> fp64 [..., D]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    D = codes.shape[-1] * 2
    rows = codes.size // (D // 2)
    out = np.empty((rows, D), np.float64)
    c2, s2 = codes.reshape(rows, D // 2), scales.reshape(rows, D // 32)
    for r in range(rows):
        lib().orc_decode_mxfp4_row(_p(c2[r]), _p(s2[r]), D, _p(out[r]))
    return out.reshape(codes.shape[:-1] + (D,))


def decode_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 rows (e4m3 codes [..., D], scales [..., D/32]) -> fp64 [..., D]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    D = codes.shape[-1]
    c2 = codes.reshape(-1, D)
    s2 = scales.reshape(-1, D // 32)
    out = np.empty((c2.shape[0], D), np.float64)
    for r in range(c2.shape[0]):
        lib().orc_decode_mxfp8_row(_p(c2[r]), _p(s2[r]), D, _p(out[r]))
    return out.reshape(codes.shape[:-1] + (D,))


def e4m3(code: int) -> float:
    return lib().orc_e4m3_to_double(code)


def e2m1(code: int) -> float:
    return lib().orc_e2m1_to_double(code)


def e8m0(byte: int) -> float:
    return lib().orc_e8m0_to_double(byte)


def compress_mean(raw: np.ndarray, m: int) -> np.ndarray:
    """One sequence raw [n_raw, D] (f32/bf16/f64) -> fp64 means [n_raw // m, D]."""
    raw = np.ascontiguousarray(raw)
    n_raw, D = raw.shape
    out = np.empty((n_raw // m, D), np.float64)
    lib().orc_compress_mean(n_raw, D, m, _dt_of(raw), _p(raw), _p(out))
    return out


def n_vis(p: int, m: int, N: int, seq_len: Optional[int] = None) -> int:
    """Visible entries of a query at position p (and, for a ragged batch, a sequence holding
    seq_len entries)."""
    if seq_len is None:
        return int(lib().orc_n_vis(int(p), int(m), int(N)))
    return int(lib().orc_n_vis_len(int(p), int(m), int(N), int(seq_len)))


def scores_row(q_I: np.ndarray, w: np.ndarray, k_I, n_visible: int,
               k_scale: Optional[np.ndarray] = None,
               q_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """One query: q_I [H_I, D_I] (or MXFP8 codes [H_I, D_I] uint8 with q_scale [H_I, D_I/32]),
    w [H_I] fp32, k_I [N, D_I] (or MXFP4 codes [N, D_I/2] / MXFP8 codes [N, D_I], uint8, with
    k_scale [N, D_I/32]) -> fp64 scores [N] (-inf for s >= n_visible)."""
    q_I = np.ascontiguousarray(q_I)
    w = np.ascontiguousarray(w, np.float32)
    H_I, D_I = q_I.shape
    if q_scale is not None:
        qdt = MXFP8
        q_I = np.ascontiguousarray(q_I, np.uint8)
        q_scale = np.ascontiguousarray(q_scale, np.uint8)
        assert q_scale.shape == (H_I, D_I // 32)
    else:
        qdt = _dt_of(q_I)
    k_I = np.ascontiguousarray(k_I)
    N = k_I.shape[0]
    if k_scale is not None:
        k_scale = np.ascontiguousarray(k_scale, np.uint8)
        assert k_I.dtype == np.uint8 and k_scale.shape == (N, D_I // 32)
        if k_I.shape[1] * 2 == D_I:
            kdt = MXFP4
        else:
            assert k_I.shape[1] == D_I
            kdt = MXFP8
    else:
        kdt = _dt_of(k_I)
        assert k_I.shape[1] == D_I
    out = np.empty(N, np.float64)
    lib().orc_scores_row(H_I, D_I, N, int(n_visible), qdt, _p(q_I), _p(q_scale), _p(w), kdt,
                         _p(k_I), _p(k_scale), _p(out))
    return out


def topk_row(scores: np.ndarray, n_visible: int, k: int) -> Tuple[np.ndarray, int]:
    """-> (idx [k] int32 ascending then -1, count)."""
    scores = np.ascontiguousarray(scores, np.float64)
    idx = np.empty(k, np.int32)
    cnt = lib().orc_topk_row(_p(scores), int(n_visible), int(k), _p(idx))
    return idx, int(cnt)


def attend_row(q: np.ndarray, kv: Optional[np.ndarray], idx: np.ndarray, D_V: int, scale: float,
               p: int = 0, W: int = 0, kv_raw: Optional[np.ndarray] = None, raw_base: int = 0,
               sink: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One query: q [H, D_K], kv [N, D_K] (f32/bf16/f64) or an MX cache (codes, scales): MXFP8
    (codes [N, D_K]) or MXFP4 (codes [N, D_K/2]), idx [k] (-1 = none), raw window rows
    kv_raw [n_raw, D_K] at positions raw_base.., optional sink logits [H] (fp32 values) ->
    (out [H, D_V] fp64, lse [H] fp64)."""
    q = np.ascontiguousarray(q)
    H, D_K = q.shape
    idx = np.ascontiguousarray(idx, np.int32)
    if isinstance(kv, tuple):
        # a low-precision cache (scales [N, D_K/32]; codes [N, D_K] e4m3 or [N, D_K/2] e2m1
        # pairs): the referenced rows decoded exactly (code x 2^(e-127)); the entry set and so
        # the softmax are order-free
        codes, scales = kv
        dec = decode_mxfp4 if codes.shape[-1] * 2 == D_K else decode_mxfp8
        assert codes.shape[-1] in (D_K, D_K // 2)
        sel = idx[idx >= 0]
        rows = dec(codes[sel], scales[sel]) if sel.size else np.zeros((1, D_K))
        remap = np.full(idx.shape, -1, np.int32)
        remap[idx >= 0] = np.arange(sel.size, dtype=np.int32)
        kv, idx = rows, remap
    if kv is None:
        kv = np.zeros((1, D_K), np.float64)
        assert (idx < 0).all()
    kv = np.ascontiguousarray(kv)
    assert kv.shape[1] == D_K
    assert idx.max(initial=-1) < kv.shape[0]
    n_raw = 0
    rawdt = F64
    if kv_raw is not None:
        kv_raw = np.ascontiguousarray(kv_raw)
        n_raw = kv_raw.shape[0]
        rawdt = _dt_of(kv_raw)
    out = np.empty((H, D_V), np.float64)
    lse = np.empty(H, np.float64)
    sk = None if sink is None else np.ascontiguousarray(sink, np.float64)
    assert sk is None or sk.shape == (H,)
    lib().orc_attend_row(H, D_K, D_V, _dt_of(q), _p(q), _dt_of(kv), _p(kv), _p(idx), idx.size,
                         rawdt, _p(kv_raw), int(raw_base), int(n_raw), int(p), int(W),
                         float(scale), _p(sk), _p(out), _p(lse))
    return out, lse


def dense_entries(n_visible: int, N: int) -> np.ndarray:
    """Entry list of heavily compressed attention (HCA; Tencent Cloud CSA/HCA snippets: the
    compressed sequence is attended densely, with no sparse selection): every visible
    compressed entry, 0 .. n_visible-1, padded with -1 to N (at least one slot)."""
    idx = np.full(max(int(N), 1), -1, np.int32)
    idx[: int(n_visible)] = np.arange(int(n_visible), dtype=np.int32)
    return idx


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---- composition over one query of a workload -----------------------------------------------

class QueryRunner:
    """Runs the oracle on individual queries (b, t) of a ``synth.Workload``.

    Holds per-sequence decoded-or-stored inputs; big query-side tensors are regenerated per row.
    For CSA workloads that compress, the compressed entries are the fp64 means of kv_raw."""

    def __init__(self, wl):
        self.wl = wl
        self.cfg = wl.cfg
        self._kvc: Dict[int, np.ndarray] = {}

    def kv_b(self, b: int) -> np.ndarray:
        c = self.cfg
        if c.compress:
            if b not in self._kvc:
                self._kvc[b] = compress_mean(self.wl.kv_raw()[b], c.m)
            return self._kvc[b]
        kv = self.wl.kv()
        if isinstance(kv, tuple):
            return kv[0][b], kv[1][b]
        return kv[b]

    def raw_b(self, b: int):
        raw = self.wl.kv_raw()
        if raw is None or self.cfg.W == 0:
            return None
        return raw[b]

    def n_vis(self, b: int, t: int) -> int:
        c = self.cfg
        lens = self.wl.seq_len()
        return n_vis(int(self.wl.q_pos()[b, t]), c.m, c.N,
                     seq_len=None if lens is None else int(lens[b]))

    def scores(self, b: int, t: int) -> np.ndarray:
        c = self.cfg
        nv = self.n_vis(b, t)
        w = self.wl.w()[b, t]
        qs = None
        if c.qi_dt == "mxfp8":
            qc, qsc = self.wl.q_I()
            qI, qs = qc[b, t], qsc[b, t]
        else:
            qI = self.wl.q_I()[b, t] if "q_I" in self.wl._cache else self.wl.q_I_rows(b, t)
        if c.k_dt in ("mxfp4", "mxfp8"):
            codes, sc = self.wl.k_I()
            return scores_row(qI, w, codes[b], nv, k_scale=sc[b], q_scale=qs)
        return scores_row(qI, w, self.wl.k_I()[b], nv, q_scale=qs)

    def attend(self, b: int, t: int, idx: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        c = self.cfg
        p = int(self.wl.q_pos()[b, t])
        q = self.wl.q()[b, t] if "q" in self.wl._cache else self.wl.q_rows(b, t)
        base, _ = self.wl.raw_extent()
        sink = self.wl.sink()
        return attend_row(q, self.kv_b(b), idx, c.D_V, c.softmax_scale, p=p, W=c.W,
                          kv_raw=self.raw_b(b), raw_base=base,
                          sink=None if sink is None else sink.astype(np.float64))

    def run(self, b: int, t: int) -> Dict[str, np.ndarray]:
        c = self.cfg
        p = int(self.wl.q_pos()[b, t])
        nv = self.n_vis(b, t)
        sc = self.scores(b, t)
        idx, cnt = topk_row(sc, nv, c.top_k)
        out, lse = self.attend(b, t, idx)
        return dict(scores=sc, idx=idx, count=cnt, out=out, lse=lse, n_vis=nv, p=p)

    def run_dense(self, b: int, t: int) -> Dict[str, np.ndarray]:
        """HCA: attention over every visible compressed entry (+ the raw window)."""
        c = self.cfg
        p = int(self.wl.q_pos()[b, t])
        nv = self.n_vis(b, t)
        out, lse = self.attend(b, t, dense_entries(nv, c.N))
        return dict(out=out, lse=lse, n_vis=nv, p=p)

    def run_many(self, queries: Sequence[Tuple[int, int]]):
        return [self.run(b, t) for (b, t) in queries]
