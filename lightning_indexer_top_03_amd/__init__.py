"""Python binding of the DSA / CSA hot-path library (include/dsa.h, libdsa.so).

Argument marshalling only: every step runs in the HIP kernels of ``csrc/``. torch tensors are
used for device memory and streams; each call passes ``data_ptr()`` values and the current HIP
stream to the C ABI and raises ``DsaError`` with the library's status text on failure. There is
no fallback: without the built library the import fails.

bf16 tensors are ``torch.bfloat16``; MX keys are pairs (codes uint8, MXFP4 [B,N,D_I/2] or MXFP8
[B,N,D_I], scales uint8 [B,N,D_I/32]); an MXFP8 q_I is (codes [B,T,H_I,D_I], scales
[B,T,H_I,D_I/32]); an MXFP8 latent KV cache is (codes [B,N,D_K], scales [B,N,D_K/32]).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple, Union

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python lightning_indexer_top_03_amd/build.py` "
        "(hipcc, gfx950). There is no non-HIP fallback.")

_lib = ctypes.CDLL(LIB_PATH)

F32, BF16, MXFP4, MXFP8 = 0, 1, 2, 3
ERR_WORKSPACE, ERR_SCRATCH = 5, 8
OP_TOPK, OP_ATTEND, OP_FORWARD, OP_HCA = 1, 2, 3, 4
# the same calls over an MXFP8 latent cache (their workspace may hold a bf16 copy of it)
OP_ATTEND_MXKV, OP_FORWARD_MXKV, OP_HCA_MXKV = 5, 6, 7

EXPORTS = ("dsa_status_str", "dsa_version", "dsa_workspace_bytes", "kv_compress_mean",
           "kv_compress_blocks", "indexer_scores", "topk_select", "sparse_mla_attend",
           "sparse_mla_attend_mxkv", "dsa_forward", "hca_forward", "dsa_forward_noalloc",
           "dsa_noalloc_scratch_bytes")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "N", "H_I", "D_I", "H", "D_K", "D_V", "top_k", "m", "W")]


class ForwardArgs(ctypes.Structure):
    _fields_ = [("dt", ctypes.c_int), ("k_dt", ctypes.c_int),
                ("q_I", ctypes.c_void_p), ("w", ctypes.c_void_p), ("k_I", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p),
                ("kv_raw", ctypes.c_void_p), ("raw_base", ctypes.c_int64),
                ("n_raw", ctypes.c_int64), ("compress", ctypes.c_int32),
                ("q_pos", ctypes.c_void_p), ("softmax_scale", ctypes.c_float),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("scores", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int32),
                ("q_scale", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("sink", ctypes.c_void_p), ("kv_scale", ctypes.c_void_p), ("kv_dt", ctypes.c_int)]


_vp, _i64, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
_D = ctypes.POINTER(Dims)
_lib.dsa_status_str.argtypes = [ctypes.c_int]
_lib.dsa_status_str.restype = ctypes.c_char_p
_lib.dsa_version.restype = ctypes.c_int
_lib.dsa_workspace_bytes.argtypes = [_D, ctypes.c_int]
_lib.dsa_workspace_bytes.restype = _sz
_lib.kv_compress_mean.argtypes = [_D, ctypes.c_int, _vp, _i64, _vp, _vp]
_lib.kv_compress_blocks.argtypes = [_D, ctypes.c_int, _vp, _i64, _vp, _i64, _i64, _i64, _vp]
_lib.indexer_scores.argtypes = [_D, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp,
                                _vp, _vp]
_lib.topk_select.argtypes = [_D, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.sparse_mla_attend.argtypes = [_D, ctypes.c_int, _vp, _vp, _vp, _vp, _i64, _i64, _vp,
                                   ctypes.c_float, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.sparse_mla_attend_mxkv.argtypes = [_D, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _i64, _i64,
                                        _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dsa_forward.argtypes = [_D, ctypes.POINTER(ForwardArgs), _vp, _sz, _vp]
_lib.hca_forward.argtypes = [_D, ctypes.POINTER(ForwardArgs), _vp, _sz, _vp]
_lib.dsa_forward_noalloc.argtypes = [_D, ctypes.POINTER(ForwardArgs), _vp]
_lib.dsa_noalloc_scratch_bytes.restype = _sz
for _f in ("kv_compress_mean", "kv_compress_blocks", "indexer_scores", "topk_select",
           "sparse_mla_attend", "sparse_mla_attend_mxkv", "dsa_forward", "hca_forward",
           "dsa_forward_noalloc"):
    getattr(_lib, _f).restype = ctypes.c_int


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.dsa_status_str(status).decode()}")


def lib():
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DsaError(status, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the DSA library must be contiguous")
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def dims(B=1, T=1, N=1, H_I=1, D_I=8, H=1, D_K=8, D_V=8, top_k=1, m=1, W=0) -> Dims:
    return Dims(B, T, N, H_I, D_I, H, D_K, D_V, top_k, m, W)


def workspace_bytes(d: Dims, op: int) -> int:
    return int(_lib.dsa_workspace_bytes(ctypes.byref(d), op))


def _workspace(d: Dims, op: int, device) -> Optional[torch.Tensor]:
    n = workspace_bytes(d, op)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


# ---- step 0 -----------------------------------------------------------------------------------

def kv_compress_mean(kv_raw: torch.Tensor, m: int, kv_c: Optional[torch.Tensor] = None):
    """kv_raw [B, n_raw, D] -> kv_c [B, n_raw // m, D] (mean of each m consecutive rows)."""
    B, n_raw, D = kv_raw.shape
    if kv_c is None:
        kv_c = torch.empty((B, n_raw // m, D), dtype=kv_raw.dtype, device=kv_raw.device)
    d = dims(B=B, D_K=D, m=m)
    _check(_lib.kv_compress_mean(ctypes.byref(d), _dt(kv_raw), _ptr(kv_raw), n_raw, _ptr(kv_c),
                                 _stream(kv_raw)), "kv_compress_mean")
    return kv_c


def kv_compress_blocks(kv_raw: torch.Tensor, m: int, kv_c: torch.Tensor, j0: int, j1: int):
    """Blocks j0 .. j1-1 of every sequence: kv_c[:, j] = mean of kv_raw[:, m*j .. m*j+m-1]
    (kv_raw [B, raw_stride, D], kv_c [B, c_stride, D]); the rest of kv_c is left alone."""
    B, raw_stride, D = kv_raw.shape
    d = dims(B=B, D_K=D, m=m)
    _check(_lib.kv_compress_blocks(ctypes.byref(d), _dt(kv_raw), _ptr(kv_raw), raw_stride,
                                   _ptr(kv_c), kv_c.shape[1], j0, j1, _stream(kv_raw)),
           "kv_compress_blocks")
    return kv_c


# ---- step 1 -----------------------------------------------------------------------------------

KeyT = Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]]


def _keys(k_I: KeyT, q_dt: int):
    """-> (codes or values, scales or None, dtype, N, D_I); MX keys are (codes, scales) pairs:
    MXFP4 codes [B,N,D_I/2] or MXFP8 codes [B,N,D_I], scales [B,N,D_I/32]."""
    if isinstance(k_I, tuple):
        codes, scales = k_I
        if codes.shape[2] == 16 * scales.shape[2]:
            return codes, scales, MXFP4, codes.shape[1], codes.shape[2] * 2
        return codes, scales, MXFP8, codes.shape[1], codes.shape[2]
    return k_I, None, _dt(k_I), k_I.shape[1], k_I.shape[2]


def _queries(q_I: KeyT):
    """-> (codes or values, scales or None, dtype); an MXFP8 q_I is (codes [B,T,H_I,D_I] uint8,
    scales [B,T,H_I,D_I/32] uint8)."""
    if isinstance(q_I, tuple):
        return q_I[0], q_I[1], MXFP8
    return q_I, None, _dt(q_I)


def indexer_scores(q_I: KeyT, w: torch.Tensor, k_I: KeyT, q_pos: torch.Tensor,
                   m: int = 1, scores: Optional[torch.Tensor] = None,
                   seq_len: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_I [B,T,H_I,D_I] or MXFP8 (codes, scales), w [B,T,H_I] fp32, k_I [B,N,D_I] or MX
    (codes, scales), q_pos [B,T] int32, seq_len [B] int32 (ragged batch) or None -> scores
    [B,T,N] fp32 (-inf where not visible)."""
    qt, qs, qdt = _queries(q_I)
    B, T, H_I, D_I = qt.shape
    kt, ks, kdt, N, _ = _keys(k_I, qdt)
    if scores is None:
        scores = torch.empty((B, T, N), dtype=torch.float32, device=qt.device)
    d = dims(B=B, T=T, N=N, H_I=H_I, D_I=D_I, m=m)
    _check(_lib.indexer_scores(ctypes.byref(d), _ptr(qt), qdt, _ptr(qs), _ptr(w), _ptr(kt),
                               _ptr(ks), kdt, _ptr(q_pos), _ptr(seq_len), _ptr(scores),
                               _stream(qt)),
           "indexer_scores")
    return scores


# ---- step 2 -----------------------------------------------------------------------------------

def topk_select(scores: torch.Tensor, q_pos: torch.Tensor, top_k: int, m: int = 1,
                idx: Optional[torch.Tensor] = None,
                seq_len: Optional[torch.Tensor] = None) -> torch.Tensor:
    """scores [B,T,N] fp32 -> idx [B,T,top_k] int32 (set semantics, -1 padded); seq_len [B]
    int32 (ragged batch) or None."""
    B, T, N = scores.shape
    if idx is None:
        idx = torch.empty((B, T, top_k), dtype=torch.int32, device=scores.device)
    d = dims(B=B, T=T, N=N, top_k=top_k, m=m)
    ws = _workspace(d, OP_TOPK, scores.device)
    _check(_lib.topk_select(ctypes.byref(d), _ptr(scores), _ptr(q_pos), _ptr(seq_len), _ptr(idx),
                            _ptr(ws), 0 if ws is None else ws.numel(), _stream(scores)),
           "topk_select")
    return idx


# ---- step 3 -----------------------------------------------------------------------------------

def _kv(kv):
    """-> (kv or codes, scales or None, codes' dtype); an MX cache is (codes, scales [B,N,D_K/32])
    with codes [B,N,D_K] (MXFP8) or [B,N,D_K/2] (MXFP4, two e2m1 codes per byte)."""
    if isinstance(kv, tuple):
        codes, scales = kv
        d_k = 32 * scales.shape[-1]
        if codes.shape[-1] not in (d_k, d_k // 2):
            raise ValueError("MX cache: codes must hold D_K (MXFP8) or D_K/2 (MXFP4) bytes per row")
        return codes, scales, (MXFP8 if codes.shape[-1] == d_k else MXFP4)
    return kv, None, F32


def sparse_mla_attend(q: torch.Tensor, kv, idx: torch.Tensor, q_pos: torch.Tensor,
                      D_V: int, softmax_scale: float, kv_raw: Optional[torch.Tensor] = None,
                      raw_base: int = 0, W: int = 0, m: int = 1,
                      out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      want_lse: bool = True, sink: Optional[torch.Tensor] = None):
    """q [B,T,H,D_K], kv [B,N,D_K] or MX (codes, scales), idx [B,T,k] int32, optional raw
    window rows kv_raw [B,n_raw,D_K] at positions raw_base.., optional attention-sink logits
    sink [H] fp32 -> (out [B,T,H,D_V], lse [B,T,H] fp32)."""
    B, T, H, D_K = q.shape
    kvt, kvs, kvdt = _kv(kv)
    N = kvt.shape[1]
    k = idx.shape[2]
    if out is None:
        out = torch.empty((B, T, H, D_V), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    d = dims(B=B, T=T, N=N, H=H, D_K=D_K, D_V=D_V, top_k=k, m=m, W=W)
    ws = _workspace(d, OP_ATTEND if kvs is None else OP_ATTEND_MXKV, q.device)
    n_raw = 0 if kv_raw is None else kv_raw.shape[1]
    if kvs is not None:
        _check(_lib.sparse_mla_attend_mxkv(ctypes.byref(d), _ptr(q), _ptr(kvt), _ptr(kvs), kvdt,
                                           _ptr(idx), _ptr(kv_raw), raw_base, n_raw, _ptr(q_pos),
                                           softmax_scale, _ptr(sink), _ptr(out), _ptr(lse),
                                           _ptr(ws), 0 if ws is None else ws.numel(), _stream(q)),
               "sparse_mla_attend_mxkv")
        return out, lse
    _check(_lib.sparse_mla_attend(ctypes.byref(d), _dt(q), _ptr(q), _ptr(kv), _ptr(idx),
                                  _ptr(kv_raw), raw_base, n_raw, _ptr(q_pos), softmax_scale,
                                  _ptr(sink), _ptr(out), _ptr(lse), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(q)),
           "sparse_mla_attend")
    return out, lse


# ---- fused ------------------------------------------------------------------------------------

class Forward:
    """A prepared dsa_forward call: dims, argument block and workspace built once, so that
    ``run()`` is a single C call (cheap to time and to capture in a HIP graph)."""

    def __init__(self, q_I, w, k_I: KeyT, q, kv, q_pos, top_k: int, D_V: int,
                 softmax_scale: float, m: int = 1, W: int = 0, kv_raw=None, raw_base: int = 0,
                 compress: bool = False, out=None, lse=None, scores=None, idx=None,
                 want_lse: bool = True, seq_len=None, sink=None):
        qt, qs, qdt = _queries(q_I)
        B, T, H_I, D_I = qt.shape
        _, _, H, D_K = q.shape
        kt, ks, kdt, N, _ = _keys(k_I, qdt)
        self.d = dims(B=B, T=T, N=N, H_I=H_I, D_I=D_I, H=H, D_K=D_K, D_V=D_V, top_k=top_k, m=m,
                      W=W)
        dev = q.device
        self.out = out if out is not None else torch.empty((B, T, H, D_V), dtype=q.dtype, device=dev)
        self.lse = lse if lse is not None else (
            torch.empty((B, T, H), dtype=torch.float32, device=dev) if want_lse else None)
        self.scores, self.idx = scores, idx
        kvt, kvs, kvdt = _kv(kv)
        self.ws = _workspace(self.d, OP_FORWARD if kvs is None else OP_FORWARD_MXKV, dev)
        self._keep = (qt, qs, w, kt, ks, q, kvt, kvs, q_pos, kv_raw, seq_len, sink)
        n_raw = 0 if kv_raw is None else kv_raw.shape[1]
        self.args = ForwardArgs(_dt(q), kdt, _ptr(qt), _ptr(w), _ptr(kt), _ptr(ks), _ptr(q),
                                _ptr(kvt), _ptr(kv_raw), raw_base, n_raw, 1 if compress else 0,
                                _ptr(q_pos), softmax_scale, _ptr(self.out), _ptr(self.lse),
                                _ptr(scores), _ptr(idx), None, 0, _ptr(qs), _ptr(seq_len),
                                _ptr(sink), _ptr(kvs), kvdt)
        self.device = dev

    def set_events(self, events) -> None:
        """Profiling aid: timing events for this call's kernels (events[2i] and events[2i+1]
        receive the start and the end of the i-th kernel), as torch.cuda.Event objects or raw
        hipEvent_t handles (int). None to clear."""
        if not events:
            self._ev = None
            self.args.events, self.args.n_events = None, 0
            return
        handles = []
        for e in events:
            if isinstance(e, int):
                handles.append(e)
                continue
            if e.cuda_event == 0:  # torch creates the HIP event lazily
                e.record()
            handles.append(e.cuda_event)
        self._ev = (ctypes.c_void_p * len(handles))(*handles)
        self.args.events = ctypes.cast(self._ev, ctypes.POINTER(ctypes.c_void_p))
        self.args.n_events = len(events)

    def run(self, stream: Optional[int] = None) -> torch.Tensor:
        st = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        _check(_lib.dsa_forward(ctypes.byref(self.d), ctypes.byref(self.args), _ptr(self.ws),
                                0 if self.ws is None else self.ws.numel(), st), "dsa_forward")
        return self.out

    def run_noalloc(self, stream: Optional[int] = None) -> torch.Tensor:
        """The same call through dsa_forward_noalloc: the library's static per-GPU scratch array
        instead of this object's workspace (calls on one GPU must not overlap)."""
        st = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        _check(_lib.dsa_forward_noalloc(ctypes.byref(self.d), ctypes.byref(self.args), st),
               "dsa_forward_noalloc")
        return self.out


def dsa_forward(q_I, w, k_I: KeyT, q, kv, q_pos, top_k: int, D_V: int, softmax_scale: float,
                **kw):
    """[compress] -> indexer -> top-k -> sparse attention. Returns (out, lse, forward)."""
    f = Forward(q_I, w, k_I, q, kv, q_pos, top_k, D_V, softmax_scale, **kw)
    f.run()
    return f.out, f.lse, f


# ---- heavily compressed attention -------------------------------------------------------------

class HcaForward(Forward):
    """A prepared hca_forward call: [compress] -> dense attention over every visible compressed
    entry (+ raw window). ``run()`` is a single C call."""

    def __init__(self, q, kv, q_pos, D_V: int, softmax_scale: float, m: int, W: int = 0,
                 kv_raw=None, raw_base: int = 0, compress: bool = False, out=None, lse=None,
                 want_lse: bool = True, seq_len=None, sink=None):
        B, T, H, D_K = q.shape
        kvt, kvs, kvdt = _kv(kv)
        N = kvt.shape[1]
        self.d = dims(B=B, T=T, N=N, H=H, D_K=D_K, D_V=D_V, m=m, W=W)
        dev = q.device
        self.out = out if out is not None else torch.empty((B, T, H, D_V), dtype=q.dtype, device=dev)
        self.lse = lse if lse is not None else (
            torch.empty((B, T, H), dtype=torch.float32, device=dev) if want_lse else None)
        self.scores = self.idx = None
        self.ws = _workspace(self.d, OP_HCA if kvs is None else OP_HCA_MXKV, dev)
        self._keep = (q, kvt, kvs, q_pos, kv_raw, seq_len, sink)
        n_raw = 0 if kv_raw is None else kv_raw.shape[1]
        self.args = ForwardArgs(_dt(q), _dt(q), None, None, None, None, _ptr(q), _ptr(kvt),
                                _ptr(kv_raw), raw_base, n_raw, 1 if compress else 0,
                                _ptr(q_pos), softmax_scale, _ptr(self.out), _ptr(self.lse),
                                None, None, None, 0, None, _ptr(seq_len), _ptr(sink), _ptr(kvs),
                                kvdt)
        self.device = dev

    def run(self, stream: Optional[int] = None) -> torch.Tensor:
        st = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        _check(_lib.hca_forward(ctypes.byref(self.d), ctypes.byref(self.args), _ptr(self.ws),
                                0 if self.ws is None else self.ws.numel(), st), "hca_forward")
        return self.out


def hca_forward(q, kv, q_pos, D_V: int, softmax_scale: float, m: int, **kw):
    """[compress] -> dense attention over every visible compressed entry. Returns (out, lse, f)."""
    f = HcaForward(q, kv, q_pos, D_V, softmax_scale, m, **kw)
    f.run()
    return f.out, f.lse, f
