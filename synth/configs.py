"""Workload recipes: shapes, dtypes, distributions and query positions of the five DSA / CSA
workloads, plus small variants for parity tests. Pure description + calls into the generator;
no arithmetic of the method lives here.

Recipes (all seeded; seed = workload id, "sharp" variants use seed 100 + id):
  tiny      B=1  T=16    N=256     H_I=4  D_I=32  H=8   D_K=64  D_V=48  k=64   fp32
            q_I,k_I ~ N(0,1); w ~ U(0,1); q,kv ~ N(0,1)/sqrt(D_K); positions 240..255
  decode    B=16 T=1     N=8192    64x128  128/576/512  k=2048  bf16 (w fp32); scale 1/24
            q_I,k_I ~ N(0,1); w ~ U(0,1); q,kv ~ N(0,1)/24; position 8191 (cache holds the token)
  prefill   B=1  T=N=32768  64x128 128/576/512 k=2048  bf16; as decode; position t
  csa_prefill  raw 131072 tokens (kv_raw ~ N(0,1)/24) -> m=4 -> N=32768 blocks; k_I[32768,128]
            ~ N(0,1) per block; last 8192 queries (positions 122880..131071); k=1024; W=128
  csa_decode   B=4 T=1 N=262144 blocks of a 1,048,576-token context; k_I MXFP4 of N(0,1);
            q_I bf16; kv_c ~ N(0,1)/48 (the law of a 4-token mean of N(0,1)/24); the 128 raw
            window rows ~ N(0,1)/24; position 1048575; k=1024; W=128
  hca_decode   B=4 T=1 N=8192 blocks of a 1,048,576-token context compressed 128:1 (HCA: no
            indexer, every visible block attends); kv_c ~ N(0,1)/(24 sqrt(128)) (the law of a
            128-token mean of N(0,1)/24); the 128 raw window rows ~ N(0,1)/24; position 1048575
  decode_fp8 / prefill_fp8   decode / prefill with an MXFP8 indexer: q_I and k_I N(0,1)
            quantised to e4m3 with one E8M0 scale per 32 (2^(floor(log2 amax) - 8), RNE,
            saturating at 448)
  hca_prefill  raw 131072 tokens (kv_raw ~ N(0,1)/24) -> m=128 -> N=1024 blocks; last 8192
            queries (positions 122880..131071); W=128
  decode_kv8 / prefill_kv8   decode / prefill over an MXFP8 latent KV cache: the same
            N(0,1)/24 entries quantised to e4m3 with one E8M0 scale per 32 elements (as above)
  decode_kv4 / prefill_kv4   the same over an MXFP4 latent KV cache: e2m1 codes (two per byte,
            low nibble first) with one E8M0 scale per 32 (2^(floor(log2 amax) - 2), RNE,
            saturating at 6)
  sharp variants: q, kv ~ N(0,1) and softmax scale 4/sqrt(D_K), so that attention outputs are
            O(1) and a wrong gather moves them by far more than the tolerance.
  sink = (lo, hi): one attention-sink logit per head, U(lo, hi), fp32, tensor id 7.
  seq_lens: entries held by each sequence of a ragged batch (visibility is clamped to them).
  w_lo < 0: head weights w ~ U(w_lo, 1) (the weights come from a learned projection, so their
            sign is not fixed): index scores of either sign, and rows whose top-k threshold is
            negative.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

from . import (TID_KI, TID_KV, TID_Q, TID_QI, TID_SINK, TID_W, TID_WIN, normal, normal_mxfp4,
               normal_mxfp8, uniform)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    B: int
    T: int
    N: int
    H_I: int
    D_I: int
    H: int
    D_K: int
    D_V: int
    top_k: int
    m: int = 1
    W: int = 0
    dt: str = "bf16"          # dtype of q_I, q, kv, kv_raw, out
    k_dt: str = "bf16"        # dtype of k_I: dt, "mxfp4" or "mxfp8"
    qi_dt: str = ""           # dtype of q_I: dt ("" ) or "mxfp8"
    kv_dt: str = ""           # dtype of the stored entries kv: dt (""), "mxfp8" or "mxfp4" (bf16 q / out)
    pos0: int = 0             # q_pos[b, t] = pos0 + pos_stride * t
    pos_stride: int = 1
    qkv_std: float = 0.0      # std of q and kv rows (0 -> 1/sqrt(D_K))
    scale: float = 0.0        # softmax scale (0 -> 1/sqrt(D_K))
    compress: bool = False    # kv is produced from kv_raw (n_raw = N*m, raw_base = 0)
    n_raw: int = 0            # raw rows held in kv_raw (window only when not compressing)
    raw_base: int = 0
    kv_std: float = 0.0       # std of stored kv entries (0 -> qkv_std)
    win_std: float = 0.0      # std of raw window rows (0 -> qkv_std)
    dense: bool = False       # HCA: no indexer / top-k, every visible entry attends
    w_lo: float = 0.0         # head weights w ~ U(w_lo, 1): a negative w_lo gives mixed signs
    sink: tuple = ()          # (lo, hi): one attention-sink logit per head ~ U(lo, hi) (fp32)
    seq_lens: tuple = ()      # entries held per sequence (ragged batch); () = N for every one

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.D_K)

    @property
    def q_std(self) -> float:
        return self.qkv_std if self.qkv_std else 1.0 / math.sqrt(self.D_K)

    @property
    def entry_std(self) -> float:
        return self.kv_std if self.kv_std else self.q_std

    @property
    def raw_std(self) -> float:
        return self.win_std if self.win_std else self.q_std

    def sharp(self) -> "Config":
        """Same shapes, q and kv ~ N(0,1), softmax scale 4/sqrt(D_K)."""
        # pooled entries keep their ratio to the raw rows (a 4-token mean of N(0,1) has std 1/2)
        kv = self.kv_std / self.q_std if self.kv_std else 0.0
        return dataclasses.replace(self, name=self.name + "_sharp", seed=100 + self.seed,
                                   qkv_std=1.0, scale=4.0 / math.sqrt(self.D_K), kv_std=kv,
                                   win_std=1.0 if self.win_std else 0.0)

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def positions(self) -> np.ndarray:
        t = np.arange(self.T, dtype=np.int64)
        p = self.pos0 + self.pos_stride * t
        return np.broadcast_to(p, (self.B, self.T)).astype(np.int32).copy()

    def dims(self) -> Dict[str, int]:
        return dict(B=self.B, T=self.T, N=self.N, H_I=self.H_I, D_I=self.D_I, H=self.H,
                    D_K=self.D_K, D_V=self.D_V, top_k=self.top_k, m=self.m, W=self.W)


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 1, B=1, T=16, N=256, H_I=4, D_I=32, H=8, D_K=64, D_V=48, top_k=64,
                   dt="f32", k_dt="f32", pos0=240),
    "decode": Config("decode", 2, B=16, T=1, N=8192, H_I=64, D_I=128, H=128, D_K=576, D_V=512,
                     top_k=2048, pos0=8191),
    "prefill": Config("prefill", 3, B=1, T=32768, N=32768, H_I=64, D_I=128, H=128, D_K=576,
                      D_V=512, top_k=2048, pos0=0),
    "csa_prefill": Config("csa_prefill", 4, B=1, T=8192, N=32768, H_I=64, D_I=128, H=128,
                          D_K=576, D_V=512, top_k=1024, m=4, W=128, pos0=122880,
                          compress=True, n_raw=131072),
    "csa_decode": Config("csa_decode", 5, B=4, T=1, N=262144, H_I=64, D_I=128, H=128, D_K=576,
                         D_V=512, top_k=1024, m=4, W=128, k_dt="mxfp4", pos0=1048575,
                         n_raw=128, raw_base=1048576 - 128, kv_std=1.0 / 48, win_std=1.0 / 24),
    "decode_fp8": Config("decode_fp8", 8, B=16, T=1, N=8192, H_I=64, D_I=128, H=128, D_K=576,
                         D_V=512, top_k=2048, pos0=8191, qi_dt="mxfp8", k_dt="mxfp8"),
    "prefill_fp8": Config("prefill_fp8", 9, B=1, T=32768, N=32768, H_I=64, D_I=128, H=128,
                          D_K=576, D_V=512, top_k=2048, pos0=0, qi_dt="mxfp8", k_dt="mxfp8"),
    "decode_kv8": Config("decode_kv8", 10, B=16, T=1, N=8192, H_I=64, D_I=128, H=128, D_K=576,
                         D_V=512, top_k=2048, pos0=8191, kv_dt="mxfp8"),
    "prefill_kv8": Config("prefill_kv8", 11, B=1, T=32768, N=32768, H_I=64, D_I=128, H=128,
                          D_K=576, D_V=512, top_k=2048, pos0=0, kv_dt="mxfp8"),
    "decode_kv4": Config("decode_kv4", 12, B=16, T=1, N=8192, H_I=64, D_I=128, H=128, D_K=576,
                         D_V=512, top_k=2048, pos0=8191, kv_dt="mxfp4"),
    "prefill_kv4": Config("prefill_kv4", 13, B=1, T=32768, N=32768, H_I=64, D_I=128, H=128,
                          D_K=576, D_V=512, top_k=2048, pos0=0, kv_dt="mxfp4"),
    "hca_decode": Config("hca_decode", 6, B=4, T=1, N=8192, H_I=64, D_I=128, H=128, D_K=576,
                         D_V=512, top_k=8192, m=128, W=128, pos0=1048575, n_raw=128,
                         raw_base=1048576 - 128, kv_std=1.0 / (24 * math.sqrt(128)),
                         win_std=1.0 / 24, dense=True),
    "hca_prefill": Config("hca_prefill", 7, B=1, T=8192, N=1024, H_I=64, D_I=128, H=128,
                          D_K=576, D_V=512, top_k=1024, m=128, W=128, pos0=122880,
                          compress=True, n_raw=131072, dense=True),
}


class Workload:
    """Lazily generated host tensors of one Config (numpy; bf16 as uint16 bit patterns).

    Tensor element indices follow each tensor's natural row-major layout, so rows can be
    regenerated independently (``q_rows``) without materialising multi-GB tensors."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self._cache: Dict[str, object] = {}

    # --- full tensors -------------------------------------------------------------------
    def q_pos(self) -> np.ndarray:
        return self.cfg.positions()

    def q_I(self):
        """[B,T,H_I,D_I] in dt, or (codes [B,T,H_I,D_I], scales [B,T,H_I,D_I/32]) for MXFP8."""
        c = self.cfg
        if c.qi_dt == "mxfp8":
            def mk():
                codes, sc = normal_mxfp8(c.seed, TID_QI, c.B * c.T * c.H_I, c.D_I, 1.0)
                return (codes.reshape(c.B, c.T, c.H_I, c.D_I),
                        sc.reshape(c.B, c.T, c.H_I, c.D_I // 32))
            return self._get("q_I", mk)
        return self._get("q_I", lambda: normal(c.seed, TID_QI, (c.B, c.T, c.H_I, c.D_I), 1.0, c.dt))

    def w(self) -> np.ndarray:
        c = self.cfg
        return self._get("w", lambda: uniform(c.seed, TID_W, (c.B, c.T, c.H_I), c.w_lo, 1.0))

    def k_I(self):
        """[B,N,D_I] in dt, or (codes [B,N,D_I/2], scales [B,N,D_I/32]) for MXFP4, or
        (codes [B,N,D_I], scales [B,N,D_I/32]) for MXFP8."""
        c = self.cfg
        if c.k_dt == "mxfp8":
            def mk8():
                codes, sc = normal_mxfp8(c.seed, TID_KI, c.B * c.N, c.D_I, 1.0)
                return codes.reshape(c.B, c.N, c.D_I), sc.reshape(c.B, c.N, c.D_I // 32)
            return self._get("k_I", mk8)
        if c.k_dt == "mxfp4":
            def mk():
                codes, sc = normal_mxfp4(c.seed, TID_KI, c.B * c.N, c.D_I, 1.0)
                return codes.reshape(c.B, c.N, c.D_I // 2), sc.reshape(c.B, c.N, c.D_I // 32)
            return self._get("k_I", mk)
        return self._get("k_I", lambda: normal(c.seed, TID_KI, (c.B, c.N, c.D_I), 1.0, c.k_dt))

    def q(self) -> np.ndarray:
        c = self.cfg
        return self._get("q", lambda: normal(c.seed, TID_Q, (c.B, c.T, c.H, c.D_K), c.q_std, c.dt))

    def kv(self):
        """Stored entries [B,N,D_K] (None when they are compressed from kv_raw), or for an MXFP8
        cache (e4m3 codes [B,N,D_K], E8M0 scales [B,N,D_K/32]): the same N(0,1) draws as the
        bf16 cache, quantised per 32 elements."""
        c = self.cfg
        if c.compress:
            return None
        if c.kv_dt in ("mxfp8", "mxfp4"):
            def mk():
                fn, w = (normal_mxfp8, c.D_K) if c.kv_dt == "mxfp8" else (normal_mxfp4, c.D_K // 2)
                codes, sc = fn(c.seed, TID_KV, c.B * c.N, c.D_K, c.entry_std)
                return codes.reshape(c.B, c.N, w), sc.reshape(c.B, c.N, c.D_K // 32)
            return self._get("kv", mk)
        return self._get("kv", lambda: normal(c.seed, TID_KV, (c.B, c.N, c.D_K), c.entry_std, c.dt))

    def kv_raw(self) -> Optional[np.ndarray]:
        """Raw rows [B,n_raw,D_K] at positions raw_base.. (None when W == 0 and no compression)."""
        c = self.cfg
        if c.compress:
            return self._get("kv_raw", lambda: normal(c.seed, TID_KV, (c.B, c.N * c.m, c.D_K),
                                                      c.q_std, c.dt))
        if c.W > 0:
            return self._get("kv_raw", lambda: normal(c.seed, TID_WIN, (c.B, c.n_raw, c.D_K),
                                                      c.raw_std, c.dt))
        return None

    def sink(self) -> Optional[np.ndarray]:
        """Attention-sink logits [H] fp32, or None."""
        c = self.cfg
        if not c.sink:
            return None
        return self._get("sink", lambda: uniform(c.seed, TID_SINK, (c.H,), c.sink[0], c.sink[1]))

    def seq_len(self) -> Optional[np.ndarray]:
        """Entries held per sequence [B] int32 (a ragged batch), or None."""
        c = self.cfg
        if not c.seq_lens:
            return None
        assert len(c.seq_lens) == c.B
        return np.array(c.seq_lens, np.int32)

    def raw_extent(self):
        """(raw_base, n_raw) of kv_raw."""
        c = self.cfg
        if c.compress:
            return 0, c.N * c.m
        if c.W > 0:
            return c.raw_base, c.n_raw
        return 0, 0

    # --- rows of the big query-side tensors ---------------------------------------------
    def q_rows(self, b: int, t: int) -> np.ndarray:
        c = self.cfg
        start = ((b * c.T + t) * c.H) * c.D_K
        return normal(c.seed, TID_Q, (c.H, c.D_K), c.q_std, c.dt, start=start)

    def q_I_rows(self, b: int, t: int) -> np.ndarray:
        c = self.cfg
        assert c.qi_dt != "mxfp8", "MXFP8 q_I is generated whole"
        start = ((b * c.T + t) * c.H_I) * c.D_I
        return normal(c.seed, TID_QI, (c.H_I, c.D_I), 1.0, c.dt, start=start)

    def q_chunk(self, start_row: int, rows: int) -> np.ndarray:
        """Flattened query rows [start_row, start_row+rows) of q as [rows, H, D_K]."""
        c = self.cfg
        return normal(c.seed, TID_Q, (rows, c.H, c.D_K), c.q_std, c.dt,
                      start=start_row * c.H * c.D_K)

    def drop(self, name: str) -> None:
        self._cache.pop(name, None)

    def _get(self, name, fn):
        if name not in self._cache:
            self._cache[name] = fn()
        return self._cache[name]


def make_workload(name_or_cfg) -> Workload:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    return Workload(cfg)
