"""C-ABI contract of libdsa.so, on the host: symbols, status codes, validation, workspace sizing.

Every call here fails validation (or the gfx950 device check) before any kernel is launched,
so these run without a GPU; the pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest
import torch

import lightning_indexer_top_03_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
P = 0x10000  # a 16-byte-aligned dummy address
L = dsa.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) -
                  {"sizeof", "defined", "floor", "min", "max"})


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert set(names) == set(dsa.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    for code in range(9):
        s = L.dsa_status_str(code).decode()
        assert s.startswith("DSA_"), s
    assert L.dsa_status_str(99).decode() == "unknown dsa_status"
    assert L.dsa_version() == 220


def _dims(**kw):
    base = dict(B=2, T=3, N=100, H_I=64, D_I=128, H=128, D_K=576, D_V=512, top_k=32, m=1, W=0)
    base.update(kw)
    return dsa.Dims(*[base[n] for n, _ in dsa.Dims._fields_])


def _idx_call(d, q_dt=dsa.BF16, k_dt=dsa.BF16, q_I=P, w=P, k_I=P, k_scale=None, q_pos=P, sc=P,
              q_scale=None, seq_len=None):
    return L.indexer_scores(ctypes.byref(d), q_I, q_dt, q_scale, w, k_I, k_scale, k_dt, q_pos,
                            seq_len, sc, None)


def test_indexer_validation():
    d = _dims()
    assert L.indexer_scores(None, P, 1, None, P, P, None, 1, P, None, P, None) == 1  # NULL dims
    assert _idx_call(d, seq_len=P + 2) == 4                                    # seq_len align
    assert _idx_call(d, q_I=None) == 1                                         # NULL q_I
    assert _idx_call(d, q_pos=None) == 1
    assert _idx_call(_dims(N=0)) == 2                                          # bad shape
    assert _idx_call(_dims(top_k=5000)) == 2
    assert _idx_call(d, q_dt=dsa.MXFP4) == 3                                   # bad q dtype
    assert _idx_call(d, q_dt=dsa.F32, k_dt=dsa.BF16) == 3                      # mixed
    assert _idx_call(d, k_dt=dsa.MXFP4) == 1                                   # FP4 w/o scales
    assert _idx_call(_dims(D_I=48), k_dt=dsa.MXFP4, k_scale=P) == 2            # D_I % 32
    assert _idx_call(d, k_scale=P) == 3                                        # scales w/o FP4
    assert _idx_call(_dims(H_I=128, D_I=128), q_dt=dsa.F32, k_dt=dsa.F32) == 2 # generic LDS cap
    assert _idx_call(d, q_I=P + 8) == 4                                        # misaligned
    assert _idx_call(d, sc=P + 4) == 4
    # MXFP8: q_I and/or k_I, each with its scales
    mx = dict(k_dt=dsa.MXFP8, k_scale=P)
    assert _idx_call(d, k_dt=dsa.MXFP8) == 1                                   # FP8 w/o scales
    assert _idx_call(d, q_dt=dsa.MXFP8, **mx) == 1                             # q w/o scales
    assert _idx_call(d, q_dt=dsa.MXFP8, q_scale=P, k_dt=dsa.BF16) == 3         # fp8 q, bf16 k
    assert _idx_call(d, q_dt=dsa.F32, **mx) == 3                               # fp32 q, MX k
    assert _idx_call(d, q_scale=P, **mx) == 3                                  # scales, bf16 q
    assert _idx_call(_dims(D_I=48), q_dt=dsa.MXFP8, q_scale=P, **mx) == 2      # D_I % 32
    assert _idx_call(d, q_dt=dsa.MXFP8, q_scale=P + 2, **mx) == 4              # scale alignment


def test_topk_validation():
    d = _dims()
    assert L.topk_select(ctypes.byref(d), None, P, None, P, None, 0, None) == 1
    assert L.topk_select(ctypes.byref(d), P + 4, P, None, P, None, 0, None) == 4
    assert L.topk_select(ctypes.byref(d), P, P, P + 1, P, None, 0, None) == 4
    assert L.topk_select(ctypes.byref(_dims(top_k=0)), P, P, None, P, None, 0, None) == 2
    assert L.topk_select(ctypes.byref(_dims(m=0)), P, P, None, P, None, 0, None) == 2


def _att(d, dt=dsa.BF16, q=P, kv=P, idx=P, raw=None, base=0, nraw=0, ws=None, wsb=0, out=P,
         sink=None):
    return L.sparse_mla_attend(ctypes.byref(d), dt, q, kv, idx, raw, base, nraw, P, 0.1, sink,
                               out, None, ws, wsb, None)


def test_attend_validation():
    d = _dims()
    assert _att(d, q=None) == 1
    assert _att(_dims(W=16)) == 1                  # window without kv_raw
    assert _att(_dims(D_V=600)) == 2               # D_V > D_K
    assert _att(_dims(D_K=1028)) == 2
    assert _att(d, dt=dsa.MXFP4) == 3
    assert _att(d, out=P + 2) == 4
    assert _att(d, sink=P + 2) == 4
    assert _att(_dims(W=16), raw=P, base=-1) == 2
    # few queries -> split partials need a workspace
    dd = _dims(B=1, T=1, top_k=2048)
    need = L.dsa_workspace_bytes(ctypes.byref(dd), dsa.OP_ATTEND)
    assert need > 0
    assert _att(dd) == 5
    assert _att(dd, ws=P, wsb=need - 1) == 5


def _mx(d, q=P, codes=P, scales=P, idx=P, raw=None, out=P, sink=None, ws=None, wsb=0,
        kv_dt=dsa.MXFP8):
    return L.sparse_mla_attend_mxkv(ctypes.byref(d), q, codes, scales, kv_dt, idx, raw, 0, 0, P,
                                    0.1, sink, out, None, ws, wsb, None)


def test_attend_mxkv_validation():
    d = _dims()
    assert _mx(d, scales=None) == 1              # MXFP8 codes need their scales
    assert _mx(d, codes=None) == 1
    assert _mx(_dims(D_K=80, D_V=64)) == 2       # D_K % 32
    assert _mx(_dims(W=16)) == 1                 # window without kv_raw
    assert _mx(d, codes=P + 8) == 4
    assert _mx(d, out=P + 2) == 4
    # the codes' format: MXFP8 or MXFP4 only
    for bad in (dsa.F32, dsa.BF16, 7):
        assert _mx(d, kv_dt=bad) == 3
    dd = _dims(B=1, T=1, top_k=2048)
    need = L.dsa_workspace_bytes(ctypes.byref(dd), dsa.OP_ATTEND_MXKV)
    assert need > 0 and _mx(dd) == 5
    # unsplit calls expand the cache into the workspace first
    need = L.dsa_workspace_bytes(ctypes.byref(d), dsa.OP_ATTEND_MXKV)
    assert need >= 2 * 100 * 576 * 2
    assert _mx(d) == 5 and _mx(d, ws=P, wsb=need - 1) == 5
    if not torch.cuda.is_available():
        assert _mx(d, ws=P, wsb=need) == 6


def test_forward_validation_and_workspace():
    d = _dims()
    a = dsa.ForwardArgs(dsa.BF16, dsa.BF16, P, P, P, None, P, P, None, 0, 0, 0, P, 0.1, P, None,
                        None, None, None, 0)
    need = L.dsa_workspace_bytes(ctypes.byref(d), dsa.OP_FORWARD)
    assert need >= 2 * 3 * 100 * 4 + 2 * 3 * 32 * 4
    assert L.dsa_forward(ctypes.byref(d), None, P, need, None) == 1
    assert L.dsa_forward(ctypes.byref(d), ctypes.byref(a), None, 0, None) == 5
    assert L.dsa_forward(ctypes.byref(d), ctypes.byref(a), P, need - 1, None) == 5
    a.compress = 1
    assert L.dsa_forward(ctypes.byref(d), ctypes.byref(a), P, need, None) == 1  # no kv_raw
    a.kv_raw, a.n_raw = P, 399
    assert L.dsa_forward(ctypes.byref(_dims(m=4)), ctypes.byref(a), P, need, None) == 2  # 399//4 != 100
    a.compress, a.kv_raw, a.n_raw = 0, None, 0
    a.q_I = P + 8
    assert L.dsa_forward(ctypes.byref(d), ctypes.byref(a), P, need, None) == 4
    a.q_I = P
    # an MX latent cache: bf16 path only, stored entries only, D_K % 32 == 0, an MX format
    a.kv_scale = P
    a.kv_dt = dsa.BF16
    assert L.dsa_forward(ctypes.byref(d), ctypes.byref(a), P, need, None) == 3
    a.kv_dt = dsa.MXFP4
    a.dt = dsa.F32
    assert L.dsa_forward(ctypes.byref(d), ctypes.byref(a), P, need, None) == 3
    a.dt = dsa.BF16
    a.compress, a.kv_raw, a.n_raw = 1, P, 400
    assert L.dsa_forward(ctypes.byref(_dims(m=4)), ctypes.byref(a), P, need, None) == 3
    a.compress, a.kv_raw, a.n_raw = 0, None, 0
    assert L.dsa_forward(ctypes.byref(_dims(D_K=80, D_V=64)), ctypes.byref(a), P, need, None) == 2


def test_forward_noalloc_validation():
    # the same argument rules as dsa_forward, and a clear error (nothing launched) when the call
    # needs more workspace than the static scratch array holds
    cap = L.dsa_noalloc_scratch_bytes()
    assert cap == 64 << 20
    a = dsa.ForwardArgs(dsa.BF16, dsa.BF16, P, P, P, None, P, P, None, 0, 0, 0, P, 0.1, P, None,
                        None, None, None, 0)
    dec = _dims(B=16, T=1, N=8192, top_k=2048)
    assert 0 < L.dsa_workspace_bytes(ctypes.byref(dec), dsa.OP_FORWARD) <= cap
    big = _dims(B=1, T=32768, N=32768, top_k=2048)
    assert L.dsa_workspace_bytes(ctypes.byref(big), dsa.OP_FORWARD) > cap
    assert L.dsa_forward_noalloc(ctypes.byref(big), ctypes.byref(a), None) == dsa.ERR_SCRATCH
    assert L.dsa_forward_noalloc(ctypes.byref(dec), None, None) == 1
    assert L.dsa_forward_noalloc(ctypes.byref(_dims(N=0)), ctypes.byref(a), None) == 2
    a.q = P + 4
    assert L.dsa_forward_noalloc(ctypes.byref(dec), ctypes.byref(a), None) == 4
    a.q = P
    if not torch.cuda.is_available():
        assert L.dsa_forward_noalloc(ctypes.byref(dec), ctypes.byref(a), None) == 6


def test_hca_validation_and_workspace():
    # the indexer fields are ignored (NULL here); top_k plays no part
    a = dsa.ForwardArgs(dsa.BF16, dsa.BF16, None, None, None, None, P, P, None, 0, 0, 0, P, 0.1,
                        P, None, None, None, None, 0)
    dec = _dims(B=2, T=1, N=8192, H=128, D_K=576, D_V=512, top_k=1, m=128, W=128)
    assert L.dsa_workspace_bytes(ctypes.byref(dec), dsa.OP_HCA) > 0  # few rows: split partials
    many = _dims(B=1, T=4096, N=1024, H=128, D_K=576, D_V=512, top_k=99999, m=128, W=128)
    assert L.dsa_workspace_bytes(ctypes.byref(many), dsa.OP_HCA) == 0
    need = L.dsa_workspace_bytes(ctypes.byref(dec), dsa.OP_HCA)
    assert L.hca_forward(ctypes.byref(dec), None, P, need, None) == 1
    assert L.hca_forward(ctypes.byref(dec), ctypes.byref(a), P, need, None) == 1  # W > 0, no kv_raw
    a.kv_raw, a.n_raw = P, 128
    assert L.hca_forward(ctypes.byref(dec), ctypes.byref(a), None, 0, None) == 5
    assert L.hca_forward(ctypes.byref(dec), ctypes.byref(a), P, need - 1, None) == 5
    too_many = _dims(B=2, T=1, N=10240, H=128, D_K=576, D_V=512, m=128, W=1)
    assert L.hca_forward(ctypes.byref(too_many), ctypes.byref(a), P, 1 << 30, None) == 2
    assert L.dsa_workspace_bytes(ctypes.byref(too_many), dsa.OP_HCA) == 0
    a.compress = 1  # compression needs raw_base == 0 and n_raw / m == N
    assert L.hca_forward(ctypes.byref(dec), ctypes.byref(a), P, need, None) == 2
    a.compress, a.q = 0, P + 4
    assert L.hca_forward(ctypes.byref(dec), ctypes.byref(a), P, need, None) == 4


def test_compress_blocks_validation():
    d = _dims(B=2, D_K=576, m=4)
    assert L.kv_compress_blocks(None, dsa.BF16, P, 400, P, 100, 0, 1, None) == 1
    assert L.kv_compress_blocks(ctypes.byref(d), dsa.MXFP4, P, 400, P, 100, 0, 1, None) == 3
    assert L.kv_compress_blocks(ctypes.byref(d), dsa.BF16, P, 400, P, 100, 5, 4, None) == 2   # j1 < j0
    assert L.kv_compress_blocks(ctypes.byref(d), dsa.BF16, P, 400, P, 100, 0, 101, None) == 2  # > c_stride
    assert L.kv_compress_blocks(ctypes.byref(d), dsa.BF16, P, 399, P, 100, 99, 100, None) == 2  # raw short
    assert L.kv_compress_blocks(ctypes.byref(d), dsa.BF16, P + 8, 400, P, 100, 0, 1, None) == 4


def test_compress_validation():
    d = _dims(m=4)
    assert L.kv_compress_mean(ctypes.byref(d), dsa.BF16, None, 400, P, None) == 1
    assert L.kv_compress_mean(ctypes.byref(d), dsa.MXFP4, P, 400, P, None) == 3
    assert L.kv_compress_mean(ctypes.byref(_dims(m=0)), dsa.BF16, P, 400, P, None) == 2
    assert L.kv_compress_mean(ctypes.byref(d), dsa.BF16, P, -1, P, None) == 2


def test_workspace_sizes():
    # decode-shaped calls split the entry list; large prefill calls do not need partials
    dec = _dims(B=16, T=1, N=8192, top_k=2048)
    pre = _dims(B=1, T=4096, N=4096, top_k=2048)
    assert L.dsa_workspace_bytes(ctypes.byref(dec), dsa.OP_ATTEND) > 0
    assert L.dsa_workspace_bytes(ctypes.byref(pre), dsa.OP_ATTEND) == 0
    assert L.dsa_workspace_bytes(ctypes.byref(_dims(N=0)), dsa.OP_FORWARD) == 0
    big = _dims(B=1, T=32768, N=32768, top_k=2048)
    # fused prefill chunks its score rows to a bounded workspace (< 0.6 GB)
    assert L.dsa_workspace_bytes(ctypes.byref(big), dsa.OP_FORWARD) < 600 << 20


def _al(n):
    return (n + 255) // 256 * 256


def test_workspace_sizes_mxfp8_cache():
    # split (few-row) attention converts gathered rows in the kernel: no extra bytes; unsplit
    # (many-row) attention reads a bf16 copy of the whole cache, B*N*D_K*2 bytes after the rest
    dec = _dims(B=16, T=1, N=8192, top_k=2048)
    pre = _dims(B=1, T=4096, N=4096, top_k=2048)
    ws = lambda d, op: L.dsa_workspace_bytes(ctypes.byref(d), op)
    assert ws(dec, dsa.OP_ATTEND_MXKV) == ws(dec, dsa.OP_ATTEND)
    assert ws(pre, dsa.OP_ATTEND_MXKV) == _al(ws(pre, dsa.OP_ATTEND)) + _al(4096 * 576 * 2)
    big = _dims(B=1, T=32768, N=32768, top_k=2048)
    assert ws(big, dsa.OP_FORWARD_MXKV) == ws(big, dsa.OP_FORWARD) + _al(32768 * 576 * 2)
    assert ws(dec, dsa.OP_FORWARD_MXKV) == ws(dec, dsa.OP_FORWARD)
    # scalar-kernel shapes decode in the kernel at any row count
    odd = _dims(B=1, T=4096, N=4096, top_k=2048, H=16, D_K=192, D_V=128)
    assert ws(odd, dsa.OP_ATTEND_MXKV) == ws(odd, dsa.OP_ATTEND)
    hca = _dims(B=1, T=4096, N=1024, top_k=99999, m=128, W=128)
    assert ws(hca, dsa.OP_HCA_MXKV) == _al(1024 * 576 * 2)
    assert ws(_dims(N=0), dsa.OP_FORWARD_MXKV) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU device error path")
def test_valid_call_without_gpu_reports_device_error():
    d = _dims(B=1, T=1, N=64, top_k=8)
    assert L.topk_select(ctypes.byref(d), P, P, None, P, None, 0, None) == 6
