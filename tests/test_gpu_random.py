"""Seeded random shapes through the same checks as the hand-written parity tests: topk_select
(lengths 1 .. 300000, k 1 .. 4096, m = 1 / 4, ties, sorted and constant rows), indexer_scores
(head counts 1 .. 64, dims 8 .. 128, fp32 / bf16 / MXFP4 / MXFP8 inputs, causal positions),
sparse_mla_attend (the MFMA shape and small generic shapes, fp32 / bf16, masked entries,
sinks), dsa_forward over ragged batches (sequence lengths below and past the query
positions, sinks, MX caches, rows longer than 32768 entries), over contexts of 4100 .. 32768
entries, and CSA / HCA calls that compress the raw cache themselves. One fixed seed per generator, so every run checks the same cases."""
import numpy as np
import pytest
import torch

import synth
from test_gpu_parity import _attend_case, _hca_case, _run_indexer, _topk_case
from test_gpu_serving import _run_checked
from test_gpu_workloads import _run

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.empty_cache()


def test_random_topk():
    rng = np.random.default_rng(77)
    for i in range(60):
        N = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(5000, 40000)),
                            int(rng.integers(40000, 300000))]))
        k = int(rng.choice([1, 7, 64, 257, 1024, 2048, 3000, 4096]))
        m = int(rng.choice([1, 4]))
        rows = int(rng.integers(1, 10))
        pos = rng.integers(0, N * m, rows).astype(np.int32)
        kind = int(rng.integers(0, 3))
        order = "sorted" if kind == 1 and rows >= 3 else None
        _topk_case(f"rand{i}_N{N}_k{k}_m{m}", rows, N, k, m=m, ties=kind == 2, pos=pos,
                   seed=100 + i, order=order)


def _indexer_cases(n, rng):
    out = []
    for i in range(n):
        H_I = int(rng.choice([1, 4, 8, 16, 32, 64]))
        D_I = int(rng.choice([8, 32, 64, 128]))
        fmt = int(rng.integers(0, 4))
        dt = "f32" if fmt == 0 else "bf16"
        k_dt, qi_dt = dt, ""
        if D_I % 32 == 0 and fmt >= 2:
            k_dt = str(rng.choice(["mxfp4", "mxfp8"]))
            if fmt == 3 and dt == "bf16":
                qi_dt = "mxfp8"
                k_dt = "mxfp8" if rng.random() < 0.5 else k_dt
        m = int(rng.choice([1, 1, 4]))
        N = int(rng.integers(1, 6000))
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 80))
        span = N * m
        pos0 = int(rng.integers(0, span))
        stride = int(rng.integers(0, max(1, (span - pos0) // max(T, 1)) + 1))
        out.append(synth.CONFIGS["tiny"].with_(B=B, T=T, N=N, H_I=H_I, D_I=D_I, m=m, dt=dt,
                                               k_dt=k_dt, qi_dt=qi_dt, pos0=pos0,
                                               pos_stride=stride, seed=3000 + i,
                                               name=f"rix{i}"))
    return out


def _attention_cases(n, rng):
    out = []
    for i in range(n):
        shape = int(rng.integers(0, 3))
        H, D_K, D_V = [(128, 576, 512), (8, 64, 48), (16, 128, 96)][shape]
        if shape == 0 and rng.random() < 0.5:
            H = 64
        dt = "bf16" if shape == 0 or rng.random() < 0.5 else "f32"
        N = int(rng.integers(1, 5000))
        k = int(rng.choice([1, 32, 100, 512, 2048]))
        B, T = int(rng.integers(1, 4)), int(rng.choice([1, 3, 70, 300] if shape else [1, 3, 70]))
        pos0 = int(rng.integers(0, N))
        stride = int(rng.integers(0, max(1, (N - pos0) // max(T, 1)) + 1))
        sink = (-2.0, 3.0) if rng.random() < 0.3 else ()
        c = synth.CONFIGS["decode"].with_(B=B, T=T, N=N, H=H, D_K=D_K, D_V=D_V, dt=dt, top_k=k,
                                          pos0=pos0, pos_stride=stride, W=0, n_raw=0,
                                          raw_base=0, sink=sink, scale=1.0 / np.sqrt(D_K),
                                          seed=4000 + i, name=f"rat{i}")
        if rng.random() < 0.4:
            c = c.sharp()
        out.append((c, float(rng.choice([0.0, 0.05, 0.5]))))
    return out


def test_random_indexer_and_attention():
    rng = np.random.default_rng(4242)
    ixs, ats = _indexer_cases(40, rng), _attention_cases(30, rng)
    for c in ixs:
        _run_indexer(c, c.name)
    for c, frac in ats:
        _attend_case(c, c.name, seed=int(c.seed), frac_masked=frac)


def ragged_cases():
    """Random ragged batches for dsa_forward (also used by the no-alloc comparison)."""
    out = []
    for seed in range(5):
        rng = np.random.default_rng(1000 + seed)
        for i, base in enumerate(("decode", "decode", "csa_decode", "decode_kv8", "decode_kv4")):
            c = synth.CONFIGS[base]
            B = int(rng.integers(1, 6))
            if base == "csa_decode":
                N, m, T = int(rng.integers(33000, 45000)), 4, 1
                p = m * N - 1 - int(rng.integers(0, 50))
                kw = dict(raw_base=p + 1 - 128, n_raw=128, W=128)
            else:
                N, m = int(rng.integers(900, 9000)), 1
                T = int(rng.integers(1, 3)) if i != 1 else int(rng.integers(30, 60))
                p = int(rng.integers(N // 3, N - T))
                kw = dict(W=0, n_raw=0, raw_base=0)
            top_k = int(rng.choice([64, 512, 1024, 2048]))
            lens = tuple(int(rng.integers(1, N + 1)) for _ in range(B))
            stride = 1 if T == 1 else int(rng.integers(1, max(2, (N * m - p) // T)))
            sink = (-2.0, 4.0) if rng.random() < 0.5 else ()
            cfg = c.with_(B=B, T=T, N=N, m=m, top_k=top_k, pos0=p, pos_stride=stride,
                          seq_lens=lens, sink=sink, w_lo=-0.5, seed=2000 + 10 * seed + i,
                          name=f"srv{seed}_{i}_{base}", **kw)
            if rng.random() < 0.5:
                cfg = cfg.sharp()
            out.append(cfg)
    return out


@pytest.mark.parametrize("cfg", ragged_cases(), ids=lambda c: c.name)
def test_random_ragged_batches(cfg):
    _run_checked(cfg, n_check=6)

def _long_context_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        base = ["decode", "prefill", "csa_decode", "prefill"][i % 4]
        c = synth.CONFIGS[base]
        m = 4 if base == "csa_decode" else int(rng.choice([1, 1, 4]))
        N = int(rng.integers(4100, 32768))
        top_k = int(rng.choice([257, 1024, 2048, 3000]))
        if base == "prefill":
            B, T = 1, int(rng.integers(65, 400))
        else:
            B, T = int(rng.integers(1, 4)), int(rng.integers(1, 24))
        span = N * m
        pos0 = int(rng.integers(span // 4, span - T))
        stride = int(rng.integers(1, max(2, (span - pos0) // max(T, 1))))
        k_dt = c.k_dt if base == "csa_decode" else "bf16"
        cfg = c.with_(B=B, T=T, N=N, m=m, top_k=top_k, pos0=pos0, pos_stride=stride, W=0,
                      n_raw=0, raw_base=0, compress=False, k_dt=k_dt, seed=900 + 10 * seed + i,
                      name=f"long{seed}_{i}_{base}_N{N}_k{top_k}")
        if i % 3 == 2:
            cfg = cfg.sharp()
        out.append(cfg)
    return out


@pytest.mark.parametrize("cfg", _long_context_cases(12, 1), ids=lambda c: c.name)
def test_random_long_context(cfg):
    # contexts of 4100 .. 32768 entries: the streaming top-k's sampled threshold and candidate
    # segments, prefill tiles across many key blocks
    _run(cfg, n_sample=24, always=(0,), bf16_scale_allowance=cfg.name.endswith("_sharp"))

def _compressing_cases(seed):
    """CSA dsa_forward (m = 4, window or not) and HCA hca_forward (m = 8 / 16 / 128) calls that
    pool kv_raw themselves."""
    rng = np.random.default_rng(seed)
    csa, hca = [], []
    for i in range(12):
        N = int(rng.integers(300, 6000))
        n_raw = 4 * N
        T, B = int(rng.choice([1, 5, 100])), int(rng.integers(1, 3))
        p0 = int(rng.integers(0, max(1, n_raw - T)))
        stride = int(rng.integers(1, max(2, (n_raw - p0) // T)))
        c = synth.CONFIGS["csa_prefill"].with_(B=B, T=T, N=N, n_raw=n_raw, raw_base=0, pos0=p0,
                                               pos_stride=stride, W=int(rng.choice([0, 128])),
                                               top_k=int(rng.choice([64, 257, 1024, 2048])),
                                               seed=5000 + i, name=f"csac{i}")
        csa.append(c.sharp() if rng.random() < 0.4 else c)
    for i in range(10):
        m = int(rng.choice([8, 16, 128]))
        N = int(rng.integers(20, 1200))
        n_raw = m * N
        T, B = int(rng.choice([1, 4, 100])), int(rng.integers(1, 3))
        p0 = int(rng.integers(0, max(1, n_raw - T)))
        stride = int(rng.integers(1, max(2, (n_raw - p0) // T)))
        c = synth.CONFIGS["hca_prefill"].with_(B=B, T=T, N=N, m=m, n_raw=n_raw, raw_base=0,
                                               pos0=p0, pos_stride=stride, seed=6000 + i,
                                               name=f"hcac{i}_m{m}")
        hca.append(c.sharp() if rng.random() < 0.4 else c)
    return csa, hca


def test_random_compressing_calls():
    csa, hca = _compressing_cases(1)
    for c in csa:
        _run(c, n_sample=24, always=(0,), bf16_scale_allowance=c.name.endswith("_sharp"))
    for c in hca:
        _hca_case(c)

def test_random_mx_prefill_indexer():
    # the prefill-shaped MX indexer (MXFP8 q_I, MXFP4 / MXFP8 keys, >= 64 query rows) and the
    # bf16 one, at 64 heads x 128
    rng = np.random.default_rng(99)
    for i in range(16):
        mx = i % 2 == 0
        m = int(rng.choice([1, 4]))
        N = int(rng.integers(100, 8000))
        T = int(rng.integers(64, 300))
        span = N * m
        pos0 = int(rng.integers(0, max(1, span - T)))
        stride = int(rng.integers(1, max(2, (span - pos0) // T)))
        c = synth.CONFIGS["prefill_fp8" if mx else "prefill"].with_(
            B=int(rng.integers(1, 3)), T=T, N=N, m=m, pos0=pos0, pos_stride=stride,
            k_dt=str(rng.choice(["mxfp4", "mxfp8"])) if mx else "bf16", seed=7000 + i,
            name=f"rpx{i}")
        _run_indexer(c, c.name)
