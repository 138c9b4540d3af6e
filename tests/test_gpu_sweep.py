"""Seeded random shapes through dsa_forward, every row against the fp64 oracle.

The workload tests run the five configurations and hand-picked edge cases; this sweep draws
batch, query count, context length, positions, top-k, compression ratio and key / query storage
at random (one fixed seed, so every run checks the same cases) to reach combinations the
hand-picked cases do not: small and odd top-k, contexts shorter than k, queries that see
nothing yet, decode- and prefill-sized row counts, bf16 / MXFP4 / MXFP8 indexer inputs, and
sharp attention inputs.
"""
import numpy as np
import pytest
import torch

import synth
from test_gpu_parity import _hca_case
from test_gpu_workloads import _run

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.empty_cache()


def _cases(n=14, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        base = ["decode", "prefill", "csa_decode", "decode_fp8"][i % 4]
        c = synth.CONFIGS[base]
        m = 4 if base == "csa_decode" else int(rng.choice([1, 1, 4]))
        N = int(rng.integers(200, 4000))
        top_k = int(rng.choice([32, 100, 257, 1024, 2048]))
        if base == "prefill":
            B, T = 1, int(rng.integers(65, 200))    # prefill-shaped kernels (>= 64 rows)
        else:
            B, T = int(rng.integers(1, 4)), int(rng.integers(1, 24))
        span = N * m
        pos0 = 0 if i % 5 == 0 else int(rng.integers(0, max(1, span // 2)))
        stride = int(rng.integers(1, max(2, (span - pos0) // max(T, 1))))
        k_dt = c.k_dt if base in ("csa_decode", "decode_fp8") else "bf16"
        cfg = c.with_(B=B, T=T, N=N, m=m, top_k=top_k, pos0=pos0, pos_stride=stride, W=0,
                      n_raw=0, raw_base=0, compress=False, k_dt=k_dt, seed=500 + i,
                      name=f"sweep{i}_{base}_m{m}_k{top_k}")
        if i % 3 == 2:
            cfg = cfg.sharp()
        cases.append(cfg)
    return cases


@pytest.mark.parametrize("cfg", _cases(), ids=lambda c: c.name)
def test_random_shapes(cfg):
    # sharp rows that see only a handful of entries have outputs of several units: their bar
    # carries the bf16 rounding of P and of the stored output (see check_attention)
    _run(cfg, n_sample=48, always=(0,), bf16_scale_allowance=cfg.name.endswith("_sharp"))


def _window_cases(n=4, seed=2025):
    # CSA blocks with the 128-token raw window: the raw rows held start at the first window row
    # of the first query and end at the last query
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        c = synth.CONFIGS["csa_decode"]
        N = int(rng.integers(300, 4000))
        top_k = int(rng.choice([64, 257, 1024]))
        B, T = int(rng.integers(1, 3)), int(rng.integers(2, 30))
        p0 = int(rng.integers(0, 2 * N))
        stride = int(rng.integers(1, max(2, (4 * N - p0) // T)))
        base = max(0, p0 - 127)
        last = p0 + stride * (T - 1)
        cfg = c.with_(B=B, T=T, N=N, top_k=top_k, pos0=p0, pos_stride=stride, raw_base=base,
                      n_raw=last - base + 1, seed=600 + i, name=f"sweepw{i}_k{top_k}")
        cases.append(cfg.sharp() if i % 2 else cfg)
    return cases


@pytest.mark.parametrize("cfg", _window_cases(), ids=lambda c: c.name)
def test_random_window_shapes(cfg):
    _run(cfg, n_sample=48, always=(0,), bf16_scale_allowance=cfg.name.endswith("_sharp"))


def _hca_cases(n=4, seed=2026):
    # HCA: every visible compressed entry plus the window, entry counts across the split rule
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        c = synth.CONFIGS["hca_decode"]
        m = int(rng.choice([8, 16, 128]))
        N = int(rng.integers(50, 3000))
        B, T = int(rng.integers(1, 3)), int(rng.integers(1, 9))
        p0 = int(rng.integers(0, N * m))
        stride = int(rng.integers(1, max(2, (N * m - p0) // T)))
        base = max(0, p0 - 127)
        last = p0 + stride * (T - 1)
        cases.append(c.with_(B=B, T=T, N=N, m=m, pos0=p0, pos_stride=stride, raw_base=base,
                             n_raw=last - base + 1, seed=700 + i, name=f"sweeph{i}_m{m}"))
    return cases


@pytest.mark.parametrize("cfg", _hca_cases(), ids=lambda c: c.name)
def test_random_hca_shapes(cfg):
    _hca_case(cfg)


def _scalar_cases(n=4, seed=2027):
    # the scalar kernels: fp32 inputs, small head counts and dims (the tiny configuration's
    # shapes), bf16 with heads or dims the MFMA kernels do not take
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        c = synth.CONFIGS["tiny"]
        N = int(rng.integers(20, 900))
        top_k = int(rng.choice([1, 7, 64, 300]))
        T = int(rng.integers(1, 40))
        p0 = int(rng.integers(0, N))
        stride = int(rng.integers(1, max(2, (N - p0) // T)))
        kw = dict(B=int(rng.integers(1, 3)), T=T, N=N, top_k=top_k, pos0=p0, pos_stride=stride,
                  seed=800 + i, name=f"sweeps{i}_k{top_k}")
        if i % 2:
            kw.update(dt="bf16", k_dt="bf16", H=16, H_I=8, D_I=64, name=kw["name"] + "_bf16")
        cases.append(c.with_(**kw))
    return cases


@pytest.mark.parametrize("cfg", _scalar_cases(), ids=lambda c: c.name)
def test_random_scalar_shapes(cfg):
    _run(cfg, n_sample=48, always=(0,))


def _kv8_cases(n=8, seed=2026, kv_dt="mxfp8"):
    # an MXFP8 latent cache at random shapes: decode-sized calls (split attention, gathered rows
    # converted in the kernel; some with the fused selection), prefill-sized ones (the cache
    # expanded to bf16 first), CSA blocks with bf16 raw window rows, ragged sequence lengths
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = ["decode", "prefill", "csa", "decode"][i % 4]
        N = int(rng.integers(300, 5000))
        top_k = int(rng.choice([64, 257, 1024, 2048]))
        if kind == "csa":
            c = synth.CONFIGS["csa_decode"]
            B, T = int(rng.integers(1, 3)), int(rng.integers(1, 20))
            p0 = int(rng.integers(128, 4 * N - 1))
            stride = int(rng.integers(1, max(2, (4 * N - p0) // max(T, 1))))
            base = max(0, p0 - 127)
            cfg = c.with_(B=B, T=T, N=N, top_k=min(top_k, 1024), pos0=p0, pos_stride=stride,
                          raw_base=base, n_raw=p0 + stride * (T - 1) - base + 1)
        else:
            c = synth.CONFIGS["decode" if kind == "decode" else "prefill"]
            if kind == "prefill":
                B, T = 1, int(rng.integers(130, 300))
            else:
                B, T = int(rng.integers(1, 5)), int(rng.integers(1, 40))
            pos0 = int(rng.integers(0, N // 2))
            stride = int(rng.integers(1, max(2, (N - pos0) // max(T, 1))))
            cfg = c.with_(B=B, T=T, N=N, top_k=top_k, pos0=pos0, pos_stride=stride)
        tag = "kv8" if kv_dt == "mxfp8" else "kv4"
        cfg = cfg.with_(kv_dt=kv_dt, seed=(700 if kv_dt == "mxfp8" else 800) + i,
                        name=f"sweep{tag}_{i}_{kind}_k{cfg.top_k}")
        if i % 4 == 3:
            cfg = cfg.with_(seq_lens=tuple(int(rng.integers(N // 2, N + 1)) for _ in range(cfg.B)))
        if i % 2 == 1:
            cfg = cfg.sharp()
        cases.append(cfg)
    return cases


@pytest.mark.parametrize("cfg", _kv8_cases() + _kv8_cases(6, 2027, "mxfp4"), ids=lambda c: c.name)
def test_random_shapes_mx_cache(cfg):
    _run(cfg, n_sample=32, always=(0,), bf16_scale_allowance=cfg.name.endswith("_sharp"))


def test_queries_past_their_sequence():
    # ragged batch whose later queries sit past their sequence's length (the visible count is
    # the length, below k, so every entry of the sequence is kept): the shape a seeded MX-cache
    # sweep drew, on an MXFP8 cache and on bf16
    base = synth.CONFIGS["decode_kv8"].with_(B=3, T=17, N=1249, top_k=1024, pos0=151,
                                             pos_stride=32, seq_lens=(655, 659, 694), seed=703,
                                             name="past_seq_kv8").sharp()
    _run(base, n_sample=32, always=(0, 16), bf16_scale_allowance=True)
    _run(base.with_(kv_dt="bf16", name="past_seq_bf16_sharp"), n_sample=32, always=(0, 16),
         bf16_scale_allowance=True)
