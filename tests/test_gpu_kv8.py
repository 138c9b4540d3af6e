"""An MX latent KV cache (DeepSeek-V4.1-Flash summary on the "sparse attention" tag page: the
main KV is stored in FP4): dsa_forward, hca_forward and sparse_mla_attend_mxkv over e4m3 (MXFP8)
or e2m1 (MXFP4) entries with one E8M0 scale per 32 elements, against the oracle decoding the same
bytes exactly. Every path the bf16 cache takes is taken once more: split and unsplit MFMA attention,
the fused decode selection, MXFP8 blocks beside bf16 raw window rows in one tile, dense HCA,
the scalar kernel for other shapes, and the attention sink; sharp variants give the attention
check teeth.
"""
import pytest
import torch

import synth
from test_gpu_workloads import _run, _run_fused, _run_hca

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.empty_cache()


def test_decode_kv8():
    # 16 rows: the attention selects the top-k itself and splits each row's entries
    _run(synth.CONFIGS["decode_kv8"])
    _run(synth.CONFIGS["decode_kv8"].sharp())


def test_prefill_kv8():
    _run(synth.CONFIGS["prefill_kv8"], n_sample=12, always=(0, 2047, 2048, 32767))


def test_prefill_kv8_sharp_8k():
    c = synth.CONFIGS["prefill_kv8"].with_(T=8192, N=8192).sharp()
    _run(c, n_sample=12, always=(0, 2047, 2048, 8191))


def test_csa_decode_kv8_with_window():
    # MXFP8 blocks and bf16 raw window rows share the last tiles of each row
    p = 4 * 40000 - 1
    c = synth.CONFIGS["csa_decode"].with_(B=2, N=40000, pos0=p, raw_base=p + 1 - 128,
                                          kv_dt="mxfp8", name="csa_decode_kv8")
    _run(c)
    _run(c.sharp())


def test_fused_selection_kv8_csa_window():
    p0 = 4 * 3000
    c = synth.CONFIGS["csa_decode"].with_(B=2, T=40, N=5003, pos0=p0, pos_stride=203,
                                          raw_base=p0 - 127, n_raw=203 * 39 + 128,
                                          kv_dt="mxfp8", name="fused_csa_kv8")
    _run_fused(c)


def test_hca_decode_kv8():
    c = synth.CONFIGS["hca_decode"].with_(kv_dt="mxfp8", name="hca_decode_kv8")
    _run_hca(c)
    _run_hca(c.sharp())


def test_scalar_kernel_kv8_with_sink():
    # D_K = 64, D_V = 48: not the MFMA shape, so the scalar kernel decodes the entries
    c = synth.CONFIGS["tiny"].with_(dt="bf16", k_dt="bf16", kv_dt="mxfp8", sink=(-1.0, 2.0),
                                    name="tiny_kv8_sink")
    _run(c)
    _run(c.sharp())


# ---- MXFP4 (e2m1 pairs, low nibble first) ----------------------------------------------------

def test_decode_kv4():
    _run(synth.CONFIGS["decode_kv4"])
    _run(synth.CONFIGS["decode_kv4"].sharp())


def test_prefill_kv4():
    _run(synth.CONFIGS["prefill_kv4"], n_sample=12, always=(0, 2047, 2048, 32767))


def test_prefill_kv4_sharp_8k():
    c = synth.CONFIGS["prefill_kv4"].with_(T=8192, N=8192).sharp()
    _run(c, n_sample=12, always=(0, 2047, 2048, 8191))


def test_csa_decode_kv4_with_window():
    p = 4 * 40000 - 1
    c = synth.CONFIGS["csa_decode"].with_(B=2, N=40000, pos0=p, raw_base=p + 1 - 128,
                                          kv_dt="mxfp4", name="csa_decode_kv4")
    _run(c)
    _run(c.sharp())


def test_fused_selection_kv4_csa_window():
    p0 = 4 * 3000
    c = synth.CONFIGS["csa_decode"].with_(B=2, T=40, N=5003, pos0=p0, pos_stride=203,
                                          raw_base=p0 - 127, n_raw=203 * 39 + 128,
                                          kv_dt="mxfp4", name="fused_csa_kv4")
    _run_fused(c)


def test_hca_decode_kv4():
    c = synth.CONFIGS["hca_decode"].with_(kv_dt="mxfp4", name="hca_decode_kv4")
    _run_hca(c)
    _run_hca(c.sharp())


def test_scalar_kernel_kv4_with_sink():
    c = synth.CONFIGS["tiny"].with_(dt="bf16", k_dt="bf16", kv_dt="mxfp4", sink=(-1.0, 2.0),
                                    name="tiny_kv4_sink")
    _run(c)
    _run(c.sharp())

