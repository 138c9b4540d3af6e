"""bench.py's accounting on the host: the algorithmic bytes and flops behind `roofline`, checked
against sums written out from the workload shapes, and the single-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

C = synth.CONFIGS


def test_decode_attention_bytes_and_flops():
    # 16 queries x 2048 gathered rows x 1152 B, q 16 x 128 x 576 x 2 B, the fused selection
    # reads 16 x 8192 fp32 scores, index list 16 x 2048 x 4 B; the output is the merge's
    byt, fl = bench._algorithmic(C["decode"], "attend_mfma_dma", split=True)
    assert byt == 16 * 2048 * 1152 + 16 * 128 * 576 * 2 + 16 * 8192 * 4 + 16 * 2048 * 4
    assert fl == 16 * 2048 * 128 * (576 + 512) * 2
    # unsplit, the attention writes the bf16 output and the fp32 log-sum-exp itself
    byt1, _ = bench._algorithmic(C["decode"], "attend_mfma_dma", split=False)
    assert byt1 - byt == 16 * 128 * (512 * 2 + 4)
    byt_c, _ = bench._algorithmic(C["decode"], "attend_combine")
    assert byt_c == 16 * 128 * (512 * 2 + 4)


def test_decode_indexer_bytes():
    # every visible key once per query (decode), q_I + w per row, one fp32 score per key
    byt, fl = bench._algorithmic(C["decode"], "indexer_decode_dma")
    assert byt == 16 * 8192 * 256 + 16 * 64 * (128 * 2 + 4) + 16 * 8192 * 4
    assert fl == 16 * 8192 * 64 * 128 * 2


def test_csa_decode_mxfp4_indexer_bytes():
    # 262144 blocks per query at 64 code bytes + 4 scale bytes
    byt, fl = bench._algorithmic(C["csa_decode"], "indexer_decode_mx_dma")
    n = 4 * 262144
    assert byt == n * 68 + 4 * 64 * (128 * 2 + 4) + n * 4
    assert fl == n * 64 * 128 * 2


def test_prefill_flops_and_attention_bytes():
    T = 32768
    pairs = T * (T + 1) // 2  # causal, a query sees itself
    _, fl = bench._algorithmic(C["prefill"], "indexer_prefill_mfma")
    assert fl == pairs * 64 * 128 * 2
    sel = sum(min(2048, p + 1) for p in range(T))
    byt, fl = bench._algorithmic(C["prefill"], "attend_mfma_dma", split=False)
    assert fl == sel * 128 * (576 + 512) * 2
    # the sequence's KV once, q, index lists, output + lse
    assert byt == 32768 * 1152 + T * 128 * 576 * 2 + T * 2048 * 4 + T * 128 * (512 * 2 + 4)


def test_csa_prefill_window_entries():
    cfg = C["csa_prefill"]
    _, fl = bench._algorithmic(cfg, "attend_mfma_dma", split=False)
    ents = 0
    for p in cfg.positions().ravel():
        ents += min(1024, (int(p) + 1) // 4) + min(128, int(p) + 1)
    assert fl == ents * 128 * (576 + 512) * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_sample_rows():
    # prefill: 128 distinct rows, always with the first rows, both sides of the k = 2048 edge
    # and the last row; decode: every row
    rows = bench.cpu_sample_rows(C["prefill"])
    assert len(rows) == 128 and len(set(rows)) == 128
    ts = {t for _, t in rows}
    assert set(bench.PREFILL_ALWAYS) <= ts
    assert rows == bench.cpu_sample_rows(C["prefill"])  # seeded
    assert sorted(bench.cpu_sample_rows(C["decode"])) == [(b, 0) for b in range(16)]
    assert len(bench.cpu_sample_rows(C["csa_prefill"])) == 64


def test_default_workload_is_the_largest_config():
    ap_src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", default="prefill"' in ap_src
