#!/usr/bin/env python3
"""Throughput of the DSA hot path (lightning indexer -> top-k -> sparse MQA-MLA) on one MI355X.

A step is one dsa_forward over one batch of seeded synthetic inputs, already resident in HBM.
Default workload (the largest single-GPU configuration): prefill, one sequence of 32768 tokens
with all 32768 queries causal, indexer 64 heads x 128 (bf16), top-k 2048, sparse MQA attention
with 128 heads over 576-wide latent rows (value = first 512 columns), bf16 storage, fp32
accumulation. The same line carries a per-config block for the four other workloads (tiny fp32,
decode, CSA prefill, CSA decode), each timed the same way.

The K timed steps replay HIP graphs of dsa_forward (after at least R warm-up replays), cycling
over R copies of the inputs so the bytes a step touches exceed the 256 MB last-level cache
(cold-cache HBM traffic, as in multi-layer decode). A second, instrumented pass runs the same dsa_forward calls eagerly with
a pair of HIP events per kernel, stamped by hipExtLaunchKernel with that dispatch's start and
end, to get each kernel's average duration; the dominant kernel's algorithmic bytes (or flops)
over that duration give the roofline fraction. The fp64 CPU oracle, timed on this host's
cores over the queries of one step, is reported beside it as a baseline.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0  # dense fp8 MFMA (the block-scaled fp8 x fp8 / fp8 x fp4 instructions)
FP8_KERNELS = ("indexer_prefill_mx", "indexer_decode_mx_dma")
METRIC = "query tokens/sec (indexer+top-k+sparse MLA); % of peak HBM BW / MFMA"

WORKLOAD_TEXT = {
    "decode": "decode DSA: B=16 sequences x 1 query token, context L=8192, indexer 64 heads x 128 "
              "(bf16 k_I), top-k 2048, sparse MQA-MLA 128 heads, key 576 / value 512 (bf16), "
              "softmax scale 1/24",
    "csa_decode": "CSA decode: B=4 x 1 query over 1,048,576 tokens (262,144 4:1 blocks), MXFP4 "
                  "k_I, top-k 1024 blocks + 128-token raw window, 128 heads, key 576 / value 512",
    "prefill": "prefill DSA: 1 sequence, L=T=32768 causal, indexer 64x128, top-k 2048, "
               "128 heads, key 576 / value 512 (bf16)",
    "csa_prefill": "CSA prefill: 131072 raw tokens mean-pooled 4:1 to 32768 blocks, last 8192 "
                   "queries, top-k 1024 + 128-token window, 128 heads, key 576 / value 512",
    "tiny": "tiny fp32 DSA: L=256, 16 queries, indexer 4x32, top-k 64, 8 heads, key 64 / value 48",
    "decode_fp8": "decode DSA with an MXFP8 indexer (e4m3 q_I and k_I, one E8M0 scale per 32): "
                  "B=16 x 1 query, context L=8192, indexer 64x128, top-k 2048, sparse MQA-MLA "
                  "128 heads, key 576 / value 512 (bf16)",
    "prefill_fp8": "prefill DSA with an MXFP8 indexer (e4m3 q_I and k_I, one E8M0 scale per "
                   "32): 1 sequence, L=T=32768 causal, top-k 2048, 128 heads, key 576 / value "
                   "512 (bf16)",
    "decode_kv8": "decode DSA over an MXFP8 latent KV cache (e4m3 entries, one E8M0 scale per "
                  "32): B=16 x 1 query, context L=8192, indexer 64x128 (bf16), top-k 2048, "
                  "sparse MQA-MLA 128 heads, key 576 / value 512, bf16 q and out",
    "prefill_kv8": "prefill DSA over an MXFP8 latent KV cache (e4m3 entries, one E8M0 scale per "
                   "32): 1 sequence, L=T=32768 causal, top-k 2048, 128 heads, key 576 / value "
                   "512, bf16 q and out",
    "decode_kv4": "decode DSA over an MXFP4 latent KV cache (e2m1 entries, one E8M0 scale per "
                  "32): B=16 x 1 query, context L=8192, indexer 64x128 (bf16), top-k 2048, "
                  "sparse MQA-MLA 128 heads, key 576 / value 512, bf16 q and out",
    "prefill_kv4": "prefill DSA over an MXFP4 latent KV cache (e2m1 entries, one E8M0 scale per "
                   "32): 1 sequence, L=T=32768 causal, top-k 2048, 128 heads, key 576 / value "
                   "512, bf16 q and out",
    "hca_decode": "HCA decode: B=4 x 1 query over 1,048,576 tokens compressed 128:1 (8192 blocks), "
                  "dense attention over every visible block + 128-token raw window, 128 heads, "
                  "key 576 / value 512 (bf16)",
    "hca_prefill": "HCA prefill: 131072 raw tokens mean-pooled 128:1 to 1024 blocks, last 8192 "
                   "queries, dense attention over the visible blocks + 128-token window, 128 heads",
}


def _fused_topk(cfg):
    """dsa_forward selects the top-k inside the attention kernel (bf16 MFMA shapes, N <= 32768,
    at most 128 query rows per chunk; cfg describes one chunk)."""
    return (not cfg.dense and cfg.dt == "bf16" and cfg.D_K == 576 and cfg.D_V == 512
            and cfg.H % 64 == 0 and cfg.N <= 32768 and cfg.B * cfg.T <= 128)


def _segments_fused(cfg):
    """The decode indexer writes the long-row top-k's candidate segments itself (MX keys over
    N > 32768 entries, with the plan of 4096 keys per indexer workgroup)."""
    if not (cfg.H_I == 64 and cfg.D_I == 128 and cfg.k_dt in ("mxfp4", "mxfp8")
            and cfg.N > 32768):
        return False
    rows = cfg.B * cfg.T
    if cfg.qi_dt == "mxfp8" and rows >= 64:
        return False
    tk = 64 if cfg.k_dt == "mxfp4" else 32
    max_it, it = 512 // tk, 1
    while it < max_it and 2 * it * tk * 8 * 256 <= rows * cfg.N:
        it *= 2
    return it == max_it


def _kernel_plan(cfg, nsplit):
    """Kernel names of one dsa_forward (per chunk) in launch order."""
    names = []
    if cfg.compress:
        names.append("compress_mean")
    mfma = cfg.dt == "bf16" and cfg.D_K == 576 and cfg.D_V == 512 and cfg.H % 64 == 0
    if cfg.dense:  # HCA: attention over every visible block, no indexer or top-k
        return names + ["attend_mfma_dma" if mfma else "attend_generic"] + (
            ["attend_combine"] if nsplit > 1 else [])
    fast = cfg.dt == "bf16" and cfg.H_I == 64 and cfg.D_I == 128
    rows = cfg.B * cfg.T
    if fast and cfg.k_dt == "bf16" and rows >= 64:
        names.append("indexer_prefill_mfma")
    elif fast and cfg.qi_dt == "mxfp8" and rows >= 64:
        names.append("indexer_prefill_mx")
    elif fast and cfg.k_dt == "bf16":
        names.append("indexer_decode_dma")
    elif fast:
        names.append("indexer_decode_mx_dma")
    else:
        names.append("indexer_generic")
    mfma = cfg.dt == "bf16" and cfg.D_K == 576 and cfg.D_V == 512 and cfg.H % 64 == 0
    if not _fused_topk(cfg):
        if cfg.N <= 32768:
            names.append("topk_stream")
        elif _segments_fused(cfg):
            names.append("topk_long_select")  # the indexer wrote the candidate segments
        else:
            names += ["topk_long_filter", "topk_long_select"]
    names.append("attend_mfma_dma" if mfma else "attend_generic")
    if nsplit > 1:
        names.append("attend_combine")
    return names


def _algorithmic(cfg, name, split=False):
    """(bytes, flops) the method must move / compute in one launch of `name` at this workload.

    Counts causal pairs and selected entries only; scratch traffic (split partials, repeated
    passes over the scores) is not algorithmic. `split`: the attention hands its partials to
    attend_combine, which then writes the output (else the attention kernel writes it)."""
    B, T, N = cfg.B, cfg.T, cfg.N
    rows = B * T
    esz = 2 if cfg.dt == "bf16" else 4
    kI_row = {"mxfp4": cfg.D_I // 2 + cfg.D_I // 32,
              "mxfp8": cfg.D_I + cfg.D_I // 32}.get(cfg.k_dt, cfg.D_I * esz)
    qI_row = cfg.D_I + cfg.D_I // 32 if cfg.qi_dt == "mxfp8" else cfg.D_I * esz
    nvis = [min(N, (int(p) + 1) // cfg.m) for p in cfg.positions().ravel()]  # visible entries
    pairs = float(sum(nvis))
    sel = float(sum(min(cfg.top_k, v) for v in nvis))
    win = 0.0
    if cfg.W > 0:
        base, n_raw = (0, N * cfg.m) if cfg.compress else (cfg.raw_base, cfg.n_raw)
        for p in cfg.positions().ravel():
            lo = max(0, int(p) - cfg.W + 1, base)
            hi = min(int(p), base + n_raw - 1)
            win += max(0, hi - lo + 1)
    if name == "compress_mean":
        return B * N * cfg.m * cfg.D_K * esz + B * N * cfg.D_K * esz, 0.0
    if name in ("mxfp8_to_bf16", "mxfp4_to_bf16"):
        # reads the MX cache (codes and scales), writes its bf16 copy
        cb = cfg.D_K if name == "mxfp8_to_bf16" else cfg.D_K // 2
        return B * N * (cb + cfg.D_K // 32) + B * N * cfg.D_K * 2, 0.0
    if name.startswith("indexer"):
        # every key row a sequence's queries can see is read once per sequence (decode: per query)
        keys = B * max(nvis) if T > 1 else pairs
        byt = keys * kI_row + rows * cfg.H_I * (qI_row + 4) + pairs * 4
        return byt, pairs * cfg.H_I * cfg.D_I * 2.0
    if name == "topk_long_filter":
        return pairs * 4, 0.0  # reads every visible score; its candidates are scratch
    if name == "topk_long_select":
        return rows * cfg.top_k * 4, 0.0
    if name.startswith("topk"):
        return pairs * 4 + rows * cfg.top_k * 4, 0.0
    if name.startswith("attend_mfma") or name == "attend_generic":
        ents = sel + win
        # each gathered row must cross HBM once per step: once per query at decode, but rows
        # shared by the queries of one sequence (prefill) count once
        rows_kv = min(sel, float(B * N)) + min(win, float(B * (T + cfg.W - 1)) if cfg.W else 0.0)
        kv_row = {"mxfp8": cfg.D_K + cfg.D_K // 32,
                  "mxfp4": cfg.D_K // 2 + cfg.D_K // 32}.get(cfg.kv_dt, cfg.D_K * esz)
        byt = rows_kv * kv_row + rows * cfg.H * cfg.D_K * esz
        if not cfg.dense:
            byt += rows * cfg.top_k * 4  # the index list (HCA has none)
        if name.startswith("attend_mfma") and _fused_topk(cfg):
            byt += pairs * 4  # the kernel selects the entries from the scores itself
        if not split:
            byt += rows * cfg.H * (cfg.D_V * esz + 4)  # output and log-sum-exp
        return byt, ents * cfg.H * (cfg.D_K + cfg.D_V) * 2.0
    if name == "attend_combine":
        return rows * cfg.H * (cfg.D_V * esz + 4), 0.0
    return 0.0, 0.0


def _src_sha(kernel):
    """Hash of the sources a kernel is built from (its file and the shared device headers)."""
    files = {"indexer": "indexer.hip", "topk": "topk.hip", "attend": "attend.hip",
             "compress": "compress.hip", "mxfp8": "compress.hip", "mxfp4": "compress.hip"}
    for k, f in files.items():
        if kernel.startswith(k):
            h = hashlib.sha1()
            for name in (f, "common.h", "select.h"):
                with open(os.path.join(ROOT, "lightning_indexer_top_03_amd", "csrc", name),
                          "rb") as fh:
                    h.update(fh.read())
            return h.hexdigest()[:12]
    return None


def _traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    e = tab.get(workload, {}).get(kernel)
    if not e or e.get("src_sha") != _src_sha(kernel):
        return None
    return e["hbm_bytes_per_launch"]


def _dev(a):
    import numpy as np
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _device_inputs(wl):
    """Device copies of a workload (q generated in chunks straight into HBM)."""
    import torch

    c = wl.cfg
    t = {"q_pos": _dev(wl.q_pos())}
    if not c.dense:  # HCA has no indexer
        q = wl.q_I()
        t["q_I"] = (_dev(q[0]), _dev(q[1])) if c.qi_dt == "mxfp8" else _dev(q)
        t["w"] = _dev(wl.w())
        k = wl.k_I()
        t["k_I"] = (_dev(k[0]), _dev(k[1])) if c.k_dt in ("mxfp4", "mxfp8") else _dev(k)
    rows = c.B * c.T
    tdt = torch.bfloat16 if c.dt == "bf16" else torch.float32
    q = torch.empty((c.B, c.T, c.H, c.D_K), dtype=tdt, device="cuda")
    qf = q.view(rows, c.H, c.D_K)
    for r0 in range(0, rows, 4096):
        n = min(4096, rows - r0)
        qf[r0:r0 + n] = _dev(wl.q_chunk(r0, n))
    t["q"] = q
    raw = wl.kv_raw()
    t["kv_raw"] = _dev(raw) if raw is not None else None
    wl.drop("kv_raw")
    if c.compress:
        t["kv"] = torch.empty((c.B, c.N, c.D_K), dtype=tdt, device="cuda")
    elif c.kv_dt in ("mxfp8", "mxfp4"):
        codes, sc = wl.kv()
        t["kv"] = (_dev(codes), _dev(sc))
    else:
        t["kv"] = _dev(wl.kv())
    wl.drop("kv")
    return t


def _forward(cfg, t, dsa, base):
    if cfg.dense:
        return dsa.HcaForward(t["q"], t["kv"], t["q_pos"], cfg.D_V, cfg.softmax_scale, cfg.m,
                              W=cfg.W, kv_raw=t["kv_raw"], raw_base=base, compress=cfg.compress)
    return dsa.Forward(t["q_I"], t["w"], t["k_I"], t["q"], t["kv"], t["q_pos"], cfg.top_k,
                       cfg.D_V, cfg.softmax_scale, m=cfg.m, W=cfg.W, kv_raw=t["kv_raw"],
                       raw_base=base, compress=cfg.compress)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# query positions every prefill CPU sample includes: the first rows, both sides of the keep-all
# edge (k = 2048) and the last row
PREFILL_ALWAYS = (0, 1, 2046, 2047, 2048, 2049, 32767)


def cpu_sample_rows(cfg):
    """Query rows the CPU baseline visits, in visiting order: every row of one step when there
    are at most 64, else a uniform sample (128 rows for the 32768-query prefill, always with the
    positions of PREFILL_ALWAYS; 64 elsewhere), drawn with the workload's seed and visited in
    random order so that a budget cut still leaves a uniform sample."""
    import numpy as np

    rows = [(b, t) for b in range(cfg.B) for t in range(cfg.T)]
    rng = np.random.default_rng(cfg.seed)
    if len(rows) > 64:
        n = 128 if cfg.T >= 32768 else 64
        always = [t for t in PREFILL_ALWAYS if t < cfg.T] if cfg.T >= 32768 else []
        rest = [int(i) for i in rng.permutation(len(rows)) if int(i) not in always]
        rows = [rows[i] for i in sorted(set(always) | set(rest[: n - len(always)]))]
    return [rows[int(i)] for i in rng.permutation(len(rows))]


def cpu_baseline(cfg, budget_s=20.0):
    """The oracle, as it stands, over the query rows of cpu_sample_rows (as many as fit the
    budget)."""
    import oracle
    import synth

    wl = synth.make_workload(cfg)
    run = oracle.QueryRunner(wl)
    rows = cpu_sample_rows(cfg)
    t0 = time.perf_counter()
    done = 0
    for b, t in rows:
        if cfg.dense:
            run.run_dense(b, t)
        else:
            run.run(b, t)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "query tokens/s", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{done} of {len(rows)} query rows drawn from the {cfg.B * cfg.T} of one "
                      f"step ({'all' if len(rows) == cfg.B * cfg.T else 'uniform sample'}"
                      f"{', incl. positions ' + str(PREFILL_ALWAYS) if cfg.T >= 32768 else ''}, "
                      f"random order), fp64, {dt:.1f} s wall"}


def log(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


def measure(name, steps, warmup, rotate=0, eager=False, copy_probe=False, n_inst=None):
    """Time `steps` dsa_forward steps of workload `name` (inputs resident in HBM) and the
    per-kernel durations of an instrumented pass. Returns the figures of one bench line."""
    import torch

    import lightning_indexer_top_03_amd as dsa
    import synth

    cfg = synth.CONFIGS[name]
    wl = synth.make_workload(cfg)
    t0 = time.time()
    inputs = [_device_inputs(wl)]
    log(f"[{name}] inputs ready in {time.time() - t0:.1f}s")

    # input copies so that one cycle touches > 512 MB
    touched = sum(_algorithmic(cfg, k)[0] for k in
                  (("attend_mfma_dma",) if cfg.dense else ("indexer_x", "attend_mfma_dma")))
    R = rotate or max(1, min(16, int(512e6 // max(touched, 1.0)) + 1))
    if cfg.B * cfg.T > 64:
        R = rotate or 1
    for _ in range(1, R):
        c = {k: (tuple(x.clone() for x in v) if isinstance(v, tuple) else
                 (v.clone() if v is not None else None)) for k, v in inputs[0].items()}
        inputs.append(c)
    base = wl.raw_extent()[0]
    fwds = [_forward(cfg, t, dsa, base) for t in inputs]
    rows = cfg.B * cfg.T
    # dsa_forward processes the query rows in chunks whose scores fit 256 MB
    chunk_rows = min(rows, max(1, (256 << 20) // (cfg.N * 4)))
    n_chunks = -(-rows // chunk_rows)
    d = dsa.dims(B=1, T=chunk_rows, N=cfg.N, H_I=cfg.H_I, D_I=cfg.D_I, H=cfg.H, D_K=cfg.D_K,
                 D_V=cfg.D_V, top_k=cfg.top_k, m=cfg.m, W=cfg.W)
    # the attention splits its entry list
    split = dsa.workspace_bytes(d, dsa.OP_HCA if cfg.dense else dsa.OP_ATTEND) > 0
    per_chunk = _kernel_plan(cfg.with_(compress=False, B=1, T=chunk_rows), 2 if split else 1)
    # an MXFP8 cache read by unsplit attention is expanded to bf16 once per call
    mfma = cfg.D_K == 576 and cfg.D_V == 512 and cfg.H % 64 == 0
    expand = cfg.kv_dt in ("mxfp8", "mxfp4") and mfma and not split
    xk = "mxfp4_to_bf16" if cfg.kv_dt == "mxfp4" else "mxfp8_to_bf16"
    kernels = ((["compress_mean"] if cfg.compress else []) + ([xk] if expand else [])
               + per_chunk * n_chunks)

    if copy_probe:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy probe: torch.neg over {} bytes read and written per launch, 3 launches"
            .format(src.numel() * 4))
        del src, dst

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graphs = []
    with torch.cuda.stream(stream):
        for f in fwds:
            f.run()
        torch.cuda.synchronize()
        if not eager:
            for f in fwds:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    f.run()
                graphs.append(g)
    torch.cuda.synchronize()

    def step(i):
        if graphs:
            graphs[i % R].replay()
        else:
            fwds[i % R].run()

    # every captured graph is replayed at least once before the timed steps
    warmup = max(warmup, R)
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps
    value = rows / (elapsed / steps)
    log(f"[{name}] {steps} steps: {ms_per_step:.4f} ms/step, {value:.1f} query tokens/s")

    # ---- instrumented pass: each kernel's own start / end events ----
    # dsa_forward hands event pair i to the i-th kernel's hipExtLaunchKernel, which stamps them
    # with that dispatch's start and end on the stream it runs on; nothing is inserted between
    # the kernels. Eager launches (graphs are captured without events). Each instrumented step
    # is queued behind a ~1 ms spin kernel, so the host has enqueued all of the step's kernels
    # before the GPU reaches them: they run back to back, as in the graph replays.
    nk = len(kernels)
    per_kernel = [0.0] * nk
    if n_inst is None:
        n_inst = 200 if rows <= 64 else 10
    n_inst = min(steps, n_inst)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nk)]
    with torch.cuda.stream(stream):
        for f in fwds:
            f.set_events(evs)
        torch.cuda.synchronize()
        for i in range(n_inst):
            torch.cuda._sleep(2_000_000)
            fwds[i % R].run()
            torch.cuda.synchronize()
            for k in range(nk):
                per_kernel[k] += evs[2 * k].elapsed_time(evs[2 * k + 1])
        for f in fwds:
            f.set_events(None)
    per_kernel = [x / n_inst for x in per_kernel]  # ms per launch

    # per kernel: summed over the query chunks of one step (one launch per chunk)
    tot = {}
    for k, kname in enumerate(kernels):
        tot[kname] = tot.get(kname, 0.0) + per_kernel[k]
    kinfo = {}
    step_bytes = step_flops = 0.0
    for kname, ms in tot.items():
        byt, fl = _algorithmic(cfg, kname, "attend_combine" in tot)
        step_bytes += byt
        step_flops += fl
        us = ms * 1e3
        kinfo[kname] = {"us_per_step": round(us, 3), "launches_per_step": kernels.count(kname),
                        "alg_GBps": round(byt / (us * 1e-6) / 1e9, 1) if us else None,
                        "alg_TFLOPs": round(fl / (us * 1e-6) / 1e12, 2) if us and fl else None}
    dname = max(tot, key=lambda k: tot[k])
    byt, fl = _algorithmic(cfg, dname, "attend_combine" in tot)
    dur = tot[dname] * 1e-3  # per step; equals the launch duration when there is one chunk
    intensity = fl / byt if byt else 0.0
    # a contraction is held to the peak of the dtype its MFMAs take
    peak = FP8_PEAK_TFLOPS if dname in FP8_KERNELS else BF16_PEAK_TFLOPS
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if fl and intensity > ridge:
        roof = {"bound": "mfma", "achieved": round(fl / dur / 1e12, 2), "peak": peak,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(byt / dur / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = _traffic(dname, name)
    roof["kernel"] = dname
    roof["kernel_us"] = round(dur * 1e6 / kernels.count(dname), 3)
    roof["launches_per_step"] = kernels.count(dname)
    roof["kernel_alg_bytes_per_step"] = byt
    roof["kernel_alg_flops_per_step"] = fl
    # the whole step: every kernel's algorithmic bytes / flops, and what the step's time gives
    roof["step_alg_bytes"] = step_bytes
    roof["step_alg_flops"] = step_flops
    roof["step_GBps"] = round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1)
    roof["step_TFLOPs"] = round(step_flops / (ms_per_step * 1e-3) / 1e12, 2)
    res = {"cfg": cfg, "value": value, "ms_per_step": ms_per_step, "steps": steps,
           "warmup": warmup, "R": R, "graphs": bool(graphs), "roofline": roof, "kernels": kinfo}
    del graphs, fwds, inputs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# the per-config block: the other four workloads the performance targets are stated for, and
# decode over an MXFP8 latent cache, with the steps each one times (decode-sized steps are
# short, so more of them)
OTHER_CONFIGS = {"tiny": 200, "decode": 400, "csa_prefill": 20, "csa_decode": 400,
                 "decode_kv8": 400}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--rotate", type=int, default=0,
                    help="input copies cycled over (0: enough to exceed 2x the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config block (the other four workloads)")
    ap.add_argument("--eager", action="store_true", help="launch without HIP graphs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a plain elementwise copy of 256 MiB (read) + 256 MiB "
                         "(written) three times, the reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.set_device(0)
    h = measure(args.workload, args.steps, args.warmup, rotate=args.rotate, eager=args.eager,
                copy_probe=args.copy_probe)
    cfg = h["cfg"]
    rows = cfg.B * cfg.T
    line = {
        "metric": METRIC, "value": round(h["value"], 1), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": h["warmup"], "ms_per_step": round(h["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if cfg.dt == "bf16" else "f32", "data": "synthetic (seeded, counter-based generator)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": args.workload,
                   "global_batch": rows, "seq_len": cfg.N * cfg.m, "parallelism": "single GPU",
                   "input_copies": h["R"], "launch": "hip graph" if h["graphs"] else "eager",
                   "event_pass": "eager behind a spin kernel"},
        "roofline": h["roofline"],
        "kernels": h["kernels"],
    }
    if not args.no_configs:
        block = {}
        for name, steps in OTHER_CONFIGS.items():
            if name == args.workload:
                continue
            r = measure(name, steps, args.warmup, eager=args.eager)
            ro = r["roofline"]
            block[name] = {"workload": WORKLOAD_TEXT[name], "value": round(r["value"], 1),
                           "unit": "query tokens/s", "ms_per_step": round(r["ms_per_step"], 5),
                           "steps": steps, "warmup": r["warmup"], "input_copies": r["R"],
                           "dominant_kernel": ro["kernel"], "bound": ro["bound"],
                           "achieved": ro["achieved"], "unit_roofline": ro["unit"],
                           "frac": ro["frac"], "step_GBps": ro["step_GBps"],
                           "step_TFLOPs": ro["step_TFLOPs"],
                           "kernels": {k: v["us_per_step"] for k, v in r["kernels"].items()}}
        line["configs"] = block
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
