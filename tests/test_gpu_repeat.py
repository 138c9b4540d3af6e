"""Every workload configuration (the prefill-sized ones shrunk), plain and sharp, through
dsa_forward (hca_forward for HCA) twice on the same workspace: every output repeats bit for bit.
No kernel's result depends on the order in which waves or workgroups finish (selections are
written by prefix scans, never by atomic appends; merges and reductions run in a fixed order)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DeviceWorkload, log, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.empty_cache()


def _small(c):
    if c.name.startswith("prefill"):
        return c.with_(T=2048, N=8192, pos0=6144)
    if c.name == "csa_prefill":
        return c.with_(T=1024, N=4096, n_raw=16384, pos0=16384 - 1024)
    return c


@pytest.mark.parametrize("name", sorted(synth.CONFIGS))
def test_outputs_repeat(name):
    for c in (_small(synth.CONFIGS[name]), _small(synth.CONFIGS[name]).sharp()):
        dw = DeviceWorkload(synth.make_workload(c))
        if c.dense:
            f = dw.hca()
            outs = lambda: (f.out, f.lse)
        else:
            f = dw.forward(keep_scores=True, keep_idx=True)
            outs = lambda: (f.out, f.lse, f.scores, f.idx)
        f.run()
        torch.cuda.synchronize()
        first = [to_host(t).copy() for t in outs()]
        f.run()
        torch.cuda.synchronize()
        for i, (a, t) in enumerate(zip(first, outs())):
            assert np.array_equal(a.view(np.uint8), to_host(t).view(np.uint8)), f"{c.name}: output {i}"
        log(f"[{c.name}] repeats bit for bit")
        del f, dw


@pytest.mark.parametrize("name", ["prefill", "prefill_fp8", "csa_prefill"])
def test_kept_scores_do_not_change_outputs(name):
    """The prefill indexers come in two forms: with the caller keeping the scores every masked
    score is written as -inf and every key group walks its key blocks; without, only visible
    scores are written and the key groups a query block does not need split its rows. Both
    must give the same selection and attention output, bit for bit. T = 1000 leaves a ragged
    last query block; N = 2048 (8 key blocks) with queries from position 0 makes early query
    blocks see one or two key blocks, so their rows are split up to four ways."""
    c = synth.CONFIGS[name]
    if name == "csa_prefill":
        c = c.with_(T=1000, N=2048, n_raw=8192, pos0=0)
    else:
        c = c.with_(T=1000, N=2048, pos0=0)
    dw = DeviceWorkload(synth.make_workload(c))
    outs = []
    for keep in (True, False):
        f = dw.forward(keep_scores=keep, keep_idx=True)
        f.run()
        torch.cuda.synchronize()
        outs.append([to_host(t).copy() for t in (f.out, f.lse, f.idx)])
        del f
    for i, (a, b) in enumerate(zip(*outs)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{c.name}: output {i}"
    log(f"[{c.name}] kept and dropped scores give the same bytes")
