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
