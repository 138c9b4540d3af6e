"""dsa_forward_noalloc (the workspace in the library's static per-GPU scratch array) against
dsa_forward (a caller's workspace) on the same inputs: the same kernels run on the same bytes,
so every output must match bit for bit. Two calls in a row, the second with a smaller input
(the scratch array keeps the first call's contents), then a CSA decode call whose long rows use
the top-k candidate region of the workspace as well, and three calls over an MX latent cache
(MXFP8 split and unsplit, then MXFP4 split): split attention converting the gathered rows, and
unsplit attention reading the cache expanded to bf16 in the workspace."""
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


def _outputs(f):
    return [to_host(t) for t in (f.out, f.lse, f.scores, f.idx)]


def _compare(c):
    dw = DeviceWorkload(synth.make_workload(c))
    ref = dw.forward(keep_scores=True, keep_idx=True)
    got = dw.forward(keep_scores=True, keep_idx=True)
    for t in (got.out, got.lse, got.scores, got.idx):
        t.fill_(7)  # anything stale would show
    log(f"[{c.name}] dsa_forward and dsa_forward_noalloc B={c.B} T={c.T} N={c.N} k={c.top_k}")
    ref.run()
    got.run_noalloc()
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "lse", "scores", "idx"), _outputs(ref), _outputs(got)):
        assert a.shape == b.shape
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{c.name}: {name} differs"
    del ref, got, dw


def test_noalloc_matches_dsa_forward_twice():
    _compare(synth.CONFIGS["decode"].with_(name="noalloc_decode"))
    _compare(synth.CONFIGS["decode"].with_(B=3, N=3001, pos0=3000, top_k=1024,
                                           name="noalloc_smaller").sharp())
    p = 4 * 40000 - 1
    _compare(synth.CONFIGS["csa_decode"].with_(B=2, N=40000, pos0=p, raw_base=p + 1 - 128,
                                               name="noalloc_csa"))


def test_noalloc_matches_dsa_forward_mx_cache():
    _compare(synth.CONFIGS["decode_kv8"].with_(B=4, name="noalloc_kv8_decode"))
    _compare(synth.CONFIGS["prefill_kv8"].with_(T=256, N=4096, pos0=3840,
                                                name="noalloc_kv8_prefill"))
    _compare(synth.CONFIGS["decode_kv4"].with_(B=4, name="noalloc_kv4_decode"))


def test_noalloc_matches_dsa_forward_ragged_long_rows():
    # ragged CSA decode rows over 34286 blocks: the short rows overflow their chunks' candidate
    # segments and take the exact whole-row select, whose output order is fixed
    p = 4 * 34286 - 1
    _compare(synth.CONFIGS["csa_decode"].with_(B=5, N=34286, pos0=p, raw_base=p + 1 - 128,
                                               seq_lens=(7238, 9668, 12360, 8585, 31308),
                                               sink=(-2.0, 4.0), w_lo=-0.5, seed=2012,
                                               name="noalloc_ragged_long").sharp())


def test_noalloc_matches_dsa_forward_random_ragged():
    # seeded random ragged batches (decode, many rows, CSA long rows, MX caches, sinks)
    from test_gpu_random import ragged_cases
    for c in ragged_cases():
        _compare(c.with_(name=c.name + "_noalloc"))
