"""gdn_prefill_noalloc, the allocation-free variant of gdn_prefill (for
callers that cannot allocate), through the C ABI: its results against those
of gdn_prefill with an allocated workspace, on two calls in a row -- the
second with a smaller input, so the static scratch array still holds the
first call's larger contents -- and on a call that needs no scratch."""
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn
import synth
from gpu_util import assert_close, require_gpu, to_dev
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _case(seed, n_tokens, hv=4):
    # slow decays, so every segment's incoming state reaches its outputs
    return synth.prefill_inputs(seed, lengths=[n_tokens], hq=2, hv=hv, dk=128, dv=128,
                                dtype="bf16", gate="log", gamma_range=(0.9985, 1.0), init_std=0.05)


def _both(x):
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    kw = dict(cu_seqlens=to_dev(x["cu_seqlens"]), initial_state=to_dev(x["initial_state"]),
              scale=x["scale"])
    need = gdn.prefill_workspace_size(q, k, v, to_dev(x["log_decay"]), to_dev(x["beta"]),
                                      cu_seqlens=kw["cu_seqlens"])
    o_n, f_n = gdn.prefill_noalloc(q, k, v, to_dev(x["log_decay"]), to_dev(x["beta"]), **kw)
    torch.cuda.synchronize()
    o_r, f_r = gdn.prefill(q, k, v, to_dev(x["log_decay"]), to_dev(x["beta"]), **kw)
    torch.cuda.synchronize()
    return need, (o_n, f_n), (o_r, f_r)


def test_noalloc_matches_prefill_on_two_calls_the_second_smaller():
    ro = {}
    for i, n in enumerate((16384, 6000)):
        x = _case(600 + i, n)
        need, (o_n, f_n), (o_r, f_r) = _both(x)
        assert 0 < need <= 32 << 20, need
        # the same kernels, segments and workspace layout: identical bits
        assert torch.equal(o_n, o_r) and torch.equal(f_n, f_r), "call %d differs" % i
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], x["log_decay"], x["beta"],
                                cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                                scale=x["scale"])
        assert_close(o_n, ro, "bf16", "call %d out" % i)
        assert_close(f_n, rf, "bf16", "call %d final" % i)


def test_noalloc_without_scratch():
    """A call the scan does not take (many heads): no scratch is used and the
    result is gdn_prefill's, bit for bit."""
    x = synth.prefill_inputs(610, lengths=[700, 0, 300], hq=16, hv=32, dk=128, dv=128,
                             dtype="bf16", gate="log", init_std=0.05)
    need, (o_n, f_n), (o_r, f_r) = _both(x)
    assert need == 0
    assert torch.equal(o_n, o_r) and torch.equal(f_n, f_r)
