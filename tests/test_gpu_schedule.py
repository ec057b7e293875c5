"""Workgroup scheduling of the prefill kernels, through the C ABI, against the
fp64 oracle.

Ragged calls of 2 to 64 requests that average at least 256 tokens take the
requests longest first and spread every request over all XCDs; the units of
rank k then belong to the k-th longest request, not to request k.  These
cases put the lengths out of order (longest in the middle, ties, an empty
request, one shorter than a chunk) so that a mix-up between rank and request
index moves a request's outputs or states, and run each prefill kernel that
orders this way: the general fp32 kernel, the bf16 pair kernel (also as the
scan over request segments), and the per-key-decay kernel.  Every output and
final-state element is compared with the oracle (the plain sequential
recurrence of "Gated DeltaNet State Update", with the request rules of
"com.microsoft.GatedDeltaNet", Inputs / Outputs).
"""
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn
import oracle
import synth
from gpu_util import assert_close, require_gpu, to_dev

pytestmark = pytest.mark.gpu

# 11 requests, 7000 tokens: two of equal length, the longest in the middle,
# an empty one and one of 5 tokens
LENGTHS = [300, 1500, 700, 0, 2400, 700, 5, 900, 250, 145, 100]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check(o, f, ro, rf, dtype):
    torch.cuda.synchronize()
    assert_close(o, ro, dtype, "out")
    for r in range(f.shape[0]):
        assert_close(f[r], rf[r], dtype, "final state of request %d" % r)


@pytest.mark.parametrize("dtype,d", [("f32", 128), ("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_ragged_longest_first(dtype, d):
    """General kernel (fp32) and pair kernel (bf16), initial states given."""
    x = synth.prefill_inputs(610 + d, lengths=LENGTHS, hq=2, hv=4, dk=d, dv=d, dtype=dtype,
                             gate="gamma", gamma_range=(0.8, 1.0), init_std=0.05)
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["gamma"]),
                       to_dev(x["beta"]), decay_kind="gamma", cu_seqlens=to_dev(x["cu_seqlens"]),
                       initial_state=to_dev(x["initial_state"]), scale=x["scale"], scan=False)
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], x["gamma"], x["beta"], decay_is_gamma=True,
                            cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                            scale=x["scale"])
    _check(o, f, ro, rf, dtype)


def test_ragged_longest_first_scan():
    """The scan over request segments (bf16, few units) with the requests
    taken longest first: the segment maps of each request stay its own."""
    lengths = [6000, 0, 20000, 9000]
    x = synth.prefill_inputs(620, lengths=lengths, hq=1, hv=2, dk=128, dv=128, dtype="bf16",
                             gate="log", gamma_range=(0.9985, 1.0), init_std=0.05)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    dec, bet, cu = to_dev(x["log_decay"]), to_dev(x["beta"]), to_dev(x["cu_seqlens"])
    assert gdn.prefill_workspace_size(q, k, v, dec, bet, cu_seqlens=cu) > 0
    o, f = gdn.prefill(q, k, v, dec, bet, cu_seqlens=cu, initial_state=to_dev(x["initial_state"]),
                       scale=x["scale"])
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], x["log_decay"], x["beta"],
                            cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                            scale=x["scale"])
    _check(o, f, ro, rf, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_longest_first_per_key(dtype):
    """The per-key-decay kernel (log decays per key) with the requests taken
    longest first."""
    x = synth.prefill_inputs(630, lengths=LENGTHS, hq=1, hv=2, dk=64, dv=64, dtype=dtype,
                             gate="log", init_std=0.05)
    g = torch.Generator().manual_seed(631)
    dec = -torch.rand(x["T"], 2, 64, generator=g) * 0.5
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(dec),
                       to_dev(x["beta"]), cu_seqlens=to_dev(x["cu_seqlens"]),
                       initial_state=to_dev(x["initial_state"]), scale=x["scale"],
                       decay_per_key=True)
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, x["beta"], cu_seqlens=x["cu_seqlens"],
                            initial_state=x["initial_state"], scale=x["scale"], decay_per_key=True)
    _check(o, f, ro, rf, dtype)
