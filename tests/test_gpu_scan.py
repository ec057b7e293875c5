"""The prefill's scan over the affine maps of request segments, through the C
ABI, against the fp64 oracle.

Calls with few (request, value head) units and long requests run as three
launches (local pass over every segment, combine, rerun) when a workspace of
gdn_prefill_workspace_size bytes is given; the binding allocates it, and
scan=False forces the serial walk on the same inputs.  Both are compared with
the oracle (the plain sequential recurrence of "Gated DeltaNet State Update"),
over one long request, ragged requests with an empty one and requests shorter
than a segment, initial states (also aliased with the final state), pooled
states with read / write slot rules, every update_rule, the fused gate and
in-kernel L2 norm, and both head sizes of the pair kernel.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn
import oracle
import synth
from gpu_util import assert_close, rel_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _print(*a):
    print(*a, flush=True)


def _inputs(seed, lengths, hq=2, hv=4, d=128, init=False):
    """Slow decays (gamma ~ U[0.9985, 1], about 0.5 over a 1024-token
    segment), so a segment's incoming state still shapes its outputs and the
    combine's maps matter; with fast decays the incoming state fades below
    fp32 resolution inside a segment and the scan equals the serial walk bit
    for bit."""
    return synth.prefill_inputs(seed, lengths=lengths, hq=hq, hv=hv, dk=d, dv=d, dtype="bf16",
                                gate="log", gamma_range=(0.9985, 1.0),
                                init_std=0.05 if init else None)


def _run(x, scan, rule="gated_delta", **kw):
    use_d = rule in ("gated_delta", "gated")
    use_b = rule in ("gated_delta", "delta")
    return gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]),
                       to_dev(x["log_decay"]) if use_d else None,
                       to_dev(x["beta"]) if use_b else None,
                       cu_seqlens=to_dev(x["cu_seqlens"]), scale=x["scale"], scan=scan,
                       update_rule=rule, **kw)


def _oracle(x, rule="gated_delta", **kw):
    use_d = rule in ("gated_delta", "gated")
    use_b = rule in ("gated_delta", "delta")
    return oracle.prefill(x["q"], x["k"], x["v"], x["log_decay"] if use_d else None,
                          x["beta"] if use_b else None, cu_seqlens=x["cu_seqlens"],
                          scale=x["scale"], update_rule=rule, **kw)


def _ws(x, **kw):
    return gdn.prefill_workspace_size(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]),
                                      to_dev(x["log_decay"]), to_dev(x["beta"]),
                                      cu_seqlens=to_dev(x["cu_seqlens"]), **kw)


@pytest.mark.parametrize("d", [128, 64])
def test_scan_one_long_request(d):
    """One request of 16384 tokens, Hq 2, Hv 4 (16 segments at d 128): the
    scan and the serial walk each against the oracle; the scan repeats bit
    for bit."""
    x = _inputs(500 + d, [16384], d=d)
    assert _ws(x) > 0
    o_s, f_s = _run(x, True)
    o_s2, f_s2 = _run(x, True)
    o_w, f_w = _run(x, False)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_s2) and torch.equal(f_s, f_s2)
    ro, rf = _oracle(x)
    es = assert_close(o_s, ro, "bf16", "scan out"), assert_close(f_s, rf, "bf16", "scan final")
    ew = assert_close(o_w, ro, "bf16", "serial out"), assert_close(f_w, rf, "bf16", "serial final")
    _print("d", d, "scan errors", es, "serial errors", ew)
    assert not torch.equal(o_s, o_w)  # the scan did run (another rounding order)


def test_scan_ragged_requests_with_initial_states():
    """Three requests (12345 tokens, an empty one, 777 tokens): partial last
    chunks, segments past a short request's end (empty: identity maps), the
    empty request's state copied bit for bit; initial states, also passed as
    the final-state buffer itself."""
    x = _inputs(510, [12345, 0, 777], init=True)
    assert _ws(x) > 0
    init = to_dev(x["initial_state"])
    o, f = _run(x, True, initial_state=init)
    ro, rf = _oracle(x, initial_state=x["initial_state"])
    torch.cuda.synchronize()
    assert_close(o[:12345], ro[:12345], "bf16", "out r0")
    assert_close(o[12345:], ro[12345:], "bf16", "out r2")
    for r in (0, 2):
        assert_close(f[r], rf[r], "bf16", "final r%d" % r)
    assert torch.equal(f[1].cpu(), x["initial_state"][1]), "empty request must keep its state"
    # final_state aliasing initial_state
    st = init.clone()
    o2, f2 = _run(x, True, initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert f2.data_ptr() == st.data_ptr()
    assert torch.equal(o2, o) and torch.equal(st, f)


def test_scan_over_a_state_pool():
    """Pooled states with the slot rules of the pool prefill: a valid read and
    a distinct write slot, a read slot outside the pool (zeros in) with write
    slot -1 (nothing stored), one slot read and written by one request; the
    pool's other slots stay bit for bit."""
    x = _inputs(520, [6000, 5000, 4500])
    P, hv, d = 10, 4, 128
    g = torch.Generator().manual_seed(521)
    pool0 = torch.randn(P, hv, d, d, generator=g) * 0.05
    rd = torch.tensor([3, 11, 6], dtype=torch.int32)
    wr = torch.tensor([7, -1, 6], dtype=torch.int32)
    pool = pool0.cuda()
    ws = gdn.prefill_workspace_size(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]),
                                    to_dev(x["log_decay"]), to_dev(x["beta"]),
                                    cu_seqlens=to_dev(x["cu_seqlens"]), state_pool=pool,
                                    read_slot=rd.cuda(), write_slot=wr.cuda())
    assert ws > 0
    o, _ = _run(x, True, state_pool=pool, read_slot=rd.cuda(), write_slot=wr.cuda())
    init = torch.stack([pool0[3], torch.zeros(hv, d, d), pool0[6]])
    ro, rf = _oracle(x, initial_state=init)
    torch.cuda.synchronize()
    pa = pool.cpu()
    assert_close(o, ro, "bf16", "out")
    assert_close(pa[7], rf[0], "bf16", "slot 7")
    assert_close(pa[6], rf[2], "bf16", "slot 6")
    keep = [s for s in range(P) if s not in (6, 7)]
    assert torch.equal(pa[keep], pool0[keep])


@pytest.mark.parametrize("rule", ["linear", "gated", "delta"])
def test_scan_update_rules(rule):
    """The other update rules of "com.microsoft.GatedDeltaNet" (Attributes):
    each step stays affine in the state, so the scan applies unchanged."""
    x = _inputs(530, [9000], init=True)
    init = to_dev(x["initial_state"])
    o, f = _run(x, True, rule=rule, initial_state=init)
    ro, rf = _oracle(x, rule=rule, initial_state=x["initial_state"])
    torch.cuda.synchronize()
    assert_close(o, ro, "bf16", "%s out" % rule)
    assert_close(f, rf, "bf16", "%s final" % rule)


def test_scan_fused_gate_and_l2_norm():
    """The fused gate (raw a, b) and the in-kernel q/k L2 norm under the scan."""
    x = synth.prefill_inputs(540, lengths=[10000], hq=2, hv=4, dk=128, dv=128, dtype="bf16",
                             gate="qwen")
    # slow fused decays: exp(A_log) about 1e-3
    x["A_log"] = x["A_log"] * 0.1 - 7.0
    # unnormalised q and k rows, so the in-kernel norm has work to do
    g = torch.Generator().manual_seed(541)
    x["k"] = (x["k"].float() * (0.5 + torch.rand(x["T"], 2, 1, generator=g))).to(torch.bfloat16)
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), None, None,
                       A_log=to_dev(x["A_log"]), dt_bias=to_dev(x["dt_bias"]), a=to_dev(x["a"]),
                       b=to_dev(x["b"]), cu_seqlens=to_dev(x["cu_seqlens"]), scale=x["scale"],
                       qk_l2norm=True)
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], None, None, A_log=x["A_log"],
                            dt_bias=x["dt_bias"], a=x["a"], b=x["b"], cu_seqlens=x["cu_seqlens"],
                            scale=x["scale"], qk_l2norm_eps=1e-12)
    torch.cuda.synchronize()
    assert_close(o, ro, "bf16", "out")
    assert_close(f, rf, "bf16", "final")


def test_scan_workspace_argument():
    """A caller's workspace of exactly the reported size is used; one byte
    short is refused by the binding."""
    x = _inputs(550, [8192])
    n = _ws(x)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o, f = _run(x, True, workspace=ws)
    o2, f2 = _run(x, True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(f, f2)
    with pytest.raises(ValueError):
        _run(x, True, workspace=torch.empty(n - 1, dtype=torch.uint8, device="cuda"))


def test_scan_long_request_workload_full_size():
    """The bench's long-request workload at full size (1 x 65536 tokens, Hq 2,
    Hv 4, d 128, bf16, qwen gates through gdn_gate; 32 segments): the scan as
    the bench launches it, and the serial walk, against the oracle on every
    output and final-state element."""
    x = synth.long_request_b1_s65536_hv4()
    g, _, beta = gdn.gate(to_dev(x["A_log"]), to_dev(x["dt_bias"]), to_dev(x["a"]), to_dev(x["b"]))
    q, k, v, cu = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["cu_seqlens"])
    n = gdn.prefill_workspace_size(q, k, v, g, beta, cu_seqlens=cu)
    assert n == 32 * 4 * 128 * 384 * 4
    o_s, f_s = gdn.prefill(q, k, v, g, beta, cu_seqlens=cu, scale=x["scale"])
    o_w, f_w = gdn.prefill(q, k, v, g, beta, cu_seqlens=cu, scale=x["scale"], scan=False)
    torch.cuda.synchronize()
    dec, _, bet = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, bet, cu_seqlens=x["cu_seqlens"],
                            scale=x["scale"])
    es = assert_close(o_s, ro, "bf16", "scan out"), assert_close(f_s, rf, "bf16", "scan final")
    ew = assert_close(o_w, ro, "bf16", "serial out"), assert_close(f_w, rf, "bf16", "serial final")
    _print("long request: scan errors", es, "serial errors", ew)
