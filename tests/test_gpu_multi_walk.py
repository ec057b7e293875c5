"""The pair kernel's multi-request walk, through the C ABI, against the fp64
oracle.  A bf16 call with more (request, value head, 64-column slice) units
than 256 workgroups and requests of four chunks or fewer on average runs
each workgroup over a run of consecutive requests (chunk preparation
pipelined across request boundaries, the state swapped at each).  Every
output and final state is compared: ragged lengths with empty and one-token
requests, uniform packing, initial states, both head sizes, the fused gate
with the in-kernel L2 norm, pooled states with read and write slots, and the
multi-token decode's chunked route (skipped rows, disable_state_update).
"""
import random

import numpy as np
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn
import oracle
import synth
from gpu_util import assert_close, require_gpu, to_dev
from test_gpu_kernels import _check_decode, _gpu_decode, _oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _lengths(seed, n, hi):
    g = np.random.default_rng(seed)
    L = g.integers(0, hi + 1, n)
    L[::7] = 0      # empty requests, also the first
    L[3::11] = 1    # one-token requests
    L[5] = 64       # exactly one chunk
    L[6] = 65       # one chunk and a token
    return [int(v) for v in L]


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
def test_multi_walk_ragged_initial_states(dk, dv):
    L = _lengths(1600 + dk + dv, 80, 200)
    x = synth.prefill_inputs(1601 + dk, lengths=L, hq=2, hv=4, dk=dk, dv=dv, dtype="bf16",
                             gate="log", gamma_range=(0.8, 1.0), init_std=0.05)
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["log_decay"]),
                       to_dev(x["beta"]), cu_seqlens=to_dev(x["cu_seqlens"]),
                       initial_state=to_dev(x["initial_state"]), scale=x["scale"])
    torch.cuda.synchronize()
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], x["log_decay"], x["beta"],
                            cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                            scale=x["scale"])
    assert_close(o, ro, "bf16", "multi-walk out")
    assert_close(f, rf, "bf16", "multi-walk final state")
    # an empty request's final state is its initial state, bit for bit
    for r, n in enumerate(L):
        if n == 0:
            assert torch.equal(f[r].cpu(), x["initial_state"][r])


def test_multi_walk_uniform_fused_gate_l2norm():
    x = synth.prefill_inputs(1610, n_seqs=96, seq_len=40, hq=2, hv=4, dk=128, dv=128,
                             dtype="bf16", gate="qwen")
    g = torch.Generator().manual_seed(1611)
    q = (x["q"].float() * (torch.rand(x["T"], 2, 1, generator=g) * 3 + 0.3)).to(torch.bfloat16)
    k = (x["k"].float() * (torch.rand(x["T"], 2, 1, generator=g) * 3 + 0.3)).to(torch.bfloat16)
    o, f = gdn.prefill(to_dev(q).view(96, 40, 2, 128), to_dev(k).view(96, 40, 2, 128),
                       to_dev(x["v"]).view(96, 40, 4, 128), None, None, A_log=to_dev(x["A_log"]),
                       dt_bias=to_dev(x["dt_bias"]), a=to_dev(x["a"]).view(96, 40, 4),
                       b=to_dev(x["b"]).view(96, 40, 4), qk_l2norm=True, scale=x["scale"])
    torch.cuda.synchronize()
    ro, rf = oracle.prefill(q, k, x["v"], None, None, n_seqs=96, seq_len=40, scale=x["scale"],
                            A_log=x["A_log"], dt_bias=x["dt_bias"], a=x["a"], b=x["b"],
                            qk_l2norm_eps=1e-12)
    assert_close(o.view(96 * 40, 4, 128), ro, "bf16", "multi-walk fused out")
    assert_close(f, rf, "bf16", "multi-walk fused final state")


def test_multi_walk_pool_slots():
    """Pooled states: reads outside the pool start from zeros, writes outside
    the pool store nothing, a request may read and write one slot; slots no
    request writes keep their bits."""
    n, P = 72, 160
    L = _lengths(1620, n, 150)
    x = synth.prefill_inputs(1621, lengths=L, hq=2, hv=4, dk=128, dv=128, dtype="bf16", gate="log")
    g = torch.Generator().manual_seed(1622)
    perm = torch.randperm(P, generator=g)
    read = perm[:n].clone().to(torch.int32)
    write = perm[n:2 * n].clone().to(torch.int32)
    read[::9] = -1
    read[4::13] = P + 3
    write[2::10] = -1
    write[1] = read[1]
    pool0 = torch.randn(P, 4, 128, 128, generator=g) * 0.05
    pool = to_dev(pool0.clone())
    o, _ = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["log_decay"]),
                       to_dev(x["beta"]), cu_seqlens=to_dev(x["cu_seqlens"]), scale=x["scale"],
                       state_pool=pool, read_slot=to_dev(read), write_slot=to_dev(write))
    torch.cuda.synchronize()
    init = np.zeros((n, 4, 128, 128))
    for r, s in enumerate(read.tolist()):
        if 0 <= s < P:
            init[r] = pool0[s].numpy()
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], x["log_decay"], x["beta"],
                            cu_seqlens=x["cu_seqlens"], initial_state=init, scale=x["scale"])
    assert_close(o, ro, "bf16", "multi-walk pooled out")
    got = pool.cpu().double().numpy()
    written = {}
    for r, s in enumerate(write.tolist()):
        if 0 <= s < P:
            written[s] = r
    for s in range(P):
        if s in written:
            assert_close(got[s], rf[written[s]], "bf16", "slot %d" % s)
        else:
            np.testing.assert_array_equal(got[s], pool0[s].double().numpy())


@pytest.mark.parametrize("T,mode", [(16, "plain"), (48, "disable"), (64, "plain"), (40, "qk_l2norm")])
def test_multi_walk_decode_route(T, mode):
    """gdn_decode with T >= 16 (one delta step per token, no scatter) over 96
    rows: the chunked route runs the multi-request walk; skipped rows keep
    their outputs and slots."""
    x = synth.decode_inputs(1630 + T, pool_size=240, batch=96, T=T, n_hh=1, hq=2, hv=4, dk=128,
                            dv=128, dtype="bf16", skip_rows=9, write_slots=True)
    kw, okw = {}, {}
    if mode == "disable":
        kw["disable_state_update"] = okw["disable_state_update"] = True
    if mode == "qk_l2norm":
        x["q"] = (x["q"].float() * 3.0).to(torch.bfloat16)
        x["k"] = (x["k"].float() * 0.3).to(torch.bfloat16)
        kw["use_qk_l2norm"] = True
        okw["qk_l2norm_eps"] = 1e-6
    out_g, pool_g = _gpu_decode(x, **kw)
    torch.cuda.synchronize()
    out_r, pool_r = _oracle_decode(x, **okw)
    _check_decode(x, out_g, pool_g, out_r, pool_r, "bf16")
    if mode == "disable":
        assert torch.equal(pool_g.cpu(), x["pool"])


@pytest.mark.parametrize("hq,hv,dk,dv", [(4, 4, 128, 128), (2, 6, 64, 64), (1, 4, 64, 128)],
                         ids=["no_gva", "gva3_d64", "gva4_dv128"])
def test_multi_walk_head_maps(hq, hv, dk, dv):
    """Value head h reads q/k head h * hq / hv inside the walk as outside it."""
    n = 96
    L = _lengths(1640 + hv + dk, n, 120)
    x = synth.prefill_inputs(1641 + hq + hv, lengths=L, hq=hq, hv=hv, dk=dk, dv=dv, dtype="bf16",
                             gate="gamma", init_std=0.05)
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["gamma"]),
                       to_dev(x["beta"]), decay_kind="gamma", cu_seqlens=to_dev(x["cu_seqlens"]),
                       initial_state=to_dev(x["initial_state"]), scale=x["scale"])
    torch.cuda.synchronize()
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], x["gamma"], x["beta"], decay_is_gamma=True,
                            cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                            scale=x["scale"])
    assert_close(o, ro, "bf16", "multi-walk out")
    assert_close(f, rf, "bf16", "multi-walk final state")


USES = {"gated_delta": (True, True), "gated": (True, False), "delta": (False, True),
        "linear": (False, False)}


def _walk_config(i):
    """A seeded draw of options inside the walk's regime: bf16 pair-kernel
    head sizes, and more (request, value head, slice) units than 256 with
    short requests."""
    r = random.Random(17000 + i)
    dk, dv = r.choice([(64, 64), (128, 128), (64, 128), (128, 64)])
    hq = r.choice([1, 2])
    hv = hq * r.choice([1, 2, 3])
    units_per_req = hv * (dv // 64)
    n = max(r.randint(40, 140), 256 // units_per_req + r.randint(1, 20))
    lengths = [r.choice([0, 1, r.randint(2, 63), 64, r.randint(65, 200)]) for _ in range(n)]
    if sum(lengths) == 0:
        lengths[0] = 7
    rule = r.choice(list(USES))
    fused = rule != "linear" and r.random() < 0.5
    return dict(dk=dk, dv=dv, hq=hq, hv=hv, lengths=lengths, rule=rule, fused=fused,
                norm=r.random() < 0.4, pool=r.random() < 0.4, init=r.random() < 0.6)


def run_walk_case(i):
    c = _walk_config(i)
    n, hq, hv, dk, dv = len(c["lengths"]), c["hq"], c["hv"], c["dk"], c["dv"]
    x = synth.prefill_inputs(17100 + i, lengths=c["lengths"], hq=hq, hv=hv, dk=dk, dv=dv,
                             dtype="bf16", gate="qwen", init_std=0.05 if c["init"] else None)
    use_d, use_b = USES[c["rule"]]
    if c["norm"]:
        g = torch.Generator().manual_seed(17200 + i)
        x["q"] = (x["q"].float() * (torch.rand(x["T"], hq, 1, generator=g) * 3 + 0.3)).to(torch.bfloat16)
        x["k"] = (x["k"].float() * (torch.rand(x["T"], hq, 1, generator=g) * 3 + 0.3)).to(torch.bfloat16)
    kw = dict(cu_seqlens=to_dev(x["cu_seqlens"]), scale=x["scale"], update_rule=c["rule"],
              qk_l2norm=c["norm"])
    okw = dict(cu_seqlens=x["cu_seqlens"], scale=x["scale"], update_rule=c["rule"],
               qk_l2norm_eps=1e-12 if c["norm"] else None)
    if c["fused"]:
        gk = {}
        if use_d:
            gk.update(A_log=x["A_log"], dt_bias=x["dt_bias"], a=x["a"])
        if use_b:
            gk["b"] = x["b"]
        kw.update({k: to_dev(v) for k, v in gk.items()})
        okw.update(gk)
        dec = bet = odec = obet = None
    else:
        gd, _, gb = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
        odec = torch.from_numpy(gd).float() if use_d else None
        obet = torch.from_numpy(gb).float() if use_b else None
        dec, bet = to_dev(odec), to_dev(obet)
    if c["pool"]:
        P = n + 8
        g = torch.Generator().manual_seed(17300 + i)
        pool0 = torch.randn(P, hv, dv, dk, generator=g) * 0.05
        perm = torch.randperm(P, generator=g)
        read = perm[:n].clone().to(torch.int32)
        read[::5] = -1                       # these start from zeros
        write = perm[:n].clone().to(torch.int32)
        write[2::7] = -1                     # these store nothing
        pool = to_dev(pool0.clone())
        out, _ = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), dec, bet, state_pool=pool,
                             read_slot=to_dev(read), write_slot=to_dev(write), **kw)
        oinit = np.zeros((n, hv, dv, dk))
        for r_, s in enumerate(read.tolist()):
            if s >= 0:
                oinit[r_] = pool0[s].numpy()
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], odec, obet, initial_state=oinit, **okw)
        torch.cuda.synchronize()
        assert_close(out, ro, "bf16", "out %s" % c)
        want = pool0.double().numpy().copy()
        for r_, s in enumerate(write.tolist()):
            if s >= 0:
                want[s] = rf[r_]
        got = pool.cpu().double().numpy()
        touched = set(s for s in write.tolist() if s >= 0)
        for s in range(P):
            if s in touched:
                assert_close(got[s], want[s], "bf16", "slot %d %s" % (s, c))
            else:
                np.testing.assert_array_equal(got[s], want[s])
    else:
        out, fin = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), dec, bet,
                               initial_state=to_dev(x["initial_state"]), **kw)
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], odec, obet, initial_state=x["initial_state"], **okw)
        torch.cuda.synchronize()
        assert_close(out, ro, "bf16", "out %s" % c)
        assert_close(fin, rf, "bf16", "final %s" % c)


@pytest.mark.parametrize("i", range(12))
def test_multi_walk_random_configuration(i):
    """Seeded cross-feature draws inside the walk's regime: head sizes, GVA,
    ragged lengths with empty, one-token and chunk-boundary requests, every
    update rule, given or fused gates, the L2 norm, dense or pooled states."""
    run_walk_case(i)
