"""Seeded cross-feature prefill configurations against the fp64 oracle.

Each case draws, from a fixed seed, a combination of the prefill's options
that the dedicated tests cover one at a time: io dtype, head sizes and the
GVA ratio, chunk hint (pair-role or general kernel), ragged lengths with
empty and partial-chunk requests, update_rule, given or fused gates, the
in-kernel q/k L2 norm, dense or pooled states.  The draw is deterministic, so
a failure names a reproducible configuration.
"""
import random

import numpy as np
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn
import oracle
import synth
from gpu_util import assert_close, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


USES = {"gated_delta": (True, True), "gated": (True, False), "delta": (False, True),
        "linear": (False, False)}


def _config(i):
    r = random.Random(9000 + i)
    dtype = r.choice(["bf16", "bf16", "f32"])
    dk = r.choice([16, 32, 64, 128])
    dv = r.choice([16, 32, 64, 128])
    if r.random() < 0.4 and dtype == "bf16":
        dk, dv = r.choice([(64, 64), (128, 128), (64, 128), (128, 64)])  # pair-role shapes
    hq = r.choice([1, 2])
    hv = hq * r.choice([1, 2, 3])
    chunk = r.choice([0, 0, 16, 32])
    n = r.randint(1, 5)
    lengths = [r.choice([0, 1, r.randint(2, 40), r.randint(41, 150)]) for _ in range(n)]
    if sum(lengths) == 0:
        lengths[0] = 7
    rule = r.choice(list(USES))
    fused = rule != "linear" and r.random() < 0.5
    norm = r.random() < 0.4
    pool = r.random() < 0.4
    init = r.random() < 0.6
    return dict(dtype=dtype, dk=dk, dv=dv, hq=hq, hv=hv, chunk=chunk, lengths=lengths, rule=rule,
                fused=fused, norm=norm, pool=pool, init=init)


@pytest.mark.parametrize("i", range(32))
def test_random_prefill_configuration(i):
    c = _config(i)
    x = synth.prefill_inputs(9100 + i, lengths=c["lengths"], hq=c["hq"], hv=c["hv"], dk=c["dk"],
                             dv=c["dv"], dtype=c["dtype"], gate="qwen",
                             init_std=0.05 if c["init"] else None)
    n, hv, dk, dv = len(c["lengths"]), c["hv"], c["dk"], c["dv"]
    use_d, use_b = USES[c["rule"]]
    if c["norm"]:
        # q and k away from unit length so the norm matters
        g = torch.Generator().manual_seed(9200 + i)
        x["q"] = (x["q"].float() * (torch.rand(x["T"], c["hq"], 1, generator=g) * 3 + 0.3)).to(x["q"].dtype)
        x["k"] = (x["k"].float() * (torch.rand(x["T"], c["hq"], 1, generator=g) * 3 + 0.3)).to(x["k"].dtype)
    kw = dict(cu_seqlens=to_dev(x["cu_seqlens"]), scale=x["scale"], chunk_size=c["chunk"],
              update_rule=c["rule"], qk_l2norm=c["norm"])
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
        dec = bet = None
        odec = obet = None
    else:
        gd, _, gb = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
        odec = torch.from_numpy(gd).float() if use_d else None
        obet = torch.from_numpy(gb).float() if use_b else None
        dec, bet = to_dev(odec), to_dev(obet)
    init = x["initial_state"]
    if c["pool"]:
        P = n + 4
        g = torch.Generator().manual_seed(9300 + i)
        pool0 = torch.randn(P, hv, dv, dk, generator=g) * 0.05
        perm = torch.randperm(P, generator=g)
        read = perm[:n].clone().to(torch.int32)
        read[0] = -1 if n > 1 else read[0]        # one request starts from zeros
        write = perm[:n].clone().to(torch.int32)  # each request writes its own read slot
        if n > 2:
            write[2] = -1                         # one stores nothing
        pool = to_dev(pool0.clone())
        out, _ = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), dec, bet, state_pool=pool,
                             read_slot=to_dev(read), write_slot=to_dev(write), **kw)
        oinit = np.zeros((n, hv, dv, dk))
        for r_, s in enumerate(read.tolist()):
            if s >= 0:
                oinit[r_] = pool0[s].numpy()
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], odec, obet, initial_state=oinit, **okw)
        torch.cuda.synchronize()
        assert_close(out, ro, c["dtype"], "out %s" % c)
        want = pool0.double().numpy().copy()
        for r_, s in enumerate(write.tolist()):
            if s >= 0:
                want[s] = rf[r_]
        got = pool.cpu().double().numpy()
        touched = sorted(s for s in write.tolist() if s >= 0)
        for s in range(P):
            if s in touched:
                assert_close(got[s], want[s], c["dtype"], "slot %d %s" % (s, c))
            else:
                np.testing.assert_array_equal(got[s], want[s])
    else:
        out, fin = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), dec, bet,
                               initial_state=to_dev(init), **kw)
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], odec, obet, initial_state=init, **okw)
        torch.cuda.synchronize()
        assert_close(out, ro, c["dtype"], "out %s" % c)
        assert_close(fin, rf, c["dtype"], "final %s" % c)
