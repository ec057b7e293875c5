"""Per-key decay (the ONNX card's per-key-dimension decay spelling: exp(g_t)
scales the key rows of the state) through the C ABI, against the fp64
oracle: the prefill's per-key kernel (ragged requests with empty, one-token
and partial-chunk requests, initial states, both rules with a decay, exact
zero decays and decays below 2^-96 per chunk -- the keys the kernel sums
term by term --, gamma input, in-kernel L2 norm, pooled states, odd head
sizes)
and the decode (single step, staged multi-token with sub-steps, per-token
scatter in the token loop; 16 or more tokens per row in the chunked form,
with and without write-back and with the L2 norm), and decode against
prefill from the same slot.
"""
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


LENGTHS = [37, 0, 16, 1, 70]


def _pk_case(seed, dtype, dk, dv, hq=1, hv=2, lengths=LENGTHS, zeros=False, strong=False):
    x = synth.prefill_inputs(seed, lengths=lengths, hq=hq, hv=hv, dk=dk, dv=dv, dtype=dtype,
                             gate="log", init_std=0.05)
    g = torch.Generator().manual_seed(seed + 1)
    T = x["T"]
    span = 4.0 if strong else 0.5
    dec = -torch.rand(T, hv, dk, generator=g) * span
    if zeros:
        pick = torch.rand(T, hv, dk, generator=g) < 0.03
        dec[pick] = -float("inf")  # exact zero decays on some keys
    return x, dec


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 64), (128, 128), (128, 64), (16, 128)])
@pytest.mark.parametrize("rule", ["gated_delta", "gated"])
def test_prefill_per_key_matches_oracle(dtype, dk, dv, rule):
    x, dec = _pk_case(1000 + dk + dv, dtype, dk, dv)
    bet = x["beta"] if rule == "gated_delta" else None
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(dec), to_dev(bet),
                       cu_seqlens=to_dev(x["cu_seqlens"]), initial_state=to_dev(x["initial_state"]),
                       scale=x["scale"], update_rule=rule, decay_per_key=True)
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, bet, cu_seqlens=x["cu_seqlens"],
                            initial_state=x["initial_state"], scale=x["scale"], update_rule=rule,
                            decay_per_key=True)
    torch.cuda.synchronize()
    assert_close(o, ro, dtype, "out")
    assert_close(f, rf, dtype, "final state")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
def test_prefill_per_key_with_fused_beta(dtype, dk, dv):
    """A given per-key decay with beta fused from the raw b (beta_activation
    sigmoid of "com.microsoft.GatedDeltaNet", Attributes, taken on its own)."""
    x, dec = _pk_case(1100 + dk + dv, dtype, dk, dv)
    g = torch.Generator().manual_seed(1101)
    b = torch.randn(x["T"], 2, generator=g).to(synth.DTYPES[dtype])
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(dec), None,
                       b=to_dev(b), cu_seqlens=to_dev(x["cu_seqlens"]),
                       initial_state=to_dev(x["initial_state"]), scale=x["scale"],
                       decay_per_key=True)
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, None, b=b, cu_seqlens=x["cu_seqlens"],
                            initial_state=x["initial_state"], scale=x["scale"], decay_per_key=True)
    torch.cuda.synchronize()
    assert_close(o, ro, dtype, "out")
    assert_close(f, rf, dtype, "final state")


@pytest.mark.parametrize("mode", ["zeros", "strong", "gamma", "qk_l2norm", "gva"])
def test_prefill_per_key_edge_cases(mode):
    kw = dict(zeros=mode == "zeros", strong=mode == "strong")
    hq, hv = (2, 6) if mode == "gva" else (1, 2)
    x, dec = _pk_case(1100, "f32", 64, 64, hq=hq, hv=hv, **kw)
    dkw, okw = {}, {}
    decay = dec
    if mode == "gamma":
        decay = torch.exp(dec)
        decay[torch.rand(decay.shape, generator=torch.Generator().manual_seed(5)) < 0.02] = 0.0
        dkw["decay_kind"] = "gamma"
        okw["decay_is_gamma"] = True
    if mode == "qk_l2norm":
        x["q"] = x["q"] * 3.0
        x["k"] = x["k"] * 0.4
        dkw["qk_l2norm"] = True
        okw["qk_l2norm_eps"] = 1e-12
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(decay),
                       to_dev(x["beta"]), cu_seqlens=to_dev(x["cu_seqlens"]),
                       initial_state=to_dev(x["initial_state"]), scale=x["scale"],
                       decay_per_key=True, **dkw)
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], decay, x["beta"], cu_seqlens=x["cu_seqlens"],
                            initial_state=x["initial_state"], scale=x["scale"], decay_per_key=True,
                            **okw)
    torch.cuda.synchronize()
    assert_close(o, ro, "f32", "out %s" % mode)
    assert_close(f, rf, "f32", "final %s" % mode)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_per_key_extreme_decays(dtype):
    """Keys whose decay over a 16-token chunk falls below 2^-96 (no zero
    among them) mixed with ordinary keys: the kernel adds the former term by
    term instead of through the factored Gram tile, and must match."""
    x, dec = _pk_case(1150, dtype, 128, 64)
    g = torch.Generator().manual_seed(1151)
    wild = torch.rand(dec.shape[1:], generator=g) < 0.3          # per (head, key)
    dec = torch.where(wild, -torch.rand(dec.shape, generator=g) * 14.0, dec)
    o, f = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(dec), to_dev(x["beta"]),
                       cu_seqlens=to_dev(x["cu_seqlens"]), initial_state=to_dev(x["initial_state"]),
                       scale=x["scale"], decay_per_key=True)
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, x["beta"], cu_seqlens=x["cu_seqlens"],
                            initial_state=x["initial_state"], scale=x["scale"], decay_per_key=True)
    torch.cuda.synchronize()
    assert_close(o, ro, dtype, "out")
    assert_close(f, rf, dtype, "final state")


def test_prefill_per_key_pool_and_odd_head_sizes():
    # pooled states
    x, dec = _pk_case(1200, "bf16", 128, 64)
    n, hv = len(LENGTHS), 2
    g = torch.Generator().manual_seed(1201)
    pool0 = torch.randn(8, hv, 64, 128, generator=g) * 0.05
    read = torch.tensor([3, -1, 5, 0, 7], dtype=torch.int32)
    pool = to_dev(pool0.clone())
    o, _ = gdn.prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(dec), to_dev(x["beta"]),
                       cu_seqlens=to_dev(x["cu_seqlens"]), scale=x["scale"], decay_per_key=True,
                       state_pool=pool, read_slot=to_dev(read))
    init = np.zeros((n, hv, 64, 128))
    for r, s in enumerate(read.tolist()):
        if s >= 0:
            init[r] = pool0[s].numpy()
    ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, x["beta"], cu_seqlens=x["cu_seqlens"],
                            initial_state=init, scale=x["scale"], decay_per_key=True)
    torch.cuda.synchronize()
    assert_close(o, ro, "bf16", "pooled out")
    for r, s in enumerate(read.tolist()):
        if s >= 0:
            assert_close(pool[s], rf[r], "bf16", "slot %d" % s)
    # head sizes 12 / 9, zero-padded by the binding (per-key decay padded too)
    g = torch.Generator().manual_seed(1202)
    T = 40
    q = torch.randn(T, 1, 12, generator=g)
    k = torch.nn.functional.normalize(torch.randn(T, 1, 12, generator=g), dim=-1)
    v = torch.randn(T, 2, 9, generator=g)
    d = -torch.rand(T, 2, 12, generator=g)
    b = torch.rand(T, 2, generator=g)
    o, f = gdn.prefill(q.cuda(), k.cuda(), v.cuda(), d.cuda(), b.cuda(), decay_per_key=True)
    ro, rf = oracle.prefill(q, k, v, d, b, n_seqs=1, seq_len=T, scale=1.0 / np.sqrt(12),
                            decay_per_key=True)
    torch.cuda.synchronize()
    assert_close(o, ro, "f32", "odd-size out")
    assert_close(f, rf, "f32", "odd-size final")


def _decode_pk(seed, dtype, T, n, scatter, dk=128, dv=64):
    x = synth.decode_inputs(seed, pool_size=48, batch=6, T=T, n_hh=n, hq=2, hv=4, dk=dk, dv=dv,
                            dtype=dtype, skip_rows=1, write_slots=not scatter, scatter=scatter)
    g = torch.Generator().manual_seed(seed + 1)
    dec = -torch.rand(6, T, 4, dk, generator=g) * 0.7
    return x, dec


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,n,scatter", [(1, 1, False), (3, 2, False), (4, 1, True), (20, 1, False),
                                         (16, 1, False), (33, 1, False), (64, 1, False)])
def test_decode_per_key_matches_oracle(dtype, T, n, scatter):
    x, dec = _decode_pk(1300 + T * 10 + n, dtype, T, n, scatter)
    pool = to_dev(x["pool"].clone())
    out = torch.zeros(6, T, 4, 64, dtype=synth.DTYPES[dtype], device="cuda")
    gdn.decode(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), None, None, None, to_dev(x["b"]),
               pool, to_dev(x["read_idx"]), write_idx=to_dev(x["write_idx"]),
               scatter_idx=to_dev(x["scatter_idx"]), scale=x["scale"], out=out,
               decay_per_key=to_dev(dec), use_qk_l2norm=False)
    ro, rp = oracle.decode(x["q"], x["k"], x["v"], None, None, None, x["b"], x["pool"], x["read_idx"],
                           write_idx=x["write_idx"], scatter_idx=x["scatter_idx"], scale=x["scale"],
                           decay_per_key=dec)
    torch.cuda.synchronize()
    active = (x["read_idx"] >= 0).numpy()
    assert_close(out[torch.from_numpy(active).cuda()], ro[active], dtype, "decode out")
    assert_close(pool, rp, dtype, "decode pool")
    skipped = torch.from_numpy(~active).cuda()
    assert torch.all(out[skipped] == 0)


@pytest.mark.parametrize("mode", ["disable", "qk_l2norm"])
def test_decode_per_key_chunked_modes(mode):
    """The multi-token decode with a per-key decay in its chunked form (T >= 16):
    no state write-back, and the in-kernel q/k L2 norm."""
    x, dec = _decode_pk(1500 + len(mode), "bf16", 24, 1, False)
    kw = dict(disable_state_update=True, use_qk_l2norm=False) if mode == "disable" else dict(use_qk_l2norm=True, qk_l2norm_eps=1e-12)
    okw = dict(disable_state_update=True) if mode == "disable" else dict(qk_l2norm_eps=1e-12)
    if mode == "qk_l2norm":
        x["q"] = x["q"] * 2.5
        x["k"] = x["k"] * 0.5
    pool = to_dev(x["pool"].clone())
    out = torch.zeros(6, 24, 4, 64, dtype=torch.bfloat16, device="cuda")
    gdn.decode(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), None, None, None, to_dev(x["b"]),
               pool, to_dev(x["read_idx"]), write_idx=to_dev(x["write_idx"]), scale=x["scale"], out=out,
               decay_per_key=to_dev(dec), **kw)
    ro, rp = oracle.decode(x["q"], x["k"], x["v"], None, None, None, x["b"], x["pool"], x["read_idx"],
                           write_idx=x["write_idx"], scale=x["scale"], decay_per_key=dec, **okw)
    torch.cuda.synchronize()
    active = (x["read_idx"] >= 0).numpy()
    assert_close(out[torch.from_numpy(active).cuda()], ro[active], "bf16", "decode out")
    if mode == "disable":
        assert torch.equal(pool.cpu(), x["pool"])
    else:
        assert_close(pool, rp, "bf16", "decode pool")


def test_decode_per_key_equals_prefill_from_the_slot():
    x, dec = _decode_pk(1400, "f32", 9, 1, False, dk=64, dv=64)
    B, T = 6, 9
    pool_a = to_dev(x["pool"].clone())
    od, _ = gdn.decode(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), None, None, None,
                       to_dev(x["b"]), pool_a, to_dev(x["read_idx"]), scale=x["scale"],
                       decay_per_key=to_dev(dec), use_qk_l2norm=False)
    pool_b = to_dev(x["pool"].clone())
    beta = torch.sigmoid(x["b"].float()).reshape(B * T, 4)
    cu = torch.arange(B + 1, dtype=torch.int32) * T
    op, _ = gdn.prefill(to_dev(x["q"].reshape(B * T, 2, 64)), to_dev(x["k"].reshape(B * T, 2, 64)),
                        to_dev(x["v"].reshape(B * T, 4, 64)), to_dev(dec.reshape(B * T, 4, 64)),
                        to_dev(beta), cu_seqlens=to_dev(cu), scale=x["scale"], decay_per_key=True,
                        state_pool=pool_b, read_slot=to_dev(x["read_idx"]))
    torch.cuda.synchronize()
    active = (x["read_idx"] >= 0).cuda()
    assert_close(op.view(B, T, 4, 64)[active], od[active].double().cpu().numpy(), "f32", "out")
    assert_close(pool_b, pool_a.double().cpu().numpy(), "f32", "pool")


def _pk_random(i):
    import random
    r = random.Random(7000 + i)
    dtype = r.choice(["bf16", "f32"])
    dk, dv = r.choice([16, 32, 64, 128]), r.choice([16, 32, 64, 128])
    hq = r.choice([1, 2])
    hv = hq * r.choice([1, 2])
    lengths = [r.choice([0, 1, r.randint(2, 40), r.randint(41, 120)]) for _ in range(r.randint(1, 4))]
    if sum(lengths) == 0:
        lengths[0] = 9
    return dict(dtype=dtype, dk=dk, dv=dv, hq=hq, hv=hv, lengths=lengths,
                rule=r.choice(["gated_delta", "gated"]), norm=r.random() < 0.3, pool=r.random() < 0.4,
                gamma=r.random() < 0.3, zeros=r.choice([0.0, 0.0, 0.02, 0.2]),
                wild=r.choice([0.0, 0.0, 0.1, 0.5]))


@pytest.mark.parametrize("i", range(16))
def test_prefill_per_key_random_configuration(i):
    """Seeded cross-feature per-key configurations: io dtype, head sizes, GVA,
    ragged lengths, rule, in-kernel L2 norm, pooled or dense states, log or
    gamma decays, exact zero decays and keys decaying below 2^-96 per chunk."""
    c = _pk_random(i)
    x = synth.prefill_inputs(7100 + i, lengths=c["lengths"], hq=c["hq"], hv=c["hv"], dk=c["dk"], dv=c["dv"],
                             dtype=c["dtype"], gate="log", init_std=0.05)
    g = torch.Generator().manual_seed(7200 + i)
    T, hv, dk, dv, n = x["T"], c["hv"], c["dk"], c["dv"], len(c["lengths"])
    dec = -torch.rand(T, hv, dk, generator=g) * 0.6
    wild = torch.rand(hv, dk, generator=g) < c["wild"]
    dec = torch.where(wild, -torch.rand(T, hv, dk, generator=g) * 12.0, dec)
    dec[torch.rand(T, hv, dk, generator=g) < c["zeros"]] = -float("inf")
    kw, okw = {}, {}
    if c["gamma"]:
        dec = torch.exp(dec)
        kw["decay_kind"] = "gamma"
        okw["decay_is_gamma"] = True
    if c["norm"]:
        x["q"] = (x["q"].float() * (torch.rand(T, c["hq"], 1, generator=g) * 3 + 0.3)).to(x["q"].dtype)
        x["k"] = (x["k"].float() * (torch.rand(T, c["hq"], 1, generator=g) * 3 + 0.3)).to(x["k"].dtype)
        kw["qk_l2norm"] = True
        okw["qk_l2norm_eps"] = 1e-12
    bet = x["beta"] if c["rule"] == "gated_delta" else None
    args = (to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(dec), to_dev(bet))
    oargs = (x["q"], x["k"], x["v"], dec, bet)
    common = dict(scale=x["scale"], update_rule=c["rule"], decay_per_key=True)
    if c["pool"]:
        P = n + 3
        pool0 = torch.randn(P, hv, dv, dk, generator=g) * 0.05
        slots = torch.randperm(P, generator=g)[:n].to(torch.int32)
        pool = to_dev(pool0.clone())
        o, _ = gdn.prefill(*args, cu_seqlens=to_dev(x["cu_seqlens"]), state_pool=pool,
                           read_slot=to_dev(slots), **common, **kw)
        init = np.stack([pool0[s].numpy() for s in slots.tolist()])
        ro, rf = oracle.prefill(*oargs, cu_seqlens=x["cu_seqlens"], initial_state=init, **common, **okw)
        torch.cuda.synchronize()
        assert_close(o, ro, c["dtype"], "out %s" % c)
        for r_, s_ in enumerate(slots.tolist()):
            assert_close(pool[s_], rf[r_], c["dtype"], "slot %d %s" % (s_, c))
    else:
        o, f = gdn.prefill(*args, cu_seqlens=to_dev(x["cu_seqlens"]), initial_state=to_dev(x["initial_state"]),
                           **common, **kw)
        ro, rf = oracle.prefill(*oargs, cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                                **common, **okw)
        torch.cuda.synchronize()
        assert_close(o, ro, c["dtype"], "out %s" % c)
        assert_close(f, rf, c["dtype"], "final %s" % c)
