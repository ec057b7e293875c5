"""update_rule variants of the prefill ("com.microsoft.GatedDeltaNet",
update_rule attribute) through the C ABI, against the fp64 oracle.

linear drops the decay and the delta retrieval, gated keeps only the decay,
delta keeps only the retrieval, gated_delta keeps both.  Each rule takes
exactly the gate inputs it uses, either given (fp32 decay / beta, computed by
the oracle's gate here) or fused (raw a / b in the io dtype, gated by the
kernel).  Cases cover the pair-role kernel (bf16, dk = dv in {64, 128}, the
default chunk) and the general kernel (chunk hints 16 and 32, fp32, d32),
ragged requests with partial chunks, an empty request and initial states.
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


LENGTHS = [70, 0, 129, 33]

# (name, dtype, dk, dv, chunk hint): the first two run the pair-role kernel
CONFIGS = [
    ("pair_d128", "bf16", 128, 128, 0),
    ("pair_d64", "bf16", 64, 64, 0),
    ("general_bf16_c16", "bf16", 64, 64, 16),
    ("general_f32_c32", "f32", 128, 128, 32),
    ("general_f32_d32", "f32", 32, 32, 0),
]

USES = {"gated_delta": (True, True), "gated": (True, False), "delta": (False, True),
        "linear": (False, False)}


def _case(rule, cfg, source, seed):
    name, dt, dk, dv, chunk = cfg
    x = synth.prefill_inputs(seed, lengths=LENGTHS, hq=2, hv=4, dk=dk, dv=dv, dtype=dt,
                             gate="qwen", init_std=0.05)
    use_d, use_b = USES[rule]
    kw = dict(cu_seqlens=to_dev(x["cu_seqlens"]), initial_state=to_dev(x["initial_state"]),
              scale=x["scale"], chunk_size=chunk, update_rule=rule)
    okw = dict(cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"], scale=x["scale"],
               update_rule=rule)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    if source == "fused":
        fa = dict(A_log=x["A_log"], dt_bias=x["dt_bias"], a=x["a"]) if use_d else {}
        fb = dict(b=x["b"]) if use_b else {}
        o, f = gdn.prefill(q, k, v, None, None, **{n: to_dev(t) for n, t in {**fa, **fb}.items()},
                           **kw)
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], None, None, **fa, **fb, **okw)
    else:
        g, _, beta = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
        dec = torch.from_numpy(g).float() if use_d else None
        bet = torch.from_numpy(beta).float() if use_b else None
        o, f = gdn.prefill(q, k, v, to_dev(dec), to_dev(bet), **kw)
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, bet, **okw)
    torch.cuda.synchronize()
    return o, f, ro, rf, dt


@pytest.mark.parametrize("source", ["given", "fused"])
@pytest.mark.parametrize("cfg", CONFIGS, ids=[c[0] for c in CONFIGS])
@pytest.mark.parametrize("rule", ["linear", "gated", "delta", "gated_delta"])
def test_rule_matches_oracle(rule, cfg, source):
    if rule == "linear" and source == "fused":
        # linear takes no gate inputs: raw ones are refused, never ignored
        name, dt, dk, dv, chunk = cfg
        x = synth.prefill_inputs(300, lengths=LENGTHS, hq=2, hv=4, dk=dk, dv=dv, dtype=dt,
                                 gate="qwen")
        q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
        for raw in (dict(A_log=x["A_log"], dt_bias=x["dt_bias"], a=x["a"]), dict(b=x["b"])):
            with pytest.raises(ValueError, match="linear takes no"):
                gdn.prefill(q, k, v, None, None, cu_seqlens=to_dev(x["cu_seqlens"]),
                            chunk_size=chunk, update_rule="linear",
                            **{n: to_dev(t) for n, t in raw.items()})
        return
    o, f, ro, rf, dt = _case(rule, cfg, source, seed=300 + CONFIGS.index(cfg))
    assert_close(o, ro, dt, "%s %s %s out" % (rule, cfg[0], source))
    assert_close(f, rf, dt, "%s %s %s final state" % (rule, cfg[0], source))


def test_rules_differ_where_they_should():
    """The four rules give four different results on the same inputs (a rule
    silently falling back to another would pass its oracle comparison only if
    the oracle had the same fault)."""
    outs = {}
    for rule in USES:
        o, f, ro, rf, dt = _case(rule, CONFIGS[0], "given", seed=350)
        outs[rule] = o.float().cpu()
    names = list(outs)
    for i in range(len(names)):
        for j in range(i + 1, len(names)):
            d = (outs[names[i]] - outs[names[j]]).abs().max().item()
            assert d > 1e-2, (names[i], names[j], d)


def test_gated_delta_default_is_unchanged_bitwise():
    """update_rule="gated_delta" passed explicitly and the zero default build
    the same launch: identical bits."""
    x = synth.prefill_inputs(351, lengths=LENGTHS, hq=2, hv=4, dk=128, dv=128, dtype="bf16",
                             gate="qwen")
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    g, _, beta = gdn.gate(to_dev(x["A_log"]), to_dev(x["dt_bias"]), to_dev(x["a"]),
                          to_dev(x["b"]))
    cu = to_dev(x["cu_seqlens"])
    o1, f1 = gdn.prefill(q, k, v, g, beta, cu_seqlens=cu)
    o2, f2 = gdn.prefill(q, k, v, g, beta, cu_seqlens=cu, update_rule="gated_delta")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("mix", ["fused_decay_given_beta", "given_log_decay_fused_beta",
                                 "given_gamma_fused_beta"])
@pytest.mark.parametrize("cfg", CONFIGS, ids=[c[0] for c in CONFIGS])
def test_mixed_gate_sources(mix, cfg):
    """"com.microsoft.GatedDeltaNet", Attributes: gate_activation and
    beta_activation are separate attributes, so one input may be fused while
    the other is given (already activated, fp32).  Each mix against the
    oracle, which takes each source on its own, on every kernel shape
    (mixed problems run on the general kernel)."""
    name, dt, dk, dv, chunk = cfg
    x = synth.prefill_inputs(360 + CONFIGS.index(cfg), lengths=LENGTHS, hq=2, hv=4, dk=dk, dv=dv,
                             dtype=dt, gate="qwen", init_std=0.05)
    g, gam, beta = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
    kw = dict(cu_seqlens=to_dev(x["cu_seqlens"]), initial_state=to_dev(x["initial_state"]),
              scale=x["scale"], chunk_size=chunk)
    okw = dict(cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"], scale=x["scale"])
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    if mix == "fused_decay_given_beta":
        bet = torch.from_numpy(beta).float()
        fa = dict(A_log=x["A_log"], dt_bias=x["dt_bias"], a=x["a"])
        o, f = gdn.prefill(q, k, v, None, to_dev(bet), **{n: to_dev(t) for n, t in fa.items()}, **kw)
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], None, bet, **fa, **okw)
    else:
        is_gamma = mix == "given_gamma_fused_beta"
        dec = torch.from_numpy(gam if is_gamma else g).float()
        o, f = gdn.prefill(q, k, v, to_dev(dec), None, b=to_dev(x["b"]),
                           decay_kind="gamma" if is_gamma else "log", **kw)
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, None, b=x["b"],
                                decay_is_gamma=is_gamma, **okw)
    torch.cuda.synchronize()
    assert_close(o, ro, dt, "%s %s out" % (mix, name))
    assert_close(f, rf, dt, "%s %s final state" % (mix, name))
