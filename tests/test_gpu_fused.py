"""In-kernel q/k L2 norm and the fused gate inside prefill, and use_qk_l2norm
in decode, against the fp64 oracle (the ONNX card's qk_l2_norm attribute, the
FlashInfer page's use_qk_l2norm and fused gate).

q and k are drawn far from unit length (per-token scales 0.2 .. 5) so that a
missing or misplaced normalisation shows.  Cases cover both prefill kernels
(bf16 d64/d128 with the default chunk; fp32 and chunk hints 16/32 on the
general one), ragged requests with partial chunks and empty requests, zero
vectors, and both decode paths (single step, staged multi-token).
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


def _raw(x, seed):
    """Rescale q and k rows of a synth input dict by per-token factors."""
    g = torch.Generator().manual_seed(seed)
    T, hq = x["q"].shape[0], x["q"].shape[1]
    sq = torch.rand(T, hq, 1, generator=g) * 4.8 + 0.2
    sk = torch.rand(T, hq, 1, generator=g) * 4.8 + 0.2
    y = dict(x)
    y["q"] = (x["q"].float() * sq).to(x["q"].dtype)
    y["k"] = (x["k"].float() * sk).to(x["k"].dtype)
    return y


def _run(x, *, norm, fused, chunk_size=0, eps=1e-12):
    kw = dict(cu_seqlens=to_dev(x["cu_seqlens"]), initial_state=to_dev(x["initial_state"]),
              scale=x["scale"], chunk_size=chunk_size, qk_l2norm=norm, qk_l2norm_eps=eps)
    okw = dict(cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"], scale=x["scale"],
               qk_l2norm_eps=eps if norm else None)
    assert x["cu_seqlens"] is not None, "these cases pack requests through cu_seqlens"
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    if fused:
        o, f = gdn.prefill(q, k, v, None, None, A_log=to_dev(x["A_log"]),
                           dt_bias=to_dev(x["dt_bias"]), a=to_dev(x["a"]), b=to_dev(x["b"]), **kw)
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], None, None, A_log=x["A_log"],
                                dt_bias=x["dt_bias"], a=x["a"], b=x["b"], **okw)
    else:
        g, _, beta = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
        dec = torch.from_numpy(g).float()
        bet = torch.from_numpy(beta).float()
        o, f = gdn.prefill(q, k, v, to_dev(dec), to_dev(bet), **kw)
        ro, rf = oracle.prefill(x["q"], x["k"], x["v"], dec, bet, **okw)
    return o, f, ro, rf


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
@pytest.mark.parametrize("norm,fused", [(True, True), (True, False), (False, True)])
def test_pair_kernel_norm_and_fused_gate(dk, dv, norm, fused):
    x = synth.prefill_inputs(800 + dk + dv, lengths=[130, 0, 64, 77, 1], hq=2, hv=4, dk=dk, dv=dv,
                             dtype="bf16", gate="qwen", init_std=0.2)
    x = _raw(x, 801)
    o, f, ro, rf = _run(x, norm=norm, fused=fused)
    assert_close(o, ro, "bf16", "out")
    assert_close(f, rf, "bf16", "final")


@pytest.mark.parametrize("dtype,dk,dv,chunk", [("f32", 128, 64, 0), ("f32", 32, 16, 16),
                                               ("bf16", 128, 128, 32), ("bf16", 16, 128, 16),
                                               ("f32", 64, 128, 64)])
def test_general_kernel_norm_and_fused_gate(dtype, dk, dv, chunk):
    x = synth.prefill_inputs(810 + dk, lengths=[100, 33, 0, 48], hq=1, hv=2, dk=dk, dv=dv,
                             dtype=dtype, gate="qwen", init_std=0.1)
    x = _raw(x, 811)
    o, f, ro, rf = _run(x, norm=True, fused=True, chunk_size=chunk)
    assert_close(o, ro, dtype, "out")
    assert_close(f, rf, dtype, "final")


def test_norm_is_invariant_to_power_of_two_rescaling_on_gpu():
    """Scaling q and k rows by powers of two is exact in bf16 and in every
    fp32 step of the norm, so with the norm on the results are bit-identical."""
    x = synth.prefill_inputs(820, lengths=[200, 200], hq=2, hv=2, dk=128, dv=128,
                             dtype="bf16", gate="qwen")
    x = _raw(x, 821)
    o1, f1, ro, rf = _run(x, norm=True, fused=True)
    assert_close(o1, ro, "bf16", "out")
    g = torch.Generator().manual_seed(822)
    y = dict(x)
    for key in ("q", "k"):
        e = torch.randint(-3, 4, (x[key].shape[0], x[key].shape[1], 1), generator=g).float()
        y[key] = (x[key].float() * torch.exp2(e)).to(torch.bfloat16)
    o2, f2, _, _ = _run(y, norm=True, fused=True)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_query_and_key_rows(dtype):
    x = synth.prefill_inputs(830, lengths=[90, 40], hq=1, hv=2, dk=64, dv=64, dtype=dtype,
                             gate="qwen", init_std=0.3)
    x = _raw(x, 831)
    q, k = x["q"].clone(), x["k"].clone()
    q[[3, 64, 100]] = 0
    k[[5, 64, 101]] = 0
    x["q"], x["k"] = q, k
    for chunk in (0, 16):
        o, f, ro, rf = _run(x, norm=True, fused=True, chunk_size=chunk)
        assert_close(o, ro, dtype, "out")
        assert_close(f, rf, dtype, "final")


def test_fused_gate_equals_separate_gate_call():
    """The fused gate and gdn_gate + prefill compute the same gates (fp32
    arithmetic in both): the results agree to rounding."""
    x = synth.prefill_inputs(840, lengths=[300, 50], hq=2, hv=4, dk=128, dv=128, dtype="bf16",
                             gate="qwen")
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    cu = to_dev(x["cu_seqlens"])
    g, _, beta = gdn.gate(to_dev(x["A_log"]), to_dev(x["dt_bias"]), to_dev(x["a"]), to_dev(x["b"]))
    o1, f1 = gdn.prefill(q, k, v, g, beta, cu_seqlens=cu, scale=x["scale"])
    o2, f2 = gdn.prefill(q, k, v, None, None, cu_seqlens=cu, scale=x["scale"],
                         A_log=to_dev(x["A_log"]), dt_bias=to_dev(x["dt_bias"]),
                         a=to_dev(x["a"]), b=to_dev(x["b"]))
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2 * o1.float().abs().max().item()
    assert (f1 - f2).abs().max().item() <= 1e-3 * f1.abs().max().item()


def _dec(seed, T, n, dtype, **kw):
    x = synth.decode_inputs(seed, pool_size=40, batch=6, T=T, n_hh=n, hq=2, hv=4, dk=128, dv=64,
                            dtype=dtype, skip_rows=1, **kw)
    g = torch.Generator().manual_seed(seed + 1)
    x["q"] = (x["q"].float() * (torch.rand(*x["q"].shape[:3], 1, generator=g) * 4.8 + 0.2)).to(x["q"].dtype)
    x["k"] = (x["k"].float() * (torch.rand(*x["k"].shape[:4], 1, generator=g) * 4.8 + 0.2)).to(x["k"].dtype)
    return x


@pytest.mark.parametrize("T,n", [(1, 1), (3, 2), (9, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_use_qk_l2norm(T, n, dtype):
    x = _dec(850 + T * 10 + n, T, n, dtype, scatter=(T == 3))
    pool = x["pool"].cuda()
    o, pool = gdn.decode(*(to_dev(x[kk]) for kk in ("q", "k", "v", "A_log", "dt_bias", "a", "b")),
                         pool, to_dev(x["read_idx"]), write_idx=to_dev(x["write_idx"]),
                         scatter_idx=to_dev(x["scatter_idx"]), scale=x["scale"],
                         use_qk_l2norm=True, qk_l2norm_eps=1e-6)
    ro, rp = oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                           x["pool"], x["read_idx"], write_idx=x["write_idx"],
                           scatter_idx=x["scatter_idx"], scale=x["scale"], qk_l2norm_eps=1e-6)
    assert_close(o, ro, dtype, "out")
    assert_close(pool, rp, dtype, "pool")
    # without the norm the rescaled inputs give a different result
    ro2, _ = oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                           x["pool"], x["read_idx"], write_idx=x["write_idx"],
                           scatter_idx=x["scatter_idx"], scale=x["scale"])
    assert np.abs(ro2 - ro).max() > 1e-2 * np.abs(ro).max()


def test_decode_l2norm_on_by_default():
    """The binding's use_qk_l2norm defaults to True with eps 1e-6, as the
    FlashInfer page's decode: a call that names neither is bit-identical to
    one that asks for the norm explicitly."""
    x = _dec(870, 2, 2, "bf16", scatter=False)
    args = [to_dev(x[kk]) for kk in ("q", "k", "v", "A_log", "dt_bias", "a", "b")]
    p1, p2 = x["pool"].cuda(), x["pool"].cuda()
    o1, _ = gdn.decode(*args, p1, to_dev(x["read_idx"]), write_idx=to_dev(x["write_idx"]), scale=x["scale"])
    o2, _ = gdn.decode(*args, p2, to_dev(x["read_idx"]), write_idx=to_dev(x["write_idx"]), scale=x["scale"],
                       use_qk_l2norm=True, qk_l2norm_eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


@pytest.mark.parametrize("fused", [False, True])
def test_prefill_float16_inputs(fused):
    """float16 q, k, v (the ONNX card's T includes f16): the float32 path on
    exact widenings, the output rounded to float16 once."""
    x = synth.prefill_inputs(760, lengths=[70, 0, 33], hq=2, hv=4, dk=64, dv=64, dtype="f32",
                             gate="qwen", init_std=0.05)
    q, k, v = (x[n].half() for n in ("q", "k", "v"))
    kw = dict(cu_seqlens=to_dev(x["cu_seqlens"]), initial_state=to_dev(x["initial_state"]),
              scale=x["scale"])
    okw = dict(cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"], scale=x["scale"])
    if fused:
        a, b = x["a"].half(), x["b"].half()
        o, f = gdn.prefill(q.cuda(), k.cuda(), v.cuda(), None, None, A_log=to_dev(x["A_log"]),
                           dt_bias=to_dev(x["dt_bias"]), a=a.cuda(), b=b.cuda(), **kw)
        ro, rf = oracle.prefill(q, k, v, None, None, A_log=x["A_log"], dt_bias=x["dt_bias"], a=a,
                                b=b, **okw)
    else:
        g, _, beta = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
        dec, bet = torch.from_numpy(g).float(), torch.from_numpy(beta).float()
        o, f = gdn.prefill(q.cuda(), k.cuda(), v.cuda(), dec.cuda(), bet.cuda(), **kw)
        ro, rf = oracle.prefill(q, k, v, dec, bet, **okw)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    e = np.abs(o.double().cpu().numpy() - ro).max() / np.abs(ro).max()
    assert e <= 2e-3, e  # float32 arithmetic, one float16 rounding (2^-11 relative)
    assert_close(f, rf, "f32", "final state")


def test_decode_float16_inputs_go_through_bfloat16():
    x = synth.decode_inputs(761, pool_size=20, batch=5, T=3, n_hh=2, hq=2, hv=4, dk=64, dv=64,
                            dtype="f32", skip_rows=1)
    h = {n: x[n].half() for n in ("q", "k", "v", "a", "b")}
    pool = to_dev(x["pool"].clone())
    out = torch.full((5, 3, 4, 64), 3.0, dtype=torch.float16, device="cuda")
    o, _ = gdn.decode(h["q"].cuda(), h["k"].cuda(), h["v"].cuda(), to_dev(x["A_log"]),
                      to_dev(x["dt_bias"]), h["a"].cuda(), h["b"].cuda(), pool,
                      to_dev(x["read_idx"]), write_idx=to_dev(x["write_idx"]), scale=x["scale"],
                      out=out, use_qk_l2norm=False)
    # the oracle on the bfloat16 values the kernel saw
    bf = {n: t.to(torch.bfloat16) for n, t in h.items()}
    ro, rp = oracle.decode(bf["q"], bf["k"], bf["v"], x["A_log"], x["dt_bias"], bf["a"], bf["b"],
                           x["pool"], x["read_idx"], write_idx=x["write_idx"], scale=x["scale"])
    torch.cuda.synchronize()
    assert o is out and out.dtype == torch.float16
    act = (x["read_idx"] >= 0).numpy()
    assert_close(out[torch.from_numpy(act).cuda()], ro[act], "bf16", "out")
    assert torch.all(out[torch.from_numpy(~act).cuda()] == 3.0)
    assert_close(pool, rp, "bf16", "pool")
