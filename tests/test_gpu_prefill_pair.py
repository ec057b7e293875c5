"""Parity of the bf16 pair-role prefill kernel (bf16, dk and dv in {64, 128},
default chunk) with the fp64 oracle.

Every case here is routed to that kernel by gdn_prefill; chunk_size=32 routes
the same problem to the general kernel, which is checked beside it.  Lengths
are chosen to cover empty requests, single tokens, exact chunk multiples and
ragged tails, with every head-size combination the kernel instantiates.
"""
import pytest
import torch

import synth
from gpu_util import assert_close, gpu_prefill_from, oracle_prefill_from, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


LENGTHS = [1, 63, 0, 64, 65, 130, 200]


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_pair_ragged_all_shapes(dk, dv):
    x = synth.prefill_inputs(700 + dk + dv, lengths=LENGTHS, hq=2, hv=4, dk=dk, dv=dv,
                             dtype="bf16", gate="gamma", gamma_range=(0.7, 1.0), init_std=0.2)
    out_g, fin_g = gpu_prefill_from(x)
    out_r, fin_r = oracle_prefill_from(x)
    assert_close(out_g, out_r, "bf16", "out")
    assert_close(fin_g, fin_r, "bf16", "final")
    assert torch.equal(fin_g[2].cpu(), x["initial_state"][2])  # empty request copies


@pytest.mark.parametrize("gate", ["qwen", "log"])
def test_pair_packed_batches(gate):
    x = synth.prefill_inputs(710, n_seqs=3, seq_len=257, hq=2, hv=4, dk=128, dv=128, dtype="bf16",
                             gate=gate, gamma_range=(0.3, 1.0))
    out_g, fin_g = gpu_prefill_from(x)
    out_r, fin_r = oracle_prefill_from(x)
    assert_close(out_g, out_r, "bf16", "out")
    assert_close(fin_g, fin_r, "bf16", "final")


def test_pair_matches_general_kernel_within_tolerance():
    x = synth.prefill_inputs(720, lengths=[300, 90], hq=1, hv=2, dk=128, dv=128, dtype="bf16",
                             gate="log", gamma_range=(0.5, 1.0), init_std=0.1)
    out_p, fin_p = gpu_prefill_from(x, chunk_size=0)
    out_h, fin_h = gpu_prefill_from(x, chunk_size=64)
    assert torch.equal(out_p, out_h) and torch.equal(fin_p, fin_h)  # same kernel
    out_g, fin_g = gpu_prefill_from(x, chunk_size=32)                # general kernel
    out_r, fin_r = oracle_prefill_from(x)
    for o, f, what in ((out_p, fin_p, "pair"), (out_g, fin_g, "general")):
        assert_close(o, out_r, "bf16", what + " out")
        assert_close(f, fin_r, "bf16", what + " final")


def test_pair_exact_zero_gamma_gamma_and_log_inputs():
    x = synth.prefill_inputs(730, lengths=[150, 64], hq=1, hv=2, dk=64, dv=64, dtype="bf16",
                             gate="gamma", gamma_range=(0.8, 1.0), init_std=0.5)
    gam = x["gamma"].clone()
    gam[[0, 17, 18, 63, 64, 100, 149], 0] = 0.0
    gam[[5, 127, 128, 150, 213], 1] = 0.0
    x["gamma"] = gam
    out_g, fin_g = gpu_prefill_from(x)
    out_r, fin_r = oracle_prefill_from(x)
    assert_close(out_g, out_r, "bf16", "out")
    assert_close(fin_g, fin_r, "bf16", "final")
    x2 = dict(x)
    x2["gate"] = "log"
    x2["log_decay"] = torch.log(gam)
    out_g2, fin_g2 = gpu_prefill_from(x2)
    assert_close(out_g2, out_r, "bf16", "out(log)")
    assert_close(fin_g2, fin_r, "bf16", "final(log)")


def test_pair_gva_alias_and_determinism():
    x = synth.prefill_inputs(740, lengths=[100, 29, 64], hq=2, hv=8, dk=128, dv=64, dtype="bf16",
                             gate="gamma", init_std=0.1)
    o1, f1 = gpu_prefill_from(x)
    x2 = dict(x)
    x2["q"] = x["q"].repeat_interleave(4, dim=1)
    x2["k"] = x["k"].repeat_interleave(4, dim=1)
    o2, f2 = gpu_prefill_from(x2)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    for _ in range(2):
        o3, f3 = gpu_prefill_from(x)
        assert torch.equal(o3, o1) and torch.equal(f3, f1)
    st = x["initial_state"].cuda().clone()
    o4, f4 = gpu_prefill_from(x, initial_state=st, final_state=st)
    assert f4.data_ptr() == st.data_ptr()
    assert torch.equal(o4, o1) and torch.equal(st, f1)


def test_pair_split_resume_and_strided_views():
    x = synth.prefill_inputs(750, lengths=[190], hq=2, hv=2, dk=128, dv=64, dtype="bf16",
                             gate="gamma", init_std=0.2)
    out_r, fin_r = oracle_prefill_from(x)
    n = 77
    xa, xb = dict(x), dict(x)
    for key in ("q", "k", "v", "gamma", "beta"):
        xa[key] = x[key][:n]
        xb[key] = x[key][n:]
    xa["cu_seqlens"] = torch.tensor([0, n], dtype=torch.int32)
    xb["cu_seqlens"] = torch.tensor([0, 190 - n], dtype=torch.int32)
    oa, fa = gpu_prefill_from(xa)
    ob, fb = gpu_prefill_from(xb, initial_state=fa)
    assert_close(torch.cat([oa, ob]), out_r, "bf16", "resumed out")
    assert_close(fb, fin_r, "bf16", "resumed final")
    import gated_deltanet_state_delta_amd as gdn
    wq = torch.zeros(190, 2, 136, dtype=torch.bfloat16)
    wq[:, :, :128] = x["q"]
    wk = torch.zeros(190, 2, 200, dtype=torch.bfloat16)
    wk[:, :, :128] = x["k"]
    wv = torch.zeros(190, 2, 72, dtype=torch.bfloat16)
    wv[:, :, :64] = x["v"]
    out_w = torch.full((190, 2, 80), 3.0, dtype=torch.bfloat16).cuda()
    o, f = gdn.prefill(wq.cuda()[:, :, :128], wk.cuda()[:, :, :128], wv.cuda()[:, :, :64],
                       x["gamma"].cuda(), x["beta"].cuda(), decay_kind="gamma",
                       cu_seqlens=x["cu_seqlens"].cuda(), initial_state=x["initial_state"].cuda(),
                       scale=x["scale"], out=out_w[:, :, :64])
    assert_close(o, out_r, "bf16", "strided out")
    assert_close(f, fin_r, "bf16", "strided final")
    assert torch.all(out_w[:, :, 64:] == 3.0), "padding columns of the output were written"
