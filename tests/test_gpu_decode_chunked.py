"""gdn_decode with many tokens per row (T >= 16, one delta step per token, no
per-token scatter) runs the chunked form over the pool.  Same contract as the
token loop ("flashinfer.cake_gdp.cake_gated_delta_product_mtp", parameters):
checked against the fp64 decode oracle with skipped rows, write slots that
default to the read slots, disable_state_update, the in-kernel L2 norm, both
io dtypes and several head sizes; skipped rows keep the caller's output and
untouched slots their bits.  Rows that keep the token loop (T < 16, n > 1,
scatter) are covered by the other decode tests.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn
import synth
from gpu_util import assert_close, require_gpu, to_dev
from test_gpu_kernels import _check_decode, _gpu_decode, _oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,dk,dv", [(16, 128, 128), (17, 64, 64), (31, 128, 64), (32, 64, 128),
                                     (47, 32, 32), (64, 128, 128), (64, 16, 64)])
def test_chunked_decode_matches_oracle(dtype, T, dk, dv):
    x = synth.decode_inputs(500 + T + dk + dv, pool_size=40, batch=10, T=T, n_hh=1, hq=2, hv=4,
                            dk=dk, dv=dv, dtype=dtype, skip_rows=3, write_slots=True)
    out = torch.zeros(10, T, 4, dv, dtype=synth.DTYPES[dtype], device="cuda")
    out_g, pool_g = _gpu_decode(x, out=out)
    torch.cuda.synchronize()
    out_r, pool_r = _oracle_decode(x)
    _check_decode(x, out_g, pool_g, out_r, pool_r, dtype)
    skipped = (x["read_idx"] < 0).cuda()
    assert torch.all(out_g[skipped] == 0), "skipped rows must keep the caller's output"


@pytest.mark.parametrize("mode", ["write_is_read", "disable", "qk_l2norm"])
def test_chunked_decode_rules(mode):
    x = synth.decode_inputs(560, pool_size=30, batch=8, T=24, n_hh=1, hq=2, hv=4, dk=128, dv=128,
                            dtype="bf16", skip_rows=2, write_slots=mode != "write_is_read")
    kw = {}
    if mode == "disable":
        kw["disable_state_update"] = True
    if mode == "qk_l2norm":
        # q and k far from unit length, so a missing norm shows
        x["q"] = (x["q"].float() * 3.0).to(torch.bfloat16)
        x["k"] = (x["k"].float() * 0.3).to(torch.bfloat16)
        kw["use_qk_l2norm"] = True
        okw = dict(qk_l2norm_eps=1e-6)
    else:
        okw = dict(disable_state_update=mode == "disable")
    out_g, pool_g = _gpu_decode(x, **kw)
    torch.cuda.synchronize()
    out_r, pool_r = _oracle_decode(x, **okw)
    _check_decode(x, out_g, pool_g, out_r, pool_r, "bf16")
    if mode == "disable":
        assert torch.equal(pool_g.cpu(), x["pool"])


def test_chunked_and_token_loop_agree():
    """T = 16 (chunked) against the same rows fed to the token loop as 16
    single-token calls: the state hand-over through the pool is the same."""
    x = synth.decode_inputs(570, pool_size=20, batch=6, T=16, n_hh=1, hq=2, hv=4, dk=64, dv=64,
                            dtype="f32", write_slots=False)
    pool_a = to_dev(x["pool"]).clone()
    out_a, _ = _gpu_decode(x, pool=pool_a)
    pool_b = to_dev(x["pool"]).clone()
    outs = []
    for t in range(16):
        sl = slice(t, t + 1)
        o, _ = gdn.decode(to_dev(x["q"][:, sl]), to_dev(x["k"][:, sl]), to_dev(x["v"][:, sl]),
                          to_dev(x["A_log"]), to_dev(x["dt_bias"]), to_dev(x["a"][:, sl]),
                          to_dev(x["b"][:, sl]), pool_b, to_dev(x["read_idx"]), scale=x["scale"], use_qk_l2norm=False)
        outs.append(o)
    torch.cuda.synchronize()
    out_b = torch.cat(outs, dim=1)
    assert_close(out_a, out_b.double().cpu().numpy(), "f32", "chunked vs token loop out")
    assert_close(pool_a, pool_b.double().cpu().numpy(), "f32", "chunked vs token loop pool")
