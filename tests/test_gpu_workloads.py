"""GPU parity on the five named workloads at their full sizes.

Each workload runs on the GPU exactly as the benchmark launches it.  The fp64
oracle then checks every output of the small workloads, and sampled
(request, value head) or (batch row) units of the large ones -- units are
independent, so a sampled unit's oracle result is exact for that unit.
Bitwise properties (skipped rows, untouched pool slots, empty requests) are
checked over the whole output.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, gpu_prefill_from, oracle_prefill_from, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _print(*a):
    print(*a, flush=True)


def oracle_prefill_units(x, units):
    """Oracle on sampled (request, value head) units, packed as one-head requests.

    Returns {(r, h): (out [len, dv], final [dv, dk])} in float64."""
    cu = x["cu_seqlens"]
    if cu is None:
        bounds = [(r * x["seq_len"], (r + 1) * x["seq_len"]) for r in range(x["n_seqs"])]
    else:
        c = cu.tolist()
        bounds = [(c[r], c[r + 1]) for r in range(len(c) - 1)]
    if x["gate"] == "qwen":
        dec_all, _, beta_all = oracle.gate(x["A_log"], x["dt_bias"], x["a"], x["b"])
        is_gamma = False
    else:
        dec_all = (x["gamma"] if x["gate"] == "gamma" else x["log_decay"]).double().numpy()
        beta_all = x["beta"].double().numpy()
        is_gamma = x["gate"] == "gamma"
    qs, ks, vs, ds, bs, inits, lens = [], [], [], [], [], [], []
    for r, h in units:
        s, e = bounds[r]
        qh = h * x["hq"] // x["hv"]
        qs.append(x["q"][s:e, qh:qh + 1])
        ks.append(x["k"][s:e, qh:qh + 1])
        vs.append(x["v"][s:e, h:h + 1])
        ds.append(torch.from_numpy(np.ascontiguousarray(dec_all[s:e, h:h + 1])))
        bs.append(torch.from_numpy(np.ascontiguousarray(beta_all[s:e, h:h + 1])))
        if x["initial_state"] is not None:
            inits.append(x["initial_state"][r:r + 1, h:h + 1])
        lens.append(e - s)
    cu_u = torch.zeros(len(units) + 1, dtype=torch.int64)
    cu_u[1:] = torch.cumsum(torch.tensor(lens), 0)
    init = torch.cat(inits) if inits else None
    out, fin = oracle.prefill(torch.cat(qs).double(), torch.cat(ks).double(),
                              torch.cat(vs).double(), torch.cat(ds), torch.cat(bs),
                              decay_is_gamma=is_gamma, cu_seqlens=cu_u, initial_state=init,
                              scale=x["scale"])
    res = {}
    for i, u in enumerate(units):
        res[u] = (out[cu_u[i]:cu_u[i + 1], 0], fin[i, 0])
    return res, bounds


def test_single_head_scan_b2_s64():
    """B=2, S=64, Dk=Dv=16 fp32: every output and the (B, Dk, Dv) final state."""
    x = synth.single_head_scan()
    out_g, fin_g = gpu_prefill_from(x)
    out_r, fin_r = oracle_prefill_from(x)
    assert_close(out_g.view(2, 64, 16), out_r.reshape(2, 64, 16), "f32", "outputs (B,S,Dv)")
    # the problem statement's final_state is (B, Dk, Dv): the transpose of the V-major state
    assert_close(fin_g[:, 0].transpose(1, 2), fin_r[:, 0].transpose(0, 2, 1), "f32", "final (B,Dk,Dv)")


def test_chunked_prefill_b4_s4096_bf16():
    x = synth.chunked_prefill_b4_s4096()
    _print("chunked prefill B4 S4096 Hq16 Hv32 d128 bf16: GPU run")
    out_g, fin_g = gpu_prefill_from(x)
    torch.cuda.synchronize()
    assert torch.isfinite(out_g).all() and torch.isfinite(fin_g).all()
    units = [(0, 0), (0, 1), (1, 17), (2, 30), (3, 31), (3, 6)]
    _print("oracle on units", units)
    ref, bounds = oracle_prefill_units(x, units)
    for (r, h), (o_r, f_r) in ref.items():
        s, e = bounds[r]
        assert_close(out_g[s:e, h], o_r, "bf16", "out r%d h%d" % (r, h))
        assert_close(fin_g[r, h], f_r, "bf16", "final r%d h%d" % (r, h))


def test_ragged_prefill_8req_f32():
    x = synth.ragged_prefill_8req()
    lengths = np.diff(x["cu_seqlens"].numpy())
    _print("ragged prefill lengths", lengths.tolist(), "total", int(lengths.sum()))
    out_g, fin_g = gpu_prefill_from(x)
    torch.cuda.synchronize()
    zero = int(np.nonzero(lengths == 0)[0][0])
    assert torch.equal(fin_g[zero].cpu(), x["initial_state"][zero]), "empty request must copy its state"
    units = [(r, h) for r in range(8) if r != zero for h in (0, 13, 31)]
    _print("oracle on", len(units), "units")
    ref, bounds = oracle_prefill_units(x, units)
    for (r, h), (o_r, f_r) in ref.items():
        s, e = bounds[r]
        assert_close(out_g[s:e, h], o_r, "f32", "out r%d h%d" % (r, h))
        assert_close(fin_g[r, h], f_r, "f32", "final r%d h%d" % (r, h))


def _run_decode(x, pool_dev, out=None):
    import gated_deltanet_state_delta_amd as gdn
    return gdn.decode(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["A_log"]),
                      to_dev(x["dt_bias"]), to_dev(x["a"]), to_dev(x["b"]), pool_dev,
                      to_dev(x["read_idx"]), write_idx=to_dev(x["write_idx"]),
                      scatter_idx=to_dev(x["scatter_idx"]), scale=x["scale"], out=out)


def test_decode_pool1024_b256_bf16():
    x = synth.decode_pool_b256()
    pool0 = x["pool"]
    _print("decode pool [1024,32,128,128] B256: GPU run")
    pool_dev = pool0.cuda()
    out_g, _ = _run_decode(x, pool_dev)
    torch.cuda.synchronize()
    rd, wr = x["read_idx"], x["write_idx"]
    skipped = rd < 0
    assert int(skipped.sum()) == 26
    assert torch.all(out_g[skipped.cuda()] == 0)
    # slots: written = write slots of active rows; everything else bitwise unchanged
    written = torch.zeros(1024, dtype=torch.bool)
    written[wr[~skipped].long()] = True
    pool_after = pool_dev.cpu()
    assert torch.equal(pool_after[~written], pool0[~written]), "unwritten slots changed"
    # oracle on sampled rows (compact pool of their slots)
    act = torch.nonzero(~skipped).flatten()
    rows = torch.cat([act[:20], torch.nonzero(skipped).flatten()[:4]])
    slots = torch.unique(torch.cat([rd[rows][rd[rows] >= 0], wr[rows]]).long())
    remap = {int(s): i for i, s in enumerate(slots)}
    rd_c = torch.tensor([remap.get(int(s), -1) if s >= 0 else -1 for s in rd[rows]])
    wr_c = torch.tensor([remap[int(s)] for s in wr[rows]])
    sel = lambda t: t[rows]
    out_r, pool_r = oracle.decode(sel(x["q"]), sel(x["k"]), sel(x["v"]), x["A_log"],
                                  x["dt_bias"], sel(x["a"]), sel(x["b"]), pool0[slots], rd_c,
                                  write_idx=wr_c, scale=x["scale"])
    m = (rd_c >= 0).numpy()
    assert_close(out_g[rows.cuda()][torch.from_numpy(m).cuda()], out_r[m], "bf16", "out")
    for i, rrow in enumerate(rows.tolist()):
        if rd[rrow] >= 0:
            w = int(wr[rrow])
            assert_close(pool_after[w], pool_r[remap[w]], "bf16", "written slot %d" % w)


def test_mtp_decode_b64_t4_n2_bf16():
    x = synth.mtp_decode_b64_t4()
    _print("MTP decode B64 T4 n2 H16 Dk128 Dv64: GPU run")
    pool_dev = x["pool"].cuda()
    out_g, _ = _run_decode(x, pool_dev)
    torch.cuda.synchronize()
    out_r, pool_r = oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"],
                                  x["b"], x["pool"], x["read_idx"],
                                  scatter_idx=x["scatter_idx"], scale=x["scale"])
    assert_close(out_g, out_r, "bf16", "out")
    pool_after = pool_dev.cpu()
    sc = x["scatter_idx"].flatten().long()
    assert_close(pool_after[sc], pool_r[sc.numpy()], "bf16", "scattered states")
    untouched = torch.ones(512, dtype=torch.bool)
    untouched[sc] = False
    assert torch.equal(pool_after[untouched], x["pool"][untouched])


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("idx", [0, 1, 2])
def test_worked_examples_through_the_kernel(idx, dtype):
    """The three worked examples of "Gated DeltaNet State Update" (Examples),
    through gdn.state_update (one prefill launch, head sizes zero-padded to
    16): the printed outputs and (B, Dk, Dv) final states.  Every printed
    value is a small integer, exact in bf16 as well."""
    import gated_deltanet_state_delta_amd as gdn
    ex = json.load(open(GOLDEN))["examples"][idx]
    t = {n: torch.tensor(ex[n], dtype=torch.float32, device="cuda")
         for n in ("q", "k", "v", "gamma", "beta")}
    res = gdn.state_update(t["q"].to(dtype), t["k"].to(dtype), t["v"].to(dtype), t["gamma"],
                           t["beta"])
    torch.cuda.synchronize()
    assert res["outputs"].dtype == dtype and res["final_state"].dtype == dtype
    want_o = torch.tensor(ex["outputs"], dtype=torch.float64)
    want_f = torch.tensor(ex["final_state"], dtype=torch.float64)
    assert tuple(res["outputs"].shape) == tuple(want_o.shape)
    assert tuple(res["final_state"].shape) == tuple(want_f.shape)
    np.testing.assert_allclose(res["outputs"].double().cpu().numpy(), want_o.numpy(), atol=1e-5)
    np.testing.assert_allclose(res["final_state"].double().cpu().numpy(), want_f.numpy(), atol=1e-5)


@pytest.mark.parametrize("dk,dv", [(5, 3), (16, 16), (40, 100)])
def test_state_update_interface_against_the_oracle(dk, dv):
    """Random (B, S, D) inputs of the problem statement's interface, odd head
    sizes included (zero-padded), against the oracle; inputs unmodified."""
    import gated_deltanet_state_delta_amd as gdn
    g = torch.Generator().manual_seed(700 + dk + dv)
    B, S = 3, 77
    q = torch.randn(B, S, dk, generator=g)
    k = torch.randn(B, S, dk, generator=g)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(B, S, dv, generator=g)
    gam = torch.rand(B, S, generator=g) * 0.2 + 0.8
    bet = torch.rand(B, S, generator=g)
    args = [t.cuda() for t in (q, k, v, gam, bet)]
    copies = [t.clone() for t in args]
    res = gdn.state_update(*args)
    torch.cuda.synchronize()
    for a, c in zip(args, copies):
        assert torch.equal(a, c), "inputs must not be modified"
    ro, rf = oracle.prefill(q.reshape(B * S, 1, dk), k.reshape(B * S, 1, dk),
                            v.reshape(B * S, 1, dv), gam.reshape(B * S, 1), bet.reshape(B * S, 1),
                            decay_is_gamma=True, n_seqs=B, seq_len=S, scale=1.0)
    assert_close(res["outputs"], ro.reshape(B, S, dv), "f32", "outputs")
    assert_close(res["final_state"], rf[:, 0].transpose(0, 2, 1), "f32", "final (B,Dk,Dv)")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_onnx_js_example_shapes(dtype):
    """The shapes of the ONNX card's JS usage example ("Use with
    @huggingface/kernels": 4 tokens, one query head of 12, two value heads
    of 9, an initial state [1, 2, 9, 12]; the page gives no values): seeded
    values, head sizes zero-padded in the binding, against the oracle."""
    import gated_deltanet_state_delta_amd as gdn
    g = torch.Generator().manual_seed(710)
    dt = synth.DTYPES[dtype]
    q = torch.randn(4, 1, 12, generator=g).to(dt)
    k = torch.nn.functional.normalize(torch.randn(4, 1, 12, generator=g), dim=-1).to(dt)
    v = torch.randn(4, 2, 9, generator=g).to(dt)
    decay = -torch.rand(4, 2, generator=g)
    beta = torch.rand(4, 2, generator=g)
    init = torch.randn(1, 2, 9, 12, generator=g) * 0.1
    o, f = gdn.prefill(q.cuda(), k.cuda(), v.cuda(), decay.cuda(), beta.cuda(),
                       initial_state=init.cuda())
    torch.cuda.synchronize()
    assert tuple(o.shape) == (4, 2, 9) and tuple(f.shape) == (1, 2, 9, 12)
    ro, rf = oracle.prefill(q, k, v, decay, beta, initial_state=init, n_seqs=1, seq_len=4,
                            scale=1.0 / math.sqrt(12))
    assert_close(o, ro, dtype, "outputs")
    assert_close(f, rf, dtype, "final state")
