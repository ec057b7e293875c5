"""GPU parity on the five named workloads at their full sizes.

Each workload runs on the GPU exactly as the benchmark launches it.  The fp64
oracle then checks every output and every written state of each workload:
the whole tensors (error normalised by the tensor's max-abs) and each
independent unit -- (request, value head) for prefill, batch row for decode --
against its own oracle values.  Bitwise properties (skipped rows, untouched
pool slots, empty requests) are checked over the whole output.  The achieved
errors are printed and, with GDN_PARITY_REPORT set to a path, written there.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_close, gpu_prefill_from, oracle_prefill_from, rel_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _print(*a):
    print(*a, flush=True)


def _report(name, errs):
    """Print the achieved errors of one workload and, when GDN_PARITY_REPORT
    names a file, merge them into that JSON file (the margins below the
    tolerance are recorded from it)."""
    _print(name, json.dumps(errs))
    path = os.environ.get("GDN_PARITY_REPORT")
    if path:
        try:
            cur = json.load(open(path))
        except (OSError, ValueError):
            cur = {}
        cur[name] = errs
        with open(path, "w") as f:
            json.dump(cur, f, indent=1, sort_keys=True)


def _unit_errors(out_g, fin_g, out_r, fin_r, bounds, hv, dtype):
    """Per (request, value head) unit: the normalised max error of its outputs
    and of its final state, each against that unit's own oracle tensor.
    Returns (worst output error, worst state error, units checked)."""
    og = out_g.double().cpu().numpy()
    fg = fin_g.double().cpu().numpy()
    worst_o = worst_f = 0.0
    n = 0
    for r, (s, e) in enumerate(bounds):
        for h in range(hv):
            if e > s:
                eo = rel_err(og[s:e, h], out_r[s:e, h])
                assert eo <= TOL[dtype], "out r%d h%d: normalised max error %.3e" % (r, h, eo)
                worst_o = max(worst_o, eo)
            ef = rel_err(fg[r, h], fin_r[r, h])
            assert ef <= TOL[dtype], "final r%d h%d: normalised max error %.3e" % (r, h, ef)
            worst_f = max(worst_f, ef)
            n += 1
    return worst_o, worst_f, n


def _bounds(x):
    if x["cu_seqlens"] is None:
        return [(r * x["seq_len"], (r + 1) * x["seq_len"]) for r in range(x["n_seqs"])]
    c = x["cu_seqlens"].tolist()
    T = x["T"]
    return [(min(max(c[r], 0), T), max(min(max(c[r], 0), T), min(max(c[r + 1], 0), T)))
            for r in range(len(c) - 1)]


def test_single_head_scan_b2_s64():
    """B=2, S=64, Dk=Dv=16 fp32: every output and the (B, Dk, Dv) final state."""
    x = synth.single_head_scan()
    out_g, fin_g = gpu_prefill_from(x)
    out_r, fin_r = oracle_prefill_from(x)
    eo = assert_close(out_g.view(2, 64, 16), out_r.reshape(2, 64, 16), "f32", "outputs (B,S,Dv)")
    # the problem statement's final_state is (B, Dk, Dv): the transpose of the V-major state
    ef = assert_close(fin_g[:, 0].transpose(1, 2), fin_r[:, 0].transpose(0, 2, 1), "f32",
                      "final (B,Dk,Dv)")
    _report("single_head_scan_b2_s64_d16_f32", {"tol": TOL["f32"], "out": eo, "final_state": ef})


def test_chunked_prefill_b4_s4096_bf16():
    """All 128 (request, value head) units of B4 x S4096 (Hq16, Hv32, d128,
    bf16, qwen gates through gdn_gate) against the oracle, every output and
    every final-state element: the whole tensors and each unit on its own."""
    x = synth.chunked_prefill_b4_s4096()
    _print("chunked prefill B4 S4096 Hq16 Hv32 d128 bf16: GPU run")
    out_g, fin_g = gpu_prefill_from(x)
    torch.cuda.synchronize()
    assert torch.isfinite(out_g).all() and torch.isfinite(fin_g).all()
    _print("oracle on all 128 units")
    out_r, fin_r = oracle_prefill_from(x)
    eo = assert_close(out_g, out_r, "bf16", "outputs")
    ef = assert_close(fin_g, fin_r, "bf16", "final states")
    wo, wf, n = _unit_errors(out_g, fin_g, out_r, fin_r, _bounds(x), x["hv"], "bf16")
    assert n == 128
    _report("chunked_prefill_b4_s4096_hv32_d128_bf16",
            {"tol": TOL["bf16"], "out": eo, "final_state": ef, "units": n,
             "worst_unit_out": wo, "worst_unit_final_state": wf})


def test_ragged_prefill_8req_f32():
    """All 8 x 32 (request, value head) units of the ragged fp32 workload with
    initial states against the oracle; the empty request's state bitwise."""
    x = synth.ragged_prefill_8req()
    lengths = np.diff(x["cu_seqlens"].numpy())
    _print("ragged prefill lengths", lengths.tolist(), "total", int(lengths.sum()))
    out_g, fin_g = gpu_prefill_from(x)
    torch.cuda.synchronize()
    zero = int(np.nonzero(lengths == 0)[0][0])
    assert torch.equal(fin_g[zero].cpu(), x["initial_state"][zero]), "empty request must copy its state"
    _print("oracle on all 256 units")
    out_r, fin_r = oracle_prefill_from(x)
    eo = assert_close(out_g, out_r, "f32", "outputs")
    ef = assert_close(fin_g, fin_r, "f32", "final states")
    wo, wf, n = _unit_errors(out_g, fin_g, out_r, fin_r, _bounds(x), x["hv"], "f32")
    assert n == 256
    _report("ragged_prefill_8req_hv32_d128_f32",
            {"tol": TOL["f32"], "out": eo, "final_state": ef, "units": n, "tokens": int(lengths.sum()),
             "worst_unit_out": wo, "worst_unit_final_state": wf})


def _run_decode(x, pool_dev, out=None):
    import gated_deltanet_state_delta_amd as gdn
    return gdn.decode(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["A_log"]),
                      to_dev(x["dt_bias"]), to_dev(x["a"]), to_dev(x["b"]), pool_dev,
                      to_dev(x["read_idx"]), write_idx=to_dev(x["write_idx"]),
                      scatter_idx=to_dev(x["scatter_idx"]), scale=x["scale"], out=out, use_qk_l2norm=False)


def test_decode_pool1024_b256_bf16():
    """Every active row (230 of 256) of the pool-1024 decode against the
    oracle, in batches of rows over a compacted pool of their slots: each
    row's outputs and the state it wrote.  Skipped rows and every slot no
    active row writes are compared bitwise with their contents before."""
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
    del pool_dev
    assert torch.equal(pool_after[~written], pool0[~written]), "unwritten slots changed"
    out_gc = out_g.cpu()
    act = torch.nonzero(~skipped).flatten()
    assert act.numel() == 230
    # the whole tensors' normalisers, so the per-tensor error is over all rows
    worst_row_out = worst_row_state = 0.0
    d_out = d_state = 0.0
    m_out = m_state = 0.0
    for b0 in range(0, act.numel(), 58):
        rows = act[b0:b0 + 58]
        slots = torch.unique(torch.cat([rd[rows], wr[rows]]).long())
        remap = {int(s): i for i, s in enumerate(slots)}
        rd_c = torch.tensor([remap[int(s)] for s in rd[rows]])
        wr_c = torch.tensor([remap[int(s)] for s in wr[rows]])
        sel = lambda t: t[rows]
        out_r, pool_r = oracle.decode(sel(x["q"]), sel(x["k"]), sel(x["v"]), x["A_log"],
                                      x["dt_bias"], sel(x["a"]), sel(x["b"]), pool0[slots], rd_c,
                                      write_idx=wr_c, scale=x["scale"])
        og = out_gc[rows].double().numpy()
        d_out = max(d_out, float(np.abs(og - out_r).max()))
        m_out = max(m_out, float(np.abs(out_r).max()))
        for i, rrow in enumerate(rows.tolist()):
            e = rel_err(og[i], out_r[i])
            assert e <= TOL["bf16"], "out row %d: normalised max error %.3e" % (rrow, e)
            worst_row_out = max(worst_row_out, e)
            w = int(wr[rrow])
            sg = pool_after[w].double().numpy()
            sr = pool_r[remap[w]]
            e = rel_err(sg, sr)
            assert e <= TOL["bf16"], "state of row %d (slot %d): normalised max error %.3e" % (rrow, w, e)
            worst_row_state = max(worst_row_state, e)
            d_state = max(d_state, float(np.abs(sg - sr).max()))
            m_state = max(m_state, float(np.abs(sr).max()))
        _print("rows %d..%d checked" % (b0, b0 + rows.numel() - 1))
    eo, es = d_out / m_out, d_state / m_state
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)
    _report("decode_pool1024_b256_hv32_d128_bf16",
            {"tol": TOL["bf16"], "out": eo, "written_states": es, "rows": int(act.numel()),
             "worst_row_out": worst_row_out, "worst_row_state": worst_row_state})


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
