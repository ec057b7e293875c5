"""GPU parity of gdn_gate, gdn_decode and gdn_prefill against the fp64 oracle.

Small and medium seeded cases that span several tiles, chunks and a ragged
tail, plus the edge cases of the contracts: empty and decreasing requests,
skipped rows, out-of-range slots, scatter, disable_state_update, GVA head
maps, all supported head sizes, every chunk size, aliasing of the initial and
final state, and run-to-run bitwise determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (TOL, assert_close, gpu_prefill_from, oracle_prefill_from, rel_err,
                      require_gpu, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


# ------------------------------------------------------------------- gate --

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_parity(dtype):
    import gated_deltanet_state_delta_amd as gdn
    g = torch.Generator().manual_seed(101)
    hv = 12
    A_log = torch.rand(hv, generator=g) * 4 - 1
    dt_bias = torch.randn(hv, generator=g)
    a = (torch.randn(1000, hv, generator=g) * 8).to(synth.DTYPES[dtype])
    b = (torch.randn(1000, hv, generator=g) * 8).to(synth.DTYPES[dtype])
    a[0, :4] = torch.tensor([20.0, 19.0, 21.0, 0.0])  # around the softplus threshold
    ld, gam, beta = gdn.gate(A_log.cuda(), dt_bias.cuda(), a.cuda(), b.cuda(), want_gamma=True)
    rg, rgam, rbeta = oracle.gate(A_log, dt_bias, a, b)
    assert rel_err(ld, rg) < 1e-5
    assert rel_err(gam, rgam) < 1e-5
    assert rel_err(beta, rbeta) < 1e-6
    # beta only / decay only
    _, _, beta2 = gdn.gate(A_log.cuda(), dt_bias.cuda(), None, b.cuda())
    assert torch.equal(beta2, beta)
    ld2, _, _ = gdn.gate(A_log.cuda(), dt_bias.cuda(), a.cuda(), None)
    assert torch.equal(ld2, ld)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_ragged_and_unaligned(dtype):
    """The vector path (groups of eight elements, heads stepped across rows),
    its ragged end (4 985 elements) and the element path of unaligned inputs
    (views one element into their buffers) all match the oracle."""
    import gated_deltanet_state_delta_amd as gdn
    g = torch.Generator().manual_seed(102)
    hv, n = 5, 997
    A_log = torch.rand(hv, generator=g) * 4 - 1
    dt_bias = torch.randn(hv, generator=g)
    a = (torch.randn(n, hv, generator=g) * 8).to(synth.DTYPES[dtype])
    b = (torch.randn(n, hv, generator=g) * 8).to(synth.DTYPES[dtype])
    rg, rgam, rbeta = oracle.gate(A_log, dt_bias, a, b)
    ld, gam, beta = gdn.gate(A_log.cuda(), dt_bias.cuda(), a.cuda(), b.cuda(), want_gamma=True)
    assert rel_err(ld, rg) < 1e-5 and rel_err(gam, rgam) < 1e-5 and rel_err(beta, rbeta) < 1e-6
    ua = torch.empty(n * hv + 1, dtype=a.dtype, device="cuda")[1:].view(n, hv)
    ub = torch.empty(n * hv + 1, dtype=b.dtype, device="cuda")[1:].view(n, hv)
    ua.copy_(a.cuda())
    ub.copy_(b.cuda())
    ld2, gam2, beta2 = gdn.gate(A_log.cuda(), dt_bias.cuda(), ua, ub, want_gamma=True)
    assert torch.equal(ld2, ld) and torch.equal(gam2, gam) and torch.equal(beta2, beta)


# ----------------------------------------------------------------- decode --

def _gpu_decode(x, out=None, pool=None, **kw):
    import gated_deltanet_state_delta_amd as gdn
    pool = to_dev(x["pool"]).clone() if pool is None else pool
    args = dict(write_idx=to_dev(x["write_idx"]), scatter_idx=to_dev(x["scatter_idx"]),
                scale=x["scale"], out=out, use_qk_l2norm=False)
    args.update(kw)
    return gdn.decode(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["A_log"]),
                      to_dev(x["dt_bias"]), to_dev(x["a"]), to_dev(x["b"]), pool,
                      to_dev(x["read_idx"]), **args)


def _oracle_decode(x, **kw):
    args = dict(write_idx=x["write_idx"], scatter_idx=x["scatter_idx"], scale=x["scale"])
    args.update(kw)
    return oracle.decode(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                         x["pool"], x["read_idx"], **args)


def _check_decode(x, out_g, pool_g, out_r, pool_r, dtype):
    active = (x["read_idx"] >= 0) & (x["read_idx"] < x["pool_size"])
    act = active.numpy()
    if act.any():
        assert_close(out_g[active.cuda()], out_r[act], dtype, "decode out")
    # every slot: written ones to tolerance, untouched ones bitwise
    p0 = x["pool"]
    changed = np.zeros(x["pool_size"], dtype=bool)
    for s in range(x["pool_size"]):
        if not np.array_equal(pool_r[s], p0[s].double().numpy()):
            changed[s] = True
    pg = pool_g.cpu()
    if changed.any():
        idx = torch.from_numpy(np.nonzero(changed)[0])
        assert_close(pg[idx], pool_r[changed], dtype, "decode pool")
    same = torch.from_numpy(np.nonzero(~changed)[0])
    assert torch.equal(pg[same], p0[same]), "untouched pool slots changed"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 64), (16, 128)])
def test_decode_single_token(dtype, dk, dv):
    x = synth.decode_inputs(200 + dk + dv, pool_size=24, batch=8, T=1, n_hh=1, hq=2, hv=4,
                            dk=dk, dv=dv, dtype=dtype, skip_rows=2)
    out_g, pool_g = _gpu_decode(x)
    out_r, pool_r = _oracle_decode(x)
    _check_decode(x, out_g, pool_g, out_r, pool_r, dtype)
    skipped = (x["read_idx"] < 0).cuda()
    assert torch.all(out_g[skipped] == 0), "skipped rows must keep the caller's output"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,n", [(4, 2), (3, 1), (2, 4), (7, 3)])
def test_decode_multi_token_scatter(dtype, T, n):
    x = synth.decode_inputs(300 + 10 * T + n, pool_size=64, batch=6, T=T, n_hh=n, hq=4, hv=8,
                            dk=128, dv=64, dtype=dtype, scatter=True, write_slots=False)
    sc = x["scatter_idx"].clone()
    sc[0, 0] = -1     # skip one write
    sc[1, -1] = 999   # out of range: skipped as well
    x["scatter_idx"] = sc
    out_g, pool_g = _gpu_decode(x)
    out_r, pool_r = _oracle_decode(x)
    _check_decode(x, out_g, pool_g, out_r, pool_r, dtype)


def test_decode_write_slots_disable_and_skips():
    x = synth.decode_inputs(400, pool_size=40, batch=10, T=2, n_hh=2, hq=2, hv=4, dk=64, dv=64,
                            dtype="bf16", skip_rows=3)
    rd = x["read_idx"].clone()
    wr = x["write_idx"].clone()
    active = torch.nonzero(rd >= 0).flatten()
    rd[active[0]] = 40          # out of range read -> skipped
    wr[active[1]] = -1          # no write-back, output still stored
    x["read_idx"], x["write_idx"] = rd, wr
    sentinel = torch.full((10, 2, 4, 64), 3.0, dtype=torch.bfloat16)
    out_g, pool_g = _gpu_decode(x, out=sentinel.cuda().clone())
    out_r, pool_r = _oracle_decode(x, out_init=sentinel)
    _check_decode(x, out_g, pool_g, out_r, pool_r, "bf16")
    skipped = ((rd < 0) | (rd >= 40)).cuda()
    assert torch.all(out_g[skipped] == 3.0)
    assert not torch.any(out_g[active[1]] == 3.0)
    # disable_state_update: same outputs, pool untouched
    out_d, pool_d = _gpu_decode(x, out=sentinel.cuda().clone(), disable_state_update=True)
    assert torch.equal(out_d, out_g)
    assert torch.equal(pool_d.cpu(), x["pool"])


@pytest.mark.parametrize("layout", ["transposed", "strided", "offset"])
def test_decode_into_a_non_contiguous_output(layout):
    """"flashinfer...cake_gated_delta_product_mtp", Parameters (output): the
    kernel writes a dense buffer and any other caller buffer receives a copy
    after the launch.  A transposed view, a strided slice of a larger buffer
    and an unaligned offset view all end bitwise equal to the dense output,
    and rows the call skips keep their previous contents."""
    x = synth.decode_inputs(420, pool_size=40, batch=10, T=3, n_hh=2, hq=2, hv=4, dk=64, dv=64,
                            dtype="bf16", skip_rows=3)
    sentinel = torch.full((10, 3, 4, 64), 5.0, dtype=torch.bfloat16)
    ref_out, ref_pool = _gpu_decode(x, out=sentinel.cuda().clone())
    if layout == "transposed":
        base = torch.full((10, 4, 3, 64), 5.0, dtype=torch.bfloat16, device="cuda")
        out = base.transpose(1, 2)
    elif layout == "strided":
        base = torch.full((10, 3, 4, 128), 5.0, dtype=torch.bfloat16, device="cuda")
        out = base[..., 32:96]
    else:
        base = torch.full((10 * 3 * 4 * 64 + 1,), 5.0, dtype=torch.bfloat16, device="cuda")
        out = base[1:].view(10, 3, 4, 64)
    assert not (out.is_contiguous() and out.data_ptr() % 16 == 0)
    o, pool = _gpu_decode(x, out=out)
    torch.cuda.synchronize()
    assert o is out
    assert torch.equal(out, ref_out)
    assert torch.equal(pool, ref_pool)
    skipped = (x["read_idx"] < 0).cuda()
    assert torch.all(out[skipped] == 5.0)
    if layout == "strided":
        assert torch.all(base[..., :32] == 5.0) and torch.all(base[..., 96:] == 5.0)


def test_decode_in_place_default_write_slot_and_padded_pool():
    """write_idx None writes back to the read slot; a pool with padding between
    heads and slots is used as is."""
    x = synth.decode_inputs(410, pool_size=16, batch=5, T=3, n_hh=1, hq=1, hv=3, dk=32, dv=16,
                            dtype="f32", write_slots=False, skip_rows=1)
    P, hv, dv, dk = 16, 3, 16, 32
    big = torch.full((P, hv + 1, dv + 2, dk), -9.0)
    big[:, :hv, :dv] = x["pool"]
    pool_dev = big.cuda()
    view = pool_dev[:, :hv, :dv]
    out_g, _ = _gpu_decode(x, pool=view)
    out_r, pool_r = _oracle_decode(x)
    active = (x["read_idx"] >= 0).numpy()
    assert_close(out_g[torch.from_numpy(active).cuda()], out_r[active], "f32")
    got = pool_dev.cpu()
    assert_close(got[:, :hv, :dv], pool_r, "f32", "pool")
    assert torch.all(got[:, hv] == -9.0) and torch.all(got[:, :, dv:] == -9.0), "padding touched"


def test_decode_gva_equals_repeated_heads_and_scale_zero():
    x = synth.decode_inputs(420, pool_size=12, batch=4, T=2, n_hh=2, hq=2, hv=8, dk=64, dv=32,
                            dtype="bf16")
    out_g, pool_g = _gpu_decode(x)
    x2 = dict(x)
    x2["q"] = x["q"].repeat_interleave(4, dim=2)
    x2["k"] = x["k"].repeat_interleave(4, dim=3)
    x2["hq"] = 8
    out_g2, pool_g2 = _gpu_decode(x2)
    assert torch.equal(out_g, out_g2) and torch.equal(pool_g, pool_g2)
    out0, _ = _gpu_decode(x, scale=0.0)
    assert torch.all(out0 == 0)


def test_decode_deterministic():
    x = synth.decode_inputs(430, pool_size=100, batch=16, T=4, n_hh=2, hq=4, hv=8, dk=128, dv=64,
                            dtype="bf16", scatter=True, write_slots=False)
    runs = [_gpu_decode(x) for _ in range(3)]
    for o, p in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(p, runs[0][1])


def test_decode_batch_zero_is_noop():
    import gated_deltanet_state_delta_amd as gdn
    x = synth.decode_inputs(440, pool_size=4, batch=1, T=1, n_hh=1, hq=1, hv=1, dk=16, dv=16,
                            dtype="f32")
    pool = x["pool"].cuda()
    e = lambda t: t[:0].cuda()
    out, _ = gdn.decode(e(x["q"]), e(x["k"]), e(x["v"]), x["A_log"].cuda(), x["dt_bias"].cuda(),
                        e(x["a"]), e(x["b"]), pool, e(x["read_idx"]), use_qk_l2norm=False)
    assert out.numel() == 0
    assert torch.equal(pool.cpu(), x["pool"])


# ---------------------------------------------------------------- prefill --

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 16), (128, 128), (128, 32), (16, 128)])
def test_prefill_ragged_all_head_sizes(dtype, dk, dv):
    lengths = [1, 70, 0, 16, 131, 64]
    x = synth.prefill_inputs(500 + dk + dv, lengths=lengths, hq=2, hv=4, dk=dk, dv=dv,
                             dtype=dtype, gate="gamma", gamma_range=(0.7, 1.0), init_std=0.2)
    out_g, fin_g = gpu_prefill_from(x)
    out_r, fin_r = oracle_prefill_from(x)
    assert_close(out_g, out_r, dtype, "out")
    assert_close(fin_g, fin_r, dtype, "final")
    # empty request: incoming state copied bit for bit
    assert torch.equal(fin_g[2].cpu(), x["initial_state"][2])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_prefill_chunk_sizes(dtype, chunk):
    x = synth.prefill_inputs(600, lengths=[200, 37], hq=1, hv=2, dk=128, dv=64, dtype=dtype,
                             gate="log", gamma_range=(0.5, 1.0), init_std=0.1)
    out_g, fin_g = gpu_prefill_from(x, chunk_size=chunk)
    out_r, fin_r = oracle_prefill_from(x)
    assert_close(out_g, out_r, dtype, "out")
    assert_close(fin_g, fin_r, dtype, "final")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_qwen_gates_strong_decay(dtype):
    """Workload-like gates (median gamma ~ 0.1): exercises large in-chunk log-decay ranges."""
    x = synth.prefill_inputs(610, n_seqs=2, seq_len=300, hq=2, hv=4, dk=128, dv=128, dtype=dtype,
                             gate="qwen")
    out_g, fin_g = gpu_prefill_from(x)
    out_r, fin_r = oracle_prefill_from(x)
    assert_close(out_g, out_r, dtype, "out")
    assert_close(fin_g, fin_r, dtype, "final")


def test_prefill_exact_zero_gamma():
    x = synth.prefill_inputs(620, lengths=[150], hq=1, hv=2, dk=64, dv=64, dtype="f32",
                             gate="gamma", gamma_range=(0.8, 1.0), init_std=0.5)
    gam = x["gamma"].clone()
    gam[[0, 17, 18, 63, 64, 100], 0] = 0.0
    gam[[5, 127, 128], 1] = 0.0
    x["gamma"] = gam
    out_g, fin_g = gpu_prefill_from(x)
    out_r, fin_r = oracle_prefill_from(x)
    assert_close(out_g, out_r, "f32", "out")
    assert_close(fin_g, fin_r, "f32", "final")
    # the same through the log-space input, with -inf for the zeros
    x2 = dict(x)
    x2["gate"] = "log"
    x2["log_decay"] = torch.log(gam)
    out_g2, fin_g2 = gpu_prefill_from(x2)
    assert_close(out_g2, out_r, "f32", "out(log)")
    assert_close(fin_g2, fin_r, "f32", "final(log)")


def test_prefill_cu_seqlens_clamped_decreasing_and_uncovered_rows():
    x = synth.prefill_inputs(630, lengths=[40, 40, 40], hq=1, hv=1, dk=32, dv=32, dtype="f32",
                             gate="gamma", init_std=0.3)
    T = x["T"]
    x["cu_seqlens"] = torch.tensor([-5, 30, 20, T + 100], dtype=torch.int32)  # [0,30), empty, [20,T)
    sentinel = torch.full((T, 1, 32), 11.0)
    x_a = dict(x)
    x_a["cu_seqlens"] = torch.tensor([0, 30], dtype=torch.int32)
    x_a["initial_state"] = x["initial_state"][:1]
    x_b = dict(x)
    x_b["cu_seqlens"] = torch.tensor([20, T], dtype=torch.int32)
    x_b["initial_state"] = x["initial_state"][2:]
    out_g, fin_g = gpu_prefill_from(x_a, out=sentinel.cuda().clone())
    out_r, fin_r = oracle_prefill_from(x_a)
    assert_close(out_g[:30], out_r[:30], "f32")
    assert torch.all(out_g[30:] == 11.0), "rows no request covers must not be written"
    _, fin_all = gpu_prefill_from(x)
    assert torch.equal(fin_all[1].cpu(), x["initial_state"][1])   # decreasing -> empty
    assert_close(fin_all[0], fin_r[0], "f32")
    _, fin_rb = oracle_prefill_from(x_b)
    assert_close(fin_all[2], fin_rb[0], "f32")


def test_prefill_gva_matches_repeated_heads_and_deterministic():
    x = synth.prefill_inputs(640, lengths=[100, 29], hq=2, hv=8, dk=64, dv=64, dtype="bf16",
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


def test_prefill_final_state_may_alias_initial_state():
    x = synth.prefill_inputs(650, lengths=[77, 0, 5], hq=1, hv=2, dk=128, dv=128, dtype="f32",
                             gate="gamma", init_std=0.2)
    st = x["initial_state"].cuda().clone()
    _, fin = gpu_prefill_from(x, initial_state=st, final_state=st)
    _, fin_r = oracle_prefill_from(x)
    assert fin.data_ptr() == st.data_ptr()
    assert_close(st, fin_r, "f32")


def test_prefill_split_resume_and_noncontiguous_inputs():
    x = synth.prefill_inputs(660, lengths=[190], hq=2, hv=2, dk=64, dv=32, dtype="f32",
                             gate="gamma", init_std=0.2)
    out_r, fin_r = oracle_prefill_from(x)
    n = 77
    xa = dict(x)
    xb = dict(x)
    for key in ("q", "k", "v", "gamma", "beta"):
        xa[key] = x[key][:n]
        xb[key] = x[key][n:]
    xa["cu_seqlens"] = torch.tensor([0, n], dtype=torch.int32)
    xb["cu_seqlens"] = torch.tensor([0, 190 - n], dtype=torch.int32)
    oa, fa = gpu_prefill_from(xa)
    ob, fb = gpu_prefill_from(xb, initial_state=fa)
    assert_close(torch.cat([oa, ob]), out_r, "f32", "resumed out")
    assert_close(fb, fin_r, "f32", "resumed final")
    # head-strided q/k/v views (token stride larger than heads*dim)
    import gated_deltanet_state_delta_amd as gdn
    wide_q = torch.zeros(190, 2, 96)
    wide_q[:, :, :64] = x["q"]
    wide_k = torch.zeros(190, 2, 96)
    wide_k[:, :, :64] = x["k"]
    q = wide_q.cuda()[:, :, :64]
    k = wide_k.cuda()[:, :, :64]
    o, f = gdn.prefill(q, k, x["v"].cuda(), x["gamma"].cuda(), x["beta"].cuda(),
                       decay_kind="gamma", cu_seqlens=x["cu_seqlens"].cuda(),
                       initial_state=x["initial_state"].cuda(), scale=x["scale"])
    assert_close(o, out_r, "f32", "strided out")
    assert_close(f, fin_r, "f32", "strided final")


def test_prefill_zero_tokens_writes_final_state():
    import gated_deltanet_state_delta_amd as gdn
    init = torch.randn(3, 2, 16, 32).cuda()
    e = torch.zeros(0, 1, 32).cuda()
    ev = torch.zeros(0, 2, 16).cuda()
    ed = torch.zeros(0, 2).cuda()
    cu = torch.zeros(4, dtype=torch.int32).cuda()
    out, fin = gdn.prefill(e, e, ev, ed, ed, cu_seqlens=cu, initial_state=init)
    assert out.numel() == 0 and torch.equal(fin, init)
    out, fin = gdn.prefill(e, e, ev, ed, ed, cu_seqlens=cu)
    assert torch.all(fin == 0)
