"""The Python binding's argument marshalling, on the CPU (no library call).

The kernels trust the sizes and strides in the argument structs, so every
struct the binding builds must describe memory inside the tensors it points
at.  For each pointer we compute the furthest element the kernel can touch
from the struct's sizes and strides and compare it with the tensor's storage.
Includes the benchmark's exact shapes (a 4-D output buffer), which once
reached the prefill kernel with batch/sequence strides in place of
token/head strides.
"""
import pytest
import torch

import gated_deltanet_state_delta_amd as gdn


def _span_ok(ptr, max_elem, t):
    """ptr + max_elem (elements of t's dtype) lies inside t's storage."""
    base = t.untyped_storage().data_ptr()
    end = base + t.untyped_storage().nbytes()
    last = ptr + (max_elem + 1) * t.element_size()
    return base <= ptr and last <= end


def _check_prefill(a, keep, T):
    q3, k3, v3, decay, beta, cu, init, out3, fin, A_log, dt_bias, ga, gb = keep[:13]
    last_q = (T - 1) * a.q_stride_token + (a.hq - 1) * a.q_stride_head + a.dk - 1
    last_k = (T - 1) * a.k_stride_token + (a.hq - 1) * a.k_stride_head + a.dk - 1
    last_v = (T - 1) * a.v_stride_token + (a.hv - 1) * a.v_stride_head + a.dv - 1
    last_o = (T - 1) * a.out_stride_token + (a.hv - 1) * a.out_stride_head + a.dv - 1
    assert _span_ok(a.q, last_q, q3)
    assert _span_ok(a.k, last_k, k3)
    assert _span_ok(a.v, last_v, v3)
    assert _span_ok(a.out, last_o, out3)
    if a.gate_a:
        assert not a.decay and not a.beta
        assert _span_ok(a.gate_a, T * a.hv - 1, ga) and _span_ok(a.gate_b, T * a.hv - 1, gb)
        assert _span_ok(a.A_log, a.hv - 1, A_log) and _span_ok(a.dt_bias, a.hv - 1, dt_bias)
    else:
        assert _span_ok(a.decay, T * a.hv - 1, decay)
        assert _span_ok(a.beta, T * a.hv - 1, beta)
    assert _span_ok(a.final_state, a.n_seqs * a.hv * a.dv * a.dk - 1, fin)
    if a.initial_state:
        assert _span_ok(a.initial_state, a.n_seqs * a.hv * a.dv * a.dk - 1, init)
    if a.cu_seqlens:
        assert _span_ok(a.cu_seqlens, a.n_seqs, cu)
    else:
        assert a.n_seqs * a.seq_len == T


def test_bench_prefill_shapes_with_4d_out():
    B, S, hq, hv, d = 4, 4096, 16, 32, 128
    q = torch.zeros(B, S, hq, d, dtype=torch.bfloat16)
    k = torch.zeros_like(q)
    v = torch.zeros(B, S, hv, d, dtype=torch.bfloat16)
    g = torch.zeros(B * S, hv)
    out = torch.empty_like(v)
    fin = torch.empty(B, hv, d, d)
    a, keep, o, f = gdn.prefill_args(q, k, v, g.view(B, S, hv), g.view(B, S, hv), out=out,
                                     final_state=fin)
    assert o is out and f is fin
    assert (a.out_stride_token, a.out_stride_head) == (hv * d, d)
    assert (a.q_stride_token, a.q_stride_head) == (hq * d, d)
    assert (a.n_seqs, a.seq_len, a.total_tokens) == (B, S, B * S)
    _check_prefill(a, keep, B * S)


@pytest.mark.parametrize("form", ["packed3", "batched4", "ragged", "strided"])
def test_prefill_struct_in_bounds(form):
    T, hq, hv, dk, dv = 96, 2, 4, 64, 32
    g = torch.zeros(T, hv)
    kw = {}
    if form == "batched4":
        q = torch.zeros(3, 32, hq, dk)
        v = torch.zeros(3, 32, hv, dv)
    elif form == "strided":
        q = torch.zeros(T, hq, dk + 32)[:, :, :dk]
        v = torch.zeros(T, hv + 1, dv)[:, 1:]
    else:
        q = torch.zeros(T, hq, dk)
        v = torch.zeros(T, hv, dv)
    if form == "ragged":
        kw["cu_seqlens"] = torch.tensor([0, 10, 10, 96])
        kw["initial_state"] = torch.zeros(3, hv, dv, dk)
    a, keep, o, f = gdn.prefill_args(q, q.clone() if form != "strided" else q, v, g, g, **kw)
    _check_prefill(a, keep, T)
    assert tuple(o.shape) == ((3, 32, hv, dv) if form == "batched4" else (T, hv, dv))


BAD_PREFILL = [
    dict(out=torch.empty(96, 4, 16)),                 # wrong dv
    dict(out=torch.empty(2, 48, 4, 32)),              # 4-D out for a 3-D call
    dict(final_state=torch.empty(1, 4, 32, 32)),      # wrong dk
    dict(initial_state=torch.empty(2, 4, 32, 64)),    # wrong n_seqs
    dict(decay=torch.zeros(95, 4)),
    dict(beta=torch.zeros(96, 3)),
    dict(out=torch.empty(96, 4, 32, dtype=torch.bfloat16)),  # dtype
]


@pytest.mark.parametrize("bad", BAD_PREFILL)
def test_prefill_rejects_bad_shapes(bad):
    T, hq, hv, dk, dv = 96, 2, 4, 64, 32
    args = dict(q=torch.zeros(T, hq, dk), k=torch.zeros(T, hq, dk), v=torch.zeros(T, hv, dv),
                decay=torch.zeros(T, hv), beta=torch.zeros(T, hv))
    kw = {}
    for key, val in bad.items():
        (args if key in args else kw)[key] = val
    with pytest.raises(ValueError):
        gdn.prefill_args(args["q"], args["k"], args["v"], args["decay"], args["beta"], **kw)


def _dec(B=8, T=2, n=2, hq=2, hv=4, dk=64, dv=32, P=20):
    return dict(q=torch.zeros(B, T, hq, dk, dtype=torch.bfloat16),
                k=torch.zeros(B, T, n, hq, dk, dtype=torch.bfloat16),
                v=torch.zeros(B, T, n, hv, dv, dtype=torch.bfloat16),
                A_log=torch.zeros(hv), dt_bias=torch.zeros(hv),
                a=torch.zeros(B, T, hv, dtype=torch.bfloat16),
                b=torch.zeros(B, T, n, hv, dtype=torch.bfloat16),
                pool=torch.zeros(P, hv, dv, dk), read_idx=torch.zeros(B, dtype=torch.int64))


def test_decode_l2norm_default_follows_flashinfer():
    """use_qk_l2norm defaults to True (eps 1e-6) in the decode binding, as on
    the FlashInfer page; False clears the struct's flag."""
    x = _dec(B=2, T=1, n=1, hq=2, hv=4, dk=64, dv=64, P=4)
    d, _, _ = gdn.decode_args(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                              x["pool"], x["read_idx"])
    assert d.qk_l2norm == 1 and abs(d.qk_l2norm_eps - 1e-6) < 1e-12
    d, _, _ = gdn.decode_args(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                              x["pool"], x["read_idx"], use_qk_l2norm=False)
    assert d.qk_l2norm == 0


def test_decode_struct_in_bounds_bench_shapes():
    x = _dec(B=256, T=1, n=1, hq=16, hv=32, dk=128, dv=128, P=8)
    out = torch.zeros(256, 1, 32, 128, dtype=torch.bfloat16)
    d, keep, o = gdn.decode_args(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"],
                                 x["b"], x["pool"], x["read_idx"],
                                 write_idx=torch.zeros(256, dtype=torch.int32), out=out, use_qk_l2norm=False)
    assert o is out
    P = x["pool"]
    last = (d.pool_size - 1) * d.pool_slot_stride + (d.hv - 1) * d.pool_head_stride + d.dv * d.dk - 1
    assert _span_ok(d.pool, last, P)
    assert _span_ok(d.out, d.batch * d.T * d.hv * d.dv - 1, out)


BAD_DECODE = [
    ("out", torch.zeros(8, 2, 4, 16, dtype=torch.bfloat16)),
    ("pool", torch.zeros(20, 4, 32, 32)),
    ("a", torch.zeros(8, 2, 3, dtype=torch.bfloat16)),
    ("b", torch.zeros(8, 2, 1, 4, dtype=torch.bfloat16)),
    ("read_idx", torch.zeros(7, dtype=torch.int32)),
    ("write_idx", torch.zeros(9, dtype=torch.int32)),
    ("scatter_idx", torch.zeros(8, 3, dtype=torch.int32)),
    ("A_log", torch.zeros(5)),
]


@pytest.mark.parametrize("key,val", BAD_DECODE)
def test_decode_rejects_bad_shapes(key, val):
    x = _dec()
    kw = {}
    if key in x:
        x[key] = val
    else:
        kw[key] = val
    with pytest.raises(ValueError):
        gdn.decode_args(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"], x["b"],
                        x["pool"], x["read_idx"], **kw)


def test_fused_gate_and_norm_arguments():
    """The fused-gate form: [B, S, hv] a/b in q's dtype, decay and beta None;
    the norm flag and epsilon reach the struct."""
    B, S, hq, hv, d = 2, 48, 2, 4, 64
    q = torch.zeros(B, S, hq, d, dtype=torch.bfloat16)
    v = torch.zeros(B, S, hv, d, dtype=torch.bfloat16)
    ab = torch.zeros(B, S, hv, dtype=torch.bfloat16)
    A = torch.zeros(hv)
    a, keep, o, f = gdn.prefill_args(q, q, v, None, None, A_log=A, dt_bias=A, a=ab, b=ab.clone(),
                                     qk_l2norm=True, qk_l2norm_eps=1e-12)
    assert a.qk_l2norm == 1 and abs(a.qk_l2norm_eps - 1e-12) < 1e-18
    _check_prefill(a, keep, B * S)
    with pytest.raises(ValueError):
        gdn.prefill_args(q, q, v, None, None)                        # no gates at all
    with pytest.raises(ValueError):
        gdn.prefill_args(q, q, v, None, None, A_log=A, dt_bias=A, a=ab.float(), b=ab.float())


def _conv(T=40, C=64, K=4, n=3, P=5, dtype=torch.bfloat16):
    x = torch.randn(T, C).to(dtype)
    w = torch.randn(C, K).to(dtype)
    st = torch.randn(P, C, K - 1).to(dtype) if K > 1 else None
    sl = torch.tensor(list(range(n)), dtype=torch.int64)
    off = torch.tensor([0] + [T * (i + 1) // n for i in range(n)], dtype=torch.int64)
    return x, w, st, sl, off


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("K", [1, 4, 8])
def test_conv1d_struct_in_bounds(dtype, K):
    x, w, st, sl, off = _conv(K=K, dtype=dtype)
    # x as a column slice of a wider buffer: passed in place with its row stride
    wide = torch.zeros(x.shape[0], x.shape[1] + 16, dtype=dtype)
    wide[:, 8:8 + x.shape[1]] = x
    xv = wide[:, 8:8 + x.shape[1]]
    a, keep, out = gdn.conv1d_args(xv, w, st, sl, off)
    x2, w2, slots, offs = keep
    T, C = a.total_tokens, a.conv_dim
    assert (T, C, a.kernel_size, a.n_seqs) == (40, 64, K, 3)
    assert a.x_stride_token == x2.stride(0) and a.out_stride_token == out.stride(0)
    assert _span_ok(a.x, (T - 1) * a.x_stride_token + C - 1, x2)
    assert _span_ok(a.out, (T - 1) * a.out_stride_token + C - 1, out)
    assert _span_ok(a.weight, C * K - 1, w2)
    if K > 1:
        assert a.max_slots == st.shape[0]
        assert _span_ok(a.conv_state, a.max_slots * C * (K - 1) - 1, st)
    else:
        assert not a.conv_state
    assert _span_ok(a.slot_idx, a.n_seqs - 1, slots) and _span_ok(a.row_offsets, a.n_seqs, offs)


def test_conv1d_index_marshalling():
    """Indices reach the C ABI as the uint32 values the page's dtype holds:
    int64 negatives become 0xFFFFFFFF (slots: outside every pool) or 0
    (offsets), values past 2^32 - 1 are clamped, int32 passes bit for bit."""
    x, w, st, _, _ = _conv()
    sl = torch.tensor([-1, 2, 2**33], dtype=torch.int64)
    off = torch.tensor([-5, 10, 2**32 + 7, 40], dtype=torch.int64)
    a, (x2, w2, slots, offs), out = gdn.conv1d_args(x, w, st, sl, off)
    assert slots.dtype == torch.int32 and offs.dtype == torch.int32
    assert [v & 0xFFFFFFFF for v in slots.tolist()] == [0xFFFFFFFF, 2, 0xFFFFFFFF]
    assert [v & 0xFFFFFFFF for v in offs.tolist()] == [0, 10, 0xFFFFFFFF, 40]
    s32 = torch.tensor([-1, 0, 7], dtype=torch.int32)
    _, (_, _, slots32, _), _ = gdn.conv1d_args(x, w, st, s32, off)
    assert slots32.tolist() == [-1, 0, 7]


@pytest.mark.parametrize("bad", ["weight_shape", "weight_dtype", "state_shape", "state_dtype",
                                 "state_missing", "offsets_len", "x_3d", "out_shape"])
def test_conv1d_rejects_bad_shapes(bad):
    x, w, st, sl, off = _conv()
    kw = {}
    if bad == "weight_shape":
        w = torch.randn(63, 4).to(x.dtype)
    elif bad == "weight_dtype":
        w = w.float()
    elif bad == "state_shape":
        st = torch.randn(5, 64, 4).to(x.dtype)
    elif bad == "state_dtype":
        st = st.float()
    elif bad == "state_missing":
        st = None
    elif bad == "offsets_len":
        off = off[:-1]
    elif bad == "x_3d":
        x = x.view(40, 8, 8)
    elif bad == "out_shape":
        kw["out"] = torch.empty(40, 32, dtype=x.dtype)
    with pytest.raises(ValueError):
        gdn.conv1d_args(x, w, st, sl, off, **kw)


@pytest.mark.parametrize("rule,use_d,use_b", [("gated_delta", True, True), ("gated", True, False),
                                              ("delta", False, True), ("linear", False, False)])
@pytest.mark.parametrize("fused", [False, True])
def test_prefill_rule_inputs(rule, use_d, use_b, fused):
    T, hq, hv, dk, dv = 20, 2, 4, 64, 64
    q = torch.randn(T, hq, dk).to(torch.bfloat16)
    k = torch.randn(T, hq, dk).to(torch.bfloat16)
    v = torch.randn(T, hv, dv).to(torch.bfloat16)
    kw = dict(update_rule=rule)
    dec = bet = None
    if fused:
        if use_d:
            kw.update(A_log=torch.zeros(hv), dt_bias=torch.zeros(hv),
                      a=torch.randn(T, hv).to(torch.bfloat16))
        if use_b:
            kw["b"] = torch.randn(T, hv).to(torch.bfloat16)
    else:
        dec = -torch.rand(T, hv) if use_d else None
        bet = torch.rand(T, hv) if use_b else None
    a, keep, out, fin = gdn.prefill_args(q, k, v, dec, bet, **kw)
    assert a.update_rule == gdn.RULES[rule]
    assert bool(a.decay) == (use_d and not fused) and bool(a.beta) == (use_b and not fused)
    assert bool(a.gate_a) == (use_d and fused) and bool(a.gate_b) == (use_b and fused)
    assert bool(a.A_log) == bool(a.gate_a) and bool(a.dt_bias) == bool(a.gate_a)
    # the rule's missing input, or an input it does not take, is refused
    with pytest.raises(ValueError):
        gdn.prefill_args(q, k, v, None if use_d else -torch.rand(T, hv), bet if not fused else None,
                         update_rule=rule)


def test_prefill_mixed_sources_and_unknown_rule():
    """Each gate input is given or fused on its own ("com.microsoft.GatedDeltaNet",
    Attributes): a with beta, and decay with b, build the struct with one
    fused and one given pointer; one input given both ways is refused."""
    T, hv = 8, 2
    q = torch.randn(T, 1, 16)
    v = torch.randn(T, hv, 16)
    args, *_ = gdn.prefill_args(q, q, v, None, torch.rand(T, hv), A_log=torch.zeros(hv),
                                dt_bias=torch.zeros(hv), a=torch.randn(T, hv))
    assert args.gate_a and args.beta and not args.decay and not args.gate_b
    args, *_ = gdn.prefill_args(q, q, v, -torch.rand(T, hv), None, b=torch.randn(T, hv))
    assert args.decay and args.gate_b and not args.beta and not args.gate_a
    with pytest.raises(ValueError):
        gdn.prefill_args(q, q, v, -torch.rand(T, hv), torch.rand(T, hv), A_log=torch.zeros(hv),
                         dt_bias=torch.zeros(hv), a=torch.randn(T, hv))
    with pytest.raises(ValueError):
        gdn.prefill_args(q, q, v, -torch.rand(T, hv), torch.rand(T, hv), b=torch.randn(T, hv))
    with pytest.raises(ValueError):
        gdn.prefill_args(q, q, v, -torch.rand(T, hv), torch.rand(T, hv), update_rule="mamba")


def test_int64_slot_and_offset_narrowing():
    """int64 slot indices outside the int32 range must not wrap onto a valid
    slot (2^32 + 3 would become 3 under a plain cast): they reach the C ABI as
    -1, which the slot rules ("flashinfer...cake_gated_delta_product_mtp",
    Parameters) read as skip, as they read the original value.  int64
    cu_seqlens are clamped to the int32 range, which the kernels' clamp to
    [0, total_tokens] ("com.microsoft.GatedDeltaNet", Inputs) maps to the
    same request bounds."""
    x = _dec(B=6)
    rd = torch.tensor([2**32 + 3, 5, -2**33 + 1, 2**31, 2**31 - 1, -1], dtype=torch.int64)
    wr = torch.tensor([1, 2**40, 3, 4, 2**32, 0], dtype=torch.int64)
    d, keep, _ = gdn.decode_args(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"],
                                 x["b"], x["pool"], rd, write_idx=wr, use_qk_l2norm=False)
    rd32, wr32 = keep[7], keep[8]
    assert rd32.dtype == torch.int32 and wr32.dtype == torch.int32
    assert rd32.tolist() == [-1, 5, -1, -1, 2**31 - 1, -1]
    assert wr32.tolist() == [1, -1, 3, 4, -1, 0]
    sc = torch.tensor([[2**32 + 1, 7]] * 6, dtype=torch.int64)
    _, keep, _ = gdn.decode_args(x["q"], x["k"], x["v"], x["A_log"], x["dt_bias"], x["a"],
                                 x["b"], x["pool"], rd, scatter_idx=sc, use_qk_l2norm=False)
    assert keep[9].tolist() == [[-1, 7]] * 6
    T, hq, hv, dk, dv = 96, 2, 4, 64, 32
    cu = torch.tensor([-2**40, 10, 2**35, 2**31 - 1], dtype=torch.int64)
    args, keep, _, _ = gdn.prefill_args(torch.zeros(T, hq, dk), torch.zeros(T, hq, dk),
                                        torch.zeros(T, hv, dv), torch.zeros(T, hv),
                                        torch.zeros(T, hv), cu_seqlens=cu)
    assert keep[5].tolist() == [-2**31, 10, 2**31 - 1, 2**31 - 1]
    pool = torch.zeros(8, hv, dv, dk)
    args, keep, _, _ = gdn.prefill_args(torch.zeros(T, hq, dk), torch.zeros(T, hq, dk),
                                        torch.zeros(T, hv, dv), torch.zeros(T, hv),
                                        torch.zeros(T, hv), state_pool=pool,
                                        read_slot=torch.tensor([2**32 + 2], dtype=torch.int64),
                                        write_slot=torch.tensor([2**33], dtype=torch.int64))
    assert keep[13].tolist() == [-1] and keep[14].tolist() == [-1]
