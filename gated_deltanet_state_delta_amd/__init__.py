"""Gated delta rule on MI355X (gfx950): Python binding of libgdn.

Three calls with the names of the C ABI (include/libgdn.h).  This layer only
marshals arguments (device pointers, strides, dtype codes, the current HIP
stream); every step of the computation runs in libgdn's HIP kernels.  There
is no other implementation: a missing libgdn.so or a non-GPU tensor is an
error.  Every tensor's shape is checked against the call's contract here,
because the kernels trust the sizes and strides they are given.

  gate(A_log, dt_bias, a, b)            -> (log_decay, gamma | None, beta)
  prefill(q, k, v, decay, beta, ...)    -> (out, final_state)
  decode(q, k, v, A_log, dt_bias, a, b, pool, read_idx, ...) -> (out, pool)
  conv1d(x, weight, conv_state, slot_idx, row_offsets, ...) -> out
  state_update(q, k, v, gamma, beta) -> {"outputs", "final_state"}
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import GdnError

__all__ = ["gate", "prefill", "decode", "conv1d", "state_update", "version", "GdnError",
           "prefill_args", "decode_args", "conv1d_args", "prefill_workspace_size",
           "prefill_noalloc", "wait_timeouts"]

_DT = {torch.float32: _lib.GDN_F32, torch.bfloat16: _lib.GDN_BF16}
# update_rule of the ONNX card -> gdn_update_rule
RULES = {"gated_delta": 0, "gated": 1, "delta": 2, "linear": 3}


def version() -> str:
    return _lib.load().gdn_version().decode()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if t is not None and not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (libgdn has no CPU path)" % name)
    return t


def _io_dtype(t):
    if t.dtype not in _DT:
        raise ValueError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)
    return _DT[t.dtype]


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t


_I32_MIN, _I32_MAX = -(1 << 31), (1 << 31) - 1


def _idx32(t, name, shape, offsets=False):
    """An int32 or int64 index tensor as the int32 table the C ABI reads.

    int64 entries outside the int32 range never wrap onto a valid index:
    slot indices (offsets=False) become -1, which every slot rule reads as
    "skip" exactly as it reads the original out-of-range value; offsets
    (cu_seqlens) are clamped to the int32 range, which the kernels' clamp to
    [0, total_tokens] maps to the same request bounds."""
    if t is None:
        return None
    if t.dtype not in (torch.int32, torch.int64):
        raise ValueError("%s must be int32 or int64" % name)
    _shape(t, name, shape)
    if t.dtype == torch.int64:
        if offsets:
            t = t.clamp(_I32_MIN, _I32_MAX)
        else:
            t = torch.where((t < _I32_MIN) | (t > _I32_MAX), torch.full_like(t, -1), t)
    return t.to(torch.int32).contiguous()


def _f32c(t, name, shape):
    _shape(t, name, shape)
    return t.to(torch.float32).contiguous()


def _strided3(t):
    """A [tokens, heads, dim] view the kernels can read in place: dense last dim,
    outer strides multiples of 8 elements, 16-byte aligned base; else a copy."""
    if t.stride(-1) != 1 or any(s % 8 for s in t.stride()[:-1]) or t.data_ptr() % 16:
        t = t.contiguous()
    return t


def gate(A_log, dt_bias, a=None, b=None, *, want_gamma=False, log_decay_out=None,
         beta_out=None, stream=None):
    """Fused gates: log_decay = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b).

    a, b: [..., hv] float32 or bfloat16 (either may be None).  Returns
    (log_decay, gamma, beta) as float32 tensors shaped like a / b; gamma only
    when want_gamma.  log_decay_out / beta_out: optional preallocated
    contiguous float32 outputs of a's / b's shape.
    """
    lib = _lib.load()
    ref = a if a is not None else b
    if ref is None:
        return None, None, None
    hv = ref.shape[-1]
    dt = _io_dtype(ref)
    a = None if a is None else _dev(a, "a").contiguous()
    b = None if b is None else _dev(b, "b").contiguous()
    if a is not None and b is not None:
        if a.dtype != b.dtype or b.shape[-1] != hv or b.numel() != a.numel():
            raise ValueError("a and b must share dtype and element count")
    if a is not None:
        A_log = _f32c(_dev(A_log, "A_log"), "A_log", (hv,))
        dt_bias = _f32c(_dev(dt_bias, "dt_bias"), "dt_bias", (hv,))
    else:
        A_log = dt_bias = None
    n = ref.numel() // hv
    def _outbuf(t, ref_t, name):
        if ref_t is None:
            return None
        if t is None:
            return torch.empty(ref_t.shape, dtype=torch.float32, device=ref_t.device)
        _dev(t, name)
        if tuple(t.shape) != tuple(ref_t.shape) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("%s must be contiguous float32 of shape %s" % (name, tuple(ref_t.shape)))
        return t

    g = _outbuf(log_decay_out, a, "log_decay_out")
    gam = torch.empty_like(g) if (a is not None and want_gamma) else None
    bet = _outbuf(beta_out, b, "beta_out")
    _lib.check(lib.gdn_gate(_ptr(A_log), _ptr(dt_bias), _ptr(a), _ptr(b), dt, n, hv, _ptr(g),
                            _ptr(gam), _ptr(bet), _stream(stream)))
    return g, gam, bet


def prefill_args(q, k, v, decay, beta, *, decay_kind="log", cu_seqlens=None,
                 initial_state=None, scale=None, chunk_size=0, out=None, final_state=None,
                 qk_l2norm=False, qk_l2norm_eps=1e-12, A_log=None, dt_bias=None, a=None,
                 b=None, update_rule="gated_delta", state_pool=None, read_slot=None,
                 write_slot=None, decay_per_key=False):
    """Validate shapes and build the gdn_prefill_args struct (device-agnostic).

    Returns (args, keep, out, final_state): `keep` holds every tensor whose
    pointer is in args (converted copies included), `out` is the caller-shaped
    output tensor; with state_pool, final_state is the pool.
    """
    batched = q.dim() == 4
    if batched:
        B, S = q.shape[0], q.shape[1]
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens requires the [T, heads, dim] form")
        _shape(k, "k", q.shape)
        if v.dim() != 4 or tuple(v.shape[:2]) != (B, S):
            raise ValueError("v must be [B, S, hv, dv] like q")
        q3, k3, v3 = q.reshape(B * S, *q.shape[2:]), k.reshape(B * S, *k.shape[2:]), \
            v.reshape(B * S, *v.shape[2:])
    else:
        if q.dim() != 3 or v.dim() != 3:
            raise ValueError("q, k, v must be [T, heads, dim] (or [B, S, heads, dim])")
        q3, k3, v3 = q, k, v
    T, hq, dk = q3.shape
    hv, dv = v3.shape[1], v3.shape[2]
    _shape(k3, "k", (T, hq, dk))
    _shape(v3, "v", (T, hv, dv))
    if k3.dtype != q3.dtype or v3.dtype != q3.dtype:
        raise ValueError("q, k and v must share a dtype")
    dt = _io_dtype(q3)
    q3, k3, v3 = _strided3(q3), _strided3(k3), _strided3(v3)
    if update_rule not in RULES:
        raise ValueError("update_rule must be one of %s" % sorted(RULES))
    uses_decay = update_rule in ("gated_delta", "gated")
    uses_beta = update_rule in ("gated_delta", "delta")
    if a is not None and decay is not None:
        raise ValueError("give the decay either fused (a) or given (decay), not both")
    if b is not None and beta is not None:
        raise ValueError("give beta either fused (b) or given (beta), not both")
    if (a is not None or (decay is not None)) != uses_decay:
        raise ValueError("update_rule %s %s a decay input (decay or a)"
                         % (update_rule, "needs" if uses_decay else "takes no"))
    if (b is not None or (beta is not None)) != uses_beta:
        raise ValueError("update_rule %s %s a beta input (beta or b)"
                         % (update_rule, "needs" if uses_beta else "takes no"))
    ga = gb = None
    if a is not None:
        if A_log is None or dt_bias is None:
            raise ValueError("the fused decay needs A_log and dt_bias")
        ga = a.reshape(-1, hv) if a.dim() == 3 else a
        _shape(ga, "a", (T, hv))
        if ga.dtype != q3.dtype:
            raise ValueError("a must have q's dtype")
        ga = ga.contiguous()
        A_log = _f32c(A_log, "A_log", (hv,))
        dt_bias = _f32c(dt_bias, "dt_bias", (hv,))
    else:
        A_log = dt_bias = None
    if b is not None:
        gb = b.reshape(-1, hv) if b.dim() == 3 else b
        _shape(gb, "b", (T, hv))
        if gb.dtype != q3.dtype:
            raise ValueError("b must have q's dtype")
        gb = gb.contiguous()
    if decay_per_key and a is not None:
        raise ValueError("decay_per_key takes the decay as a given input (not a)")
    if decay is not None and decay_per_key:
        decay = _f32c(decay.reshape(-1, hv, dk) if decay.dim() == 4 else decay, "decay",
                      (T, hv, dk))
    elif decay is not None:
        decay = _f32c(decay.reshape(-1, hv) if decay.dim() == 3 else decay, "decay", (T, hv))
    if beta is not None:
        beta = _f32c(beta.reshape(-1, hv) if beta.dim() == 3 else beta, "beta", (T, hv))
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be [N + 1]")
        cu = _idx32(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), offsets=True)
        n_seqs, seq_len = cu.numel() - 1, 0
    else:
        cu = None
        n_seqs, seq_len = (B, S) if batched else (1, T)
    if initial_state is not None:
        _shape(initial_state, "initial_state", (n_seqs, hv, dv, dk))
        if initial_state.dtype != torch.float32 or not initial_state.is_contiguous():
            initial_state = initial_state.to(torch.float32).contiguous()
    dev = q3.device
    if out is None:
        out = torch.empty((B, S, hv, dv) if batched else (T, hv, dv), dtype=q3.dtype, device=dev)
    if out.dtype != q3.dtype:
        raise ValueError("out must have q's dtype")
    _shape(out, "out", (B, S, hv, dv) if (batched and out.dim() == 4) else (T, hv, dv))
    out3 = out.view(T, hv, dv)  # a view, never a copy: the kernel writes through it
    if out3.stride(-1) != 1 or any(s % 8 for s in out3.stride()[:-1]) or out3.data_ptr() % 16:
        raise ValueError("out must have a dense last dim, 8-aligned strides and a 16-byte base")
    if state_pool is not None:
        if initial_state is not None or final_state is not None:
            raise ValueError("state_pool replaces initial_state and final_state")
        if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (hv, dv, dk):
            raise ValueError("state_pool must be [P, hv, dv, dk]")
        if state_pool.dtype != torch.float32 or state_pool.stride(3) != 1 or \
                state_pool.stride(2) != dk:
            raise ValueError("state_pool must be float32 with dense [dv, dk] heads")
        read_slot = _idx32(read_slot, "read_slot", (n_seqs,))
        write_slot = _idx32(write_slot, "write_slot", (n_seqs,))
    elif read_slot is not None or write_slot is not None:
        raise ValueError("read_slot / write_slot need state_pool")
    else:
        if final_state is None:
            final_state = torch.empty((n_seqs, hv, dv, dk), dtype=torch.float32, device=dev)
        _shape(final_state, "final_state", (n_seqs, hv, dv, dk))
        if final_state.dtype != torch.float32 or not final_state.is_contiguous():
            raise ValueError("final_state must be contiguous float32")
    args = _lib.PrefillArgs()
    args.n_seqs, args.seq_len, args.total_tokens = n_seqs, seq_len, T
    args.hq, args.hv, args.dk, args.dv = hq, hv, dk, dv
    args.io_dtype = dt
    args.decay_kind = _lib.GDN_DECAY_GAMMA if decay_kind == "gamma" else _lib.GDN_DECAY_LOG
    args.chunk_size = int(chunk_size)
    args.scale = (1.0 / math.sqrt(dk)) if scale is None else float(scale)
    args.q, args.q_stride_token, args.q_stride_head = q3.data_ptr(), q3.stride(0), q3.stride(1)
    args.k, args.k_stride_token, args.k_stride_head = k3.data_ptr(), k3.stride(0), k3.stride(1)
    args.v, args.v_stride_token, args.v_stride_head = v3.data_ptr(), v3.stride(0), v3.stride(1)
    args.out, args.out_stride_token, args.out_stride_head = \
        out3.data_ptr(), out3.stride(0), out3.stride(1)
    args.decay = None if decay is None else decay.data_ptr()
    args.beta = None if beta is None else beta.data_ptr()
    args.cu_seqlens = None if cu is None else cu.data_ptr()
    args.initial_state = None if initial_state is None else initial_state.data_ptr()
    args.final_state = None if final_state is None else final_state.data_ptr()
    if state_pool is not None:
        args.state_pool, args.pool_size = state_pool.data_ptr(), state_pool.shape[0]
        args.pool_slot_stride, args.pool_head_stride = state_pool.stride(0), state_pool.stride(1)
        args.read_slot = None if read_slot is None else read_slot.data_ptr()
        args.write_slot = None if write_slot is None else write_slot.data_ptr()
        final_state = state_pool
    args.qk_l2norm = 1 if qk_l2norm else 0
    args.qk_l2norm_eps = float(qk_l2norm_eps)
    if ga is not None:
        args.A_log, args.dt_bias = A_log.data_ptr(), dt_bias.data_ptr()
        args.gate_a = ga.data_ptr()
    if gb is not None:
        args.gate_b = gb.data_ptr()
    args.update_rule = RULES[update_rule]
    args.decay_per_key = 1 if decay_per_key else 0
    keep = (q3, k3, v3, decay, beta, cu, initial_state, out3, final_state, A_log, dt_bias, ga, gb,
            read_slot, write_slot)
    return args, keep, out, final_state


def prefill(q, k, v, decay, beta, *, decay_kind="log", cu_seqlens=None, initial_state=None,
            scale=None, chunk_size=0, out=None, final_state=None, stream=None,
            qk_l2norm=False, qk_l2norm_eps=1e-12, A_log=None, dt_bias=None, a=None, b=None,
            update_rule="gated_delta", state_pool=None, read_slot=None, write_slot=None,
            decay_per_key=False, scan=True, workspace=None):
    """Chunked prefill.

    q, k: [T, hq, dk] (or [B, S, hq, dk], then uniform packing with seq_len S);
    v: [T, hv, dv] (or [B, S, hv, dv]); decay, beta: [T, hv] float32 (decay is
    log-space for decay_kind="log", gamma for "gamma"); cu_seqlens: [N+1]
    int32/int64 or None; initial_state: [N, hv, dv, dk] float32 or None.
    scale None means 1/sqrt(dk).  qk_l2norm: use every q and k head vector as
    x / sqrt(sum x^2 + qk_l2norm_eps) (the ONNX card's qk_l2_norm).  a, b
    ([T, hv] or [B, S, hv] in q's dtype): the fused gate, computed in the
    kernel -- the qwen decay from a with A_log, dt_bias [hv], beta = sigmoid(b);
    each gate input is given or fused on its own (the ONNX card's separate
    gate_activation and beta_activation), so a with beta, or decay with b,
    is accepted too.  Head sizes other than 16, 32, 64, 128
    (up to 128) run zero-padded to the next kernel size, with dense states
    only; the results are exact.  update_rule ("gated_delta", "gated",
    "delta", "linear"; the ONNX card's attribute) selects which terms of the
    recurrence survive; a rule takes exactly the gate inputs it uses (gated:
    decay or a only; delta: beta or b only; linear: neither).
    state_pool [P, hv, dv, dk] float32 (updated in place) with read_slot /
    write_slot [N]: the states come from and go to pool slots instead of
    initial_state / final_state (read slot outside the pool: zeros; write slot
    None: the read slot; outside the pool: not stored); returns (out, pool).
    decay_per_key: decay is [T, hv, dk] (or [B, S, hv, dk]), one decay per
    key dimension (the ONNX card's per-key spelling; a given decay, with a
    given beta or a fused b); it runs a separate, slower kernel.
    float16 q, k, v (the ONNX card's T includes f16) run the float32 path on
    exact widenings and the output is rounded back to float16.
    scan: calls with few (request, head) units and long requests may run as a
    scan over request segments (gdn_prefill_workspace_size > 0), which needs a
    device workspace: `workspace` (a uint8 CUDA tensor of at least that many
    bytes) or, when None, one allocated here; scan=False runs the serial
    walk instead (no workspace).  Both compute the same recurrence; only the
    rounding order differs.
    Returns (out, final_state [N, hv, dv, dk] float32); out is [T, hv, dv] (or
    [B, S, hv, dv]) in q's dtype.
    """
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("decay", decay), ("beta", beta),
                    ("cu_seqlens", cu_seqlens), ("initial_state", initial_state),
                    ("out", out), ("final_state", final_state), ("A_log", A_log),
                    ("dt_bias", dt_bias), ("a", a), ("b", b), ("state_pool", state_pool),
                    ("read_slot", read_slot), ("write_slot", write_slot)):
        _dev(t, name)
    if q.dtype == torch.float16:
        if out is not None and out.dtype != torch.float16:
            raise ValueError("out must have q's dtype")
        w = lambda t: None if t is None else t.float()
        o32, fin = prefill(w(q), w(k), w(v), decay, beta, decay_kind=decay_kind,
                           cu_seqlens=cu_seqlens, initial_state=initial_state, scale=scale,
                           chunk_size=chunk_size, final_state=final_state, stream=stream,
                           qk_l2norm=qk_l2norm, qk_l2norm_eps=qk_l2norm_eps, A_log=A_log,
                           dt_bias=dt_bias, a=w(a), b=w(b), update_rule=update_rule,
                           state_pool=state_pool, read_slot=read_slot, write_slot=write_slot,
                           decay_per_key=decay_per_key)
        if out is None:
            return o32.half(), fin
        out.copy_(o32)
        return out, fin
    dk, dv = q.shape[-1], v.shape[-1]
    pk, pv = _head_pad(dk), _head_pad(dv)
    if (pk, pv) != (dk, dv):
        return _prefill_padded(q, k, v, decay, beta, pk, pv, decay_kind=decay_kind,
                               cu_seqlens=cu_seqlens, initial_state=initial_state, scale=scale,
                               chunk_size=chunk_size, out=out, final_state=final_state,
                               stream=stream, qk_l2norm=qk_l2norm, qk_l2norm_eps=qk_l2norm_eps,
                               A_log=A_log, dt_bias=dt_bias, a=a, b=b, update_rule=update_rule,
                               state_pool=state_pool, decay_per_key=decay_per_key)
    args, keep, out, final_state = prefill_args(
        q, k, v, decay, beta, decay_kind=decay_kind, cu_seqlens=cu_seqlens,
        initial_state=initial_state, scale=scale, chunk_size=chunk_size, out=out,
        final_state=final_state, qk_l2norm=qk_l2norm, qk_l2norm_eps=qk_l2norm_eps,
        A_log=A_log, dt_bias=dt_bias, a=a, b=b, update_rule=update_rule,
        state_pool=state_pool, read_slot=read_slot, write_slot=write_slot,
        decay_per_key=decay_per_key)
    ws = None
    if scan:
        need = lib.gdn_prefill_workspace_size(ctypes.byref(args))
        if need > 0:
            if workspace is None:
                ws = torch.empty(need, dtype=torch.uint8, device=q.device)
            else:
                _dev(workspace, "workspace")
                if workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
                    raise ValueError("workspace must be a contiguous buffer of at least %d bytes" % need)
                ws = workspace
            args.workspace, args.workspace_bytes = ws.data_ptr(), need
    _lib.check(lib.gdn_prefill(ctypes.byref(args), _stream(stream)))
    del keep, ws
    return out, final_state


def prefill_noalloc(q, k, v, decay, beta, *, stream=None, **kw):
    """prefill through gdn_prefill_noalloc: the same call and result as
    prefill, with any scratch taken from the library's static per-device
    array instead of an allocated workspace (for callers that cannot
    allocate; calls that overlap on one device race).  q, k, v in float32 or
    bfloat16 with head sizes of 16, 32, 64 or 128; out and final_state are
    allocated here when not given.  Returns (out, final_state)."""
    for name in ("scan", "workspace"):
        if name in kw:
            raise ValueError("prefill_noalloc takes no %s argument" % name)
    for name, t in (("q", q), ("k", k), ("v", v), ("decay", decay), ("beta", beta)):
        _dev(t, name)
    for name, t in kw.items():
        if isinstance(t, torch.Tensor):
            _dev(t, name)
    args, keep, out, final_state = prefill_args(q, k, v, decay, beta, **kw)
    _lib.check(_lib.load().gdn_prefill_noalloc(ctypes.byref(args), _stream(stream)))
    del keep
    return out, final_state


def prefill_workspace_size(q, k, v, decay, beta, **kw) -> int:
    """Bytes of device workspace a prefill call with these arguments would use
    (gdn_prefill_workspace_size): 0 unless the call runs as the scan over
    request segments."""
    args, keep, _, _ = prefill_args(q, k, v, decay, beta, **kw)
    return int(_lib.load().gdn_prefill_workspace_size(ctypes.byref(args)))


def wait_timeouts(clear=True) -> int:
    """The current device's count of in-kernel waits that ran out of polls
    (gdn_wait_timeouts): 0 in every correct run.  clear resets it.  Waits
    for all work on the device."""
    n = ctypes.c_uint32(0)
    _lib.check(_lib.load().gdn_wait_timeouts(ctypes.byref(n), 1 if clear else 0))
    return int(n.value)


_HEAD_SIZES = (16, 32, 64, 128)


def _head_pad(d):
    """The kernel head size a head of size d runs at: the next of 16, 32, 64,
    128 (d itself when it is one; d above 128 is refused by the C ABI)."""
    return next((n for n in _HEAD_SIZES if n >= d), d)


def _pad_last(t, n):
    """t with its last dimension zero-padded to n (t itself when already n)."""
    if t.shape[-1] == n:
        return t
    out = torch.zeros(*t.shape[:-1], n, dtype=t.dtype, device=t.device)
    out[..., :t.shape[-1]] = t
    return out


def _prefill_padded(q, k, v, decay, beta, pk, pv, *, out, final_state, initial_state,
                    state_pool, decay_per_key=False, **kw):
    """prefill for head sizes the kernels do not take (the ONNX card's head
    sizes are free, e.g. its JS example's 12 and 9): q, k and v are
    zero-padded to the kernel sizes pk, pv, the initial state likewise, and
    the results are sliced back.  This is exact: a zero key or query
    component adds nothing to any dot product, and a value row that starts at
    zero with zero values stays zero."""
    if state_pool is not None:
        raise ValueError("head sizes other than 16, 32, 64, 128 need dense states "
                         "(a pool slot cannot be padded in place)")
    dk, dv = q.shape[-1], v.shape[-1]
    if kw.get("scale") is None:
        kw["scale"] = 1.0 / math.sqrt(dk)  # the caller's head size, not the padded one
    init = None
    if initial_state is not None:
        init = torch.zeros(*initial_state.shape[:-2], pv, pk, dtype=torch.float32,
                           device=initial_state.device)
        init[..., :dv, :dk] = initial_state
    if decay_per_key and decay is not None:
        decay = _pad_last(decay, pk)  # padded keys: zero k, q and state; their decay is moot
    o_p, f_p = prefill(_pad_last(q, pk), _pad_last(k, pk), _pad_last(v, pv), decay, beta,
                       initial_state=init, decay_per_key=decay_per_key, **kw)
    o = o_p[..., :dv]
    f = f_p[..., :dv, :dk]
    if out is not None:
        out.copy_(o)
    else:
        out = o.contiguous()
    if final_state is not None:
        final_state.copy_(f)
    else:
        final_state = f.contiguous()
    return out, final_state


def state_update(q, k, v, gamma, beta):
    """The interface of "Gated DeltaNet State Update" (statement, Constraints):
    q, k [B, S, Dk], v [B, S, Dv] (float32 or bfloat16), gamma, beta [B, S]
    float32; every batch item starts from a zero state; y_t = q_t^T S_t (no
    scale).  Returns {"outputs": [B, S, Dv], "final_state": [B, Dk, Dv]} in
    q's dtype and device.

    The call is one gdn_prefill launch with one head (decay given as gamma,
    scale 1; head sizes the kernels do not take are zero-padded by prefill);
    its V-major final state is returned transposed, as the statement's
    (B, Dk, Dv).
    """
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B, S, Dk] and v [B, S, Dv]")
    B, S, dk = q.shape
    dv = v.shape[2]
    _shape(gamma, "gamma", (B, S))
    _shape(beta, "beta", (B, S))
    if dk > 128 or dv > 128:
        raise ValueError("Dk and Dv up to 128 are supported (got %d, %d)" % (dk, dv))
    out, fin = prefill(q.unsqueeze(2), k.unsqueeze(2), v.unsqueeze(2), gamma.unsqueeze(-1),
                       beta.unsqueeze(-1), decay_kind="gamma", scale=1.0)
    return {"outputs": out[:, :, 0], "final_state": fin[:, 0].transpose(1, 2).to(q.dtype)}


def decode_args(q, k, v, A_log, dt_bias, a, b, pool, read_idx, *, write_idx=None,
                scatter_idx=None, disable_state_update=False, scale=None, out=None,
                use_qk_l2norm=True, qk_l2norm_eps=1e-6, decay_per_key=None):
    """Validate shapes and build the gdn_decode_args struct (device-agnostic).

    Returns (args, keep, out)."""
    if q.dim() != 4 or k.dim() != 5 or v.dim() != 5:
        raise ValueError("q [B,T,hq,dk], k [B,T,n,hq,dk], v [B,T,n,hv,dv] expected")
    B, T, hq, dk = q.shape
    n = k.shape[2]
    hv, dv = v.shape[3], v.shape[4]
    _shape(k, "k", (B, T, n, hq, dk))
    _shape(v, "v", (B, T, n, hv, dv))
    _shape(b, "b", (B, T, n, hv))
    dt = _io_dtype(q)
    if decay_per_key is not None:
        # the per-key decay replaces the fused gate's decay: a, A_log, dt_bias unused
        decay_per_key = _f32c(decay_per_key, "decay_per_key", (B, T, hv, dk))
        a = A_log = dt_bias = None
    else:
        _shape(a, "a", (B, T, hv))
        A_log = _f32c(A_log, "A_log", (hv,))
        dt_bias = _f32c(dt_bias, "dt_bias", (hv,))
    if any(t.dtype != q.dtype for t in (k, v, b) + ((a,) if a is not None else ())):
        raise ValueError("q, k, v, a and b must share one dtype")
    q, k, v, b = (t.contiguous() for t in (q, k, v, b))
    a = None if a is None else a.contiguous()
    if pool.dim() != 4 or tuple(pool.shape[1:]) != (hv, dv, dk):
        raise ValueError("pool must be [P, %d, %d, %d], got %s" % (hv, dv, dk, tuple(pool.shape)))
    if pool.dtype != torch.float32 or pool.stride(-1) != 1 or pool.stride(-2) != dk:
        raise ValueError("pool must be float32 with dense [dv][dk] rows")
    if out is None:
        out = torch.zeros((B, T, hv, dv), dtype=q.dtype, device=q.device)
    _shape(out, "out", (B, T, hv, dv))
    if not out.is_contiguous() or out.dtype != q.dtype:
        raise ValueError("out must be contiguous and of q's dtype")
    read_idx = _idx32(read_idx, "read_idx", (B,))
    write_idx = _idx32(write_idx, "write_idx", (B,))
    scatter_idx = _idx32(scatter_idx, "scatter_idx", (B, T))
    d = _lib.DecodeArgs()
    d.batch, d.T, d.n_householder = B, T, n
    d.hq, d.hv, d.dk, d.dv = hq, hv, dk, dv
    d.io_dtype = dt
    d.disable_state_update = 1 if disable_state_update else 0
    d.scale = (1.0 / math.sqrt(dk)) if scale is None else float(scale)
    d.q, d.k, d.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    d.A_log = None if A_log is None else A_log.data_ptr()
    d.dt_bias = None if dt_bias is None else dt_bias.data_ptr()
    d.a = None if a is None else a.data_ptr()
    d.b = b.data_ptr()
    d.decay_per_key = None if decay_per_key is None else decay_per_key.data_ptr()
    d.pool, d.pool_size = pool.data_ptr(), pool.shape[0]
    d.pool_slot_stride, d.pool_head_stride = pool.stride(0), pool.stride(1)
    d.read_idx = read_idx.data_ptr()
    d.write_idx = None if write_idx is None else write_idx.data_ptr()
    d.scatter_idx = None if scatter_idx is None else scatter_idx.data_ptr()
    d.out = out.data_ptr()
    d.qk_l2norm = 1 if use_qk_l2norm else 0
    d.qk_l2norm_eps = float(qk_l2norm_eps)
    keep = (q, k, v, a, b, A_log, dt_bias, read_idx, write_idx, scatter_idx, decay_per_key)
    return d, keep, out


def decode(q, k, v, A_log, dt_bias, a, b, pool, read_idx, *, write_idx=None, scatter_idx=None,
           disable_state_update=False, scale=None, out=None, stream=None, use_qk_l2norm=True,
           qk_l2norm_eps=1e-6, decay_per_key=None):
    """Slot-pool decode with Householder sub-steps (one fused launch).

    q [B, T, hq, dk]; k [B, T, n, hq, dk]; v [B, T, n, hv, dv]; A_log, dt_bias
    [hv] float32; a [B, T, hv]; b [B, T, n, hv]; pool [P, hv, dv, dk] float32
    (updated in place); read_idx [B]; write_idx [B] or None; scatter_idx [B, T]
    or None.  scale None means 1/sqrt(dk).  use_qk_l2norm: use every q and k
    head vector as x / sqrt(sum x^2 + qk_l2norm_eps) (the FlashInfer page's
    use_qk_l2norm, on by default as there; pass False for inputs already
    normalised).  decay_per_key [B, T, hv, dk] float32
    log-decay per key dimension: replaces the gate's decay (a, A_log, dt_bias
    may then be None).  float16 q, k, v, a, b are converted to bfloat16 for
    the kernel and the output is copied into a float16 buffer (skipped rows
    keep their values through a bfloat16 round trip), as the FlashInfer page
    describes.  out may be any [B, T, hv, dv] tensor of q's dtype: a
    non-contiguous (or unaligned) one receives a copy of the kernel's dense
    output after the launch, as the FlashInfer page's output parameter says.
    Returns (out [B, T, hv, dv], pool); rows of skipped batch rows keep out's
    previous contents (zeros when out is None).
    """
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("A_log", A_log), ("dt_bias", dt_bias),
                    ("a", a), ("b", b), ("pool", pool), ("read_idx", read_idx),
                    ("write_idx", write_idx), ("scatter_idx", scatter_idx), ("out", out),
                    ("decay_per_key", decay_per_key)):
        _dev(t, name)
    if q.dtype == torch.float16:
        c = lambda t: None if t is None else t.to(torch.bfloat16)
        o16 = None if out is None else out.to(torch.bfloat16)
        o, pool = decode(c(q), c(k), c(v), A_log, dt_bias, c(a), c(b), pool, read_idx,
                         write_idx=write_idx, scatter_idx=scatter_idx,
                         disable_state_update=disable_state_update, scale=scale, out=o16,
                         stream=stream, use_qk_l2norm=use_qk_l2norm, qk_l2norm_eps=qk_l2norm_eps,
                         decay_per_key=decay_per_key)
        if out is None:
            return o.half(), pool
        out.copy_(o)
        return out, pool
    if out is not None and out.dtype == q.dtype and out.dim() == 4 and \
            (not out.is_contiguous() or out.data_ptr() % 16):
        # "flashinfer...cake_gated_delta_product_mtp", Parameters (output): the
        # kernel writes a dense buffer and any other buffer receives a copy
        # after the launch.  The dense buffer starts as a copy of out, so rows
        # the call skips keep their previous contents.
        dense = out.clone(memory_format=torch.contiguous_format)
        _, pool = decode(q, k, v, A_log, dt_bias, a, b, pool, read_idx, write_idx=write_idx,
                         scatter_idx=scatter_idx, disable_state_update=disable_state_update,
                         scale=scale, out=dense, stream=stream, use_qk_l2norm=use_qk_l2norm,
                         qk_l2norm_eps=qk_l2norm_eps, decay_per_key=decay_per_key)
        out.copy_(dense)
        return out, pool
    d, keep, out = decode_args(q, k, v, A_log, dt_bias, a, b, pool, read_idx,
                               write_idx=write_idx, scatter_idx=scatter_idx,
                               disable_state_update=disable_state_update, scale=scale, out=out,
                               use_qk_l2norm=use_qk_l2norm, qk_l2norm_eps=qk_l2norm_eps,
                               decay_per_key=decay_per_key)
    _lib.check(lib.gdn_decode(ctypes.byref(d), _stream(stream)))
    del keep
    return out, pool


_U32_MAX = 0xFFFFFFFF


def _u32(t, name, shape, negative):
    """An index tensor as the uint32 bit pattern the C ABI reads (held in an
    int32 tensor).  int32 tensors pass through as their bit pattern (no extra
    launch); in int64 / uint32 tensors negative entries become `negative` and
    entries above 2^32-1 are clamped to it."""
    if t.dtype not in (torch.int32, torch.int64, torch.uint32):
        raise ValueError("%s must be int32, int64 or uint32" % name)
    _shape(t, name, shape)
    if t.dtype == torch.int32:
        return t.contiguous()
    t64 = t.to(torch.int64)
    t64 = torch.where(t64 < 0, torch.full_like(t64, negative), t64.clamp(max=_U32_MAX))
    return torch.where(t64 > 0x7FFFFFFF, t64 - (1 << 32), t64).to(torch.int32).contiguous()


def conv1d_args(x, weight, conv_state, slot_idx, row_offsets, *, write_state=True, out=None):
    """Marshal a gdn_conv1d call: returns (args struct, tensors to keep alive, out)."""
    if x.dim() != 2:
        raise ValueError("x must be [total_tokens, conv_dim]")
    T, C = x.shape
    dt = _io_dtype(x)
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError("weight must be [conv_dim, kernel_size]")
    K = weight.shape[1]
    if weight.dtype != x.dtype:
        raise ValueError("weight must have x's dtype")
    weight = weight.contiguous()
    n = slot_idx.shape[0] if slot_idx.dim() == 1 else -1
    if n < 0:
        raise ValueError("slot_idx must be [n_seqs]")
    if conv_state is not None:
        if conv_state.dim() != 3 or conv_state.shape[1:] != (C, K - 1):
            raise ValueError("conv_state must be [max_slots, conv_dim, kernel_size - 1]")
        if conv_state.dtype != x.dtype or not conv_state.is_contiguous() or conv_state.data_ptr() % 16:
            raise ValueError("conv_state must be dense, 16-byte aligned, with x's dtype "
                             "(it is updated in place)")
    elif K > 1:
        raise ValueError("conv_state is required when kernel_size > 1")
    slots = _u32(slot_idx, "slot_idx", (n,), _U32_MAX)
    offs = _u32(row_offsets, "row_offsets", (n + 1,), 0)
    ve = 8 if dt == _lib.GDN_BF16 else 4
    if x.stride(1) != 1 or x.stride(0) % ve or x.stride(0) < C or x.data_ptr() % 16:
        x = x.contiguous()
    if out is None:
        out = torch.zeros((T, C), dtype=x.dtype, device=x.device)
    else:
        _shape(out, "out", (T, C))
        if out.dtype != x.dtype or out.stride(1) != 1 or out.stride(0) % ve or out.data_ptr() % 16:
            raise ValueError("out must have x's dtype, a dense last dim, 16-byte rows")
    d = _lib.Conv1dArgs()
    d.total_tokens, d.conv_dim, d.kernel_size, d.n_seqs = T, C, K, n
    d.io_dtype, d.write_state = dt, 1 if write_state else 0
    d.max_slots = 0 if conv_state is None else conv_state.shape[0]
    d.x, d.x_stride_token = x.data_ptr(), x.stride(0)
    d.weight = weight.data_ptr()
    d.conv_state = None if conv_state is None else conv_state.data_ptr()
    d.slot_idx, d.row_offsets = slots.data_ptr(), offs.data_ptr()
    d.out, d.out_stride_token = out.data_ptr(), out.stride(0)
    keep = (x, weight, slots, offs)
    return d, keep, out


def conv1d(x, weight, conv_state, slot_idx, row_offsets, *, write_state=True, out=None,
           stream=None):
    """Causal depthwise conv1d over a ragged batch with a slot-indexed conv-state
    pool ("gated_delta_conv1d_fwd").

    x [T, conv_dim]; weight [conv_dim, K] (x's dtype); conv_state
    [max_slots, conv_dim, K-1] (x's dtype, dense, updated in place when
    write_state); slot_idx [n_seqs]; row_offsets [n_seqs + 1], uint32-valued
    as on the page (int32 tensors are read as their uint32 bit pattern, so a
    negative int32 slot is out of range and a negative int32 offset is past
    the end; int64 offsets below 0 count as 0).  Slots outside the pool read
    zeros and are not written.  Returns out
    [T, conv_dim]; rows no sequence covers keep out's previous contents (zeros
    when out is None).
    """
    lib = _lib.load()
    for name, t in (("x", x), ("weight", weight), ("conv_state", conv_state),
                    ("slot_idx", slot_idx), ("row_offsets", row_offsets), ("out", out)):
        _dev(t, name)
    d, keep, out = conv1d_args(x, weight, conv_state, slot_idx, row_offsets,
                               write_state=write_state, out=out)
    _lib.check(lib.gdn_conv1d(ctypes.byref(d), _stream(stream)))
    del keep
    return out
