"""Gated delta rule on MI355X (gfx950): Python binding of libgdn.

Three calls with the names of the C ABI (include/libgdn.h).  This layer only
marshals arguments (device pointers, strides, dtype codes, the current HIP
stream); every step of the computation runs in libgdn's HIP kernels.  There
is no other implementation: a missing libgdn.so or a non-GPU tensor is an
error.

  gate(A_log, dt_bias, a, b)            -> (log_decay, gamma | None, beta)
  prefill(q, k, v, decay, beta, ...)    -> (out, final_state)
  decode(q, k, v, A_log, dt_bias, a, b, pool, read_idx, ...) -> (out, pool)
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import GdnError

__all__ = ["gate", "prefill", "decode", "version", "GdnError"]

_DT = {torch.float32: _lib.GDN_F32, torch.bfloat16: _lib.GDN_BF16}


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


def _idx32(t):
    if t is None:
        return None
    if t.dtype != torch.int32:
        t = t.to(torch.int32)
    return t.contiguous()


def _last_dense(t, name):
    """Keep views whose last dim is dense with 8-aligned outer strides, copy others."""
    if t.stride(-1) != 1 or any(s % 8 for s in t.stride()[:-1]) or t.data_ptr() % 16:
        t = t.contiguous()
    return t


def gate(A_log, dt_bias, a=None, b=None, *, want_gamma=False, stream=None):
    """Fused gates: log_decay = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b).

    a, b: [..., hv] float32 or bfloat16 (either may be None).  Returns
    (log_decay, gamma, beta) as float32 tensors shaped like a / b; gamma only
    when want_gamma.
    """
    lib = _lib.load()
    ref = a if a is not None else b
    if ref is None:
        return None, None, None
    hv = ref.shape[-1]
    dt = _io_dtype(ref)
    a = None if a is None else _dev(a, "a").contiguous()
    b = None if b is None else _dev(b, "b").contiguous()
    if a is not None and b is not None and a.dtype != b.dtype:
        raise ValueError("a and b must share a dtype")
    A_log = None if A_log is None else _dev(A_log, "A_log").float().contiguous()
    dt_bias = None if dt_bias is None else _dev(dt_bias, "dt_bias").float().contiguous()
    n = ref.numel() // hv
    if a is not None and b is not None and b.numel() != a.numel():
        raise ValueError("a and b must have the same number of elements")
    g = torch.empty(a.shape, dtype=torch.float32, device=a.device) if a is not None else None
    gam = torch.empty_like(g) if (a is not None and want_gamma) else None
    bet = torch.empty(b.shape, dtype=torch.float32, device=b.device) if b is not None else None
    _lib.check(lib.gdn_gate(_ptr(A_log), _ptr(dt_bias), _ptr(a), _ptr(b), dt, n, hv, _ptr(g),
                            _ptr(gam), _ptr(bet), _stream(stream)))
    return g, gam, bet


def prefill(q, k, v, decay, beta, *, decay_kind="log", cu_seqlens=None, initial_state=None,
            scale=None, chunk_size=0, out=None, final_state=None, stream=None):
    """Chunked prefill.

    q, k: [T, hq, dk] (or [B, S, hq, dk], then uniform packing with seq_len S);
    v: [T, hv, dv] (or [B, S, hv, dv]); decay, beta: [T, hv] float32 (decay is
    log-space for decay_kind="log", gamma for "gamma"); cu_seqlens: [N+1]
    int32/int64 or None; initial_state: [N, hv, dv, dk] float32 or None.
    scale None means 1/sqrt(dk).  Returns (out [T, hv, dv] in q's dtype,
    final_state [N, hv, dv, dk] float32).
    """
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("decay", decay), ("beta", beta)):
        _dev(t, name)
    batched = q.dim() == 4
    if batched:
        B, S = q.shape[0], q.shape[1]
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens requires the [T, heads, dim] form")
        q = q.reshape(B * S, *q.shape[2:])
        k = k.reshape(B * S, *k.shape[2:])
        v = v.reshape(B * S, *v.shape[2:])
        decay = decay.reshape(B * S, -1)
        beta = beta.reshape(B * S, -1)
    T, hq, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k must match q in shape and dtype; v must share q's dtype")
    dt = _io_dtype(q)
    q, k, v = _last_dense(q, "q"), _last_dense(k, "k"), _last_dense(v, "v")
    decay = decay.float().contiguous()
    beta = beta.float().contiguous()
    cu = _idx32(_dev(cu_seqlens, "cu_seqlens"))
    if cu is not None:
        n_seqs, seq_len = cu.numel() - 1, 0
    elif batched:
        n_seqs, seq_len = B, S
    else:
        n_seqs, seq_len = 1, T
    if initial_state is not None:
        initial_state = _dev(initial_state, "initial_state")
        if initial_state.dtype != torch.float32 or not initial_state.is_contiguous():
            initial_state = initial_state.float().contiguous()
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=q.device)
    if final_state is None:
        final_state = torch.empty((n_seqs, hv, dv, dk), dtype=torch.float32, device=q.device)
    a = _lib.PrefillArgs()
    a.n_seqs, a.seq_len, a.total_tokens = n_seqs, seq_len, T
    a.hq, a.hv, a.dk, a.dv = hq, hv, dk, dv
    a.io_dtype = dt
    a.decay_kind = _lib.GDN_DECAY_GAMMA if decay_kind == "gamma" else _lib.GDN_DECAY_LOG
    a.chunk_size = int(chunk_size)
    a.scale = (1.0 / math.sqrt(dk)) if scale is None else float(scale)
    a.q, a.q_stride_token, a.q_stride_head = q.data_ptr(), q.stride(0), q.stride(1)
    a.k, a.k_stride_token, a.k_stride_head = k.data_ptr(), k.stride(0), k.stride(1)
    a.v, a.v_stride_token, a.v_stride_head = v.data_ptr(), v.stride(0), v.stride(1)
    a.out, a.out_stride_token, a.out_stride_head = out.data_ptr(), out.stride(0), out.stride(1)
    a.decay, a.beta = decay.data_ptr(), beta.data_ptr()
    a.cu_seqlens = None if cu is None else cu.data_ptr()
    a.initial_state = None if initial_state is None else initial_state.data_ptr()
    a.final_state = final_state.data_ptr()
    _lib.check(lib.gdn_prefill(ctypes.byref(a), _stream(stream)))
    if batched:
        out = out.view(B, S, hv, dv)
    return out, final_state


def decode(q, k, v, A_log, dt_bias, a, b, pool, read_idx, *, write_idx=None, scatter_idx=None,
           disable_state_update=False, scale=None, out=None, stream=None):
    """Slot-pool decode with Householder sub-steps (one fused launch).

    q [B, T, hq, dk]; k [B, T, n, hq, dk]; v [B, T, n, hv, dv]; A_log, dt_bias
    [hv] float32; a [B, T, hv]; b [B, T, n, hv]; pool [P, hv, dv, dk] float32
    (updated in place); read_idx [B]; write_idx [B] or None; scatter_idx [B, T]
    or None.  scale None means 1/sqrt(dk).  Returns (out [B, T, hv, dv], pool);
    rows of skipped batch rows keep out's previous contents (zeros when out is
    None).
    """
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("a", a), ("b", b), ("pool", pool),
                    ("read_idx", read_idx)):
        _dev(t, name)
    B, T, hq, dk = q.shape
    n = k.shape[2]
    hv, dv = v.shape[3], v.shape[4]
    dt = _io_dtype(q)
    q, k, v, a, b = (t.contiguous() for t in (q, k, v, a, b))
    if a.dtype != q.dtype or b.dtype != q.dtype or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v, a and b must share one dtype")
    A_log = _dev(A_log, "A_log").float().contiguous()
    dt_bias = _dev(dt_bias, "dt_bias").float().contiguous()
    if pool.dtype != torch.float32 or pool.stride(-1) != 1 or pool.stride(-2) != dk:
        raise ValueError("pool must be float32 with dense [dv][dk] rows")
    if out is None:
        out = torch.zeros((B, T, hv, dv), dtype=q.dtype, device=q.device)
    elif not out.is_contiguous() or out.dtype != q.dtype:
        raise ValueError("out must be contiguous and of q's dtype")
    read_idx = _idx32(read_idx)
    write_idx = _idx32(write_idx)
    scatter_idx = _idx32(scatter_idx)
    d = _lib.DecodeArgs()
    d.batch, d.T, d.n_householder = B, T, n
    d.hq, d.hv, d.dk, d.dv = hq, hv, dk, dv
    d.io_dtype = dt
    d.disable_state_update = 1 if disable_state_update else 0
    d.scale = (1.0 / math.sqrt(dk)) if scale is None else float(scale)
    d.q, d.k, d.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    d.A_log, d.dt_bias = A_log.data_ptr(), dt_bias.data_ptr()
    d.a, d.b = a.data_ptr(), b.data_ptr()
    d.pool, d.pool_size = pool.data_ptr(), pool.shape[0]
    d.pool_slot_stride, d.pool_head_stride = pool.stride(0), pool.stride(1)
    d.read_idx = read_idx.data_ptr()
    d.write_idx = None if write_idx is None else write_idx.data_ptr()
    d.scatter_idx = None if scatter_idx is None else scatter_idx.data_ptr()
    d.out = out.data_ptr()
    _lib.check(lib.gdn_decode(ctypes.byref(d), _stream(stream)))
    return out, pool
