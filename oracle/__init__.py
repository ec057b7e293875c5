"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and the two share no
code.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision); this
module only widens inputs exactly to float64, converts index tables to int64
and marshals pointers.  Outputs are float64 and are never rounded.

Page citations (by title and section):
  * "Gated DeltaNet State Update": recurrence, readout after the update,
    zero initial state, per-batch independence, constraints.
  * "com.microsoft.GatedDeltaNet": GVA head map h*Hq/Hv, cu_seqlens clamping,
    V-major fp32 states, empty-request copy-through, qwen gate, scale,
    update_rule (linear / gated / delta / gated_delta).
  * "flashinfer.cake_gdp.cake_gated_delta_product_mtp": slot-pool decode,
    Householder sub-steps, skip / write-slot / scatter / disable rules.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so with gcc (plain -O2)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            lib.gdno_gate.restype = None
            lib.gdno_gate.argtypes = [ctypes.c_int64, ctypes.c_int32, _dp, _dp, _dp, _dp,
                                      _dp, _dp, _dp]
            lib.gdno_prefill.restype = ctypes.c_int
            lib.gdno_prefill.argtypes = [
                ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                _dp, _dp, _dp, _dp, ctypes.c_int32, _dp, _ip, _dp, ctypes.c_double,
                _dp, _dp, ctypes.c_int32, ctypes.c_double, _dp, _dp, _dp, _dp, ctypes.c_int32,
                ctypes.c_int32]
            lib.gdno_decode.restype = ctypes.c_int
            lib.gdno_decode.argtypes = [
                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                ctypes.c_int32, ctypes.c_int32,
                _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                _dp, ctypes.c_int32, _ip, _ip, _ip, ctypes.c_int32, ctypes.c_double,
                _dp, ctypes.c_int32, ctypes.c_double, _dp]
            lib.gdno_conv1d.restype = ctypes.c_int
            lib.gdno_conv1d.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, _dp, _dp, _dp, ctypes.c_int64, _ip,
                                        _ip, ctypes.c_int32, _dp]
            _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x):
    """Exact widening of a torch tensor / array-like to a dense float64 array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (any dtype, any device)
        import torch
        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu", torch.int64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _p(a, ptype=_dp):
    return None if a is None else a.ctypes.data_as(ptype)


def gate(A_log, dt_bias, a=None, b=None):
    """Returns (log_decay, gamma, beta) as float64 arrays of a's / b's shape.

    a is [..., hv] and b is [..., hv]; either may be None (its outputs are None).
    """
    lib = _load()
    A = _f64(A_log).reshape(-1)
    dt = _f64(dt_bias).reshape(-1)
    hv = A.shape[0]
    a64 = _f64(a)
    b64 = _f64(b)
    shape_a = a64.shape if a64 is not None else None
    shape_b = b64.shape if b64 is not None else None
    g = gam = bet = None
    if a64 is not None:
        n = a64.size // hv
        g = np.empty(n * hv)
        gam = np.empty(n * hv)
        lib.gdno_gate(n, hv, _p(A), _p(dt), _p(a64), None, _p(g), _p(gam), None)
        g = g.reshape(shape_a)
        gam = gam.reshape(shape_a)
    if b64 is not None:
        n = b64.size // hv
        bet = np.empty(n * hv)
        lib.gdno_gate(n, hv, _p(A), _p(dt), None, _p(b64), None, None, _p(bet))
        bet = bet.reshape(shape_b)
    return g, gam, bet


RULES = {"gated_delta": 0, "gated": 1, "delta": 2, "linear": 3}


def prefill(q, k, v, decay, beta, *, decay_is_gamma=False, cu_seqlens=None,
            n_seqs=None, seq_len=None, initial_state=None, scale=1.0,
            out_init=None, nthreads=None, qk_l2norm_eps=None, A_log=None, dt_bias=None,
            a=None, b=None, update_rule="gated_delta", decay_per_key=False):
    """Sequential fp64 prefill.

    q, k: [T, hq, dk]; v: [T, hv, dv]; decay, beta: [T, hv];
    cu_seqlens: [N+1] or None (then n_seqs * seq_len == T);
    initial_state: [N, hv, dv, dk] V-major or None.
    qk_l2norm_eps: None (q, k used as given) or the epsilon of the in-kernel
    L2 norm x / sqrt(sum x^2 + eps).  a [T, hv] with A_log, dt_bias [hv]: the
    fused qwen decay (decay is then ignored); b [T, hv]: beta = sigmoid(b)
    (beta is then ignored).  update_rule: "gated_delta", "gated", "delta" or
    "linear" (the ONNX card's update_rule); rules without the decay ignore
    decay / a, rules without beta ignore beta / b.  decay_per_key: decay is
    [T, hv, dk], one decay per key dimension (given, not fused).
    Returns (out [T, hv, dv], final_state [N, hv, dv, dk]) as float64 arrays.
    out rows no request covers hold out_init (default NaN).
    """
    lib = _load()
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    T, hq, dk = q64.shape
    hv, dv = v64.shape[1], v64.shape[2]
    d64, b64 = _f64(decay), _f64(beta)
    cu = _i64(cu_seqlens)
    if cu is not None:
        n_seqs = cu.shape[0] - 1
        seq_len = 0
    else:
        if n_seqs is None:
            n_seqs = T // seq_len if seq_len else 1
        if seq_len is None:
            seq_len = T // n_seqs if n_seqs else 0
    init = _f64(initial_state)
    if out_init is None:
        out = np.full((T, hv, dv), np.nan)
    else:
        out = _f64(out_init).copy()
    fin = np.zeros((n_seqs, hv, dv, dk))
    fused = [_f64(x) for x in (A_log, dt_bias, a, b)]
    rc = lib.gdno_prefill(n_seqs, T, seq_len, hq, hv, dk, dv, _p(q64), _p(k64), _p(v64),
                          _p(d64), 1 if decay_is_gamma else 0, _p(b64), _p(cu, _ip),
                          _p(init), float(scale), _p(out), _p(fin),
                          nthreads or default_threads(),
                          -1.0 if qk_l2norm_eps is None else float(qk_l2norm_eps),
                          *[_p(x) for x in fused], RULES[update_rule],
                          1 if decay_per_key else 0)
    if rc != 0:
        raise ValueError("gdno_prefill rejected its arguments")
    return out, fin


def decode(q, k, v, A_log, dt_bias, a, b, pool, read_idx, *, write_idx=None,
           scatter_idx=None, disable_state_update=False, scale=1.0, out_init=None,
           nthreads=None, qk_l2norm_eps=None, decay_per_key=None):
    """fp64 slot-pool decode.

    q [B,T,hq,dk]; k [B,T,n,hq,dk]; v [B,T,n,hv,dv]; A_log, dt_bias [hv];
    a [B,T,hv]; b [B,T,n,hv]; pool [P,hv,dv,dk] (not modified: a float64 copy is
    updated and returned); read_idx [B]; write_idx [B] or None;
    scatter_idx [B,T] or None; qk_l2norm_eps: None or the epsilon of the
    in-kernel L2 norm of q and k (use_qk_l2norm); decay_per_key [B,T,hv,dk]
    log-decay per key dimension or None (then the fused gate on a).
    Returns (out [B,T,hv,dv], pool_after [P,hv,dv,dk]) as float64 arrays;
    out rows of skipped batch rows hold out_init (default zeros).
    """
    lib = _load()
    q64, k64, v64 = _f64(q), _f64(k), _f64(v)
    B, T, hq, dk = q64.shape
    n_hh = k64.shape[2]
    hv, dv = v64.shape[3], v64.shape[4]
    pool64 = _f64(pool).copy()
    P = pool64.shape[0]
    out = np.zeros((B, T, hv, dv)) if out_init is None else _f64(out_init).copy()
    rc = lib.gdno_decode(B, T, n_hh, hq, hv, dk, dv, _p(q64), _p(k64), _p(v64),
                         _p(_f64(A_log)), _p(_f64(dt_bias)), _p(_f64(a)), _p(_f64(b)),
                         _p(pool64), P, _p(_i64(read_idx), _ip), _p(_i64(write_idx), _ip),
                         _p(_i64(scatter_idx), _ip), 1 if disable_state_update else 0,
                         float(scale), _p(out), nthreads or default_threads(),
                         -1.0 if qk_l2norm_eps is None else float(qk_l2norm_eps),
                         _p(_f64(decay_per_key)))
    if rc != 0:
        raise ValueError("gdno_decode rejected its arguments")
    return out, pool64


def conv1d(x, weight, conv_state, slot_idx, row_offsets, *, write_state=True, out_init=None):
    """fp64 causal depthwise conv1d with a slot-indexed conv-state pool.

    x [T, conv_dim]; weight [conv_dim, K]; conv_state [max_slots, conv_dim, K-1]
    (not modified: a float64 copy is updated and returned); slot_idx [B];
    row_offsets [B+1].  Returns (out [T, conv_dim], state_after) as float64
    arrays; out rows no sequence covers hold out_init (default NaN).
    """
    lib = _load()
    x64, w64 = _f64(x), _f64(weight)
    T, conv_dim = x64.shape
    K = w64.shape[1]
    st = _f64(conv_state).copy()
    slots, offs = _i64(slot_idx), _i64(row_offsets)
    out = np.full((T, conv_dim), np.nan) if out_init is None else _f64(out_init).copy()
    rc = lib.gdno_conv1d(T, conv_dim, K, slots.shape[0], _p(x64), _p(w64), _p(st), st.shape[0],
                         _p(slots, _ip), _p(offs, _ip), 1 if write_state else 0, _p(out))
    if rc != 0:
        raise ValueError("gdno_conv1d rejected its arguments")
    return out, st
